"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake (a dropped term, a wrong sign or index,
a transposed operand, an off-by-one mask) in a temporary copy of the oracle's
C source, builds it, points the oracle binding at it and runs the pin tests:
at least one pin must fail.  The real oracle is restored afterwards.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as oracle_mod
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "osattn_oracle.c")

MUTATIONS = {
    "causal_excludes_diagonal": ("if (causal && b > i + 1) b = i + 1;",
                                 "if (causal && b > i) b = i;"),
    "varlen_boundary_off_by_one": ("i < cu_seqlens[s + 1]", "i <= cu_seqlens[s + 1]"),
    "dot_drops_last_term": ("for (int d = 0; d < D; ++d) acc += a[d] * b[d];",
                            "for (int d = 0; d < D - 1; ++d) acc += a[d] * b[d];"),
    "scale_missing_in_fwd": ("s[j] = dot(kh + j * D, qi, D) * scale;",
                             "s[j] = dot(kh + j * D, qi, D);"),
    "normaliser_unshifted": ("for (int64_t j = lo; j < hi; ++j) sum += exp(s[j] - mx);",
                             "for (int64_t j = lo; j < hi; ++j) sum += exp(s[j]);"),
    "delta_sign": ("dSi[j] = Pi[j] * (dSi[j] - delta);", "dSi[j] = Pi[j] * (dSi[j] + delta);"),
    "dq_scale_dropped": ("dqh[i * D + d] = scale * acc;", "dqh[i * D + d] = acc;"),
    "dk_scale_dropped": ("for (int d = 0; d < D; ++d) dkj[d] *= scale;", ""),
    "dv_uses_dS": ("dvj[d] += p * doh[i * D + d];", "dvj[d] += ds * doh[i * D + d];"),
    "dk_uses_do": ("dkj[d] += ds * qh[i * D + d];", "dkj[d] += ds * doh[i * D + d];"),
    "dq_uses_v": ("acc += dSi[j] * kh[j * D + d];", "acc += dSi[j] * vh[j * D + d];"),
    # tile pruning
    "prune_strict_comparison": ("adm[t] = (unsigned char)(m_tile >= thr);",
                                "adm[t] = (unsigned char)(m_tile > thr);"),
    "prune_log_base_2": ("const double log_rho = log(rho);", "const double log_rho = log2(rho);"),
    "prune_threshold_sign": ("const double thr = m_run + log_rho;", "const double thr = m_run - log_rho;"),
    "prune_tile_max_first_row_only": (
        "for (int64_t i = i0; i < i1; ++i)\n                    for (int64_t j = j0; j < j1; ++j)",
        "for (int64_t i = i0; i < i0 + 1; ++i)\n                    for (int64_t j = j0; j < j1; ++j)"),
    "prune_running_max_never_moves": ("if (adm[t] && m_tile > m_run) m_run = m_tile;", ""),
    # CSR segment softmax
    "csr_segment_end_inclusive": ("for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) sum += exp(sh[e] - mx);",
                                  "for (int64_t e = row_ptr[i]; e <= row_ptr[i + 1]; ++e) sum += exp(sh[e] - mx);"),
    "csr_gathers_destination_row": ("oi[d] += p * vh[(int64_t)col_idx[e] * D + d];",
                                    "oi[d] += p * vh[i * D + d];"),
    "csr_head_offset_dropped": ("const double *sh = scores + h * nnz;", "const double *sh = scores;"),
    "prune_tile_overlaps_next": ("const int64_t j0 = t * bc, j1 = (j0 + bc < n_k) ? j0 + bc : n_k;",
                                 "const int64_t j0 = t * bc, j1 = (j0 + bc + 1 < n_k) ? j0 + bc + 1 : n_k;"),
}

PIN_CALLS = [
    lambda o: [pins.test_golden_forward(o, c) for c in pins.load_golden()["forward"]],
    lambda o: [pins.test_golden_backward(o, c) for c in pins.load_golden()["backward"]],
    lambda o: pins.test_brute_force_dense(o, 7, 4, 3),
    lambda o: pins.test_brute_force_causal(o, 6, 4),
    lambda o: pins.test_brute_force_varlen(o, True),
    lambda o: pins.test_brute_force_varlen(o, False),
    lambda o: pins.test_sdpa_dense(o, 33, 129, 64),
    lambda o: pins.test_causal_row0_is_v0_exactly(o),
    lambda o: pins.test_backward_autograd_sdpa(o, False),
    lambda o: pins.test_backward_autograd_sdpa(o, True),
    lambda o: pins.test_backward_identities(o, True, [0, 10, 11, 40]),
    lambda o: [pins.test_pruning_golden(o, c) for c in pins.load_pruning()["cases"]],
    lambda o: pins.test_pruning_tiny_rho_is_exact(o, 300, 200, 128, 128),
    lambda o: pins.test_csr_relation_equals_attention(o, True, [0, 5, 6, 19, 40]),
    lambda o: pins.test_csr_empty_rows_and_duplicate_edges(o),
]


def _build(src_text, tmpdir):
    c = os.path.join(tmpdir, "mut.c")
    so = os.path.join(tmpdir, "libmut.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", so,
                           c, "-lm"])
    return so


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation anchor not found uniquely: " + name
    so = _build(text.replace(old, new), str(tmp_path))
    saved_lib, saved_path = oracle_mod._lib, oracle_mod._LIB_PATH
    try:
        oracle_mod._lib = None
        oracle_mod._LIB_PATH = so
        oracle_mod._load()
        caught = 0
        for call in PIN_CALLS:
            try:
                with np.errstate(all="ignore"):
                    call(oracle_mod)
            except (AssertionError, ValueError):
                caught += 1
        assert caught > 0, "no pin caught the planted mistake " + name
    finally:
        oracle_mod._lib, oracle_mod._LIB_PATH = saved_lib, saved_path
