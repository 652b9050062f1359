"""CPU oracle for exact scaled-dot-product attention (f64) -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
does, and shares no code with it: the oracle is the plain two-pass softmax
definition and its chain-rule gradient written in C (``osattn_oracle.c``),
loaded here through ctypes.

Definitions followed (cited per function in the C file):
  * forward: TIGA-lang "Attention and dense relations", the equations of the
    full, causal and varlen causal sections;
  * backward: OCANNL "Module Ir.Online_softmax", the composed-backward bullet,
    in Jacobian form (no D = rowsum(dO * O) shortcut);
  * tile-pruned forward: TIGA-lang "Tile-pruned sparse attention", the
    admission rule on (query block, key tile) pairs;
  * CSR segment softmax over given edge scores: the relation view of the
    TIGA-lang attention pages (each destination row's softmax over its edges).

Inputs are float arrays laid out (H, N, D); they are upcast exactly to f64.
bf16 inputs must be passed already widened to f32 (exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "osattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE f64: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.oracle_attn_fwd_rows.argtypes = [
            ctypes.c_int, i64, i64, ctypes.c_int, dp, dp, dp, ctypes.c_double,
            ctypes.c_int, ip, ctypes.c_int, lp, i64, dp, dp, dp]
        lib.oracle_attn_fwd_rows.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [
            ctypes.c_int, i64, i64, ctypes.c_int, dp, dp, dp, dp, ctypes.c_double,
            ctypes.c_int, ip, ctypes.c_int, dp, dp, dp, dp, dp, dp]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_fwd_pruned.argtypes = [
            ctypes.c_int, i64, i64, ctypes.c_int, dp, dp, dp, ctypes.c_double, ctypes.c_double,
            ctypes.c_int, ctypes.c_int, dp, dp, dp, ctypes.POINTER(ctypes.c_uint8), dp]
        lib.oracle_attn_fwd_pruned.restype = ctypes.c_int
        lib.oracle_csr_softmax.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, ip, ip, dp, dp,
                                           dp, dp, dp]
        lib.oracle_csr_softmax.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, 0, ctypes.POINTER(ctypes.c_int32)()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    return cu, len(cu) - 1, _ptr(cu, ctypes.c_int32)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def attn_fwd(q, k, v, scale, causal=False, cu_seqlens=None, rows=None):
    """Exact attention forward.

    q: (H, n_q, D); k, v: (H, n_k, D).  Returns (o, m, l): o (H, n_q, D),
    m and l (H, n_q), all f64.  With ``rows`` (an int array of flat indices
    h * n_q + i), only those rows are computed and the results have a leading
    dimension len(rows) instead.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, n_q, D = q.shape
    n_k = k.shape[1]
    assert k.shape == (H, n_k, D) and v.shape == (H, n_k, D)
    cu, ns, cup = _cu(cu_seqlens)
    if rows is None:
        rows_arr, n_rows, rp = None, H * n_q, ctypes.POINTER(ctypes.c_int64)()
        o = np.empty((H, n_q, D))
        m = np.empty((H, n_q))
        l = np.empty((H, n_q))
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows, rp = len(rows_arr), _ptr(rows_arr, ctypes.c_int64)
        o = np.empty((n_rows, D))
        m = np.empty(n_rows)
        l = np.empty(n_rows)
    st = _load().oracle_attn_fwd_rows(
        H, n_q, n_k, D, _ptr(q), _ptr(k), _ptr(v), float(scale), int(bool(causal)),
        cup, ns, rp, n_rows, _ptr(o), _ptr(m), _ptr(l))
    if st != 0:
        raise ValueError("oracle_attn_fwd_rows failed with status %d" % st)
    return o, m, l


def attn_bwd(q, k, v, dout, scale, causal=False, cu_seqlens=None):
    """Exact attention backward in chain-rule form.

    Returns (dq, dk, dv, m, l, delta) in f64, where delta_i = sum_j P_ij dP_ij.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    H, n_q, D = q.shape
    n_k = k.shape[1]
    assert dout.shape == q.shape
    cu, ns, cup = _cu(cu_seqlens)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    m = np.empty((H, n_q))
    l = np.empty((H, n_q))
    delta = np.empty((H, n_q))
    st = _load().oracle_attn_bwd(
        H, n_q, n_k, D, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), float(scale),
        int(bool(causal)), cup, ns, _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(m), _ptr(l), _ptr(delta))
    if st != 0:
        raise ValueError("oracle_attn_bwd failed with status %d" % st)
    return dq, dk, dv, m, l, delta


def attn_fwd_pruned(q, k, v, scale, rho, br=128, bc=128):
    """Tile-pruned dense forward (an approximation; see the C source).

    Query blocks of ``br`` rows, key tiles of ``bc`` keys, admission
    m_tile >= m_run + ln(rho) per (head, query block).  Returns
    (o, m, l, admit, min_margin): o (H, n_q, D), m and l (H, n_q) in f64,
    admit (H, ceil(n_q / br), ceil(n_k / bc)) uint8, and the smallest distance
    of a tile maximum from its threshold over the decisions taken against a
    finite running maximum.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, n_q, D = q.shape
    n_k = k.shape[1]
    assert k.shape == (H, n_k, D) and v.shape == (H, n_k, D)
    o = np.empty((H, n_q, D))
    m = np.empty((H, n_q))
    l = np.empty((H, n_q))
    admit = np.zeros((H, (n_q + br - 1) // br, (n_k + bc - 1) // bc), dtype=np.uint8)
    margin = ctypes.c_double(0.0)
    st = _load().oracle_attn_fwd_pruned(
        H, n_q, n_k, D, _ptr(q), _ptr(k), _ptr(v), float(scale), float(rho), int(br), int(bc),
        _ptr(o), _ptr(m), _ptr(l), _ptr(admit, ctypes.c_uint8), ctypes.byref(margin))
    if st != 0:
        raise ValueError("oracle_attn_fwd_pruned failed with status %d" % st)
    return o, m, l, admit, margin.value


def csr_softmax(row_ptr, col_idx, scores, v):
    """Segment softmax over CSR rows with given edge scores.

    row_ptr (n_dst + 1,) and col_idx (nnz,) int; scores (H, nnz); v (H, n_src, D).
    Returns (o, m, l) in f64: o (H, n_dst, D), m and l (H, n_dst); empty rows
    give o = 0, m = -inf, l = 0.
    """
    rp = np.ascontiguousarray(np.asarray(row_ptr, dtype=np.int32))
    ci = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int32))
    scores, v = _f64(scores), _f64(v)
    H, n_src, D = v.shape
    n_dst = len(rp) - 1
    assert scores.shape == (H, int(rp[-1]))
    o = np.empty((H, n_dst, D))
    m = np.empty((H, n_dst))
    l = np.empty((H, n_dst))
    ci_p = _ptr(ci, ctypes.c_int32) if len(ci) else ctypes.POINTER(ctypes.c_int32)()
    st = _load().oracle_csr_softmax(H, n_dst, n_src, D, _ptr(rp, ctypes.c_int32), ci_p,
                                    _ptr(scores), _ptr(v), _ptr(o), _ptr(m), _ptr(l))
    if st != 0:
        raise ValueError("oracle_csr_softmax failed with status %d" % st)
    return o, m, l
