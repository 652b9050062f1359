"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these re-types the oracle's formula.  They use hand-derived closed forms
(tests/golden), a separately written pure-Python brute force with exact
summation on tiny inputs, torch's CPU f64 scaled_dot_product_attention and its
autograd (the library routine the TIGA-lang examples test against), invariants
of softmax attention, and central finite differences for the gradient.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- brute force
def brute_fwd(q, k, v, scale, admitted):
    """Pure-Python attention with exact (fsum) summation; admitted(i) -> keys."""
    H, n_q, D = q.shape
    o = np.zeros_like(q)
    m = np.zeros((H, n_q))
    l = np.zeros((H, n_q))
    for h in range(H):
        for i in range(n_q):
            js = list(admitted(i))
            s = [math.fsum(float(k[h, j, d]) * float(q[h, i, d]) for d in range(D)) * scale
                 for j in js]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = math.fsum(w)
            for d in range(D):
                o[h, i, d] = math.fsum(w[t] * float(v[h, j, d]) for t, j in enumerate(js)) / tot
            m[h, i] = mx
            l[h, i] = tot
    return o, m, l


def dense_keys(n_k):
    return lambda i: range(n_k)


def causal_keys():
    return lambda i: range(i + 1)


def varlen_keys(cu, causal):
    def f(i):
        b = max(t for t in range(len(cu) - 1) if cu[t] <= i)
        hi = min(cu[b + 1], i + 1) if causal else cu[b + 1]
        return range(cu[b], hi)
    return f


def sdpa_ref(q, k, v, scale, causal=False, mask=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=causal, scale=scale)
    return out.numpy()


def block_diag_mask(cu, causal):
    n = cu[-1]
    mask = np.zeros((n, n), dtype=bool)
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        blk = np.ones((e - a, e - a), dtype=bool)
        mask[a:e, a:e] = np.tril(blk) if causal else blk
    return mask


# ------------------------------------------------------------------- golden
def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", load_golden()["forward"], ids=lambda c: c["name"])
def test_golden_forward(oracle, case):
    q, k, v = (np.array(case[x], dtype=np.float64) for x in "qkv")
    rel = case["relation"]
    o, m, l = oracle.attn_fwd(q, k, v, case["scale"], causal=rel != "dense",
                              cu_seqlens=case.get("cu_seqlens"))
    np.testing.assert_allclose(o, np.array(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, np.array(case["m"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(case["l"]), rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", load_golden()["backward"], ids=lambda c: c["name"])
def test_golden_backward(oracle, case):
    q, k, v, do = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v", "do"))
    dq, dk, dv, m, l, delta = oracle.attn_bwd(q, k, v, do, case["scale"])
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(got, np.array(case[name]), rtol=0, atol=1e-12, err_msg=name)
    o, _, _ = oracle.attn_fwd(q, k, v, case["scale"])
    np.testing.assert_allclose(o, np.array(case["o"]), rtol=0, atol=1e-12)


# -------------------------------------------------------- brute force, tiny N
@pytest.mark.parametrize("n_q,n_k,D", [(1, 1, 1), (3, 5, 2), (7, 4, 3), (8, 8, 5)])
def test_brute_force_dense(oracle, n_q, n_k, D):
    q, k, v = rand((2, n_q, D), 1), rand((2, n_k, D), 2), rand((2, n_k, D), 3)
    scale = 0.37
    o, m, l = oracle.attn_fwd(q, k, v, scale)
    bo, bm, bl = brute_fwd(q, k, v, scale, dense_keys(n_k))
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(m, bm, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, bl, rtol=1e-13)


@pytest.mark.parametrize("n,D", [(1, 3), (6, 4), (9, 2)])
def test_brute_force_causal(oracle, n, D):
    q, k, v = rand((2, n, D), 4), rand((2, n, D), 5), rand((2, n, D), 6)
    o, m, l = oracle.attn_fwd(q, k, v, 0.8, causal=True)
    bo, bm, bl = brute_fwd(q, k, v, 0.8, causal_keys())
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(m, bm, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, bl, rtol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_varlen(oracle, causal):
    cu = [0, 3, 4, 9, 11]
    n, D = cu[-1], 3
    q, k, v = rand((2, n, D), 7), rand((2, n, D), 8), rand((2, n, D), 9)
    o, m, l = oracle.attn_fwd(q, k, v, 0.5, causal=causal, cu_seqlens=cu)
    bo, bm, bl = brute_fwd(q, k, v, 0.5, varlen_keys(cu, causal))
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(m, bm, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, bl, rtol=1e-13)


# ---------------------------------------------------- library routine (SDPA)
@pytest.mark.parametrize("n_q,n_k,D", [(64, 64, 16), (100, 37, 8), (33, 129, 64)])
def test_sdpa_dense(oracle, n_q, n_k, D):
    q, k, v = rand((3, n_q, D), 10), rand((3, n_k, D), 11), rand((3, n_k, D), 12)
    scale = D ** -0.5
    o, m, l = oracle.attn_fwd(q, k, v, scale)
    np.testing.assert_allclose(o, sdpa_ref(q, k, v, scale), rtol=0, atol=1e-12)
    # m + log l is the log-sum-exp of the scores
    s = np.einsum("hid,hjd->hij", q, k) * scale
    lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
    np.testing.assert_allclose(m + np.log(l), lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, s.max(-1), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,D", [(65, 16), (128, 64), (200, 8)])
def test_sdpa_causal(oracle, n, D):
    q, k, v = rand((2, n, D), 13), rand((2, n, D), 14), rand((2, n, D), 15)
    scale = D ** -0.5
    o, m, l = oracle.attn_fwd(q, k, v, scale, causal=True)
    np.testing.assert_allclose(o, sdpa_ref(q, k, v, scale, causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_sdpa_varlen(oracle, causal):
    cu = [0, 37, 38, 138, 201]
    n, D = cu[-1], 16
    q, k, v = rand((2, n, D), 16), rand((2, n, D), 17), rand((2, n, D), 18)
    o, _, _ = oracle.attn_fwd(q, k, v, 0.25, causal=causal, cu_seqlens=cu)
    ref = sdpa_ref(q, k, v, 0.25, mask=block_diag_mask(cu, causal))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- invariants
def test_zero_query_gives_mean_of_values(oracle):
    n, D = 40, 8
    q = np.zeros((2, n, D))
    k, v = rand((2, n, D), 19), rand((2, n, D), 20)
    o, m, l = oracle.attn_fwd(q, k, v, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(1, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_array_equal(m, 0.0)
    np.testing.assert_array_equal(l, float(n))
    oc, mc, lc = oracle.attn_fwd(q, k, v, 0.3, causal=True)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, n + 1)[None, :, None]
    np.testing.assert_allclose(oc, prefix_mean, atol=1e-14)
    np.testing.assert_array_equal(lc, np.broadcast_to(np.arange(1, n + 1, dtype=float), lc.shape))


def test_causal_row0_is_v0_exactly(oracle):
    q, k, v = rand((3, 50, 16), 21), rand((3, 50, 16), 22), rand((3, 50, 16), 23)
    o, m, l = oracle.attn_fwd(q, k, v, 0.25, causal=True)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    np.testing.assert_array_equal(l[:, 0], 1.0)
    np.testing.assert_allclose(m[:, 0], np.einsum("hd,hd->h", q[:, 0], k[:, 0]) * 0.25, atol=1e-14)


def test_varlen_first_rows_and_length_one(oracle):
    cu = [0, 1, 5, 6, 20]
    q, k, v = rand((2, 20, 8), 24), rand((2, 20, 8), 25), rand((2, 20, 8), 26)
    o, _, l = oracle.attn_fwd(q, k, v, 0.5, causal=True, cu_seqlens=cu)
    for b in range(len(cu) - 1):
        np.testing.assert_array_equal(o[:, cu[b]], v[:, cu[b]])
        np.testing.assert_array_equal(l[:, cu[b]], 1.0)


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_is_concatenation_of_sequences(oracle, causal):
    cu = [0, 13, 14, 50, 77]
    q, k, v = rand((2, 77, 8), 27), rand((2, 77, 8), 28), rand((2, 77, 8), 29)
    o, m, l = oracle.attn_fwd(q, k, v, 0.4, causal=causal, cu_seqlens=cu)
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        ob, mb, lb = oracle.attn_fwd(q[:, a:e], k[:, a:e], v[:, a:e], 0.4, causal=causal)
        np.testing.assert_array_equal(o[:, a:e], ob)
        np.testing.assert_array_equal(m[:, a:e], mb)
        np.testing.assert_array_equal(l[:, a:e], lb)


def test_key_shift_invariance(oracle):
    q, k, v = rand((2, 30, 8), 30), rand((2, 45, 8), 31), rand((2, 45, 8), 32)
    c = rand((2, 1, 8), 33)
    scale = 0.35
    o, m, l = oracle.attn_fwd(q, k, v, scale)
    o2, m2, l2 = oracle.attn_fwd(q, k + c, v, scale)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(l2, l, rtol=1e-12)
    np.testing.assert_allclose(m2, m + scale * np.einsum("hid,hd->hi", q, c[:, 0]), atol=1e-12)


def test_convex_hull_and_linearity_in_v(oracle):
    q, k = rand((2, 30, 8), 34), rand((2, 60, 8), 35)
    v1, v2 = rand((2, 60, 8), 36), rand((2, 60, 8), 37)
    o1, _, _ = oracle.attn_fwd(q, k, v1, 0.5, causal=False)
    assert np.all(o1 <= v1.max(1, keepdims=True) + 1e-14)
    assert np.all(o1 >= v1.min(1, keepdims=True) - 1e-14)
    o2, _, _ = oracle.attn_fwd(q, k, v2, 0.5)
    o12, _, _ = oracle.attn_fwd(q, k, 2.0 * v1 - 3.0 * v2, 0.5)
    np.testing.assert_allclose(o12, 2.0 * o1 - 3.0 * o2, atol=1e-12)


@pytest.mark.parametrize("n", [63, 64, 65])
def test_masked_keys_contribute_nothing(oracle, n):
    """Keys outside a row's relation leave its output unchanged (guarded tail)."""
    D = 8
    q, k, v = rand((1, n, D), 38), rand((1, n, D), 39), rand((1, n, D), 40)
    o, m, l = oracle.attn_fwd(q, k, v, 0.5, causal=True)
    # Huge keys and values appended past the end (and masked by causality
    # for every earlier row) must not leak into rows < n.
    k2 = np.concatenate([k, 1e3 * np.ones((1, 5, D))], axis=1)
    v2 = np.concatenate([v, 1e6 * np.ones((1, 5, D))], axis=1)
    q2 = np.concatenate([q, rand((1, 5, D), 41)], axis=1)
    o2, m2, l2 = oracle.attn_fwd(q2, k2, v2, 0.5, causal=True)
    np.testing.assert_array_equal(o2[:, :n], o)
    np.testing.assert_array_equal(m2[:, :n], m)
    np.testing.assert_array_equal(l2[:, :n], l)


def test_row_subset_matches_full(oracle):
    q, k, v = rand((3, 40, 8), 42), rand((3, 40, 8), 43), rand((3, 40, 8), 44)
    o, m, l = oracle.attn_fwd(q, k, v, 0.5, causal=True)
    rows = np.array([0, 39, 41, 80, 119, 7])
    os_, ms, ls = oracle.attn_fwd(q, k, v, 0.5, causal=True, rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(ms, m.reshape(-1)[rows])
    np.testing.assert_array_equal(ls, l.reshape(-1)[rows])


def online_block_model(q, k, v, scale, B):
    """The block recurrence of OCANNL 'Module Ir.Online_softmax' (fourth bullet)
    for one head, dense, in f64: per key block the new max, the rescale factor,
    the exponentials, the rescaled sum and the rescaled numerator; O = U / l.
    It documents that the recurrence the GPU runs equals the definition."""
    n_q, D = q.shape
    n_k = k.shape[0]
    o = np.zeros((n_q, D))
    for i in range(n_q):
        m, l, U = -math.inf, 0.0, np.zeros(D)
        for c0 in range(0, n_k, B):
            s = np.array([float(k[j] @ q[i]) * scale if j < n_k else -math.inf
                          for j in range(c0, c0 + B)])
            m_new = max(m, float(s.max()))
            alpha = math.exp(m - m_new)
            p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            vb = np.zeros((B, D))
            vb[: min(B, n_k - c0)] = v[c0:c0 + B]
            U = alpha * U + p @ vb
            m = m_new
        o[i] = U / l
    return o


@pytest.mark.parametrize("B", [1, 7, 64])
def test_online_recurrence_equals_definition(oracle, B):
    q, k, v = rand((1, 9, 6), 45), rand((1, 50, 6), 46), rand((1, 50, 6), 47)
    o, _, _ = oracle.attn_fwd(q, k, v, 0.7)
    np.testing.assert_allclose(online_block_model(q[0], k[0], v[0], 0.7, B), o[0], atol=1e-12)


# ------------------------------------------------------------------ backward
def loss_of(oracle, q, k, v, do, scale, causal, cu):
    o, _, _ = oracle.attn_fwd(q, k, v, scale, causal=causal, cu_seqlens=cu)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal,cu", [(False, None), (True, None), (True, [0, 2, 6]),
                                       (False, [0, 4, 6])])
def test_backward_finite_differences(oracle, causal, cu):
    n, D = 6, 3
    q, k, v, do = (rand((2, n, D), s) for s in (48, 49, 50, 51))
    scale = 0.6
    dq, dk, dv, _, _, _ = oracle.attn_bwd(q, k, v, do, scale, causal=causal, cu_seqlens=cu)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss_of(oracle, args["q"], args["k"], args["v"], do, scale, causal, cu)
            args[name] = xm
            lm = loss_of(oracle, args["q"], args["k"], args["v"], do, scale, causal, cu)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_autograd_sdpa(oracle, causal):
    n_q = n_k = 70
    D = 16
    q, k, v, do = rand((2, n_q, D), 52), rand((2, n_k, D), 53), rand((2, n_k, D), 54), \
        rand((2, n_q, D), 55)
    scale = D ** -0.5
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale)
    out.backward(torch.from_numpy(do))
    dq, dk, dv, _, _, _ = oracle.attn_bwd(q, k, v, do, scale, causal=causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_backward_rectangular_autograd(oracle):
    q, k, v, do = rand((1, 50, 8), 56), rand((1, 20, 8), 57), rand((1, 20, 8), 58), \
        rand((1, 50, 8), 59)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3).backward(
        torch.from_numpy(do))
    dq, dk, dv, _, _, _ = oracle.attn_bwd(q, k, v, do, 0.3)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal,cu", [(False, None), (True, None), (True, [0, 10, 11, 40])])
def test_backward_identities(oracle, causal, cu):
    n, D = 40, 8
    q, k, v, do = (rand((2, n, D), s) for s in (60, 61, 62, 63))
    dq, dk, dv, m, l, delta = oracle.attn_bwd(q, k, v, do, 0.5, causal=causal, cu_seqlens=cu)
    o, mo, lo = oracle.attn_fwd(q, k, v, 0.5, causal=causal, cu_seqlens=cu)
    # the per-row shortcut: delta_i = <dO_i, O_i>
    np.testing.assert_allclose(delta, np.sum(do * o, -1), atol=1e-12)
    np.testing.assert_allclose(m, mo, atol=0)
    np.testing.assert_allclose(l, lo, rtol=1e-15)
    segs = [(0, n)] if cu is None else list(zip(cu[:-1], cu[1:]))
    for a, e in segs:
        # shift invariance of each row's softmax => sum_j dK_j = 0 per segment
        np.testing.assert_allclose(dk[:, a:e].sum(1), 0.0, atol=1e-12)
        # rows of P sum to one => sum_j dV_j = sum_i dO_i per segment
        np.testing.assert_allclose(dv[:, a:e].sum(1), do[:, a:e].sum(1), atol=1e-12)


def test_backward_degenerate(oracle):
    n, D = 12, 4
    k, v, do = rand((1, n, D), 64), rand((1, n, D), 65), rand((1, n, D), 66)
    dq, dk, dv, *_ = oracle.attn_bwd(np.zeros((1, n, D)), k, v, do, 0.5)
    np.testing.assert_array_equal(dk, 0.0)
    q = rand((1, n, D), 67)
    dq, dk, dv, *_ = oracle.attn_bwd(q, k, v, np.zeros((1, n, D)), 0.5, causal=True)
    for g in (dq, dk, dv):
        np.testing.assert_array_equal(g, 0.0)


def test_invalid_arguments_rejected(oracle):
    q = rand((1, 4, 2), 68)
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, rand((1, 5, 2), 69), rand((1, 5, 2), 70), 1.0, causal=True)
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, q, q, 1.0, cu_seqlens=[1, 4])
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, q, q, 1.0, cu_seqlens=[0, 3, 2, 4])


def test_thread_count_does_not_change_results(oracle):
    """Every output element has one fixed summation order."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import numpy as np, oracle;"
            "r = np.random.default_rng(0); q = r.standard_normal((2, 97, 8));"
            "o, m, l = oracle.attn_fwd(q, q, q, 0.5, causal=True);"
            "sys.stdout.write(o.tobytes().hex()[:4000] + l.tobytes().hex())" %
            os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    outs = []
    for t in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env))
    assert outs[0] == outs[1]


# ------------------------------------------------------------------- tile pruning
PRUNE_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tile_pruning_cases.json")


def load_pruning():
    with open(PRUNE_GOLDEN) as f:
        return json.load(f)


def test_pruning_page_ratio():
    # The page prints exp(1 - 10) as about 0.00012.
    r = load_pruning()["page_ratio"]
    assert abs(math.exp(1 - 10) - r["printed"]) < 5e-6 and r["value"] == math.exp(-9)


@pytest.mark.parametrize("case", load_pruning()["cases"], ids=lambda c: c["name"])
def test_pruning_golden(oracle, case):
    q, k, v = (np.array(case[x], dtype=np.float64) for x in "qkv")
    o, m, l, admit, _ = oracle.attn_fwd_pruned(q, k, v, case["scale"], case["rho"], case["br"],
                                               case["bc"])
    assert admit.tolist() == case["admit"]
    np.testing.assert_allclose(o, np.array(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, np.array(case["m"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(case["l"]), rtol=1e-12, atol=0)


@pytest.mark.parametrize("n_q,n_k,br,bc", [(300, 200, 128, 128), (130, 257, 64, 32)])
def test_pruning_tiny_rho_is_exact(oracle, n_q, n_k, br, bc):
    # rho -> 0 admits every tile: the exact dense attention.
    q, k, v = rand((2, n_q, 16), 1), rand((2, n_k, 16), 2), rand((2, n_k, 16), 3)
    o, m, l, admit, _ = oracle.attn_fwd_pruned(q, k, v, 0.25, 1e-300, br, bc)
    ro, rm, rl = oracle.attn_fwd(q, k, v, 0.25)
    assert admit.all()
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, rm, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=1e-12, atol=0)


def test_pruning_rejects_bad_rho(oracle):
    q = rand((1, 4, 8), 1)
    for rho in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.attn_fwd_pruned(q, q, q, 0.5, rho, 2, 2)


# ------------------------------------------------------------ CSR segment softmax
def relation_csr(n_q, n_k, causal=False, cu=None):
    """CSR (row_ptr, col_idx) of the dense / causal / varlen relations."""
    rows = []
    for i in range(n_q):
        lo, hi = 0, n_k
        if cu is not None:
            for a, b in zip(cu[:-1], cu[1:]):
                if a <= i < b:
                    lo, hi = a, b
        if causal:
            hi = min(hi, i + 1)
        rows.append(list(range(lo, hi)))
    row_ptr = np.cumsum([0] + [len(r) for r in rows])
    col_idx = np.array([j for r in rows for j in r], dtype=np.int64)
    return row_ptr, col_idx


def edge_scores(q, k, scale, row_ptr, col_idx):
    """Scores of every edge, s_e = scale <q_i, k_col(e)>, as a (H, nnz) field."""
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    return np.einsum("hed,hed->he", q[:, rows], k[:, col_idx]) * scale


@pytest.mark.parametrize("causal,cu", [(False, None), (True, None), (True, [0, 5, 6, 19, 40]),
                                       (False, [0, 7, 7, 30, 40])])
def test_csr_relation_equals_attention(oracle, causal, cu):
    # The dense, causal and varlen relations written as CSR with q.k scores
    # give exactly the attention definition.
    n = 40
    q, k, v = rand((2, n, 8), 11), rand((2, n, 8), 12), rand((2, n, 8), 13)
    row_ptr, col_idx = relation_csr(n, n, causal, cu)
    o, m, l = oracle.csr_softmax(row_ptr, col_idx, edge_scores(q, k, 0.4, row_ptr, col_idx), v)
    ro, rm, rl = oracle.attn_fwd(q, k, v, 0.4, causal=causal, cu_seqlens=cu)
    empty = np.diff(row_ptr) == 0
    np.testing.assert_allclose(o[:, ~empty], ro[:, ~empty], rtol=0, atol=1e-12)
    np.testing.assert_allclose(m[:, ~empty], rm[:, ~empty], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l[:, ~empty], rl[:, ~empty], rtol=1e-12, atol=0)


def test_csr_rectangular_dense_equals_attention(oracle):
    q, k, v = rand((1, 9, 4), 21), rand((1, 30, 4), 22), rand((1, 30, 4), 23)
    row_ptr, col_idx = relation_csr(9, 30)
    o, m, l = oracle.csr_softmax(row_ptr, col_idx, edge_scores(q, k, 0.5, row_ptr, col_idx), v)
    ro, rm, rl = oracle.attn_fwd(q, k, v, 0.5)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", load_golden()["forward"], ids=lambda c: c["name"])
def test_csr_golden(oracle, case):
    # The hand-derived forward cases, with their scores given as an edge field.
    q, k, v = (np.array(case[x], dtype=np.float64) for x in "qkv")
    rel = case["relation"]
    n_q, n_k = q.shape[1], k.shape[1]
    row_ptr, col_idx = relation_csr(n_q, n_k, causal=rel != "dense", cu=case.get("cu_seqlens"))
    o, m, l = oracle.csr_softmax(row_ptr, col_idx, edge_scores(q, k, case["scale"], row_ptr, col_idx), v)
    np.testing.assert_allclose(o, np.array(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, np.array(case["m"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(case["l"]), rtol=1e-12, atol=0)


def test_csr_empty_rows_and_duplicate_edges(oracle):
    # Row 0 has no edges: o = 0, m = -inf, l = 0.  Row 1 lists source 2 twice
    # with score 0 and source 0 once with score ln 2: weights 1 : 1 : 2, which
    # is the same as one edge to source 2 with score ln 2 (1 : 1 of mass 2).
    v = np.array([[[8.0], [100.0], [2.0]]])
    o, m, l = oracle.csr_softmax([0, 0, 3], [2, 2, 0], np.array([[0.0, 0.0, math.log(2)]]), v)
    assert o[0, 0, 0] == 0.0 and m[0, 0] == -math.inf and l[0, 0] == 0.0
    assert abs(o[0, 1, 0] - (2 + 2 + 2 * 8) / 4) < 1e-12
    assert abs(m[0, 1] - math.log(2)) < 1e-15 and abs(l[0, 1] - 2.0) < 1e-12


def test_csr_edge_order_is_free(oracle):
    rng = np.random.default_rng(5)
    deg = rng.integers(0, 9, size=50)
    row_ptr = np.concatenate([[0], np.cumsum(deg)])
    col_idx = rng.integers(0, 30, size=row_ptr[-1])
    s = rng.standard_normal((2, row_ptr[-1]))
    v = rng.standard_normal((2, 30, 5))
    perm = np.concatenate([rng.permutation(np.arange(a, b)) for a, b in zip(row_ptr[:-1], row_ptr[1:])]
                          ).astype(np.int64)
    a = oracle.csr_softmax(row_ptr, col_idx, s, v)
    b = oracle.csr_softmax(row_ptr, col_idx[perm], s[:, perm], v)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_csr_rejects_malformed(oracle):
    v = np.zeros((1, 3, 2))
    for rp, ci in (([1, 2], [0]), ([0, 2, 1], [0, 1]), ([0, 1], [3]), ([0, 1], [-1])):
        with pytest.raises(ValueError):
            oracle.csr_softmax(rp, ci, np.zeros((1, max(rp[-1], 0))), v)
