"""Helpers for the GPU parity tests: upload seeded inputs, compare to the oracle."""
import numpy as np
import torch

# Forward max-abs-error bounds against the f64 oracle, by stored input dtype.
# Gradients use the same bound scaled by max |reference| per tensor.
TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 1e-2}
# Row statistics are f32 accumulations of exactly representable products:
# |m - m_ref| <= STAT_TOL * max(1, |m_ref|), |l / l_ref - 1| <= STAT_TOL.
STAT_TOL = 1e-4

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored host array (bf16 as uint16 bit patterns) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to("cuda")


def cu_dev(cu):
    return None if cu is None else torch.tensor(np.asarray(cu), dtype=torch.int32, device="cuda")


def assert_fwd_close(o, m, l, ro, rm, rl, dtype, what=""):
    o = np.asarray(o, dtype=np.float64)
    err = np.max(np.abs(o - ro)) if o.size else 0.0
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    assert err <= TOL[dtype], "%s: max |O - O_ref| = %.3g > %.1g" % (what, err, TOL[dtype])
    merr = np.max(np.abs(np.asarray(m, np.float64) - rm) / np.maximum(1.0, np.abs(rm)))
    lerr = np.max(np.abs(np.asarray(l, np.float64) / rl - 1.0))
    assert merr <= STAT_TOL, "%s: m error %.3g" % (what, merr)
    assert lerr <= STAT_TOL, "%s: l error %.3g" % (what, lerr)
    return err


# Gradient scale: max|ref| of the tensor.  Only a reference that is identically
# zero -- dQ and dK when every row admits a single key (dS = P (dP - D) with
# P = 1 and D = dP, exactly, in the f64 oracle) -- takes GRAD_SCALE_FLOOR
# instead, which makes the bound an absolute 1e-6 (f32) on the kernel's
# rounding residue of dP - D.
GRAD_SCALE_FLOOR = 1e-2


def grad_scale(ref) -> float:
    top = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    return top if top > 0.0 else GRAD_SCALE_FLOOR


def assert_grad_close(g, ref, dtype, name):
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), name + ": non-finite gradient"
    scale = grad_scale(ref)
    err = np.max(np.abs(g - ref))
    assert err <= TOL[dtype] * scale, "%s: max err %.3g > %.1g * %.3g" % (name, err, TOL[dtype], scale)
    return err / scale


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy()


# The 16-bit forward's a-priori bound (include/osattn.h, "Accuracy"): the only
# rounding beyond f32 is that of the probabilities to the input type, so per row
#   |O_i - O_ref,i| <= (u + n_i t) max_{j in A(i)} |v_j| + e32
# with u the type's unit roundoff, t fp16's half-step below its normal range
# (2^-25; bf16 has f32's range), n_i the admitted key count and e32 <= 1e-5
# max|v| for the f32 arithmetic.  It holds at any softmax temperature.
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
SUBNORMAL_HALF_STEP = {"bf16": 0.0, "f16": 2.0 ** -25}
F32_SLACK = 1e-5


def admitted_vmax(v32: np.ndarray, n_q: int, causal: bool, cu=None):
    """(max_{j in A(i)} |v_j|, n_i) for every (head, query row)."""
    H, n_k, _ = v32.shape
    av = np.abs(np.asarray(v32, np.float64)).max(axis=2)  # (H, n_k)
    mx = np.zeros((H, n_q))
    cnt = np.zeros(n_q)
    spans = [(0, n_q)] if cu is None else [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:])]
    for a, b in spans:
        if b <= a:
            continue
        if causal:
            mx[:, a:b] = np.maximum.accumulate(av[:, a:b], axis=1)
            cnt[a:b] = np.arange(1, b - a + 1)
        else:
            kb = (a, b) if cu is not None else (0, n_k)
            mx[:, a:b] = av[:, kb[0]:kb[1]].max(axis=1, keepdims=True)
            cnt[a:b] = kb[1] - kb[0]
    return mx, np.broadcast_to(cnt, (H, n_q))


def assert_fwd_within_bound(o, m, l, ro, rm, rl, v32, dtype, causal, cu=None, what=""):
    """Forward against the a-priori bound, row by row (16-bit), or the f32
    tolerance; row statistics as in assert_fwd_close."""
    o = np.asarray(o, dtype=np.float64)
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    if dtype == "f32":
        return assert_fwd_close(o, m, l, ro, rm, rl, dtype, what)
    vmax, cnt = admitted_vmax(v32, o.shape[1], causal, cu)
    bound = (UNIT_ROUNDOFF[dtype] + cnt * SUBNORMAL_HALF_STEP[dtype] + F32_SLACK) * vmax
    err = np.abs(o - ro).max(axis=2)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), "%s: row %s error %.3g above its bound %.3g" % (
        what, worst, err[worst], bound[worst])
    merr = np.max(np.abs(np.asarray(m, np.float64) - rm) / np.maximum(1.0, np.abs(rm)))
    lerr = np.max(np.abs(np.asarray(l, np.float64) / rl - 1.0))
    assert merr <= STAT_TOL, "%s: m error %.3g" % (what, merr)
    assert lerr <= STAT_TOL, "%s: l error %.3g" % (what, lerr)
    return float(np.max(err / bound))


# Gradients at twice the pages' softmax scale: held to 2 tol max|ref| (the
# documented bound for scale 2 D^-1/2 with unit-normal inputs).
SHARP_GRAD_FACTOR = 2.0


def assert_grad_close_sharp(g, ref, dtype, name):
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), name + ": non-finite gradient"
    scale = grad_scale(ref)
    err = np.max(np.abs(g - ref))
    lim = SHARP_GRAD_FACTOR * TOL[dtype] * scale
    assert err <= lim, "%s: max err %.3g > %.1g * %.1g * %.3g" % (
        name, err, SHARP_GRAD_FACTOR, TOL[dtype], scale)
    return err / scale
