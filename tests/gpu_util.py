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


# Floor of the gradient scale: with a single admitted key the reference dQ and dK
# are identically zero (dS = P (dP - D) with P = 1 and D = dP), so the relative
# bound is taken against max(max|ref|, GRAD_SCALE_FLOOR) -- an absolute 1e-6 for
# f32 in that degenerate case, irrelevant wherever max|ref| is O(1).
GRAD_SCALE_FLOOR = 1e-2


def assert_grad_close(g, ref, dtype, name):
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), name + ": non-finite gradient"
    scale = max(np.max(np.abs(ref)), GRAD_SCALE_FLOOR)
    err = np.max(np.abs(g - ref))
    assert err <= TOL[dtype] * scale, "%s: max err %.3g > %.1g * %.3g" % (name, err, TOL[dtype], scale)
    return err / scale


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy()
