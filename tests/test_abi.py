"""C-ABI boundary tests that need no GPU.

The library must load, export every function include/osattn.h declares, and
reject invalid arguments on the host -- before any HIP call -- with the
documented status codes.  Pointers handed to rejected calls are fake values
that must never be dereferenced; every case below fails a host check first.
"""
import ctypes
import os
import re

import pytest

import online_softmax_attention_amd as osa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osattn.h")
F32, F16, BF16 = osa.F32, osa.F16, osa.BF16

# Fake, 256-byte aligned addresses; never dereferenced (every call fails first).
A = 0x7F0000000000
B, C, O, M, L = A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(osa.LIB_PATH):
        import online_softmax_attention_amd.build as b
        b.build()
    return osa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(osattn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(osa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    codes = (osa.OK, osa.ERR_INVALID_ARG, osa.ERR_UNSUPPORTED, osa.ERR_ALIGNMENT, osa.ERR_HIP,
             osa.ERR_WORKSPACE)
    assert codes == (0, -1, -2, -3, -4, -5)  # zero is success, failures are negative
    for s in codes:
        assert osa.status_string(s).startswith("OSATTN_")
    assert "unknown" in osa.status_string(99)
    assert "unknown" in osa.status_string(1)
    assert lib.osattn_version() >= 100


# m defaults to NULL so that no combination of the other arguments can pass every
# host check and reach a launch with the fake pointers.
def fwd(lib, dtype=F16, H=2, n_q=128, n_k=128, d=64, q=A, k=B, v=C, qs=(128 * 64, 64),
        kvs=(128 * 64, 64), o=O, os_=(128 * 64, 64), m=None, l=L, scale=0.125, causal=0,
        cu=None, num_seqs=0, max_seqlen=0, ws=None, ws_bytes=0, o_dtype=F32):
    return lib.osattn_fwd(dtype, o_dtype, H, n_q, n_k, d, q, k, v, qs[0], qs[1], kvs[0], kvs[1], o,
                          os_[0], os_[1], m, l, scale, causal, cu, num_seqs, max_seqlen, ws,
                          ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), osa.ERR_INVALID_ARG),
    (dict(H=0), osa.ERR_INVALID_ARG),
    (dict(n_q=0), osa.ERR_INVALID_ARG),
    (dict(n_k=0), osa.ERR_INVALID_ARG),
    (dict(d=96), osa.ERR_UNSUPPORTED),
    (dict(d=0), osa.ERR_INVALID_ARG),
    (dict(scale=float("nan")), osa.ERR_UNSUPPORTED),
    (dict(scale=float("inf")), osa.ERR_UNSUPPORTED),
    (dict(scale=-1.0), osa.ERR_UNSUPPORTED),
    (dict(q=None), osa.ERR_INVALID_ARG),
    (dict(k=None), osa.ERR_INVALID_ARG),
    (dict(v=None), osa.ERR_INVALID_ARG),
    (dict(o=None), osa.ERR_INVALID_ARG),
    (dict(m=M, l=None), osa.ERR_INVALID_ARG),
    (dict(q=A + 8), osa.ERR_ALIGNMENT),
    (dict(o=O + 4), osa.ERR_ALIGNMENT),
    (dict(qs=(128 * 64, 60)), osa.ERR_ALIGNMENT),
    (dict(kvs=(-64, 64)), osa.ERR_INVALID_ARG),
    (dict(os_=(128 * 64, 66)), osa.ERR_ALIGNMENT),
    (dict(causal=1, n_k=100), osa.ERR_INVALID_ARG),
    (dict(cu=A, num_seqs=0, max_seqlen=10), osa.ERR_INVALID_ARG),
    (dict(cu=A, num_seqs=2, max_seqlen=0), osa.ERR_INVALID_ARG),
    (dict(cu=A, num_seqs=2, max_seqlen=200), osa.ERR_INVALID_ARG),
    (dict(cu=A, num_seqs=2, max_seqlen=64, n_k=100), osa.ERR_INVALID_ARG),
    (dict(n_q=(1 << 30) + 1, n_k=(1 << 30) + 1), osa.ERR_UNSUPPORTED),
    # o is f32, or the input's own 16-bit type
    (dict(o_dtype=BF16), osa.ERR_INVALID_ARG),
    (dict(o_dtype=7), osa.ERR_INVALID_ARG),
    (dict(dtype=F32, o_dtype=F16, qs=(128 * 64, 64), kvs=(128 * 64, 64)), osa.ERR_INVALID_ARG),
    # a 16-bit o needs 16-byte alignment in its own element size (8 elements)
    (dict(o_dtype=F16, os_=(128 * 64, 68)), osa.ERR_ALIGNMENT),
])
def test_fwd_rejects_on_host(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert osa.last_error() != ""


def test_fwd_stride_units_follow_dtype(lib):
    # f32 strides must be multiples of 4 elements, 16-bit strides of 8.
    assert fwd(lib, dtype=F32, qs=(128 * 64, 66)) == osa.ERR_ALIGNMENT
    assert fwd(lib, dtype=F16, qs=(128 * 64, 68)) == osa.ERR_ALIGNMENT
    assert fwd(lib, dtype=F32, qs=(128 * 64, 68)) == osa.ERR_INVALID_ARG  # reaches m == NULL


# The workspace defaults to NULL so no case can pass every host check.
def bwd(lib, dtype=F32, H=1, n_q=256, n_k=128, d=64, ptrs=None, ws=None, ws_bytes=1 << 30,
        causal=0, scale=0.125, o_dtype=F32):
    p = dict(q=A, k=B, v=C, o=O, do=A + 0x600000, m=M, l=L, dq=A + 0x700000,
             dk=A + 0x800000, dv=A + 0x900000)
    p.update(ptrs or {})
    return lib.osattn_bwd(dtype, o_dtype, H, n_q, n_k, d, p["q"], p["k"], p["v"], p["o"], p["do"],
                          n_q * d, d, n_k * d, d, n_q * d, d, p["m"], p["l"], scale, causal,
                          None, 0, 0, p["dq"], p["dk"], p["dv"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=F16, d=96), osa.ERR_UNSUPPORTED),
    (dict(d=32), osa.ERR_UNSUPPORTED),
    (dict(d=128, ws=None), osa.ERR_WORKSPACE),  # f32 d = 128 passes the width checks
    (dict(ws=None), osa.ERR_WORKSPACE),
    (dict(dtype=F16, ws=None), osa.ERR_WORKSPACE),  # fp16 d = 64 passes the dtype checks
    (dict(dtype=BF16, d=128, ws=None), osa.ERR_WORKSPACE),
    (dict(ws=A, ws_bytes=16), osa.ERR_WORKSPACE),
    (dict(ws=A + 16), osa.ERR_ALIGNMENT),
    (dict(ptrs={"do": None}), osa.ERR_INVALID_ARG),
    (dict(ptrs={"dk": None}), osa.ERR_INVALID_ARG),
    (dict(ptrs={"dq": A + 4}), osa.ERR_ALIGNMENT),
    (dict(causal=1), osa.ERR_INVALID_ARG),
])
def test_bwd_rejects_on_host(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_fwd_workspace_bytes(lib):
    # decode-like dense shapes (few query tiles, long keys) split their key range
    n = lib.osattn_fwd_workspace_bytes(F16, 4, 128, 16384, 64, 0, None, 0, 0)
    assert n > 0 and n % 256 == 0
    # short key ranges do not (a split costs a second launch)
    assert lib.osattn_fwd_workspace_bytes(F16, 4, 1024, 1024, 64, 0, None, 0, 0) == 0
    # causal problems never split
    assert lib.osattn_fwd_workspace_bytes(F16, 4, 1024, 1024, 64, 1, None, 0, 0) == 0
    assert lib.osattn_fwd_workspace_bytes(F32, 4, 1024, 1024, 64, 1, None, 0, 0) == 0
    assert lib.osattn_fwd_workspace_bytes(F16, 4, 1024, 1024, 96, 0, None, 0, 0) == 0
    # f32 dense splits when its 128-row tiles cannot fill the device, the keys
    # span at least 512 and (d = 64) 32-row tiles cannot fill it either:
    # (splits, H, n_q, D + 4) f32 partial states
    n = lib.osattn_fwd_workspace_bytes(F32, 1, 1024, 2048, 64, 0, None, 0, 0)
    assert n > 0 and n % 256 == 0 and n % (1024 * 68 * 4) == 0
    n = lib.osattn_fwd_workspace_bytes(F32, 1, 8192, 2048, 128, 0, None, 0, 0)
    assert n > 0 and n % 256 == 0 and n % (8192 * 132 * 4) == 0
    # 8192 / 32 = 256 tiles of 32 rows fill the device at d = 64: no partials
    assert lib.osattn_fwd_workspace_bytes(F32, 1, 8192, 2048, 64, 0, None, 0, 0) == 0
    assert lib.osattn_fwd_workspace_bytes(F32, 4, 1024, 384, 64, 0, None, 0, 0) == 0
    assert lib.osattn_fwd_workspace_bytes(F32, 1, 128, 128, 64, 0, None, 0, 0) == 0
    # enough tiles to fill the device: no split
    assert lib.osattn_fwd_workspace_bytes(BF16, 64, 8192, 8192, 128, 0, None, 0, 0) == 0


def test_fwd_workspace_bytes_varlen_work_list(lib):
    # 16-bit varlen with more than 64 sequences: a 16-byte header plus one
    # 16-byte entry per tile pair, at most (sum_s T_s + S) / 2 with
    # sum_s T_s <= (n + 127 S) / 128, and at most S ceil(ceil(max_seqlen / 128) / 2).
    # Up to 64 sequences the workgroups rank their items themselves: no list.
    cu = ctypes.c_void_p(0x1000)  # only tested for NULL on the host
    r256 = lambda x: (x + 255) // 256 * 256
    for causal in (0, 1):
        assert lib.osattn_fwd_workspace_bytes(F16, 8, 16384, 16384, 64, causal, cu, 20, 1894) == 0
        n = lib.osattn_fwd_workspace_bytes(F16, 8, 16384, 16384, 64, causal, cu, 100, 1894)
        assert n == r256(16 + 16 * (((16384 + 127 * 100) // 128 + 100) // 2))
    assert lib.osattn_fwd_workspace_bytes(BF16, 2, 4096, 4096, 128, 1, cu, 64, 100) == 0
    n = lib.osattn_fwd_workspace_bytes(BF16, 2, 4096, 4096, 128, 1, cu, 65, 100)
    assert n == r256(16 + 16 * 65)  # 65 one-tile sequences
    # equal lengths (n == S * max_seqlen): the natural order is balanced, no list
    assert lib.osattn_fwd_workspace_bytes(F16, 8, 16384, 16384, 64, 1, cu, 16, 1024) == 0
    assert lib.osattn_fwd_workspace_bytes(F32, 8, 16384, 16384, 64, 1, cu, 20, 1894) == 0


def test_bwd_workspace_bytes(lib):
    n = lib.osattn_bwd_workspace_bytes(F32, 1, 8192, 2048, 64, 0, None, 0, 0)
    assert n >= 3 * 8192 * 4 and n % 256 == 0
    assert lib.osattn_bwd_workspace_bytes(F16, 1, 8192, 2048, 64, 0, None, 0, 0) >= 3 * 8192 * 4
    assert lib.osattn_bwd_workspace_bytes(BF16, 1, 8192, 2048, 128, 0, None, 0, 0) >= 3 * 8192 * 4
    assert lib.osattn_bwd_workspace_bytes(F16, 1, 8192, 2048, 96, 0, None, 0, 0) == 0
    # f32 at d = 128: the same plan (dK/dV split over queries) with partials twice as wide
    n128 = lib.osattn_bwd_workspace_bytes(F32, 1, 8192, 2048, 128, 0, None, 0, 0)
    assert n128 > n and n128 % 256 == 0
    assert lib.osattn_bwd_workspace_bytes(F32, 1, 8192, 2048, 32, 0, None, 0, 0) == 0
    assert lib.osattn_bwd_workspace_bytes(F32, 0, 8192, 2048, 64, 0, None, 0, 0) == 0


def test_fwd_rejects_huge_row_stride(lib):
    big = (1 << 22) // 2 + 8  # f16 elements: just above 4 MiB per row
    assert fwd(lib, qs=(big * 128, big)) == osa.ERR_UNSUPPORTED
    assert fwd(lib, kvs=(big * 128, big)) == osa.ERR_UNSUPPORTED


def test_bwd_rejects_huge_row_stride(lib):
    # The backward kernels form in-block row offsets in 32 bits, as the
    # forward's do: the same 4 MiB limit, checked before the workspace (NULL).
    def call(qs, kvs, dtype=F16, d=64):
        return lib.osattn_bwd(dtype, F32, 1, 256, 256, d, A, B, C, O, A + 0x600000, qs[0], qs[1],
                              kvs[0], kvs[1], 256 * d, d, M, L, 0.125, 0, None, 0, 0,
                              A + 0x700000, A + 0x800000, A + 0x900000, None, 0, None)
    big = (1 << 22) // 2 + 8
    assert call((big * 256, big), (256 * 64, 64)) == osa.ERR_UNSUPPORTED
    assert call((256 * 64, 64), (big * 256, big)) == osa.ERR_UNSUPPORTED
    assert call((256 * 64, 64), (256 * 64, 64)) == osa.ERR_WORKSPACE  # the stride check alone
    assert "workspace" in osa.last_error()
    f32big = (1 << 22) // 4 + 4
    assert call((f32big * 256, f32big), (256 * 64, 64), dtype=F32) == osa.ERR_UNSUPPORTED


def test_bwd_noalloc_refuses_problems_above_its_scratch_before_any_hip_call(lib):
    # 3 f32 rows of statistics per (head, query): H=64, n=65536 needs 48 MiB > 32 MiB
    def call(H, n, ptrs=None, scale=0.125):
        p = dict(q=A, k=B, v=C, o=O, do=A + 0x600000, m=M, l=L, dq=A + 0x700000,
                 dk=A + 0x800000, dv=A + 0x900000)
        p.update(ptrs or {})
        return lib.osattn_bwd_noalloc(F16, F32, H, n, n, 64, p["q"], p["k"], p["v"], p["o"],
                                      p["do"], n * 64, 64, n * 64, 64, n * 64, 64, p["m"], p["l"],
                                      scale, 0, None, 0, 0, p["dq"], p["dk"], p["dv"], None)
    assert lib.osattn_bwd_workspace_bytes(F16, 64, 65536, 65536, 64, 0, None, 0, 0) > osa.NOALLOC_SCRATCH_BYTES
    assert call(64, 65536) == osa.ERR_WORKSPACE
    assert "static" in osa.last_error()
    # argument errors come first, as in osattn_bwd
    assert call(64, 65536, ptrs={"q": None}) == osa.ERR_INVALID_ARG
    assert call(64, 65536, ptrs={"dk": A + 4}) == osa.ERR_ALIGNMENT
    assert call(64, 65536, scale=float("nan")) == osa.ERR_UNSUPPORTED
    assert call(1, 256, ptrs={"m": None}) == osa.ERR_INVALID_ARG


_NO_DEVICE_CALL = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
try:
    hip = ctypes.CDLL("libamdhip64.so")
    n = ctypes.c_int(0)
    if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
        print("HAS_DEVICE")  # a real device: never launch with fake pointers
        sys.exit(0)
except OSError:
    pass
import online_softmax_attention_amd as osa
lib = osa.load()
A = 0x7F0000000000
st = lib.osattn_fwd(osa.F16, osa.F32, 2, 128, 128, 64, A, A + 0x100000, A + 0x200000,
                    128 * 64, 64, 128 * 64, 64, A + 0x300000, 128 * 64, 64, A + 0x400000,
                    A + 0x500000, 0.125, 0, None, 0, 0, None, 0, None)
print("STATUS", st, osa.last_error())
"""


def test_valid_call_without_a_device_returns_hip_error():
    """A call that passes every host check, on a host with no usable GPU,
    returns OSATTN_ERR_HIP instead of crashing (run in a child process; skipped
    where a device is visible, since the pointers here are fake)."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, "-c", _NO_DEVICE_CALL, ROOT], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=120)
    assert res.returncode == 0, res.stdout
    if "HAS_DEVICE" in res.stdout:
        pytest.skip("a HIP device is visible")
    line = [x for x in res.stdout.splitlines() if x.startswith("STATUS")][0]
    assert int(line.split()[1]) == osa.ERR_HIP, line
    assert "device" in line.lower()


# Tile-pruned forward: every case fails a host check before any launch.
def fwd_pruned(lib, dtype=F16, H=1, n_q=256, n_k=128, d=64, rho=0.5, m=None, scale=0.125,
               o_dtype=F32):
    return lib.osattn_fwd_pruned(dtype, o_dtype, H, n_q, n_k, d, A, B, C, n_q * d, d, n_k * d, d,
                                 O, n_q * d, d, m, L, scale, rho, None)


@pytest.mark.parametrize("kw,status", [
    (dict(rho=0.0), osa.ERR_INVALID_ARG),
    (dict(rho=-0.5), osa.ERR_INVALID_ARG),
    (dict(rho=1.5), osa.ERR_INVALID_ARG),
    (dict(rho=float("nan")), osa.ERR_INVALID_ARG),
    (dict(dtype=F32), osa.ERR_UNSUPPORTED),
    (dict(d=96), osa.ERR_UNSUPPORTED),
    (dict(scale=0.0), osa.ERR_UNSUPPORTED),
    (dict(n_q=0), osa.ERR_INVALID_ARG),
    (dict(), osa.ERR_INVALID_ARG),  # m is NULL: the last check
])
def test_fwd_pruned_rejects_on_host(lib, kw, status):
    assert fwd_pruned(lib, **kw) == status


# CSR segment softmax: every case fails a host check before any launch.
def csr(lib, dtype=F16, H=1, n_dst=16, n_src=16, d=64, nnz=32, rp=A + 0x100000, ci=A + 0x200000,
        sc=A + 0x300000, v=B, o=O, m=None, l=L):
    return lib.osattn_csr_softmax(dtype, H, n_dst, n_src, d, rp, ci, nnz, sc, nnz, v, n_src * d, d,
                                  o, n_dst * d, d, m, l, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), osa.ERR_INVALID_ARG),
    (dict(n_dst=0), osa.ERR_INVALID_ARG),
    (dict(nnz=-1), osa.ERR_INVALID_ARG),
    (dict(nnz=1 << 31), osa.ERR_UNSUPPORTED),
    (dict(d=96), osa.ERR_UNSUPPORTED),
    (dict(rp=None), osa.ERR_INVALID_ARG),
    (dict(ci=None), osa.ERR_INVALID_ARG),
    (dict(sc=None), osa.ERR_INVALID_ARG),
    (dict(v=B + 4), osa.ERR_ALIGNMENT),
    (dict(o=O + 8), osa.ERR_ALIGNMENT),
    (dict(), osa.ERR_INVALID_ARG),  # m is NULL: the last check
])
def test_csr_rejects_on_host(lib, kw, status):
    assert csr(lib, **kw) == status


# ------------------------------------------------------------ Python binding
# The binding validates what the raw pointers cannot carry -- device, dtype,
# shapes and the strides the ABI reuses -- before any GPU call, so these run on
# the host (CPU tensors are rejected before the library sees them).
def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float16)


def test_binding_rejects_host_tensors():
    q = _cpu(2, 64, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        osa.fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU tensor"):
        osa.fwd_pruned(q, q, q, 0.5)
    import torch
    o32 = _cpu(2, 64, 64, dtype=torch.float32)
    ml = _cpu(2, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        osa.bwd(q, q, q, o32, q, ml, ml)
    rp = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError):
        osa.csr_softmax(rp, rp, _cpu(1, 3, dtype=torch.float32), _cpu(1, 4, 64))


def test_binding_rejects_mismatched_shapes_before_the_device_check():
    import torch
    q, k = _cpu(2, 64, 64), _cpu(2, 32, 64)
    with pytest.raises(ValueError, match="same shape and strides"):
        osa.fwd(q, k, _cpu(2, 33, 64))
    with pytest.raises(ValueError, match="same shape and strides"):
        osa.bwd(q, k, _cpu(2, 64, 64), _cpu(2, 64, 64, dtype=torch.float32), q,
                _cpu(2, 64, dtype=torch.float32), _cpu(2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="float32 or the input dtype"):  # o in a third dtype
        osa.bwd(q, k, k, _cpu(2, 64, 64, dtype=torch.bfloat16), q, _cpu(2, 64, dtype=torch.float32),
                _cpu(2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="float32 or the input dtype"):
        osa.fwd(q, q, q, out_dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="do must match"):
        osa.bwd(q, k, k, _cpu(2, 64, 64, dtype=torch.float32), _cpu(2, 63, 64),
                _cpu(2, 64, dtype=torch.float32), _cpu(2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match=r"m must be a contiguous float32 tensor of shape \(2, 64\)"):
        osa.bwd(q, k, k, _cpu(2, 64, 64, dtype=torch.float32), q,
                _cpu(2, 63, dtype=torch.float32), _cpu(2, 64, dtype=torch.float32))
