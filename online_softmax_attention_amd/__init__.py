"""Online-softmax attention on AMD MI355X (gfx950): thin Python binding.

This module only marshals arguments: it checks shapes, allocates outputs with
torch, and calls the C ABI of libosattn.so (declared in include/osattn.h)
through ctypes on torch's current HIP stream.  Every step of the attention
computation runs in the library's HIP kernels; there is no fallback of any
kind -- if the library is missing, every call raises.

    o, m, l = fwd(q, k, v, scale=None, causal=False, cu_seqlens=None, max_seqlen=None)
    o, m, l = fwd_pruned(q, k, v, rho, scale=None)     # tile-pruned approximation
    dq, dk, dv = bwd(q, k, v, o, do, m, l, scale=None, causal=False, ...)

Tensors are (H, N, D) by default (``layout="hnd"``) or (N, H, D)
(``layout="nhd"``), with the feature dimension contiguous.  o is float32;
m and l are float32 of shape (H, N_q), m in natural-log units of the scaled
score.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libosattn.so")

F32, F16, BF16 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4, -5
EXPORTS = ("osattn_fwd", "osattn_fwd_workspace_bytes", "osattn_fwd_pruned", "osattn_bwd",
           "osattn_bwd_workspace_bytes", "osattn_bwd_noalloc", "osattn_csr_softmax",
           "osattn_status_string", "osattn_last_error_message", "osattn_version")
# Scratch bytes osattn_bwd_noalloc can use (OSATTN_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20

_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_lib = None


class OsattnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__("%s: %s (%s)" % (where, status_string(status), detail))
        self.status = status


def load(path: Optional[str] = None):
    """Load libosattn.so (built by online_softmax_attention_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libosattn.so is not built (%s); run online_softmax_attention_amd.build" % p)
    lib = ctypes.CDLL(p)
    i32, i64, f32, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.osattn_fwd.argtypes = [i32, i32, i32, i64, i64, i32, vp, vp, vp, i64, i64, i64, i64,
                               vp, i64, i64, vp, vp, f32, i32, vp, i32, i32, vp, ctypes.c_size_t, vp]
    lib.osattn_fwd.restype = i32
    lib.osattn_fwd_pruned.argtypes = [i32, i32, i32, i64, i64, i32, vp, vp, vp, i64, i64, i64,
                                      i64, vp, i64, i64, vp, vp, f32, f32, vp]
    lib.osattn_fwd_pruned.restype = i32
    lib.osattn_csr_softmax.argtypes = [i32, i32, i64, i64, i32, vp, vp, i64, vp, i64, vp, i64, i64,
                                       vp, i64, i64, vp, vp, vp]
    lib.osattn_csr_softmax.restype = i32
    lib.osattn_fwd_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i32, vp, i32, i32]
    lib.osattn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osattn_bwd_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i32, vp, i32, i32]
    lib.osattn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osattn_bwd.argtypes = [i32, i32, i32, i64, i64, i32, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                               i64, i64, vp, vp, f32, i32, vp, i32, i32, vp, vp, vp, vp,
                               ctypes.c_size_t, vp]
    lib.osattn_bwd.restype = i32
    lib.osattn_bwd_noalloc.argtypes = lib.osattn_bwd.argtypes[:-3] + [vp]
    lib.osattn_bwd_noalloc.restype = i32
    lib.osattn_status_string.argtypes = [i32]
    lib.osattn_status_string.restype = ctypes.c_char_p
    lib.osattn_last_error_message.argtypes = []
    lib.osattn_last_error_message.restype = ctypes.c_char_p
    lib.osattn_version.argtypes = []
    lib.osattn_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().osattn_status_string(int(status)).decode()


def last_error() -> str:
    return load().osattn_last_error_message().decode()


def _check(status: int, where: str):
    if status != OK:
        raise OsattnError(status, where, last_error())


def _hn(t: torch.Tensor, layout: str):
    """(H, N, D, stride_h, stride_n) of a 3-D tensor in the given layout."""
    if t.dim() != 3:
        raise ValueError("expected a 3-D tensor, got shape %s" % (tuple(t.shape),))
    if layout == "hnd":
        H, N, D = t.shape
        sh, sn = t.stride(0), t.stride(1)
    elif layout == "nhd":
        N, H, D = t.shape
        sh, sn = t.stride(1), t.stride(0)
    else:
        raise ValueError("layout must be 'hnd' or 'nhd'")
    if t.stride(2) != 1:
        raise ValueError("the feature dimension must be contiguous")
    return H, N, D, sh, sn


def _cu_args(cu_seqlens, max_seqlen, n, check):
    if cu_seqlens is None:
        return None, 0, 0
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
    if check or max_seqlen is None:
        host = cu_seqlens.cpu().tolist()
        if len(host) < 2 or host[0] != 0 or host[-1] != n:
            raise ValueError("cu_seqlens must start at 0 and end at the token count %d" % n)
        lens = [b - a for a, b in zip(host[:-1], host[1:])]
        if min(lens) < 0:
            raise ValueError("cu_seqlens must be non-decreasing")
        longest = max(lens)
        if max_seqlen is None:
            max_seqlen = longest
        elif max_seqlen < longest:
            raise ValueError("max_seqlen %d is below the longest sequence %d" % (max_seqlen, longest))
    return cu_seqlens, cu_seqlens.numel() - 1, int(max_seqlen)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _one_gpu(*named):
    """The device of the first tensor; every named tensor (None skipped) must be
    on that same GPU (a host pointer reaching a kernel would fault it)."""
    dev = named[0][0].device
    if not named[0][0].is_cuda:
        raise ValueError("%s must be a GPU tensor (got %s)" % (named[0][1], dev))
    for t, name in named:
        if t is None:
            continue
        if not t.is_cuda or t.device != dev:
            raise ValueError("%s must be on the GPU device %s (got %s)" % (name, dev, t.device))
    return dev


def _rows_f32(t: torch.Tensor, H: int, n: int, name: str):
    """m and l: contiguous float32 (H, n)."""
    if t.dtype != torch.float32 or tuple(t.shape) != (H, n) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 tensor of shape (%d, %d)" % (name, H, n))


def _like(t: torch.Tensor, ref: torch.Tensor, dtype: torch.dtype, name: str):
    """An output the ABI addresses with ref's strides: same shape and strides."""
    if t.dtype != dtype or t.shape != ref.shape or t.stride() != ref.stride():
        raise ValueError("%s must have dtype %s and the shape and strides of %s" %
                         (name, dtype, tuple(ref.shape)))


def _bytes(ws: torch.Tensor) -> int:
    return ws.numel() * ws.element_size()


# Forward split-KV workspaces, one per (device, stream).
_fwd_ws = {}


def _fwd_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """The cached split-KV / work-list buffer of (device, stream).  Under graph
    capture every call gets its own buffer instead: torch captures all graphs on
    one stream, so a cached buffer would be shared by graphs that may replay
    concurrently, and replacing it would hand memory a graph still uses back to
    the allocator (the graph's private pool keeps a fresh tensor alive)."""
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _fwd_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _fwd_ws[key] = ws
    return ws


def _o_code(o: torch.Tensor, q: torch.Tensor) -> int:
    """o_dtype of the ABI: float32 for any input, or the 16-bit input dtype."""
    if o.dtype == torch.float32 or (o.dtype == q.dtype and q.dtype != torch.float32):
        return _DT[o.dtype]
    raise ValueError("o must be float32 or the input dtype %s (got %s)" % (q.dtype, o.dtype))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
        causal: bool = False, cu_seqlens: Optional[torch.Tensor] = None,
        max_seqlen: Optional[int] = None, layout: str = "hnd", check: bool = True,
        out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
        workspace: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32):
    """Attention forward on the GPU; returns (o, m, l).

    ``out_dtype``: o's dtype, float32 (default) or q's 16-bit dtype (the same
    values rounded once); with ``out`` given, o's own dtype decides.
    ``workspace``: optional device buffer for split-KV partial states (see
    osattn_fwd_workspace_bytes); by default a cached one per (device, stream).
    An empty tensor forces the unsplit forward."""
    lib = load()
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype of float32/float16/bfloat16")
    H, n_q, D, q_sh, q_sn = _hn(q, layout)
    Hk, n_k, Dk, kv_sh, kv_sn = _hn(k, layout)
    Hv, n_v, Dv, v_sh, v_sn = _hn(v, layout)
    if (Hk, Dk) != (H, D) or (Hv, n_v, Dv) != (H, n_k, D) or (v_sh, v_sn) != (kv_sh, kv_sn):
        raise ValueError("k and v must have the same shape and strides, matching q's H and D")
    scale = D ** -0.5 if scale is None else float(scale)
    cu, num_seqs, max_seqlen = _cu_args(cu_seqlens, max_seqlen, n_q, check)
    if out is None:
        shape = (H, n_q, D) if layout == "hnd" else (n_q, H, D)
        o = torch.empty(shape, dtype=out_dtype, device=q.device)
        m = torch.empty((H, n_q), dtype=torch.float32, device=q.device)
        l = torch.empty((H, n_q), dtype=torch.float32, device=q.device)
    else:
        o, m, l = out
    o_code = _o_code(o, q)
    dev = _one_gpu((q, "q"), (k, "k"), (v, "v"), (o, "o"), (m, "m"), (l, "l"), (cu, "cu_seqlens"),
                   (workspace, "workspace"))
    Ho, n_o, Do, o_sh, o_sn = _hn(o, layout)
    if (Ho, n_o, Do) != (H, n_q, D):
        raise ValueError("o must have q's shape")
    _rows_f32(m, H, n_q, "m")
    _rows_f32(l, H, n_q, "l")
    cu_ptr = None if cu is None else cu.data_ptr()
    with torch.cuda.device(dev):
        if workspace is None:
            need = lib.osattn_fwd_workspace_bytes(_DT[q.dtype], H, n_q, n_k, D, int(bool(causal)),
                                                  cu_ptr, num_seqs, max_seqlen)
            workspace = _fwd_workspace(dev, int(need)) if need else None
        ws_ptr = None if workspace is None else workspace.data_ptr()
        ws_bytes = 0 if workspace is None else _bytes(workspace)
        st = lib.osattn_fwd(_DT[q.dtype], o_code, H, n_q, n_k, D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            q_sh, q_sn, kv_sh, kv_sn, o.data_ptr(), o_sh, o_sn, m.data_ptr(),
                            l.data_ptr(), scale, int(bool(causal)), cu_ptr, num_seqs, max_seqlen,
                            ws_ptr, ws_bytes, _stream())
    _check(st, "osattn_fwd")
    return o, m, l


def fwd_pruned(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: float,
               scale: Optional[float] = None, layout: str = "hnd",
               out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
               out_dtype: torch.dtype = torch.float32):
    """Tile-pruned dense forward (an approximation; see osattn_fwd_pruned); returns (o, m, l)."""
    lib = load()
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype of float16/bfloat16")
    H, n_q, D, q_sh, q_sn = _hn(q, layout)
    Hk, n_k, Dk, kv_sh, kv_sn = _hn(k, layout)
    Hv, n_v, Dv, v_sh, v_sn = _hn(v, layout)
    if (Hk, Dk) != (H, D) or (Hv, n_v, Dv) != (H, n_k, D) or (v_sh, v_sn) != (kv_sh, kv_sn):
        raise ValueError("k and v must have the same shape and strides, matching q's H and D")
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        shape = (H, n_q, D) if layout == "hnd" else (n_q, H, D)
        o = torch.empty(shape, dtype=out_dtype, device=q.device)
        m = torch.empty((H, n_q), dtype=torch.float32, device=q.device)
        l = torch.empty((H, n_q), dtype=torch.float32, device=q.device)
    else:
        o, m, l = out
    o_code = _o_code(o, q)
    dev = _one_gpu((q, "q"), (k, "k"), (v, "v"), (o, "o"), (m, "m"), (l, "l"))
    Ho, n_o, Do, o_sh, o_sn = _hn(o, layout)
    if (Ho, n_o, Do) != (H, n_q, D):
        raise ValueError("o must have q's shape")
    _rows_f32(m, H, n_q, "m")
    _rows_f32(l, H, n_q, "l")
    with torch.cuda.device(dev):
        st = lib.osattn_fwd_pruned(_DT[q.dtype], o_code, H, n_q, n_k, D, q.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), q_sh, q_sn, kv_sh, kv_sn, o.data_ptr(), o_sh,
                                   o_sn, m.data_ptr(), l.data_ptr(), scale, float(rho), _stream())
    _check(st, "osattn_fwd_pruned")
    return o, m, l


def csr_softmax(row_ptr: torch.Tensor, col_idx: torch.Tensor, scores: torch.Tensor,
                v: torch.Tensor, out=None):
    """CSR segment softmax with given edge scores; returns (o, m, l).

    row_ptr (n_dst + 1,), col_idx (nnz,) int32 device tensors; scores (H, nnz)
    float32 with a contiguous last dimension; v (H, n_src, D)."""
    lib = load()
    if v.dtype not in _DT:
        raise ValueError("v must be float32, float16 or bfloat16")
    for t, name in ((row_ptr, "row_ptr"), (col_idx, "col_idx")):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 1-D int32 device tensor" % name)
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a float32 (H, nnz) tensor with a contiguous last dimension")
    H, n_src, D, v_sh, v_sn = _hn(v, "hnd")
    n_dst, nnz = row_ptr.numel() - 1, col_idx.numel()
    if scores.shape != (H, nnz):
        raise ValueError("scores must be (H, nnz) = (%d, %d)" % (H, nnz))
    if out is None:
        o = torch.empty((H, n_dst, D), dtype=torch.float32, device=v.device)
        m = torch.empty((H, n_dst), dtype=torch.float32, device=v.device)
        l = torch.empty((H, n_dst), dtype=torch.float32, device=v.device)
    else:
        o, m, l = out
    dev = _one_gpu((v, "v"), (row_ptr, "row_ptr"), (col_idx, "col_idx"), (scores, "scores"),
                   (o, "o"), (m, "m"), (l, "l"))
    Ho, n_o, Do, _, _ = _hn(o, "hnd")
    if o.dtype != torch.float32 or (Ho, n_o, Do) != (H, n_dst, D):
        raise ValueError("o must be float32 of shape (%d, %d, %d)" % (H, n_dst, D))
    _rows_f32(m, H, n_dst, "m")
    _rows_f32(l, H, n_dst, "l")
    with torch.cuda.device(dev):
        st = lib.osattn_csr_softmax(_DT[v.dtype], H, n_dst, n_src, D, row_ptr.data_ptr(),
                                    col_idx.data_ptr() if nnz else None, nnz,
                                    scores.data_ptr() if nnz else None, scores.stride(0),
                                    v.data_ptr(), v_sh, v_sn, o.data_ptr(), o.stride(0),
                                    o.stride(1), m.data_ptr(), l.data_ptr(), _stream())
    _check(st, "osattn_csr_softmax")
    return o, m, l


def bwd_workspace_bytes(dtype: torch.dtype, H: int, n_q: int, n_k: int, D: int,
                        causal: bool = False, cu_seqlens=None, max_seqlen: int = 0) -> int:
    num_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    return int(load().osattn_bwd_workspace_bytes(
        _DT[dtype], H, n_q, n_k, D, int(bool(causal)),
        None if cu_seqlens is None else cu_seqlens.data_ptr(), num_seqs, int(max_seqlen or 0)))


def bwd(q, k, v, o, do, m, l, scale: Optional[float] = None, causal: bool = False,
        cu_seqlens=None, max_seqlen: Optional[int] = None, layout: str = "hnd",
        check: bool = True, workspace: Optional[torch.Tensor] = None, out=None,
        noalloc: bool = False):
    """Attention backward on the GPU; returns (dq, dk, dv) in the input dtype.

    ``noalloc``: call osattn_bwd_noalloc, which uses the library's static
    per-device scratch instead of a workspace (nothing is allocated for it;
    problems needing more than NOALLOC_SCRATCH_BYTES are refused)."""
    lib = load()
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype of float32/float16/bfloat16")
    H, n_q, D, q_sh, q_sn = _hn(q, layout)
    Hk, n_k, Dk, kv_sh, kv_sn = _hn(k, layout)
    Hv, n_v, Dv, v_sh, v_sn = _hn(v, layout)
    if (Hk, Dk) != (H, D) or (Hv, n_v, Dv) != (H, n_k, D) or (v_sh, v_sn) != (kv_sh, kv_sn):
        raise ValueError("k and v must have the same shape and strides, matching q's H and D")
    Ho, n_o, Do, o_sh, o_sn = _hn(o, layout)
    if (Ho, n_o, Do) != (H, n_q, D):
        raise ValueError("o must be the forward's output, with q's shape")
    o_code = _o_code(o, q)
    _, _, _, do_sh, do_sn = _hn(do, layout)
    if do.shape != q.shape or (do_sh, do_sn) != (q_sh, q_sn) or do.dtype != q.dtype:
        raise ValueError("do must match q's dtype, shape and strides")
    _rows_f32(m, H, n_q, "m")
    _rows_f32(l, H, n_q, "l")
    scale = D ** -0.5 if scale is None else float(scale)
    cu, num_seqs, max_seqlen = _cu_args(cu_seqlens, max_seqlen, n_q, check)
    if out is None:
        # the ABI writes dq with q's strides and dk, dv with k's: allocate with them
        dq, dk, dv = (torch.empty_strided(t.size(), t.stride(), dtype=q.dtype, device=q.device)
                      for t in (q, k, k))
    else:
        dq, dk, dv = out
        _like(dq, q, q.dtype, "dq")
        _like(dk, k, q.dtype, "dk")
        _like(dv, k, q.dtype, "dv")
    dev = _one_gpu((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do"), (m, "m"), (l, "l"),
                   (cu, "cu_seqlens"), (dq, "dq"), (dk, "dk"), (dv, "dv"), (workspace, "workspace"))
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        with torch.cuda.device(dev):
            st = lib.osattn_bwd_noalloc(
                _DT[q.dtype], o_code, H, n_q, n_k, D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                o.data_ptr(), do.data_ptr(), q_sh, q_sn, kv_sh, kv_sn, o_sh, o_sn, m.data_ptr(),
                l.data_ptr(), scale, int(bool(causal)), None if cu is None else cu.data_ptr(),
                num_seqs, max_seqlen, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream())
        _check(st, "osattn_bwd_noalloc")
        return dq, dk, dv
    with torch.cuda.device(dev):
        need = lib.osattn_bwd_workspace_bytes(_DT[q.dtype], H, n_q, n_k, D, int(bool(causal)),
                                              None if cu is None else cu.data_ptr(), num_seqs,
                                              max_seqlen)
        if workspace is None:
            workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
        st = lib.osattn_bwd(_DT[q.dtype], o_code, H, n_q, n_k, D, q.data_ptr(), k.data_ptr(),
                            v.data_ptr(), o.data_ptr(), do.data_ptr(), q_sh, q_sn, kv_sh, kv_sn,
                            o_sh, o_sn, m.data_ptr(), l.data_ptr(), scale, int(bool(causal)),
                            None if cu is None else cu.data_ptr(), num_seqs, max_seqlen,
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                            _bytes(workspace), _stream())
    _check(st, "osattn_bwd")
    return dq, dk, dv
