"""osattn_bwd_noalloc (the backward without a workspace, for callers that cannot
allocate) against osattn_bwd on the same inputs, through the C ABI.

Three calls in a row on one GPU share its static scratch: the first needs the
most scratch (24 MiB of split partial sums), the later ones less, so stale
contents of a larger call sit in the array when a smaller one runs.  Each must
equal osattn_bwd with its own workspace bit for bit (same kernels, same plan),
and the last one is also held to the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import assert_grad_close, cu_dev, host, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, D, causal, n_q, n_k, H, lengths): decreasing scratch needs
    ("bf16", 128, True, 1024, 1024, 4, None),
    ("f32", 64, False, 4096, 1024, 1, None),
    ("f16", 64, True, 0, 0, 2, [200, 1, 77, 300]),
]


def _scratch_need(lib, c):
    dtype, D, causal, n_q, n_k, H, lengths = c
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    if lengths:
        n = sum(lengths)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
        return lib.osattn_bwd_workspace_bytes(code, H, n, n, D, int(causal), cu.data_ptr(),
                                              len(lengths), max(lengths))
    return lib.osattn_bwd_workspace_bytes(code, H, n_q, n_k, D, int(causal), None, 0, 0)


def test_noalloc_backward_equals_the_workspace_backward(osattn, oracle):
    lib = osattn.load()
    needs = [_scratch_need(lib, c) for c in CASES]
    assert needs[0] > needs[1] > needs[2] > 0, needs
    assert needs[0] <= osattn.NOALLOC_SCRATCH_BYTES
    for i, (dtype, D, causal, n_q, n_k, H, lengths) in enumerate(CASES):
        print("noalloc case", i, dtype, D, causal, n_q, n_k, H, lengths, flush=True)
        if lengths:
            n_q = n_k = sum(lengths)
        w = W.Workload("na", H, n_q, n_k, D, dtype, causal, 8100 + i, backward=True,
                       lengths=lengths)
        inp = W.make_inputs(w)
        q, k, v, do = (to_dev(x, dtype) for x in (inp.q, inp.k, inp.v, inp.do))
        cu = cu_dev(inp.cu_seqlens)
        kw = dict(scale=w.softmax_scale, causal=causal, cu_seqlens=cu)
        o, m, l = osattn.fwd(q, k, v, **kw)
        ref = osattn.bwd(q, k, v, o, do, m, l, **kw)
        got = osattn.bwd(q, k, v, o, do, m, l, noalloc=True, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), "case %d %s differs from osattn_bwd" % (i, name)
    # the last (smallest) call against the oracle as well
    rdq, rdk, rdv, *_ = oracle.attn_bwd(inp.q32, inp.k32, inp.v32, inp.do32, w.softmax_scale,
                                        causal=causal, cu_seqlens=inp.cu_seqlens)
    for name, g, r in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
        assert_grad_close(host(g), r, dtype, "noalloc %s" % name)


def test_noalloc_backward_runs_in_a_captured_graph(osattn):
    """The point of the entry: it can be captured (nothing allocates in the
    call).  Replays with new inputs between them equal eager osattn_bwd."""
    w = W.Workload("na_graph", 2, 600, 600, 128, "bf16", True, 8200, backward=True)
    inp = W.make_inputs(w)
    q, k, v, do = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, m, l = osattn.fwd(q, k, v, scale=w.softmax_scale, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        osattn.bwd(q, k, v, o, do, m, l, scale=w.softmax_scale, causal=True, noalloc=True,
                   out=(dq, dk, dv))  # warm-up outside capture
        with torch.cuda.graph(g, stream=stream):
            osattn.bwd(q, k, v, o, do, m, l, scale=w.softmax_scale, causal=True, noalloc=True,
                       out=(dq, dk, dv))
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(3):
        do.copy_(torch.randn(do.shape, generator=gen).to(do.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = osattn.bwd(q, k, v, o, do, m, l, scale=w.softmax_scale, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(a, b), "replay %d %s" % (rep, name)
