#!/usr/bin/env python3
"""Online-softmax attention throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all]

A step is one pass of the attention hot path over one batch of seeded
synthetic input already resident in HBM: the forward (one fused kernel, plus
the combine kernel when the key range is split) and the fused backward (its
pre-pass, the dK/dV and dQ kernel, and a split reduction where one is used);
--fwd-only times the forward alone.  The default workload is causal N=4096
H=16 D=128 bf16, the largest of the named workloads.  After W untimed steps, K steps are timed
between two device synchronisations, replayed from captured HIP graphs of 20
steps so host launch overhead does not gate the GPU; value is the algorithmic
TFLOP/s of the whole step (forward 4 N_q N_k D H, halved for causal, summed per
sequence for varlen; backward 2.5x the forward).  Rank 0 prints ONE JSON line
(one per workload with --all) that also carries:

  forward      : the forward kernel's algorithmic FLOPs per launch over its
                 average device duration (HIP events around a replayed graph of
                 back-to-back launches on the launch stream), against MI355X's
                 dense MFMA peak for its dtype;
                 traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE /
                 WRITE_SIZE counters recorded in profiles/traffic.json, or null
                 when the kernel sources changed since they were recorded;
  backward     : the same record for the backward's kernels (its pre-pass, the
                 dK/dV and dQ kernel, a split reduction where one runs);
  roofline     : the record, of those two, whose launch takes the longer: the
                 step's dominant kernel (the backward's, on a forward and
                 backward step);
  cpu_baseline : the f64 CPU oracle timed on this host's cores on a bounded
                 row sample of the same workload (a reported baseline only),
                 with the CPU model and the OpenMP thread setting;
  parity       : max error of sampled output rows against that oracle, taken
                 eagerly before timing and again after the last replayed step,
                 and of every gradient of one head (one per sequence, varlen).
                 A parity failure prints the line with value null and exits 1.
Only one GPU is used; --gpus above 1 exits with a message.
"""
import argparse
import dataclasses
import glob
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % of MFMA peak on 1×MI355X"
DEFAULT_WORKLOAD = "causal_n4096_h16_d128_bf16"
# MI355X dense MFMA peaks (TFLOP/s) by MFMA input type.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}
TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 1e-2}


def fwd_flops(w) -> float:
    if w.lengths is not None:
        per = 2.0 if w.causal else 4.0
        return float(sum(per * L * L * w.D * w.H for L in w.lengths))
    f = 4.0 * w.n_q * w.n_k * w.D * w.H
    return f / 2 if w.causal else f


def bwd_flops(w) -> float:
    return 2.5 * fwd_flops(w)


_COMMENT_OR_STRING = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'', re.S)


def _code_only(text: str) -> str:
    """C/C++/HIP source with comments removed and whitespace collapsed."""
    text = _COMMENT_OR_STRING.sub(lambda m: " " if m.group(0).startswith("/") else m.group(0), text)
    return " ".join(text.split())


def kernel_source_sha() -> str:
    """Hash of the kernel sources' code (comments and layout ignored): recorded
    counters are reported only while the code they were taken on is unchanged."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "online_softmax_attention_amd", "csrc", "*"))):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# The backward's kernels (fp16/bf16, f32), as named in profiles/traffic.json.
# The varlen backward writes its work list first; the reductions run only when
# the plan splits keys or queries over partial sums.
BWD_KERNELS = {False: "bwd16_pre+bwd16_kernel+bwd16_reduce",
               True: "bwd_pre+bwd_dkdv32+bwd_dq32+reduce_parts_f32"}


def fwd_kernel_name(w, torch, split: bool) -> str:
    """The forward kernel the library's plan picks for workload w: 16-bit
    dense / causal problems whose 128-row tiles (causal: tile pairs) fill the
    device, or that split the keys, and varlen problems whose sequences average
    2048 rows or more run the 8-wave pipelined kernel; the rest the tiled one."""
    if w.dtype == "f32":
        return "fwd32_kernel"
    if w.lengths:
        return "fwd_wide_kernel" if w.n_q >= 2048 * len(w.lengths) else "fwd16_kernel"
    if split:
        return "fwd_wide_kernel"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t = (w.n_q + 127) // 128
    pair = w.causal and w.H * t >= cus
    items = w.H * ((t + 1) // 2 if pair else t)
    return "fwd_wide_kernel" if items >= cus else "fwd16_kernel"


# FETCH_SIZE and WRITE_SIZE scale factors to true bytes, from the calibration
# runs in profiles/hbm_counter_calibration.md (a 256 MiB copy: 262144 KiB moved,
# FETCH_SIZE 131084.0 KiB, WRITE_SIZE 262144.0 KiB per dispatch).
FETCH_SCALE = 262144.0 / 131084.0
WRITE_SCALE = 1.0


def kernel_identifiers(name: str) -> set:
    """The identifiers in a kernel name as rocprofv3 prints it, mangled
    (_ZN6osattn12bwd16_kernelI...: length-prefixed) or demangled."""
    if name.startswith("_Z"):
        out, i = set(), 0
        while i < len(name):
            m = re.match(r"\d+", name[i:])
            if not m:
                i += 1
                continue
            n, j = int(m.group(0)), i + len(m.group(0))
            out.add(name[j:j + n])
            i = j + n
        return out
    return set(re.findall(r"[A-Za-z_][A-Za-z0-9_]*", name))


def counter_kib_per_launch(csv_path: str, kernels: str, counter: str):
    """The counter's KiB per launch of the '+'-separated kernels, from a rocprofv3
    counter_collection CSV: the sum over every dispatch of those kernels divided
    by the launch count (the fewest dispatches of any kernel present), with the
    dispatches per launch of each kernel. A launch may run a listed kernel more
    than once (one reduction per gradient) or not at all (no split partials)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            idents = kernel_identifiers(r["Kernel_Name"])
            for k in kernels.split("+"):
                if k in idents or k + "_kernel" in idents:
                    per.setdefault(k, []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit("no %s dispatches of %s in %s" % (counter, kernels, csv_path))
    launches = min(len(v) for v in per.values())
    counts = {k: len(per.get(k, [])) / launches for k in kernels.split("+")}
    return sum(sum(v) for v in per.values()) / launches, counts


def record_traffic(key: str, kernels: str, fetch_csv: str, write_csv: str) -> dict:
    """Write profiles/traffic.json[key] from a FETCH_SIZE and a WRITE_SIZE pass."""
    fetch, counts = counter_kib_per_launch(fetch_csv, kernels, "FETCH_SIZE")
    write, _ = counter_kib_per_launch(write_csv, kernels, "WRITE_SIZE")
    rec = {"kernel": kernels, "dispatches_per_launch": counts,
           "fetch_kib": fetch, "write_kib": write, "fetch_scale": FETCH_SCALE,
           "write_scale": WRITE_SCALE, "source_sha": kernel_source_sha(),
           "traffic_bytes": (fetch * FETCH_SCALE + write * WRITE_SCALE) * 1024.0}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = {}
    if os.path.exists(path):
        with open(path) as f:
            allrec = json.load(f)
    allrec[key] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def recorded_traffic(workload: str, kernel: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel") != kernel or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("traffic_bytes")


def upload(inp, torch, np):
    def up(x):
        if x is None:
            return None
        if inp.w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    cu = None
    if inp.cu_seqlens is not None:
        cu = torch.tensor(inp.cu_seqlens, dtype=torch.int32, device="cuda")
    return up(inp.q), up(inp.k), up(inp.v), up(inp.do), cu


def sample_rows(w, np, per_head=24, seed=1):
    rng = np.random.default_rng(seed)
    rows = []
    for h in range(w.H):
        pick = set(rng.integers(0, w.n_q, per_head).tolist()) | {0, w.n_q - 1}
        rows += [h * w.n_q + i for i in sorted(pick)]
    return np.array(rows, dtype=np.int64)


def admitted_count(w, i, cu):
    if cu is not None:
        b = int(np.searchsorted(cu, i, side="right")) - 1
        lo, hi = int(cu[b]), int(cu[b + 1])
        return (i + 1 - lo) if w.causal else (hi - lo)
    return (i + 1) if w.causal else w.n_k


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, oracle, np, budget_s=10.0):
    """Time the oracle forward on row chunks of the workload until ~budget_s."""
    rng = np.random.default_rng(12345)
    order = rng.permutation(w.H * w.n_q)
    chunk = 256
    flops = 0.0
    spent = 0.0
    rows_done = 0
    passes = 0
    pos = 0
    cu = inp.cu_seqlens
    while spent < budget_s and passes < 1000:
        rows = np.sort(order[pos:pos + chunk])
        t0 = time.perf_counter()
        oracle.attn_fwd(inp.q32, inp.k32, inp.v32, w.softmax_scale, causal=w.causal,
                        cu_seqlens=cu, rows=rows)
        spent += time.perf_counter() - t0
        flops += sum(4.0 * admitted_count(w, int(r % w.n_q), cu) * w.D for r in rows)
        rows_done += len(rows)
        pos += chunk
        if pos >= len(order):
            pos = 0
            passes += 1
        chunk = min(chunk * 2, 16384)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS", "unset"),
            "sample": "f64 two-pass oracle forward on %d random (head, query) rows of the "
                      "workload (%d full passes over its %d rows; %.1f s wall on %d threads)"
                      % (rows_done, passes, w.H * w.n_q, spent, oracle.num_threads())}


def capture(fn, n, torch, stream):
    """A graph of n back-to-back calls of fn() on `stream` (nothing allocates)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                fn()
    return g


def run_workload(name, steps, warmup, torch, np, osa, W, oracle, with_cpu=True, backward=True):
    w = W.WORKLOADS[name]
    if w.backward != backward:  # same q, k, v draws; dO drawn after them
        w = dataclasses.replace(w, backward=backward)
    inp = W.make_inputs(w)
    q, k, v, do, cu = upload(inp, torch, np)
    max_seqlen = max(w.lengths) if w.lengths else None
    H, D = w.H, w.D
    o = torch.empty((H, w.n_q, D), dtype=torch.float32, device="cuda")
    m = torch.empty((H, w.n_q), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    fwd_out = (o, m, l)
    num_seqs = 0 if cu is None else cu.numel() - 1
    fws_bytes = osa.load().osattn_fwd_workspace_bytes(
        osa._DT[q.dtype], H, w.n_q, w.n_k, D, int(w.causal),
        None if cu is None else cu.data_ptr(), num_seqs, max_seqlen or 0)
    fws = torch.empty(max(int(fws_bytes), 256), dtype=torch.uint8, device="cuda")

    def fwd():
        osa.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal, cu_seqlens=cu,
                max_seqlen=max_seqlen, check=False, out=fwd_out, workspace=fws)

    bw = None
    if w.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nbytes = osa.bwd_workspace_bytes(q.dtype, H, w.n_q, w.n_k, D, w.causal, cu, max_seqlen or 0)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")

        def bw():
            osa.bwd(q, k, v, o, do, m, l, scale=w.softmax_scale, causal=w.causal, cu_seqlens=cu,
                    max_seqlen=max_seqlen, check=False, workspace=ws, out=(dq, dk, dv))

    def step():
        fwd()
        if bw is not None:
            bw()

    rows = sample_rows(w, np)
    ro, rm, rl = oracle.attn_fwd(inp.q32, inp.k32, inp.v32, w.softmax_scale, causal=w.causal,
                                 cu_seqlens=inp.cu_seqlens, rows=rows)

    def parity():
        torch.cuda.synchronize()
        og = o.reshape(-1, D).cpu().numpy()[rows]
        return float(np.max(np.abs(og - ro)))

    def grad_parity(head):
        """Largest max|g - g_ref| / max|g_ref| over dq, dk, dv of one head."""
        torch.cuda.synchronize()
        got = [t[head].float().cpu().numpy() for t in (dq, dk, dv)]
        spans = ([(0, w.n_q)] if inp.cu_seqlens is None else
                 [(int(a), int(b)) for a, b in zip(inp.cu_seqlens[:-1], inp.cu_seqlens[1:]) if b > a])
        ref = [np.zeros((w.n_q, D)), np.zeros((w.n_k, D)), np.zeros((w.n_k, D))]
        for a, b in spans:
            cut = (lambda x: np.ascontiguousarray(x[head:head + 1, a:b])) if inp.cu_seqlens is not None \
                else (lambda x: np.ascontiguousarray(x[head:head + 1]))
            r = oracle.attn_bwd(cut(inp.q32), cut(inp.k32), cut(inp.v32), cut(inp.do32),
                                w.softmax_scale, causal=w.causal)
            for i in range(3):
                if inp.cu_seqlens is None:
                    ref[i] = r[i][0]
                else:
                    ref[i][a:b] = r[i][0]
        return max(float(np.max(np.abs(g - rf)) / max(float(np.max(np.abs(rf))), 1e-2))
                   for g, rf in zip(got, ref))

    stream = torch.cuda.Stream()
    grad_head = H - 1
    with torch.cuda.stream(stream):
        step()
        err_eager = parity()  # eager parity on sampled rows, before any timing
        gerr_eager = grad_parity(grad_head) if bw is not None else None
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()

    # Timed region: K steps replayed from captured graphs of G steps each, so
    # that host launch overhead does not gate the GPU.
    G = 20
    g_steps = capture(step, G, torch, stream)
    if steps <= 0:  # auto: about 0.5 s of timed work, at least 100 steps
        t0 = time.perf_counter()
        g_steps.replay()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / G
        steps = int(min(20000, max(100, 0.5 / max(per, 1e-7))))
    steps = (steps + G - 1) // G * G
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record()
        for _ in range(steps // G):
            g_steps.replay()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    err_graph = parity()  # outputs of the last replayed step
    gerr_graph = grad_parity(grad_head) if bw is not None else None
    ms_per_step = wall * 1e3 / steps
    step_flops = fwd_flops(w) + (bwd_flops(w) if w.backward else 0.0)
    value = step_flops / (wall / steps) / 1e12
    err_o = max(err_eager, err_graph)
    parity_rec = {"max_abs_err_o": err_o, "tol": TOL[w.dtype], "rows": int(len(rows)),
                  "ok": bool(err_o <= TOL[w.dtype])}
    if bw is not None:
        gerr = max(gerr_eager, gerr_graph)
        parity_rec.update({"max_rel_err_grad": gerr, "grad_tol": TOL[w.dtype] ,
                           "grad_head": grad_head,
                           "ok": bool(parity_rec["ok"] and gerr <= TOL[w.dtype])})

    # The forward kernel's record: FLOPs per launch over its average device
    # duration, from HIP events around replays of a graph of back-to-back
    # forward launches on the launch stream.
    kern = fwd_kernel_name(w, torch, bool(fws_bytes) and not w.lengths)
    if fws_bytes:  # varlen work list before, or split-KV combine after, the forward
        kern = ("varlen_schedule_kernel+" + kern) if w.lengths else (kern + "+fwd_combine_kernel")
    n_per, reps = 50, 10
    g_fwd = capture(fwd, n_per, torch, stream)
    with torch.cuda.stream(stream):
        g_fwd.replay()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(reps):
            g_fwd.replay()
        f1.record()
    torch.cuda.synchronize()
    avg_ms = f0.elapsed_time(f1) / (n_per * reps)
    achieved = fwd_flops(w) / (avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    fwd_rec = {"pass": "forward", "bound": "mfma", "achieved": achieved, "peak": peak,
               "unit": "TFLOP/s", "frac": achieved / peak, "traffic": recorded_traffic(name, kern),
               "kernel": kern, "launch_us_avg": avg_ms * 1e3, "launches": n_per * reps,
               "flops_per_launch": fwd_flops(w)}
    bwd_rec = None
    if bw is not None:
        # Backward alone: same protocol as the forward's record above.
        g_bwd = capture(bw, n_per, torch, stream)
        with torch.cuda.stream(stream):
            g_bwd.replay()
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b0.record()
            for _ in range(reps):
                g_bwd.replay()
            b1.record()
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / (n_per * reps)
        bwd_ach = bwd_flops(w) / (bwd_ms * 1e-3) / 1e12
        bkern = BWD_KERNELS[w.dtype == "f32"]
        if w.lengths:
            bkern = "varlen_schedule_kernel+" + bkern
        bwd_rec = {"pass": "backward", "bound": "mfma", "achieved": bwd_ach, "peak": peak,
                   "unit": "TFLOP/s", "frac": bwd_ach / peak,
                   "traffic": recorded_traffic(name + "+bwd", bkern), "kernel": bkern,
                   "launch_us_avg": bwd_ms * 1e3, "launches": n_per * reps,
                   "flops_per_launch": bwd_flops(w)}
    # The step's dominant kernel: the launch that takes the longer.
    roofline = fwd_rec
    if bwd_rec is not None and bwd_rec["launch_us_avg"] > fwd_rec["launch_us_avg"]:
        roofline = bwd_rec
    if not parity_rec["ok"]:
        value = None  # a step that computes the wrong result has no throughput
    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic: seeded N(0,1) q,k,v%s (numpy default_rng seed %d) rounded to %s"
                   % (",dO" if w.backward else "", w.seed, w.dtype),
           "config": {"workload": name, "H": H, "n_q": w.n_q, "n_k": w.n_k, "D": D,
                      "causal": w.causal, "varlen_seqs": len(w.lengths) if w.lengths else 0,
                      "pass": "fwd+bwd" if w.backward else "fwd",
                      "layout": "(H, N, D)", "output": "O f32, m and l f32",
                      "launch": "graphs of %d steps replayed" % G},
           "pct_of_peak": None if value is None else 100.0 * value / peak,
           "event_ms_per_step": e0.elapsed_time(e1) / steps,
           "roofline": roofline, "forward": fwd_rec, "parity": parity_rec}
    if bwd_rec is not None:
        out["backward"] = bwd_rec
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp, oracle, np)
    return out


def run_pruned(name, rho, steps, warmup, torch, np, osa, W, oracle):
    """Tile-pruned dense forward against the exact forward at one workload's shape."""
    w = W.WORKLOADS[name]
    if w.causal or w.lengths or w.dtype == "f32":
        raise SystemExit("--prune needs a dense fp16/bf16 workload (got %s)" % name)
    inp = W.make_inputs(w)
    q, k, v, _, _ = upload(inp, torch, np)
    H, D = w.H, w.D
    o = torch.empty((H, w.n_q, D), dtype=torch.float32, device="cuda")
    m = torch.empty((H, w.n_q), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    o2, m2, l2 = torch.empty_like(o), torch.empty_like(m), torch.empty_like(m)
    ws = torch.empty(0, dtype=torch.uint8, device="cuda")

    def pruned():
        osa.fwd_pruned(q, k, v, rho, scale=w.softmax_scale, out=(o, m, l))

    def exact():
        osa.fwd(q, k, v, scale=w.softmax_scale, check=False, out=(o2, m2, l2), workspace=ws)

    hs = min(H, 2)  # the pruned oracle on the first heads only (it scores every tile)
    ro, rm, rl, admit, margin = oracle.attn_fwd_pruned(inp.q32[:hs], inp.k32[:hs], inp.v32[:hs],
                                                       w.softmax_scale, rho, 128, 128)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(warmup, 1)):
            pruned()
            exact()
    torch.cuda.synchronize()
    err = float(np.max(np.abs(o[:hs].cpu().numpy() - ro)))
    n_per = 50  # the launch protocol of the exact forward's roofline
    reps = max(10, steps // n_per)
    times = {}
    for tag, fn in (("pruned", pruned), ("exact", exact)):
        g = capture(fn, n_per, torch, stream)
        with torch.cuda.stream(stream):
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
        torch.cuda.synchronize()
        times[tag] = e0.elapsed_time(e1) / (n_per * reps)
    pruned_frac = float(1.0 - admit.mean())
    flops_exact = fwd_flops(w)
    # executed: every tile's scores, the P.V product of admitted tiles only
    flops_exec = flops_exact / 2 * (1.0 + float(admit.mean()))
    peak = PEAK_TFLOPS[w.dtype]
    value = flops_exec / (times["pruned"] * 1e-3) / 1e12
    return {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
            "steps": n_per * reps, "warmup": warmup, "ms_per_step": times["pruned"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic: seeded N(0,1) q,k,v (numpy default_rng seed %d) rounded to %s"
                    % (w.seed, w.dtype),
            "config": {"workload": name, "H": H, "n_q": w.n_q, "n_k": w.n_k, "D": D,
                       "pass": "fwd_pruned", "rho": rho, "tile": "128 queries x 128 keys",
                       "flops": "executed: all tile scores + P.V of admitted tiles"},
            "pct_of_peak": 100.0 * value / peak,
            "roofline": {"bound": "mfma", "achieved": value, "peak": peak, "unit": "TFLOP/s",
                         "frac": value / peak, "kernel": "fwd16_pruned_kernel",
                         "traffic": recorded_traffic(name + "+prune", "fwd16_pruned_kernel"),
                         "launch_us_avg": times["pruned"] * 1e3},
            "pruning": {"rho": rho, "tiles_pruned_frac": pruned_frac, "oracle_heads": hs,
                        "min_decision_margin": margin, "pruned_ms": times["pruned"],
                        "exact_ms": times["exact"], "speedup": times["exact"] / times["pruned"],
                        "exact_tflops": flops_exact / (times["exact"] * 1e-3) / 1e12},
            "parity": {"max_abs_err_o_vs_pruned_oracle": err, "tol": TOL[w.dtype],
                       "ok": bool(err <= TOL[w.dtype]),
                       # a decision within 1e-4 of its threshold may round either way
                       "decisions_unambiguous": bool(margin > 1e-4)}}


def run_csr(steps, warmup, torch, np, osa, W, oracle):
    """CSR segment softmax on the synthetic CSR workload: HBM roofline."""
    c = W.CSR_WORKLOAD
    row_ptr, col_idx = W.csr_graph(c["seed"], c["n_dst"], c["n_src"], c["mean_degree"],
                                   c["max_degree"])
    H, D, nnz = c["H"], c["D"], len(col_idx)
    scores, v, vw = W.csr_inputs(c["seed"], H, c["n_src"], nnz, D, c["dtype"])
    rp, ci = torch.tensor(row_ptr, device="cuda"), torch.tensor(col_idx, device="cuda")
    sc = torch.tensor(scores, device="cuda")
    if c["dtype"] == "bf16":
        vd = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        vd = torch.from_numpy(np.ascontiguousarray(v)).cuda()
    o = torch.empty((H, c["n_dst"], D), dtype=torch.float32, device="cuda")
    m = torch.empty((H, c["n_dst"]), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)

    def run():
        osa.csr_softmax(rp, ci, sc, vd, out=(o, m, l))

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(warmup, 1)):
            run()
    torch.cuda.synchronize()
    ro, rm, rl = oracle.csr_softmax(row_ptr, col_idx, scores, vw)
    nonempty = np.diff(row_ptr) > 0
    err = float(np.max(np.abs(o.cpu().numpy()[:, nonempty] - ro[:, nonempty])))
    n_per = 50
    reps = max(10, steps // n_per)
    g = capture(run, n_per, torch, stream)
    with torch.cuda.stream(stream):
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (n_per * reps)
    esz = 4 if c["dtype"] == "f32" else 2
    # algorithmic bytes: CSR once, every edge's score and gathered value row per
    # head, the outputs once
    nbytes = (4 * (c["n_dst"] + 1) + 4 * nnz + H * nnz * (4 + D * esz)
              + H * c["n_dst"] * (D * 4 + 8))
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "CSR segment softmax GB/s on 1\u00d7MI355X", "value": achieved, "unit": "GB/s",
            "n_gpus": 1, "steps": n_per * reps, "warmup": warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c["dtype"],
            "data": "synthetic: seeded heavy-tailed random CSR (mean degree %d), N(0,1) edge scores "
                    "and values" % c["mean_degree"],
            "config": {"workload": c["name"], "H": H, "n_dst": c["n_dst"], "n_src": c["n_src"],
                       "nnz": nnz, "D": D, "pass": "csr_softmax"},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": 8000.0, "unit": "GB/s",
                         "frac": achieved / 8000.0, "kernel": "csr_softmax_kernel",
                         "traffic": recorded_traffic(c["name"], "csr_softmax_kernel"),
                         "algorithmic_bytes": nbytes, "launch_us_avg": ms * 1e3},
            "parity": {"max_abs_err_o": err, "tol": TOL[c["dtype"]], "ok": bool(err <= TOL[c["dtype"]])}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0 = auto, ~0.5 s)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true", help="one JSON line per workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--prune", type=float, default=None, metavar="RHO",
                    help="time the tile-pruned dense forward (threshold RHO) against the exact one")
    ap.add_argument("--csr", action="store_true",
                    help="time the CSR segment softmax on the synthetic CSR workload")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (the default; kept for old command lines)")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the forward alone (the step is one forward pass)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 10 plain device copies of BYTES bytes (calibrates the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters against a known size)")
    ap.add_argument("--read-probe", type=int, default=0, metavar="BYTES",
                    help="only run 10 reads of BYTES bytes with 16-byte buffer loads "
                         "(libosattn_probe.so), to calibrate FETCH_SIZE for those loads")
    ap.add_argument("--probe-lds", action="store_true",
                    help="with --read-probe: the loads go to LDS (buffer_load ... lds)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("KEY", "KERNELS", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json[KEY] from rocprofv3 FETCH_SIZE and WRITE_SIZE "
                         "counter_collection CSVs, summed over the '+'-separated KERNELS (no GPU)")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(--gpus %d requested)\n" % args.gpus)
        sys.exit(2)

    import torch

    import online_softmax_attention_amd as osa
    import oracle
    import workloads as W

    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(1)
    if args.copy_probe:
        n = args.copy_probe // 4
        src = torch.arange(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "copies": 10}), flush=True)
        return
    if args.read_probe:
        import ctypes
        probe = ctypes.CDLL(os.path.join(ROOT, "online_softmax_attention_amd", "libosattn_probe.so"))
        probe.osattn_probe_read16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]
        probe.osattn_probe_read16.restype = ctypes.c_int
        src = torch.arange(args.read_probe // 4, dtype=torch.int32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(10):
            rc = probe.osattn_probe_read16(src.data_ptr(), args.read_probe, int(args.probe_lds),
                                           sink.data_ptr(), stream)
            if rc != 0:
                sys.stderr.write("read probe failed: %d\n" % rc)
                sys.exit(1)
        torch.cuda.synchronize()
        print(json.dumps({"read_probe_bytes": args.read_probe, "to_lds": bool(args.probe_lds),
                          "reads": 10}), flush=True)
        return
    osa.load()
    if args.csr:
        print(json.dumps(run_csr(args.steps, args.warmup, torch, np, osa, W, oracle)), flush=True)
        return
    if args.prune is not None:
        res = run_pruned(args.workload, args.prune, args.steps, args.warmup, torch, np, osa, W,
                         oracle)
        print(json.dumps(res), flush=True)
        return
    names = W.ORDER if args.all else [args.workload]
    failed = False
    for name in names:
        res = run_workload(name, args.steps, args.warmup, torch, np, osa, W, oracle,
                           with_cpu=not args.no_cpu, backward=not args.fwd_only)
        print(json.dumps(res), flush=True)
        failed |= not res["parity"]["ok"]
    if failed:
        sys.stderr.write("parity against the oracle failed: see the parity record\n")
        sys.exit(1)


if __name__ == "__main__":
    main()
