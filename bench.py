"""Benchmark: one quantized linear layer step on one MI355X.

A step is one pass of the layer's hot path over a batch of synthetic input:
[rotate +] quantize the activations (and the fused low-rank down projection
where the layer has one), then the block-scaled GEMM against weights that
were quantized beforehand (weights are prepared once per layer, outside the
timed region).  Inputs are resident in HBM before timing starts; the timed
steps cycle through enough independent buffer sets (activations, codes,
weights, outputs) that the working set exceeds 512 MB, twice the 256 MB
Infinity Cache, so every step reads from HBM.

Prints one JSON line.  ``value`` is whole-step GEMM throughput (the layer's
GEMM work, 2 M N K plus 2 M N r for a rank-r branch, per step / step time) in
TFLOP/s.  ``roofline`` describes the dominant kernel (the GEMM): its launches
over all buffer sets are captured in a HIP graph and replayed between HIP
events on the replay stream, which gives the average launch duration without
host launch gaps (the quantize kernel is timed the same way).  Its peak is the
route's: dense MXFP4 for MXFP4 x MXFP4, dense FP8 for an FP8 (MXFP8)
activation operand against 4-bit weights, bf16 for NVFP4 and the 16-bit
routes; the record also gives the fraction against the MFMA type the kernel
actually issues.  ``cpu_baseline`` times the CPU oracle on a bounded sample of
the same workload, on a pinned number of BLAS threads.

Default workload: svdq_r32, the MXFP4 x MXFP4 layer (4096 x 3072 x 3072 with
a rank-32 branch) on which the GEMM's MXFP4 roofline fraction is judged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time


def _host_threads() -> int:
    """Threads the CPU oracle may use: the CPUs this process may run on,
    capped at 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# the oracle's BLAS thread count is pinned before numpy loads its BLAS
BLAS_THREADS = _host_threads()
for _v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = str(BLAS_THREADS)

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fp8_quantized_linear_mxq_amd import workloads as wl  # noqa: E402

PEAK_TFLOPS = {"mxfp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0, "fp16": 2500.0}
HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "svdq_r32"
CSRC = os.path.join(ROOT, "fp8_quantized_linear_mxq_amd", "csrc")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def gemm_dtype(act_fmt: str, w_fmt: str) -> str:
    """The MFMA type the GEMM kernel issues for this pair."""
    if act_fmt == "MXFP4" and w_fmt == "MXFP4":
        return "mxfp4"
    if act_fmt == "NVFP4" and w_fmt == "NVFP4":
        return "fp16"
    return "bf16"


def route_peak_dtype(act_fmt: str, w_fmt: str) -> str:
    """The peak each route is judged against: dense MXFP4 for MXFP4 x MXFP4,
    dense FP8 for FP8 (MXFP8) activations against 4-bit MX / INT4 weights,
    bf16 for NVFP4 operands and unquantized bf16 activations."""
    if act_fmt == "MXFP4" and w_fmt == "MXFP4":
        return "mxfp4"
    if act_fmt == "MXFP8" and w_fmt in ("MXFP4", "INT4", "MIXED"):
        return "fp8"
    return "bf16"


def gemm_flops(w) -> float:
    """The layer's GEMM work: 2 M N K plus 2 M N r for the rank-r branch."""
    return 2.0 * w.m * w.n * w.k + 2.0 * w.m * w.n * w.rank


def quantize_bytes(w: wl.Workload, cols: int | None = None, rows: int | None = None) -> int:
    """Algorithmic HBM bytes of one activation quantize: read x once, write
    codes and scales (and u for the low-rank branch).  ``cols``/``rows``: the
    quantized shape when it is not M x K (the convolution's input pixels).
    NVFP4's dynamic tensor scale reads x a second time; that re-read is not
    algorithmic (it can come from the Infinity Cache) and is reported as
    measured traffic instead."""
    esz = 2 if w.act_dtype == "bf16" else 4
    k = w.k if cols is None else cols
    m = w.m if rows is None else rows
    rd = m * k * esz
    code = m * k // (1 if w.act_fmt == "MXFP8" else 2)
    scale = m * k // (16 if w.act_fmt == "NVFP4" else 32)
    wr = code + scale + (m * w.rank * 4 if w.rank else 0)
    return rd + wr


def mixed_weights(w: wl.Workload, mxq, torch):
    """Per-output-channel format choice on the conv weight and its groups,
    quantized once (outside the timed region).  Also returns the format
    choice's average duration (HIP events around five further calls)."""
    w0 = torch.from_numpy(wl.weights(w)).cuda()
    _, _, perm, counts, g = mxq.select_format(w0)
    cnt = counts.cpu().tolist()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        mxq.select_format(w0)
    e1.record()
    torch.cuda.synchronize()
    select_us = e0.elapsed_time(e1) / 5 * 1e3
    groups, off = [], 0
    for ci, fmt in enumerate((mxq.INT4, mxq.MXFP4, mxq.NVFP4)):
        rows = perm[off:off + cnt[ci]].long()
        groups.append(mxq.quantize(w0.index_select(0, rows).contiguous(), fmt,
                                   static_tensor_scale=g if fmt == mxq.NVFP4 else None)
                      if cnt[ci] else mxq.empty_qtensor(fmt, 0, w.k))
        off += cnt[ci]
    del w0
    return groups, perm, cnt, select_us


def make_sets(w: wl.Workload, n_sets: int, mxq, torch, mixed=None, conv="implicit"):
    """Device buffer sets: activations, pre-quantized weights, outputs.  The
    convolution layer's activations are the input's pixel rows (implicit
    im2col) or the explicit im2col matrix."""
    if w.w_fmt == "MIXED":
        lat = wl.conv_latent(w)
        act = lat.reshape(-1, lat.shape[2]) if conv == "implicit" else wl.im2col(lat)
        x0 = torch.from_numpy(np.ascontiguousarray(act).view(np.int16)).view(torch.bfloat16).cuda()
        del act, lat
        groups, perm = mixed[0], mixed[1]
        ws_n = max([mxq.workspace_size(mxq.OP_GEMM, w.m, g.rows, g.fmt) for g in groups] + [16])
        sets = []
        for i in range(n_sets):
            sets.append(dict(x=x0 if i == 0 else x0.clone(), groups=groups, perm=perm,
                             qa=mxq.empty_qtensor(mxq.MXFP8, w.m, x0.shape[1]),
                             ws=torch.empty((ws_n,), dtype=torch.uint8, device="cuda"),
                             out=torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")))
        torch.cuda.synchronize()
        return sets
    act = wl.activations(w)
    wt = wl.weights(w)
    fa, fw = wl_fmt(mxq, w.act_fmt), wl_fmt(mxq, w.w_fmt)
    bf16_act = w.act_fmt == "BF16"   # unquantized activations: the GEMM reads x itself
    if w.act_dtype == "bf16":
        x0 = torch.from_numpy(act.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x0 = torch.from_numpy(act).cuda()
    w0 = torch.from_numpy(wt).cuda()
    l1t = l2t = None
    if w.rank:
        l1, l2 = wl.lowrank_factors(w)
        l1t = torch.from_numpy(np.ascontiguousarray(l1.T).view(np.int16)).view(torch.bfloat16).cuda()
        l2t = torch.from_numpy(np.ascontiguousarray(l2.T).view(np.int16)).view(torch.bfloat16).cuda()
    sets = []
    for i in range(n_sets):
        x = x0.clone()
        qw = mxq.quantize(w0, fw, hadamard=w.hadamard)
        qa = mxq.bf16_operand(x) if bf16_act else mxq.empty_qtensor(fa, w.m, w.k)
        ws = torch.empty((max(16, mxq.workspace_size(mxq.OP_GEMM, w.m, w.n, fw),
                              0 if bf16_act else mxq.workspace_size(mxq.OP_QUANTIZE, w.m, w.k, fa)),),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")
        u = torch.empty((w.m, w.rank), dtype=torch.float32, device="cuda") if w.rank else None
        # L1 is part of the weight: where the fused quantize + projection
        # kernel runs (bf16 x, no rotation), it is packed once here, outside
        # the timed steps, into the order that kernel reads
        l1 = l1t.clone() if l1t is not None else None
        l1p = None
        if l1 is not None and x.dtype == torch.bfloat16 and w.hadamard == 0 and w.k % 128 == 0:
            l1p, l1 = mxq.pack_l1t(l1), None
        sets.append(dict(x=x, qw=qw, qa=qa, ws=ws, out=out, u=u, l1t=l1, l1p=l1p,
                         l2t=l2t.clone() if l2t is not None else None))
    del w0
    torch.cuda.synchronize()
    return sets


def wl_fmt(mxq, name: str) -> int:
    return {"MXFP4": mxq.MXFP4, "MXFP8": mxq.MXFP8, "NVFP4": mxq.NVFP4, "INT4": mxq.INT4,
            "BF16": mxq.BF16}[name]


def set_bytes(s) -> int:
    tot = 0
    vals = []
    for v in s.values():
        vals.extend(v if isinstance(v, list) else [v])
    for v in vals:
        if v is None:
            continue
        if hasattr(v, "codes"):
            for t in (v.codes, v.scales, v.tensor_scale):
                if t is not None:
                    tot += t.numel() * t.element_size()
        else:
            tot += v.numel() * v.element_size()
    return tot


def graph_avg_ms(torch, calls, min_launches: int) -> float:
    """Average duration of one call, from HIP-graph replays of all calls."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-min_launches // len(calls)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([t.get("num_threads", 1) for t in threadpool_info()
                if t.get("user_api") == "blas"] + [1])


def _oracle_conv_weights(w: wl.Workload):
    """The convolution layer's weights as the oracle prepares them: per-row
    format choice over {INT4, MXFP4, NVFP4} (one NVFP4 tensor scale over all
    of W), each row quantized in its chosen format and dequantized; returns
    float64 [N, K] in output-channel order and the rows per format."""
    from oracle import quantize as oq
    from oracle import select as osel

    wt = wl.weights(w)
    choice, _, _ = osel.select_formats(wt)
    g = oq.nvfp4_tensor_scale(wt)
    w_deq = np.empty(wt.shape, dtype=np.float64)
    counts = []
    for ci, fmt in enumerate(osel.PALETTE):
        rows = np.nonzero(choice == ci)[0]
        counts.append(int(rows.size))
        if rows.size:
            q = oq.quantize(wt[rows], fmt, tensor_scale=g if fmt == oq.NVFP4 else None)
            w_deq[rows] = oq.dequantize(q)
    return w_deq, counts


def cpu_baseline(w: wl.Workload, budget_s: float = 12.0) -> dict:
    """The oracle, as it stands, on a bounded row sample of the workload:
    activation quantize + float64 GEMM (+ low-rank branch) per row, in chunks
    of growing size, passing over the (at most 4096) sampled rows again until
    about budget_s seconds of CPU work are done.  For the convolution layer
    the rows are the first output pixels' im2col rows (MXFP8) against the
    mixed-format weights the oracle selects and quantizes beforehand (not
    timed)."""
    from oracle import gemm as og
    from oracle import hadamard as oh
    from oracle import quantize as oq
    from oracle.formats import round_to_bf16

    conv = w.w_fmt == "MIXED"
    prep = time.perf_counter()
    if conv:
        w_deq, counts = _oracle_conv_weights(w)
        lh, lw, lc = w.extra["latent"]
        lat_rows = 24                      # output image rows sampled
        # their im2col rows read latent rows 0 .. lat_rows (one row below)
        lat = wl.conv_latent(w)[:lat_rows + 1]
        cols = wl.im2col(lat)[:lat_rows * lw]
        vals = wl.bf16_to_f32(cols)
        del lat, cols
    else:
        wt = wl.weights(w)
        w_rot = oh.rotate(wt, w.hadamard, 7) if w.hadamard else wt
        w_deq = oq.dequantize(oq.quantize(w_rot, w.w_fmt))
        act = wl.activations(w, rows=min(w.m, 4096))
        vals = wl.bf16_to_f32(act) if w.act_dtype == "bf16" else act
    prep = time.perf_counter() - prep
    if w.rank:
        l1, l2 = wl.lowrank_factors(w)
        l1v = wl.bf16_to_f32(l1).astype(np.float64)
        l2v = wl.bf16_to_f32(l2).astype(np.float64)
    rows = 64 if not conv else 16
    done_rows, elapsed, pos = 0, 0.0, 0
    while elapsed < budget_s:
        pos = 0 if pos >= vals.shape[0] else pos
        chunk = vals[pos:pos + rows]
        pos += chunk.shape[0]
        t0 = time.perf_counter()
        r = oh.rotate(chunk, w.hadamard, 7) if w.hadamard else chunk
        a_deq = r if w.act_fmt == "BF16" else oq.dequantize(oq.quantize(r, w.act_fmt))
        y = og.linear(a_deq, w_deq)
        if w.rank:
            y = y + og.lowrank_down(chunk, l1v) @ l2v
        round_to_bf16(y)
        elapsed += time.perf_counter() - t0
        done_rows += chunk.shape[0]
        rows = min(rows * 2, 1024 if not conv else 256)
    flops = gemm_flops(w) * done_rows / w.m
    what = (f"{w.act_fmt} quantize of im2col rows + float64 GEMM against the oracle's "
            f"per-row formats (INT4/MXFP4/NVFP4 rows {counts[0]}/{counts[1]}/{counts[2]}; "
            f"selection and weight quantization {prep:.1f} s, not timed)") if conv else (
        f"{'bf16 activations' if w.act_fmt == 'BF16' else w.act_fmt + ' quantize'}"
        f"{' + H' + str(w.hadamard) if w.hadamard else ''} + float64 GEMM "
        f"against {w.w_fmt} weights{' + rank-' + str(w.rank) + ' branch' if w.rank else ''}")
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{done_rows} rows ({done_rows / vals.shape[0]:.1f} passes over {vals.shape[0]} "
                      f"of the {w.m} rows): oracle {what}, {elapsed:.1f} s",
            "cpu_model": cpu_model(), "blas_threads_pinned": BLAS_THREADS}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--conv", default="implicit", choices=["implicit", "im2col"],
                    help="convolution layer: gather the taps inside the GEMM from the "
                         "quantized input (implicit) or quantize the explicit im2col matrix")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the layer would shard by output channels, each GPU holding its own "
              "weight rows)", file=sys.stderr)
        return 2
    w = wl.WORKLOADS[args.workload]

    import torch

    import fp8_quantized_linear_mxq_amd as mxq
    mxq.load()
    torch.cuda.set_device(0)
    mixed = mixed_weights(w, mxq, torch) if w.w_fmt == "MIXED" else None
    one = make_sets(w, 1, mxq, torch, mixed, args.conv)
    per_set = set_bytes(one[0])
    n_sets = max(2, int(np.ceil(512e6 / per_set)) + 1)
    sets = one + make_sets(w, n_sets - 1, mxq, torch, mixed, args.conv)
    implicit = mixed is not None and args.conv == "implicit"
    if implicit:
        lat_h, lat_w, lat_c = w.extra["latent"]
    fa = wl_fmt(mxq, w.act_fmt)
    if mixed:
        # the activation format is read per step from the layer's table of
        # ten timestep buckets (every bucket MXFP8 for this convolution)
        act_table = wl.chameleon_act_table(1, mxq.MXFP8).reshape(-1)
        num_steps = max(1, args.steps)

    bf16_act = w.act_fmt == "BF16"

    def quant(s, i=0):
        if bf16_act:
            return
        if mixed:
            f = mxq.act_format_for_step(act_table, 1, wl.ACT_TABLE_BUCKETS, 0, i % num_steps,
                                        num_steps)
            if f != s["qa"].fmt:
                raise RuntimeError(f"table routes format {f}; the buffers hold {s['qa'].fmt}")
            mxq.quantize(s["x"], f, out=s["qa"])
        else:
            mxq.quantize(s["x"], fa, hadamard=w.hadamard, l1t=s["l1t"], l1p=s["l1p"], u=s["u"],
                         out=s["qa"], workspace=s["ws"])

    def gemm(s):
        if implicit:
            mxq.conv3x3_gemm_mixed(s["qa"], lat_h, lat_w, s["groups"], s["perm"], w.n,
                                   out=s["out"], workspace=s["ws"])
        elif mixed:
            mxq.gemm_mixed(s["qa"], s["groups"], s["perm"], w.n, out=s["out"],
                           workspace=s["ws"])
        else:
            mxq.gemm(s["qa"], s["qw"], u=s["u"], l2t=s["l2t"], out=s["out"], workspace=s["ws"])

    def route(s, i):
        # the activation format of step i from the timestep table (host)
        if mixed and not bf16_act:
            f = mxq.act_format_for_step(act_table, 1, wl.ACT_TABLE_BUCKETS, 0, i % num_steps,
                                        num_steps)
            if f != s["qa"].fmt:
                raise RuntimeError(f"table routes format {f}; the buffers hold {s['qa'].fmt}")

    # A step is the layer's launches (quantize, then GEMM) on one buffer set.
    # The steps are replayed from HIP graphs: one graph holds a sweep of
    # steps over every buffer set in order, so neither a small layer's
    # launches nor a graph launch per step sets the pace; a count of steps
    # that is not a whole number of sweeps ends with one-step graphs.  The
    # routing lookup still runs on the host for every step.  Graph replays
    # are bit-identical to the eager calls (tests/test_gpu_graph.py).
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        return g

    def one(s):
        quant(s)
        gemm(s)

    sweep_graph = capture(lambda: [one(s) for s in sets])
    step_graphs = [capture(lambda s=s: one(s)) for s in sets]
    torch.cuda.synchronize()

    def run_steps(first, count):
        i = first
        while i < first + count:
            if i % n_sets == 0 and first + count - i >= n_sets:
                for k in range(n_sets):
                    route(sets[k], i + k)
                sweep_graph.replay()
                i += n_sets
            else:
                route(sets[i % n_sets], i)
                step_graphs[i % n_sets].replay()
                i += 1

    run_steps(0, args.warmup)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, wall clock, synchronized both sides
    t0 = time.perf_counter()
    run_steps(0, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel durations: each kernel's launches over all buffer sets are
    # captured in a HIP graph and replayed between two HIP events on the
    # replay stream, so host launch gaps do not count
    q_ms = None if bf16_act else graph_avg_ms(torch, [lambda s=s: quant(s) for s in sets],
                                              args.steps)
    g_ms = graph_avg_ms(torch, [lambda s=s: gemm(s) for s in sets], args.steps)
    group_us = {}
    if mixed:
        # each format group's GEMM alone (same graph timing, output columns
        # through the group's slice of the permutation)
        off = 0
        for name, grp in zip(("INT4", "MXFP4", "NVFP4"), mixed[0]):
            if grp.rows:
                cols = mixed[1][off:off + grp.rows]
                if implicit:
                    one = [lambda s=s: mxq.conv3x3_gemm_mixed(s["qa"], lat_h, lat_w, [grp], cols,
                                                              w.n, out=s["out"], workspace=s["ws"])
                           for s in sets]
                else:
                    one = [lambda s=s: mxq.gemm(s["qa"], grp, n_out=w.n, w_out_col=cols,
                                                out=s["out"], workspace=s["ws"]) for s in sets]
                group_us[name] = round(graph_avg_ms(torch, one, args.steps // 4 or 1) * 1e3, 1)
            off += grp.rows
    if args.copy_probe:
        a = torch.empty((1 << 28,), dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    ms = wall / args.steps * 1e3
    flops = gemm_flops(w)
    gdt = gemm_dtype(w.act_fmt, w.w_fmt)
    rdt = route_peak_dtype(w.act_fmt, w.w_fmt)
    achieved = flops / (g_ms * 1e-3) / 1e12
    traffic = q2_fetch = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        # the counters were taken on the default form of each workload (the
        # convolution through the implicit im2col)
        ent = t.get(w.name) if (mixed is None or implicit) else None
        if ent and ent.get("kernel_source_digest") == kernel_source_digest():
            traffic = ent.get("gemm_hbm_bytes_per_launch")
            q2_fetch = ent.get("quantize_second_pass_fetch_bytes")
    qbytes = None if bf16_act else quantize_bytes(
        w, lat_c if implicit else None, lat_h * lat_w if implicit else None)
    rec = {
        "metric": "block-scaled GEMM TFLOP/s & % MXFP4 peak; quantize GB/s & % HBM BW",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gdt,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.m, "K": w.k, "N": w.n,
                   "activations": f"{w.act_dtype} -> {w.act_fmt}", "weights": w.w_fmt,
                   "hadamard": w.hadamard, "lowrank": w.rank, "buffer_sets": n_sets,
                   "working_set_MB": round(n_sets * per_set / 1e6, 1),
                   "gemm_flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_TFLOPS[rdt], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS[rdt], 4), "traffic": traffic,
                     "kernel": "gemm", "avg_launch_us": round(g_ms * 1e3, 3),
                     "route_peak_dtype": rdt, "mfma_dtype_issued": gdt,
                     "frac_vs_issued_mfma_peak": round(achieved / PEAK_TFLOPS[gdt], 4)},
        "gemm_pct_mxfp4_peak": round(achieved / PEAK_TFLOPS["mxfp4"], 4),
        "quantize": None if bf16_act else {
            "avg_launch_us": round(q_ms * 1e3, 3), "algorithmic_bytes": qbytes,
            "GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(qbytes / (q_ms * 1e-3) / 1e9 / HBM_GBPS, 4),
            "second_pass_fetch_bytes": q2_fetch if w.act_fmt == "NVFP4" else None},
        "kernel_source_digest": kernel_source_digest(),
    }
    if mixed:
        rec["config"]["weight_groups"] = {"INT4": mixed[2][0], "MXFP4": mixed[2][1],
                                          "NVFP4": mixed[2][2]}
        rec["format_choice_us"] = round(mixed[3], 1)
        rec["group_gemm_us"] = group_us
        rec["config"]["conv"] = ("implicit im2col: quantize the 128x128x2560 input once, "
                                 "gather the 3x3 taps in the GEMM") if implicit else \
            "explicit im2col: quantize the 16384x23040 matrix"
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
