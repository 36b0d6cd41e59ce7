"""Benchmark of the gfx950 low-bit-weight GEMM on one MI355X.

One step = the ternary MLP pair of a 1024x1024 denoising step at 4608 tokens
(4096 image + 512 text): X bf16 [4608 x 3072] -> up-proj [9216 x 3072] with the
exact-erf GELU fused into its epilogue -> down-proj [3072 x 9216], group-128
fp16 scales. Inputs are seeded synthetic data, resident in HBM before timing;
the one-time packing is not in the step.

Printed: ONE JSON line with TFLOP/s of the step (value), the roofline object of
the dominant kernel (the large-M MFMA GEMM; per-launch time from HIP events on
the launch stream), the CPU oracle timed on a bounded sample (cpu_baseline),
and the small-M weight-streaming GB/s over a 100-linear MMDiT weight set at
M = 16 and M = 1 (small_m).

    python bench.py [--gpus 1] [--steps 100] [--warmup 300] [--no-cpu] [--no-small]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ternary W×A16 GEMM TFLOP/s + % MFMA peak at M=4608; GB/s % HBM peak at M≤16"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_large_config3_traffic.json")


def kernel_source_sha() -> str:
    """Hash of the large-M kernel source (gemm_large.hip and common.h) with
    comments and blank lines removed, so that counter data stays attached to
    the code it was measured on."""
    h = hashlib.sha256()
    for f in ("gemm_large.hip", "common.h"):
        with open(os.path.join(ROOT, "bit_weight_gemm_int2_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def dev16(torch, bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(dtype)


def bench_large(torch, lb, steps, warmup, settle_s=0.0):
    import workloads as wl
    up, down = wl.config3()
    M, K1, N1, N2 = up.M, up.K, up.N, down.N
    x = dev16(torch, up.x, torch.bfloat16)
    pu = lb.pack_ternary(torch.from_numpy(up.codes).cuda())
    su = dev16(torch, up.scales, torch.float16)
    pd = lb.pack_ternary(torch.from_numpy(down.codes).cuda())
    sd = dev16(torch, down.scales, torch.float16)
    h = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
    ws = lb.new_workspace(max(lb.workspace_bytes("ternary", M, N1, K1), lb.workspace_bytes("ternary", M, N2, N1)))

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        lb.gemm(x, pu, su, "ternary", activation="gelu", out=h, workspace=ws)
        if evs is not None:
            evs[1].record()
        lb.gemm(h, pd, sd, "ternary", out=y, workspace=ws)
        if evs is not None:
            evs[2].record()

    # The GPU's clock ramps up over the first fraction of a second of load:
    # the step first runs untimed for settle_s seconds of wall time (in
    # batches of 50), then the W warm-up steps, then the K timed steps.
    settle_steps = 0
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(50):
            step()
        settle_steps += 50
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    launches = []
    for e in evs:
        launches.append(e[0].elapsed_time(e[1]))
        launches.append(e[1].elapsed_time(e[2]))
    flop_launch = 2.0 * M * N1 * K1                     # == 2 * M * N2 * K2
    flop_step = 2 * flop_launch
    avg_launch_ms = float(np.mean(launches))
    up_ms = float(np.mean(launches[0::2]))
    down_ms = float(np.mean(launches[1::2]))

    def spread(v):
        return {"min": round(float(np.min(v)), 4), "median": round(float(np.median(v)), 4),
                "max": round(float(np.max(v)), 4)}
    return dict(M=M, N1=N1, K1=K1, N2=N2, total_ms=total_ms, wall_s=wall, flop_step=flop_step,
                flop_launch=flop_launch, avg_launch_ms=avg_launch_ms, up_ms=up_ms, down_ms=down_ms,
                settle_steps=settle_steps, up_spread=spread(launches[0::2]), down_spread=spread(launches[1::2]),
                step_spread=spread([a + b for a, b in zip(launches[0::2], launches[1::2])]))


def bench_dense(torch, M, N1, K1, N2, steps=50, warmup=50):
    """Context: the dense bf16 GEMM that the low-bit layer replaces, through
    PyTorch's library path (torch.matmul -> hipBLASLt), on the same two shapes
    (no activation). 2-D contiguous operands only."""
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((M, K1), generator=g, device="cuda").bfloat16()
    wu = (torch.randn((K1, N1), generator=g, device="cuda") * 0.02).bfloat16().contiguous()
    wd = (torch.randn((N1, N2), generator=g, device="cuda") * 0.02).bfloat16().contiguous()
    h = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        torch.matmul(x, wu, out=h)
        torch.matmul(h, wd, out=y)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        torch.matmul(x, wu, out=h)
        e[1].record()
        torch.matmul(h, wd, out=y)
        e[2].record()
    torch.cuda.synchronize()
    up = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    down = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    flop = 2.0 * M * N1 * K1
    return {"what": "torch.matmul (hipBLASLt) with dense bf16 weights on the same two shapes, "
                    "no activation: the library GEMM the low-bit layer replaces",
            "up_ms": round(up, 4), "down_ms": round(down, 4),
            "tflops": round(2 * flop / ((up + down) * 1e-3) / 1e12, 1)}


def bench_small(torch, lb, reps=10, fuse_qkv=False, grouped=False):
    """Weight streaming at M = 16 and M = 1 over the 100 ternary linears of one
    transformer pass (and the 1-bit equivalent); with fuse_qkv, the same
    weights with each stream's Q, K, V rows concatenated at load time (80
    linears); with grouped as well, each double-stream block's image and text
    linears of one shape (independent of each other) run as one
    lowbit_gemm_grouped launch, each stream with its own activations (60
    launches). One code matrix is drawn per distinct shape and copied into its
    own device buffer per linear, so every launch streams distinct memory
    (about 0.75 GB ternary, 0.4 GB binary, far above the 256 MB last-level
    cache)."""
    import workloads as wl
    assert fuse_qkv or not grouped
    shapes = wl.mmdit_linear_shapes(fuse_qkv)
    # launches: lists of linear indices (an image / text pair of a double-stream block, or one linear)
    ops = []
    for i, (name, _, _) in enumerate(shapes):
        if grouped and ".img." in name:
            ops.append([i, shapes.index((name.replace(".img.", ".txt."),) + shapes[i][1:])])
        elif not (grouped and ".txt." in name):
            ops.append([i])
    distinct = sorted({(N, K) for _, N, K in shapes})
    out = {}
    for fmt in ("ternary", "binary"):
        g = wl.generator(4 if fmt == "ternary" else 5)
        base = {}
        for (N, K) in distinct:
            codes = wl.ternary_codes(g, N, K, 0.35) if fmt == "ternary" else wl.binary_codes(g, N, K)
            c = torch.from_numpy(codes).cuda()
            p = lb.pack_ternary(c) if fmt == "ternary" else lb.pack_binary(c)
            del c
            base[(N, K)] = (p, dev16(torch, wl.group_scales(g, N, K), torch.float16))
        layers = [(base[(N, K)][0].clone(), base[(N, K)][1].clone(), N, K) for _, N, K in shapes]
        del base
        gx = wl.generator(6)
        for M in (16, 1):
            xs = {K: dev16(torch, wl.activations(gx, M, K, "bf16"), torch.bfloat16)
                  for K in sorted({K for _, _, K in shapes})}
            # the text stream's own activations (grouped launches only)
            xt = {K: dev16(torch, wl.activations(gx, M, K, "bf16"), torch.bfloat16)
                  for K in sorted({K for _, _, K in shapes})} if grouped else xs
            ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, _, N, _ in layers]
            need = max(lb.workspace_bytes(fmt, M, N, K) for _, _, N, K in layers)
            if grouped:
                need = max(need, max(int(lb.lib().lowbit_gemm_grouped_workspace_bytes(
                    len(op), lb._FMT[fmt], M, layers[op[0]][2], layers[op[0]][3])) for op in ops))
            ws = lb.new_workspace(need)

            def sweep():
                for op in ops:
                    if len(op) == 1:
                        p, s, N, K = layers[op[0]]
                        lb.gemm(xs[K], p, s, fmt, out=ys[op[0]], workspace=ws)
                    else:
                        K = layers[op[0]][3]
                        lb.gemm_grouped([xs[K], xt[K]], [layers[i][0] for i in op], [layers[i][1] for i in op],
                                        fmt, outs=[ys[i] for i in op], workspace=ws)
            # the 100 launches are captured once in a HIP graph and replayed,
            # so the host's per-call Python cost is not what gets timed
            sweep()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                sweep()
            for _ in range(20):                       # warm replays (clocks settle)
                graph.replay()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                graph.replay()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / reps
            wbytes = sum(lb.packed_bytes(fmt, N, K) + 2 * N * K // 128 for _, _, N, K in layers)
            io = sum(2 * M * K + 2 * M * N for _, _, N, K in layers)
            gbs = (wbytes + io) / (ms * 1e-3) / 1e9
            out[f"{fmt}_M{M}"] = dict(ms_per_pass=round(ms, 4), bytes_per_pass=wbytes + io,
                                      GBps=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4),
                                      launches=len(ops))
            del ys, xs, xt, ws, graph
        del layers
        torch.cuda.empty_cache()
    return out


def bench_large_sweep(torch, lb, passes=3):
    """The 100 ternary linears of one transformer pass at M = 4608 tokens, each
    with its own weights (about 0.7 GB in all); one activation per distinct K
    and one output buffer per distinct N; one pass after a warm pass, then
    `passes` timed passes."""
    import workloads as wl
    M = 4608
    shapes = wl.mmdit_linear_shapes()
    g = wl.generator(4)
    base = {}
    for (N, K) in sorted({(N, K) for _, N, K in shapes}):
        c = torch.from_numpy(wl.ternary_codes(g, N, K, 0.35)).cuda()
        base[(N, K)] = (lb.pack_ternary(c), dev16(torch, wl.group_scales(g, N, K), torch.float16))
        del c
    layers = [(base[(N, K)][0].clone(), base[(N, K)][1].clone(), N, K) for _, N, K in shapes]
    del base
    tg = torch.Generator(device="cuda").manual_seed(12)
    xs = {K: torch.randn((M, K), generator=tg, device="cuda").bfloat16() for K in sorted({K for _, _, K in shapes})}
    ys = {N: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N in sorted({N for _, N, _ in shapes})}
    ws = lb.new_workspace(max(lb.workspace_bytes("ternary", M, N, K) for _, _, N, K in layers))

    def one_pass():
        for p, sc, N, K in layers:
            lb.gemm(xs[K], p, sc, "ternary", out=ys[N], workspace=ws)
    one_pass()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(passes):
        one_pass()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / passes
    flop = sum(2.0 * M * N * K for _, _, N, K in layers)
    tf = flop / (ms * 1e-3) / 1e12
    del layers, xs, ys, ws
    torch.cuda.empty_cache()
    return dict(M=M, launches=len(shapes), ms_per_pass=round(ms, 3), flop_per_pass=flop,
                tflops=round(tf, 1), frac_mfma_peak=round(tf / PEAK_BF16_TFLOPS, 4))


def bench_m1536(torch, lb, reps=200):
    """Context: the 512x512 step's token count (M = 1536) on the linears of the
    workloads quoted there: ternary 3072 x 3072 with bias (bf16), binary
    3072 x 3072 and the binary fused QKV 9216 x 3072, each beside torch.matmul
    (hipBLASLt) with dense bf16 weights of the same shape."""
    import workloads as wl
    out = {}
    for name, fmt, N, K, bias in (("ternary_3072x3072_bias", "ternary", 3072, 3072, True),
                                  ("binary_3072x3072", "binary", 3072, 3072, False),
                                  ("binary_9216x3072", "binary", 9216, 3072, False)):
        lin = wl.make_linear(name, fmt, 1536, N, K, seed=13, with_bias=bias)
        c = torch.from_numpy(lin.codes).cuda()
        p = lb.pack_ternary(c) if fmt == "ternary" else lb.pack_binary(c)
        del c
        sc = dev16(torch, lin.scales, torch.float16)
        x = dev16(torch, lin.x, torch.bfloat16)
        b = dev16(torch, lin.bias, torch.float16) if bias else None
        y = torch.empty((1536, N), dtype=torch.bfloat16, device="cuda")
        wd = torch.randn((K, N), generator=torch.Generator(device="cuda").manual_seed(14), device="cuda").bfloat16()

        def timed(fn):
            for _ in range(50):
                fn()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / reps
        ms = timed(lambda: lb.gemm(x, p, sc, fmt, bias=b, out=y))
        msd = timed(lambda: torch.matmul(x, wd))
        flop = 2.0 * 1536 * N * K
        out[name] = dict(us=round(ms * 1e3, 1), tflops=round(flop / (ms * 1e-3) / 1e12, 1),
                         dense_bf16_us=round(msd * 1e3, 1), dense_bf16_tflops=round(flop / (msd * 1e-3) / 1e12, 1))
        del p, sc, x, b, y, wd
    torch.cuda.empty_cache()
    return out


def hbm_copy(torch, nbytes=1 << 30, reps=10):
    """Context: a device-to-device copy of 1 GiB (reads and writes counted)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return dict(bytes_moved_per_copy=2 * nbytes, GBps=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))


def bench_small_single(torch, lb, reps=5, rotate_bytes=1 << 30):
    """The binary workload's weight-streaming cases: one 1-bit linear of
    3072 x 3072 and the fused QKV of 9216 x 3072, at M = 16 and M = 1. The
    launches rotate over distinct weight copies totalling at least 1 GiB
    (four times the 256 MB last-level cache, so each launch streams its
    weights from HBM); they are captured in a HIP graph and replayed."""
    import workloads as wl
    out = {}
    g = wl.generator(7)
    gx = wl.generator(8)
    for (N, K) in ((3072, 3072), (9216, 3072)):
        c = torch.from_numpy(wl.binary_codes(g, N, K)).cuda()
        p0 = lb.pack_binary(c)
        del c
        s0 = dev16(torch, wl.group_scales(g, N, K), torch.float16)
        per_copy = p0.numel() + 2 * s0.numel()
        copies = -(-rotate_bytes // per_copy)
        ws_ = [(p0.clone(), s0.clone()) for _ in range(copies)]
        for M in (16, 1):
            x = dev16(torch, wl.activations(gx, M, K, "bf16"), torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ws = lb.new_workspace(lb.workspace_bytes("binary", M, N, K))

            def run():
                for p, sc in ws_:
                    lb.gemm(x, p, sc, "binary", out=y, workspace=ws)
            run()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                run()
            for _ in range(10):
                graph.replay()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                graph.replay()
            t1.record()
            torch.cuda.synchronize()
            us = t0.elapsed_time(t1) * 1e3 / (reps * copies)
            nbytes = lb.packed_bytes("binary", N, K) + 2 * N * K // 128 + 2 * M * K + 2 * M * N
            gbs = nbytes / (us * 1e-6) / 1e9
            out[f"binary_{N}x{K}_M{M}"] = dict(us_per_launch=round(us, 2), bytes_per_launch=nbytes,
                                               GBps=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4),
                                               weight_copies=copies)
            del graph, x, y, ws
        del ws_, p0, s0
        torch.cuda.empty_cache()
    return out


def bench_base3_transcode(torch, lb, reps=10):
    """Load-time transcoding of the 100-linear sweep's ternary weights from the
    base-3 storage (five values per byte) to the INT2 form the GEMM reads
    (0.57 GB read, 0.71 GB written per pass). Two ways a loader can issue it:
    one base3_to_int2 launch per linear, each on its own buffers (100 launches,
    2.5-15 MB each, captured in a HIP graph and replayed), and one launch per
    distinct K over the rows of every linear with that K stored back to back
    (3 launches; rows are independent, so this is the same transcoding)."""
    import workloads as wl
    shapes = wl.mmdit_linear_shapes()
    g = wl.generator(9)
    base = {}
    for (N, K) in sorted({(N, K) for _, N, K in shapes}):
        c = torch.from_numpy(wl.ternary_codes(g, N, K, 0.35)).cuda()
        base[(N, K)] = lb.pack_base3(c)
        del c
    ins = [(base[(N, K)].clone(), N, K) for _, N, K in shapes]
    del base
    outs = [torch.empty((N, K // 4), dtype=torch.uint8, device="cuda") for _, N, K in ins]
    rd = sum(lb.packed_bytes("base3", N, K) for _, N, K in ins)
    wr = sum(lb.packed_bytes("ternary", N, K) for _, N, K in ins)

    def timed(one_pass):
        one_pass()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass()
        for _ in range(5):
            graph.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            graph.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        gbs = (rd + wr) / (ms * 1e-3) / 1e9
        del graph
        return ms, gbs

    def per_linear():
        for (p, N, K), o in zip(ins, outs):
            lb.base3_to_int2(p, K, check=False, out=o)
    ms1, gbs1 = timed(per_linear)
    del outs
    # the same rows grouped by K, each group one contiguous matrix
    stacked = {}
    for K in sorted({K for _, _, K in ins}):
        rows = [p for p, _, k in ins if k == K]
        stacked[K] = torch.cat(rows, 0)
    del ins
    souts = {K: torch.empty((p.shape[0], K // 4), dtype=torch.uint8, device="cuda") for K, p in stacked.items()}

    def per_k():
        for K, p in stacked.items():
            lb.base3_to_int2(p, K, check=False, out=souts[K])
    ms3, gbs3 = timed(per_k)
    del stacked, souts
    torch.cuda.empty_cache()
    return dict(bytes_read=rd, bytes_written=wr,
                per_linear=dict(launches=len(shapes), ms_per_pass=round(ms1, 4), GBps=round(gbs1, 1),
                                frac_hbm_peak=round(gbs1 / PEAK_HBM_GBS, 4)),
                per_k=dict(launches=3, ms_per_pass=round(ms3, 4), GBps=round(gbs3, 1),
                           frac_hbm_peak=round(gbs3 / PEAK_HBM_GBS, 4)))


def bench_quantize(torch, lb, reps=10):
    """Load-time quantisation of the 100-linear sweep's dense FP16 weights into
    ternary codes and group scales (lowbit_quantize): 5.66 GB of FP16 read,
    0.75 GB of codes and scales written per pass. Per linear (100 launches,
    each on its own buffers, replayed from a HIP graph) and per distinct K over
    the rows of every linear with that K stored back to back (3 launches; the
    rule is row-local, so that is the same quantisation). Weights: normal with
    standard deviation 0.02, drawn on the device (torch, seed 15)."""
    import workloads as wl
    shapes = wl.mmdit_linear_shapes()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(15)
    ins = []
    for _, N, K in shapes:
        w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32).mul_(0.02).half()
        ins.append((w, N, K))
    outs = [(torch.empty((N, K // 4), dtype=torch.uint8, device="cuda"),
             torch.empty((N, K // 128), dtype=torch.float16, device="cuda")) for _, N, K in ins]
    rd = sum(2 * N * K for _, N, K in ins)
    wr = sum(N * K // 4 + 2 * N * K // 128 for _, N, K in ins)

    def timed(one_pass):
        one_pass()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            graph.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        del graph
        return ms, (rd + wr) / (ms * 1e-3) / 1e9

    def per_linear():
        for (w, N, K), o in zip(ins, outs):
            lb.quantize(w, "ternary", check=False, out=o)
    ms1, gbs1 = timed(per_linear)
    del outs
    stacked = {}
    for K in sorted({K for _, _, K in ins}):
        stacked[K] = torch.cat([w for w, _, k in ins if k == K], 0)
    del ins
    souts = {K: (torch.empty((w.shape[0], K // 4), dtype=torch.uint8, device="cuda"),
                 torch.empty((w.shape[0], K // 128), dtype=torch.float16, device="cuda"))
             for K, w in stacked.items()}

    def per_k():
        for K, w in stacked.items():
            lb.quantize(w, "ternary", check=False, out=souts[K])
    ms3, gbs3 = timed(per_k)
    del stacked, souts
    torch.cuda.empty_cache()
    return dict(bytes_read=rd, bytes_written=wr,
                per_linear=dict(launches=len(shapes), ms_per_pass=round(ms1, 4), GBps=round(gbs1, 1),
                                frac_hbm_peak=round(gbs1 / PEAK_HBM_GBS, 4)),
                per_k=dict(launches=3, ms_per_pass=round(ms3, 4), GBps=round(gbs3, 1),
                           frac_hbm_peak=round(gbs3 / PEAK_HBM_GBS, 4)))


def bench_int4(torch, lb, reps=50, fused=False):
    """The text encoder's 4-bit linears (lowbit_gemm_int4): the seven linears
    of one Qwen3-4B-shaped layer (q, k, v, o, gate, up, down) at 512 prompt
    tokens, bf16 activations, uniform 4-bit codes, FP16 scales and zero points
    per 128 (device draws, seed 16), each call with its row-sum pre-pass,
    back to back on one stream; beside torch.matmul (hipBLASLt) on dense bf16
    weights of the same shapes. fused: the linears that share an input run as
    one, their weight rows concatenated (q|k|v 6144 x 2560, gate|up
    19456 x 2560; four calls), on both sides."""
    import workloads as wl
    M = wl.TE_TOKENS
    gen = torch.Generator(device="cuda")
    gen.manual_seed(16)
    layer = []
    shapes = wl.text_encoder_shapes()
    if fused:
        d = {n: (N, K) for n, N, K in shapes}
        shapes = [("qkv", d["q"][0] + d["k"][0] + d["v"][0], d["q"][1]), ("o",) + d["o"],
                  ("gate_up", d["gate"][0] + d["up"][0], d["gate"][1]), ("down",) + d["down"]]
    for name, N, K in shapes:
        q = torch.randint(0, 16, (N, K), generator=gen, device="cuda", dtype=torch.uint8)
        packed = lb.pack_int4(q)
        s = (torch.rand((N, K // 128), generator=gen, device="cuda") * 0.003 + 1e-4).half()
        z = (torch.randn((N, K // 128), generator=gen, device="cuda") * 0.5 + 7.5).half()
        x = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).bfloat16()
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(int(lb.lib().lowbit_gemm_int4_workspace_bytes(M, N, K)), 256), dtype=torch.uint8,
                         device="cuda")
        wd = torch.randn((K, N), generator=gen, device="cuda", dtype=torch.float32).bfloat16()
        layer.append((name, N, K, x, packed, s, z, y, ws, wd))
        del q
    flop = sum(2 * M * N * K for _, N, K, *_ in layer)

    def lowbit():
        for _, N, K, x, packed, s, z, y, ws, _ in layer:
            lb.gemm_int4(x, packed, s, z, out=y, workspace=ws)

    def dense():
        for *_, x, _p, _s, _z, _y, _w, wd in layer:
            torch.matmul(x, wd)

    def timed(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    ms, dms = timed(lowbit), timed(dense)
    del layer
    torch.cuda.empty_cache()
    out = dict(M=M, linears=len(shapes), flop_per_layer=flop, ms_per_layer=round(ms, 4),
               tflops=round(flop / (ms * 1e-3) / 1e12, 1), dense_bf16_ms=round(dms, 4),
               dense_bf16_tflops=round(flop / (dms * 1e-3) / 1e12, 1))
    if not fused:
        out["fused_same_input"] = bench_int4(torch, lb, reps, fused=True)
    return out


def traffic_probe(torch, lb):
    """Workload for the rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes: first a
    plain 256 MiB device copy (calibration: its byte counts are known), then two
    passes of the MLP pair."""
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    bench_large(torch, lb, steps=1, warmup=1)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)


def traffic_summary(fetch_csv: str, write_csv: str) -> dict:
    """Write TRAFFIC_FILE from the two rocprofv3 --pmc counter files of the
    --traffic-probe workload (FETCH_SIZE run, WRITE_SIZE run). The counters
    are scaled by what they read for the calibration copy (the largest
    __amd_rocclr_copyBuffer dispatch: 256 MiB read and written); the GEMM
    launches are told apart by grid size (up-projection, down-projection)."""
    import csv

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        calib = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        gemm = {}
        for r in rows:
            if "gemm_large_kernel" in r["Kernel_Name"]:
                gemm.setdefault(int(r["Grid_Size"]), (r["Kernel_Name"], []))[1].append(float(r["Counter_Value"]))
        return calib, gemm

    copy_kib = (256 << 20) / 1024
    f_cal, f_gemm = read(fetch_csv, "FETCH_SIZE")
    w_cal, w_gemm = read(write_csv, "WRITE_SIZE")
    ff, wf = copy_kib / f_cal, copy_kib / w_cal
    import workloads as wl
    up, down = wl.config3()
    alg = {name: lin.N * lin.K // 4 + lin.N * lin.K // 64 + 2 * lin.M * lin.K + 2 * lin.M * lin.N
           for name, lin in (("up", up), ("down", down))}
    out = {
        "kernel": "gemm_large_kernel<bf16, ternary>",
        "workload": "MLP pair of a 1024x1024 step: up 4608x9216x3072 (+GELU), down 4608x3072x9216, "
                    "bf16, ternary, group 128",
        "kernel_source_sha": kernel_source_sha(),
        "kernel_source_sha_note": "sha256 of gemm_large.hip + common.h with // comments and blank lines removed "
                                  "(bench.py kernel_source_sha)",
        "how": "hbm_bytes = (FETCH_SIZE_KiB * fetch_factor + WRITE_SIZE_KiB * write_factor) * 1024, mean over "
               "dispatches; factors = 262144 KiB / the counter value of a plain 256 MiB device copy",
        "calibration": {"copy_bytes": 256 << 20, "fetch_kib": f_cal, "write_kib": w_cal,
                        "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
    }
    # the up-projection has the larger grid (more, smaller tiles or more rows of tiles)
    grids = sorted(f_gemm, reverse=True)
    if len(grids) != 2 or sorted(w_gemm, reverse=True) != grids:
        raise SystemExit(f"expected two GEMM launch shapes, found grids {grids}")
    total = 0.0
    for name, g in zip(("up", "down"), grids):
        fk = float(np.mean(f_gemm[g][1]))
        wk = float(np.mean(w_gemm[g][1]))
        hb = (fk * ff + wk * wf) * 1024
        total += hb
        out[name] = {"kernel_name": f_gemm[g][0], "grid": g, "dispatches": len(f_gemm[g][1]),
                     "fetch_kib": fk, "write_kib": wk, "hbm_bytes": int(round(hb)),
                     "algorithmic_bytes": int(alg[name])}
    out["bytes_per_launch"] = int(round(total / 2))
    out["commands"] = [
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
        "-d $OUT/tr_FETCH_SIZE -o run -- python $REPO/bench.py --traffic-probe",
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv "
        "-d $OUT/tr_WRITE_SIZE -o run -- python $REPO/bench.py --traffic-probe",
        "python bench.py --traffic-summary $OUT/tr_FETCH_SIZE/run_counter_collection.csv "
        "$OUT/tr_WRITE_SIZE/run_counter_collection.csv",
    ]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    return out


def counter_table(csvs, num_simd: int = 1024, num_xcd: int = 8) -> str:
    """Markdown table of per-kernel means of the rocprofv3 --pmc counters in
    the given counter_collection.csv files (one row per kernel name and grid
    size), with MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES (summed over all
    SIMDs) / (GRBM_GUI_ACTIVE / XCDs x SIMDs) -- GRBM_GUI_ACTIVE reads as the
    sum over the 8 XCDs -- and VALU instructions per MFMA where those
    counters are there."""
    import csv
    agg = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "lowbit::gemm" not in name:
                continue
            key = (name.split("(")[0].replace("void ", ""), int(r["Grid_Size"]))
            agg.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cols = sorted({c for d in agg.values() for c in d})
    head = ["kernel", "grid", "dispatches"] + cols
    derived = []
    if {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"} <= set(cols):
        derived.append("MFMA busy %")
    if {"SQ_INSTS_VALU", "SQ_INSTS_MFMA"} <= set(cols):
        derived.append("VALU per MFMA")
    out = ["| " + " | ".join(head + derived) + " |", "|" + "---|" * (len(head) + len(derived))]
    for (name, grid), d in sorted(agg.items(), key=lambda kv: -len(next(iter(kv[1].values())))):
        m = {c: float(np.mean(v)) for c, v in d.items()}
        row = [f"`{name}`", str(grid), str(len(next(iter(d.values()))))] + [f"{m[c]:.4g}" if c in m else "" for c in cols]
        if "MFMA busy %" in derived:
            row.append(f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (m['GRBM_GUI_ACTIVE'] / num_xcd * num_simd):.1f}")
        if "VALU per MFMA" in derived:
            row.append(f"{(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / max(m['SQ_INSTS_MFMA'], 1):.2f}")
        out.append("| " + " | ".join(row) + " |")
    return "\n".join(out)


def stats_table(stats_csv: str, limit: int = 24) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv
    (durations converted from ns to us)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    out = ["| kernel | calls | total us | average us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:limit]:
        out.append("| `{}` | {} | {:.1f} | {:.1f} | {:.1f} | {:.1f} | {:.2f} |".format(
            r["Name"][:110], r["Calls"], float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def cpu_configs(torch, lb):
    """The oracle (float64 NumPy, all host cores) per workload configuration,
    its dequantisation and its matrix product timed separately, beside the
    GPU time of the same call (HIP events, inputs resident): the 64 x 256 x 256
    case, the 1536-token ternary linear with bias, the MLP pair of the
    1024 x 1024 step, the binary linears at M = 1536, 16 and 1, and one pass
    of the 100 linears at M = 4608, whose oracle runs on a seeded sample of
    256 rows per linear and is scaled to 4608 rows (an extrapolation)."""
    import oracle
    import workloads as wl

    def gpu_ms(lin, x_bits=None, reps=20):
        xb = lin.x if x_bits is None else x_bits
        x = dev16(torch, xb, torch.bfloat16 if lin.x_dtype == "bf16" else torch.float16)
        c = torch.from_numpy(lin.codes).cuda()
        p = lb.pack_ternary(c) if lin.fmt == "ternary" else lb.pack_binary(c)
        del c
        sc = dev16(torch, lin.scales, torch.float16)
        b = dev16(torch, lin.bias, torch.float16) if lin.bias is not None else None
        for _ in range(5):
            lb.gemm(x, p, sc, lin.fmt, bias=b)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            lb.gemm(x, p, sc, lin.fmt, bias=b)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    def oracle_s(lin, rows=None):
        xb = lin.x if rows is None else lin.x[rows]
        t0 = time.perf_counter()
        W = oracle.dequantize(lin.codes, lin.scales)
        t1 = time.perf_counter()
        A = oracle.decode(xb, lin.x_dtype) @ W.T
        if lin.bias is not None:
            A = A + lin.bias.astype(np.float64)[None, :]
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    out = {"cores": len(os.sched_getaffinity(0))}
    cases = [("64x256x256_ternary_f16", wl.config1()), ("1536x3072x3072_ternary_bias", wl.config2())]
    up, down = wl.config3()
    if down.x is None:       # its input is the up-projection's GELU; any bf16 of that shape times the same
        down.x = wl.activations(wl.generator(78), down.M, down.K, "bf16")
    cases += [("4608x9216x3072_mlp_up", up), ("4608x3072x9216_mlp_down", down)]
    for M in (1536, 16, 1):
        for lin in wl.config4(M):
            cases.append((f"{M}x{lin.N}x{lin.K}_binary", lin))
    for name, lin in cases:
        print(f"[cpu-configs] {name}", file=sys.stderr, flush=True)
        dq, mm = oracle_s(lin)
        g = gpu_ms(lin)
        out[name] = dict(oracle_dequant_s=round(dq, 4), oracle_matmul_s=round(mm, 4), gpu_ms=round(g, 4),
                         speedup=round((dq + mm) / (g * 1e-3), 1))
    # one pass of the 100 linears at M = 4608 (oracle on 256 rows per linear, scaled)
    xs = wl.config5_activations()
    rows = np.sort(wl.generator(77).choice(4608, size=256, replace=False))
    dq = mm = g = 0.0
    for i, (name, codes, scales) in enumerate(wl.config5_weights()):
        if i % 10 == 0:
            print(f"[cpu-configs] 100 linears: {i}", file=sys.stderr, flush=True)
        N, K = codes.shape
        lin = wl.Linear(name, "ternary", 4608, N, K, "bf16", "bf16", xs[K], codes, scales)
        d, m = oracle_s(lin, rows)
        dq += d
        mm += m * 4608 / 256
        g += gpu_ms(lin, reps=3)
    out["100_linears_M4608"] = dict(oracle_dequant_s=round(dq, 2), oracle_matmul_s_extrapolated=round(mm, 1),
                                    gpu_ms=round(g, 3), speedup=round((dq + mm) / (g * 1e-3), 1),
                                    oracle_sample="256 of 4608 rows per linear, matmul time x 18")
    return out


def dispatch_table(trace_csv: str, kernel: str) -> str:
    """Markdown table of the dispatches of one kernel in a rocprofv3
    --kernel-trace kernel_trace.csv, grouped by grid size (threads)."""
    import csv
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        if kernel not in r["Kernel_Name"]:
            continue
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault(int(r["Grid_Size_X"]), []).append(d)
    out = ["| grid (threads) | workgroups | dispatches | average us | min us | max us |",
           "|---|---|---|---|---|---|"]
    for grid in sorted(groups):
        ds = groups[grid]
        out.append("| {} | {} | {} | {:.2f} | {:.2f} | {:.2f} |".format(
            grid, grid // 256, len(ds), sum(ds) / len(ds), min(ds), max(ds)))
    return "\n".join(out)


def _blas_name() -> str:
    """The BLAS library numpy uses (for the report)."""
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        return "unknown"


def cpu_baseline(seconds_target=10.0):
    """The oracle as it stands (float64 dequantise + BLAS matmul) on a bounded
    sample of the step: the first R rows of the MLP pair (R grown up to all 4608),
    repeated until about `seconds_target` seconds of CPU work are timed."""
    import oracle
    import workloads as wl
    up, down = wl.config3()
    cores = len(os.sched_getaffinity(0))

    def one(rows):
        A = oracle.linear(up.x[:rows], "bf16", up.codes, up.scales)
        H = oracle.encode(oracle.gelu(A), "bf16")
        oracle.linear(H, "bf16", down.codes, down.scales)

    rows = 64
    while True:
        t0 = time.perf_counter()
        one(rows)
        dt = time.perf_counter() - t0
        if dt > seconds_target / 3 or rows >= up.M:
            break
        rows = min(up.M, rows * 4)
    reps, total = 1, dt
    while total < seconds_target:
        t0 = time.perf_counter()
        one(rows)
        total += time.perf_counter() - t0
        reps += 1
    flop = reps * (2.0 * rows * up.N * up.K + 2.0 * rows * down.N * down.K)

    # the FP32-BLAS form of the same layer (exact FP32 dequantisation, sgemm),
    # on the same sample, timed for about a third of the time
    def one32(r):
        A = oracle.linear_f32(up.x[:r], "bf16", up.codes, up.scales)
        H = oracle.encode(oracle.gelu(A), "bf16")
        oracle.linear_f32(H, "bf16", down.codes, down.scales)
    reps32, total32 = 0, 0.0
    while total32 < seconds_target / 3 or reps32 == 0:
        t0 = time.perf_counter()
        one32(rows)
        total32 += time.perf_counter() - t0
        reps32 += 1
    flop32 = reps32 * (2.0 * rows * up.N * up.K + 2.0 * rows * down.N * down.K)
    return dict(value=round(flop / total / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{reps} pass(es) of the first {rows} of 4608 rows through up-proj, GELU and "
                       f"down-proj (float64 oracle, {total:.1f} s)",
                fp32_blas=dict(value=round(flop32 / total32 / 1e12, 6), unit="TFLOP/s",
                               sample=f"{reps32} pass(es) of the same rows with the layer in FP32 "
                                      f"(oracle.linear_f32: exact FP32 dequantisation and sgemm), "
                                      f"{total32:.1f} s"),
                blas=_blas_name())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of untimed steps before the warm-up steps, so the timed steps run at "
                         "the clock the GPU settles to under this load")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context runs that launch the same kernels as the timed paths "
                         "(the 100-linear pass at M = 4608, the M = 1536 linears, the single binary "
                         "linears) and the device copy, so that kernel traces and counters cover the "
                         "timed paths only")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run the counter-calibration workload instead of the benchmark")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary from the two counter runs and exit")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="time the oracle per workload configuration beside the GPU (about two minutes "
                         "of host work) and print that JSON instead of the benchmark line")
    ap.add_argument("--dispatch-table", nargs=2, metavar=("TRACE_CSV", "KERNEL"),
                    help="print one kernel's dispatches from a rocprofv3 kernel_trace.csv by grid size")
    ap.add_argument("--stats-table", metavar="STATS_CSV",
                    help="print a rocprofv3 kernel_stats.csv as a markdown table and exit")
    ap.add_argument("--only", choices=["int4", "quantize", "base3", "small", "small_grouped"],
                    help="run one of the context legs alone and print its JSON (for kernel traces of it)")
    ap.add_argument("--counter-table", nargs="+", metavar="COUNTER_CSV",
                    help="print per-kernel means of rocprofv3 --pmc counter files and exit")
    args = ap.parse_args()
    if args.counter_table:
        print(counter_table(args.counter_table))
        return
    if args.traffic_summary:
        print(json.dumps(traffic_summary(*args.traffic_summary)))
        return
    if args.dispatch_table:
        print(dispatch_table(*args.dispatch_table))
        return
    if args.stats_table:
        print(stats_table(args.stats_table))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the low-bit linear layer runs on a single "
              "device here; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_gemm_int2_amd as lb
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    lb.lib()
    if args.traffic_probe:
        traffic_probe(torch, lb)
        return
    if args.cpu_configs:
        print(json.dumps(cpu_configs(torch, lb)), flush=True)
        return
    if args.only:
        leg = {"int4": lambda: bench_int4(torch, lb), "quantize": lambda: bench_quantize(torch, lb),
               "base3": lambda: bench_base3_transcode(torch, lb), "small": lambda: bench_small(torch, lb),
               "small_grouped": lambda: bench_small(torch, lb, fuse_qkv=True, grouped=True)}[args.only]
        print(json.dumps({args.only: leg()}), flush=True)
        return

    r = bench_large(torch, lb, args.steps, args.warmup, args.settle_s)
    ms_step = r["total_ms"] / args.steps
    tflops = r["flop_step"] / (ms_step * 1e-3) / 1e12
    achieved = r["flop_launch"] / (r["avg_launch_ms"] * 1e-3) / 1e12
    traffic = load_traffic()
    dense = bench_dense(torch, r["M"], r["N1"], r["K1"], r["N2"])
    sweep = None if args.no_context else bench_large_sweep(torch, lb)
    copy = None if args.no_context else hbm_copy(torch)
    m1536 = None if args.no_context else bench_m1536(torch, lb)
    small = None if args.no_small else bench_small(torch, lb)
    small_fused = None if args.no_small else bench_small(torch, lb, fuse_qkv=True)
    small_grouped = None if args.no_small else bench_small(torch, lb, fuse_qkv=True, grouped=True)
    small_single = None if (args.no_small or args.no_context) else bench_small_single(torch, lb)
    base3 = None if args.no_small else bench_base3_transcode(torch, lb)
    quant = None if args.no_small else bench_quantize(torch, lb)
    int4 = None if args.no_context else bench_int4(torch, lb)
    cpu = None if args.no_cpu else cpu_baseline()
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "ternary MLP pair of a 1024x1024 step: X bf16 [4608x3072] -> up [9216x3072] "
                        "+ fused exact GELU -> down [3072x9216], INT2 codes P(0)=0.35, fp16 scales per 128",
            "M": r["M"], "hidden": r["K1"], "mlp": r["N1"], "group": 128,
            "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "up_ms": round(r["up_ms"], 4), "down_ms": round(r["down_ms"], 4),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "gemm_large_kernel<bf16, ternary>, mean of its two launches per step "
                      "(up: 96x256 tiles, two workgroups per CU; down: 128x512 tiles)",
            "avg_launch_ms": round(r["avg_launch_ms"], 4),
            "flop_per_launch": r["flop_launch"],
            "launch_ms": {"up": r["up_spread"], "down": r["down_spread"], "step": r["step_spread"]},
            "settle": {"seconds": args.settle_s, "untimed_steps": r["settle_steps"]},
        },
        "cpu_baseline": cpu,
        "dense_bf16_matmul": dense,
        "large_m_sweep": sweep,
        "hbm_copy": copy,
        "m1536": m1536,
        "small_m": small,
        "small_m_fused_qkv": small_fused,
        "small_m_grouped": small_grouped,
        "small_m_binary_single": small_single,
        "base3_to_int2_sweep": base3,
        "quantize_sweep": quant,
        "int4_text_encoder_layer": int4,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
