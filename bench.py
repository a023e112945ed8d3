"""Benchmark of the W4A16 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Headline workload: decode GEMV, M=1 K=4096 N=12800 G=128, symmetric zero point
8 (the 8B-class MLP up-projection).  One step = one w4a16_gemm call (host
validation and dispatch, weight stream, nibble unpack, zero/scale, fp32
accumulate, split-K reduction, fp16 epilogue).  The weights, scales and
activations rotate over enough copies (> 256 MB) that every step reads them
from HBM rather than from the 256 MB Infinity Cache; everything is resident on
the GPU before the timed region.  The K timed steps are one captured HIP graph
replayed on the stream the kernels run on, bracketed by synchronisation and
HIP events; `value` is algorithmic bytes x K / elapsed.

The same JSON line carries the other measured rows (batched M=32 GEMM, prefill
M=256 GEMM, repack, the 40-layer decode step at M=1 and M=32), the roofline of
the dominant kernel and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA
KERNEL_SOURCES = ["w4a16_weight_only_amd/csrc/gemv.hip", "w4a16_weight_only_amd/csrc/device.h"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemv_M1_K4096_N12800_counters.md")


TRIAGE_STOP = 1.3  # [Floor-First] methodology step 3: measured / floor below this means stop tuning


def floors(measured_us, nbytes, flops, extra_floor_us=0.0):
    """Floor-first triage of one row: t_hbm (bytes at peak HBM), t_mfma (2MNK
    at peak fp16 MFMA), t_opt = the larger (the binding roof), t_sum = both in
    sequence (no overlap), residual = measured / t_opt, and the triage verdict
    at 1.3x the floor.  extra_floor_us: a further lower bound (the decode
    step's launch floor), folded into t_opt when larger."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = flops / (FP16_PEAK_TFLOPS * 1e12) * 1e6
    t_opt = max(t_hbm, t_mfma, extra_floor_us)
    res = measured_us / t_opt
    return dict(t_hbm_us=t_hbm, t_mfma_us=t_mfma, floor_us=t_opt, t_sum_us=t_hbm + t_mfma, residual=res,
                triage="stop" if res < TRIAGE_STOP else "escalate")


def alg_bytes(M, K, N, G, asym):
    b = K * N // 2 + (K // G) * N * 2 + 2 * M * K + 2 * M * N
    if asym:
        b += (K // G) * N // 2
    return b


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the GEMV kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def timed_graph(torch, stream, launch, steps, warmup):
    """Warm up eagerly, capture `steps` launches into one graph, replay once
    untimed, then time one replay with events on `stream`.  Returns
    (ms per step from events, ms per step from the host clock)."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            launch(i)
    with torch.cuda.stream(stream):
        g.replay()
    stream.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        t1 = time.perf_counter()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / steps, (t1 - t0) * 1e3 / steps


def timed_eager(torch, stream, launch, steps, warmup):
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(steps):
            launch(i)
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def rotated_problem(torch, M, K, N, G, asym, copies, seed):
    """`copies` independent synthetic problems on the GPU; copy 0 is the seeded
    workload of the parity tests, the others are drawn on the device."""
    from w4a16_weight_only_amd import synth
    p = synth.problem(M, K, N, G, asym, seed)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 12345)

    def words(r, c):
        return torch.randint(-2 ** 31, 2 ** 31, (r, c), dtype=torch.int32, device=dev, generator=gen)

    out = dict(a=[], b=[], s=[], z=[])
    for i in range(copies):
        if i == 0:
            out["a"].append(torch.from_numpy(p["a"]).to(dev))
            out["b"].append(torch.from_numpy(p["b_packed"]).to(dev))
            out["s"].append(torch.from_numpy(p["scales"]).to(dev))
            out["z"].append(torch.from_numpy(p["qzeros"]).to(dev) if asym else None)
        else:
            out["a"].append(torch.randn(M, K, device=dev, generator=gen).half())
            out["b"].append(words(K, N // 8))
            out["s"].append(((torch.rand(K // G, N, device=dev, generator=gen) + 0.5) / K ** 0.5).half())
            out["z"].append(words(K // G, N // 8) if asym else None)
    out["o"] = torch.empty(M, N, dtype=torch.float16, device=dev)
    return out


def bench_gemm(torch, w4, stream, M, K, N, G, asym, steps, warmup, seed):
    nbytes = alg_bytes(M, K, N, G, asym)
    copies = max(2, -(-512 * 2 ** 20 // nbytes))  # > 512 MB rotated
    P = rotated_problem(torch, M, K, N, G, asym, copies, seed)
    L = w4.lib()
    ptrs = [(P["a"][i].data_ptr(), P["b"][i].data_ptr(), P["s"][i].data_ptr(),
             P["z"][i].data_ptr() if asym else None) for i in range(copies)]
    optr = P["o"].data_ptr()
    sp = stream.cuda_stream

    def launch(i):
        a, b, s, z = ptrs[i % copies]
        rc = L.w4a16_gemm(a, b, s, z, M, K, N, G, 8, optr, sp)
        if rc:
            raise RuntimeError(L.w4a16_last_error().decode())

    ms, host_ms = timed_graph(torch, stream, launch, steps, warmup)
    eager_ms = timed_eager(torch, stream, launch, min(steps, 100), 5)
    flops = 2.0 * M * N * K
    path, splits, grid = w4.w4a16_gemm_plan(M, K, N, G)
    del P
    torch.cuda.empty_cache()
    row = dict(M=M, K=K, N=N, G=G, asym=asym, path={1: "gemv", 2: "mfma", 3: "gemv_mma"}[path], splits=splits,
               grid=grid, rotated_copies=copies, us_per_call=ms * 1e3, host_us_per_call=host_ms * 1e3,
               eager_us_per_call=eager_ms * 1e3, alg_bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
               tflops=flops / (ms * 1e-3) / 1e12,
               hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               mfma_frac=flops / (ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS)
    row.update(floors(ms * 1e3, nbytes, flops))
    return row


def bench_repack(torch, w4, stream, K, N, steps, warmup):
    nbytes = 2 * K * N // 2
    copies = max(2, -(-512 * 2 ** 20 // nbytes))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    src = [torch.randint(-2 ** 31, 2 ** 31, (N, K // 8), dtype=torch.int32, device="cuda", generator=gen)
           for _ in range(copies)]
    dst = [torch.empty(K, N // 8, dtype=torch.int32, device="cuda") for _ in range(copies)]
    L = w4.lib()
    sp = stream.cuda_stream

    def launch(i):
        rc = L.w4a16_repack(src[i % copies].data_ptr(), dst[i % copies].data_ptr(), K, N, sp)
        if rc:
            raise RuntimeError(L.w4a16_last_error().decode())

    ms, _ = timed_graph(torch, stream, launch, steps, warmup)
    del src, dst
    torch.cuda.empty_cache()
    row = dict(K=K, N=N, us_per_call=ms * 1e3, alg_bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
               hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    row.update(floors(ms * 1e3, nbytes, 0.0))
    return row


def launch_floor_us(torch, w4, stream, steps=200):
    """Per-launch time of the smallest kernel of the library (a one-row,
    eight-element row-norm: one workgroup, one round trip) replayed back to
    back from a graph: what every dependent launch of a step costs at least."""
    x = torch.randn(1, 8, device="cuda").half()
    y = torch.empty_like(x)
    L = w4.lib()
    sp = stream.cuda_stream

    def launch(i):
        rc = L.w4a16_rownorm(x.data_ptr(), 8, 1, 8, y.data_ptr(), sp)
        if rc:
            raise RuntimeError(L.w4a16_last_error().decode())

    ms, _ = timed_graph(torch, stream, launch, steps, 10)
    return ms * 1e3


def decode_launches(w4, M, stack, nl):
    """Kernel launches of one decode step: one per linear, one more for each
    glue step that runs as a kernel of its own, and the final row-norm."""
    n = 1
    for l in range(nl):
        for j, glue in enumerate((w4.GLUE_NONE if l == 0 else w4.GLUE_RMSNORM, w4.GLUE_RMSNORM, w4.GLUE_RMSNORM,
                                  w4.GLUE_SWIGLU)):
            n += 1 + (w4.w4a16_gemm_glue_workspace_bytes(glue, M, stack[4 * l + j]) > 0)
    return n


def bench_decode(torch, w4, stream, Ms, steps, warmup):
    """40-layer 8B-class stack (4.1 GB of packed weights, larger than any cache),
    random weights drawn on the device from a seeded generator."""
    from w4a16_weight_only_amd import synth
    S = synth.STACK
    H, NQ, I, G, nl = S["H"], S["NQ"], S["I"], S["G"], S["layers"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(S["seed_base"])
    stack = []
    wbytes = 0
    for l in range(nl):
        for (K, N) in synth.stack_linear_shapes(H, NQ, I):
            b = torch.randint(-2 ** 31, 2 ** 31, (K, N // 8), dtype=torch.int32, device="cuda", generator=gen)
            s = ((torch.rand(K // G, N, device="cuda", generator=gen) + 0.5) / K ** 0.5).half()
            stack.append(dict(b_packed=b, scales=s, qzeros=None, G=G, zp_bias=8))
            wbytes += K * N // 2 + (K // G) * N * 2
    res = {}
    L = w4.lib()
    t_launch = launch_floor_us(torch, w4, stream)
    arr = w4._linear_array(stack)
    import ctypes
    arrp = ctypes.cast(arr, ctypes.c_void_p)
    for M in Ms:
        x = torch.randn(M, H, device="cuda", generator=gen).half()
        y = torch.empty_like(x)
        need = w4.w4a16_decode_workspace_bytes(M, stack)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        sp = stream.cuda_stream

        def launch(i):
            rc = L.w4a16_decode_step(arrp, nl, x.data_ptr(), y.data_ptr(), M, ws.data_ptr(), need, sp)
            if rc:
                raise RuntimeError(L.w4a16_last_error().decode())

        ms, _ = timed_graph(torch, stream, launch, steps, warmup)
        eager_ms = timed_eager(torch, stream, launch, steps, 1)
        act = 0
        flops = 0
        for (K, N) in synth.stack_linear_shapes(H, NQ, I):
            act += 2 * M * (K + N) * nl
            flops += 2.0 * M * K * N * nl
        rms = float(y.float().pow(2).mean(1).sqrt().mean())
        row = dict(M=M, layers=nl, us_per_step=ms * 1e3, eager_us_per_step=eager_ms * 1e3,
                   tok_per_s=M / (ms * 1e-3), eager_tok_per_s=M / (eager_ms * 1e-3),
                   weight_bytes=wbytes, gbs=(wbytes + act) / (ms * 1e-3) / 1e9,
                   hbm_frac=(wbytes + act) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   target_tok_per_s_70pct=0.7 * M / ((wbytes + act) / (HBM_PEAK_GBS * 1e9)),
                   output_row_rms=rms)
        n_launch = decode_launches(w4, M, stack, nl)
        row.update(floors(ms * 1e3, wbytes + act, flops, n_launch * t_launch))
        row.update(launches=n_launch, launch_us=t_launch, launch_floor_us=n_launch * t_launch)
        res["M%d" % M] = row
    del stack
    torch.cuda.empty_cache()
    return res


def bench_copy_context(torch, stream, nbytes, steps, warmup):
    """Context only: a plain device elementwise copy (torch's own kernel) that
    moves the same number of HBM bytes as one headline call (half read, half
    written), over rotated buffers, timed like the headline."""
    n = nbytes // 8  # int32 elements per side
    copies = max(2, -(-512 * 2 ** 20 // nbytes))
    src = [torch.empty(n, dtype=torch.int32, device="cuda").random_() for _ in range(copies)]
    dst = [torch.empty_like(src[0]) for _ in range(copies)]

    def launch(i):
        torch.neg(src[i % copies], out=dst[i % copies])

    ms, _ = timed_graph(torch, stream, launch, steps, warmup)
    del src, dst
    torch.cuda.empty_cache()
    return dict(bytes=8 * n, us_per_call=ms * 1e3, gbs=8 * n / (ms * 1e-3) / 1e9,
                hbm_frac=8 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def bench_fp16_dense(torch, stream, steps, warmup):
    """Context only: the same products with dense fp16 weights through torch's
    own GEMM (the vendor BLAS), weights rotated past the last-level cache and
    timed like the W4A16 rows.  Shows the byte saving of 4-bit weights at
    M = 1 and the compute side at M = 32 and 256."""
    rows = {}
    for (M, K, N) in [(1, 4096, 12800), (32, 4096, 12800), (256, 12800, 4096)]:
        copies = max(2, -(-768 * 2 ** 20 // (K * N * 2)))
        g = torch.Generator(device="cuda").manual_seed(M + K + N)
        A = torch.randn(M, K, device="cuda", dtype=torch.float16, generator=g)
        W = [torch.randn(K, N, device="cuda", dtype=torch.float16, generator=g) for _ in range(copies)]
        O = torch.empty(M, N, device="cuda", dtype=torch.float16)

        def launch(i):
            torch.matmul(A, W[i % copies], out=O)

        ms, _ = timed_graph(torch, stream, launch, steps, warmup)
        us = ms * 1e3
        rows["M%d_K%d_N%d" % (M, K, N)] = dict(
            us_per_call=us, weight_bytes=K * N * 2, gbs=K * N * 2 / (us * 1e-6) / 1e9,
            tflops=2.0 * M * N * K / (us * 1e-6) / 1e12,
            mfma_frac=2.0 * M * N * K / (us * 1e-6) / 1e12 / FP16_PEAK_TFLOPS)
        del A, W, O
        torch.cuda.empty_cache()
    return rows


EXTRA_ROWS = {
    "batched_M32": lambda t, w, st, k, wu: bench_gemm(t, w, st, 32, 4096, 12800, 128, True, k, wu, 3),
    "prefill_M256": lambda t, w, st, k, wu: bench_gemm(t, w, st, 256, 12800, 4096, 128, True, k, wu, 4),
    "repack_K4096_N12800": lambda t, w, st, k, wu: bench_repack(t, w, st, 4096, 12800, k, wu),
    "decode_step": lambda t, w, st, k, wu: bench_decode(t, w, st, [1, 32], max(5, k // 20), 3),
    "fp16_dense_context": lambda t, w, st, k, wu: bench_fp16_dense(t, st, min(k, 100), wu),
    "copy_context_27MB": lambda t, w, st, k, wu: bench_copy_context(
        t, st, alg_bytes(1, 4096, 12800, 128, False), k, wu),
}


def _timed(fn, seconds):
    """Run fn() at least once and until `seconds` have passed; (calls, s)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def cpu_baseline(seconds=10.0):
    """The oracle (plain C, fp64, unchanged) on the host's cores: its products
    split over column slices run on one thread per core (at most 16), each
    slice the same loops over a smaller instance.  The headline figure is the
    M = 1 workload repeated for about `seconds`; the other rows are bounded
    samples of the M = 32, M = 256 and 40-layer decode workloads, scaled to
    their metric."""
    import oracle
    from w4a16_weight_only_amd import synth
    cores = oracle.host_workers()
    p = synth.workload("gemv")
    nbytes = alg_bytes(1, 4096, 12800, 128, False)
    parts = oracle.split_columns(p["b_packed"], p["scales"], None)
    n, dt = _timed(lambda: oracle.gemm_split(p["a"], parts, 128, 8), seconds)
    head = dict(value=nbytes * n / dt / 1e9, unit="GB/s", cores=cores, kind="oracle",
                sample="%d full M=1 K=4096 N=12800 G=128 products (%.1f s, %d threads over column slices, fp64)"
                       % (n, dt, cores))
    rows = {}
    b = synth.workload("batched")
    b["b_packed"] = oracle.repack(b["b_nk8"], b["K"])
    parts = oracle.split_columns(b["b_packed"], b["scales"], b["qzeros"])
    n, dt = _timed(lambda: oracle.gemm_split(b["a"], parts, 128, 8), seconds / 4)
    f = 2.0 * 32 * 4096 * 12800
    rows["batched_M32"] = dict(value=f * n / dt / 1e12, unit="TFLOP/s", gbs=alg_bytes(32, 4096, 12800, 128, True)
                               * n / dt / 1e9, cores=cores, sample="%d full M=32 products (%.1f s)" % (n, dt))
    pf = synth.workload("prefill")
    rows_m = 32
    a32 = pf["a"][:rows_m]
    parts = oracle.split_columns(pf["b_packed"], pf["scales"], pf["qzeros"])
    n, dt = _timed(lambda: oracle.gemm_split(a32, parts, 128, 8), seconds / 4)
    f = 2.0 * rows_m * 12800 * 4096
    rows["prefill_M256"] = dict(value=f * n / dt / 1e12, unit="TFLOP/s", cores=cores,
                                sample="%d products of the first %d of the 256 rows, K=12800 N=4096 (%.1f s); the "
                                       "oracle's cost per output is the same for every row" % (n, rows_m, dt))
    layers = synth.stack_layer(0) + synth.stack_layer(1)
    x = synth.stack_input(1)
    t0 = time.perf_counter()
    y = oracle.decode_layer_columns(layers[:4], x)
    oracle.decode_layer_columns(layers[4:], y)
    dt = time.perf_counter() - t0
    per_layer = dt / 2
    rows["decode_step_M1"] = dict(value=1.0 / (per_layer * synth.STACK["layers"]), unit="tok/s", cores=cores,
                                  sample="layers 0 and 1 of the 8B-class stack at M=1 (%.1f s), scaled to 40 "
                                         "layers" % dt)
    x32 = synth.stack_input(32)
    t0 = time.perf_counter()
    oracle.decode_layer_columns(layers[:4], x32)
    dt = time.perf_counter() - t0
    rows["decode_step_M32"] = dict(value=32.0 / (dt * synth.STACK["layers"]), unit="tok/s", cores=cores,
                                   sample="layer 0 of the 8B-class stack at M=32 (%.1f s), scaled to 40 layers"
                                          % dt)
    head["rows"] = rows
    return head


def host_info():
    info = {"nproc": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        m = re.search(r"Model name:\s*(.+)", out)
        if m:
            info["cpu_model"] = m.group(1).strip()
    except Exception:
        pass
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (no extra rows, no CPU baseline)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3 runs: one 256 MiB device copy first (a plain copy kernel of "
                         "known size, to calibrate HBM byte counters); implies --quick unless --only")
    ap.add_argument("--only", default="",
                    help="comma-separated extra rows to run after the headline (%s); no CPU baseline"
                         % ",".join(EXTRA_ROWS))
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the W4A16 linear "
              "would shard column- or row-wise with one all-reduce). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a16_weight_only_amd as w4
    if not os.path.exists(w4.LIB_PATH):
        from w4a16_weight_only_amd import build
        build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    stream = torch.cuda.Stream()
    log = lambda m: print("[bench] " + m, file=sys.stderr, flush=True)
    log("gpu: %s" % torch.cuda.get_device_name(0))

    if args.profile:
        src = torch.empty(64 * 2 ** 20, dtype=torch.int32, device="cuda").random_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst
        log("profile: 256 MiB device copy done")
        args.quick = not args.only

    log("headline: M=1 K=4096 N=12800 G=128 sym, %d steps" % args.steps)
    head = bench_gemm(torch, w4, stream, 1, 4096, 12800, 128, False, args.steps, args.warmup, seed=2)
    log("headline: %.2f us/call, %.0f GB/s" % (head["us_per_call"], head["gbs"]))

    extra = {}
    cpu = None
    if args.only:
        rows = [r for r in args.only.split(",") if r]
        bad = [r for r in rows if r not in EXTRA_ROWS]
        if bad:
            print("unknown rows %s (choose from %s)" % (bad, ",".join(EXTRA_ROWS)), file=sys.stderr)
            sys.exit(2)
    else:
        rows = [] if args.quick else list(EXTRA_ROWS)
    for r in rows:
        log(r)
        extra[r] = EXTRA_ROWS[r](torch, w4, stream, args.steps, args.warmup)
    if not args.quick and not args.only:
        log("cpu baseline (oracle) ~%.0f s" % args.cpu_seconds)
        cpu = cpu_baseline(args.cpu_seconds)

    traffic = measured_traffic()
    roofline = dict(bound="hbm", achieved=round(head["gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(head["gbs"] / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=("gemv_mma_kernel<M=1>" if head["path"] == "gemv_mma" else "gemv_kernel<M=1>"),
                    alg_bytes_per_launch=head["alg_bytes"],
                    us_per_launch=round(head["us_per_call"], 3), kernel_source_sha256_16=kernel_hash())
    line = {
        "metric": "W4A16 linear: HBM GB/s at M=1, TFLOP/s at M=32/256, % of roofline",
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xf16->f32",
        "data": "synthetic (seeded; uniform int4 weights, N(0,1) fp16 activations, U[0.5,1.5)/sqrt(K) fp16 scales)",
        "config": {"workload": "decode GEMV M=1 K=4096 N=12800 G=128 symmetric zp=8",
                   "global_batch": 1, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "headline_detail": head,
        "extra": extra,
        "host": host_info(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
