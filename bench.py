#!/usr/bin/env python3
"""Throughput of the weight-quantised GEMV/GEMM path on one MI355X.

Headline (the JSON `value`): weight GB/s of the decode-shape W4A16 GEMV --
both projections of one layer, K=5120,N=17280 and K=17280,N=5120, int4 codes
with bf16 group-128 scales and zero 8, bf16 x, bf16 out -- over a batch of
c = 1, 2 and 4 activation columns.  One step is those six GEMV calls.  Each
call reads a different copy of the weights from a rotating set larger than
the 256 MB Infinity Cache, so every weight byte comes from HBM.

The same run also times the other rows of the path (quantise + pack, the
small-batch GEMV, the 8192^3 W4A16 GEMM, the ternary GEMV) and reports them
under "rows"; and, on rank 0, times the CPU oracle on a bounded sample
("cpu_baseline").  GEMV rows also give tokens-equivalent rows per second
("Mrows_per_s": output rows times activation columns per second, millions).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4 GEMV weight GB/s (% of HBM peak); W4A16 GEMM TFLOP/s (% of MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA (and fp8)
MALL_BYTES = 256 << 20
SETTLE_S = 0.4              # seconds of step replays before the warm-up steps


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def sha_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel_src):
    """Memory bytes per launch from the committed PMC summary, if it was taken
    on the current kernel source (else None): FETCH_SIZE + WRITE_SIZE, and the
    L2's DRAM-side request counters, each scaled by a plain copy."""
    path = os.path.join(ROOT, "profiles", "gemv_w4_decode_traffic.md")
    if not os.path.exists(path):
        return None, None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_sha or m_sha.group(1) != sha_of(kernel_src):
        return None, None
    vals = []
    for key in ("hbm_bytes_per_launch", "dram_bytes_per_launch"):
        m = re.search(key + r":\s*([0-9.eE+]+)", text)
        vals.append(float(m.group(1)) if m else None)
    return tuple(vals)


def copies_for(nbytes, minimum=2):
    return max(minimum, int((MALL_BYTES * 1.25) // max(nbytes, 1)) + 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the secondary rows")
    ap.add_argument("--rows", default="small,gemm,ternary",
                    help="secondary rows to time (comma list of small, gemm, ternary)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run one plain device copy of this size (PMC scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "across GPUs each would take a slice of the output rows (no collective needed)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_wq_quantize_amd as g
    import wq_inputs

    if not os.path.exists(g.LIB_PATH):
        from gemm_wq_quantize_amd import build as b
        b.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("device", torch.cuda.get_device_name(dev))

    # ------------------------------------------------------------ decode GEMV
    shapes = wq_inputs.DECODE_SHAPES
    batches = (1, 2, 4)
    sets = []
    for (k, n) in shapes:
        p = wq_inputs.decode_int4(k, n, cmax=4)
        pk = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        g.wq_pack_int4(torch.from_numpy(p.codes).to(dev), g.LAYOUT_GFX950, pk)
        sc = torch.from_numpy(p.scale_bits).view(torch.bfloat16).to(dev)
        wbytes = pk.numel() + sc.numel() * 2
        ncopy = copies_for(wbytes)
        copies = [(pk, sc)] + [(pk.clone(), sc.clone()) for _ in range(ncopy - 1)]
        x = torch.from_numpy(p.x_bits).view(torch.bfloat16).to(dev)
        out = torch.empty((4, n), dtype=torch.bfloat16, device=dev)
        sets.append(dict(k=k, n=n, copies=copies, x=x, out=out, wbytes=wbytes))
        log(f"decode K={k} N={n}: {wbytes / 1e6:.2f} MB of weights x {ncopy} copies")
    torch.cuda.synchronize()

    calls = [(si, c) for si in range(len(sets)) for c in batches]
    ncopy = min(len(s["copies"]) for s in sets)

    def call(si, c, j):
        s = sets[si]
        pk, sc = s["copies"][j % len(s["copies"])]
        g.wq_gemv_w4(pk, 1, sc, None, 8.0, s["k"], 128, s["x"][:c], s["out"][:c])

    # One HIP graph per rotation index: a step is the 6 calls, each on its own
    # weight copy; step i replays graph i % ncopy.  Graph replay removes the
    # per-launch host and dispatch gaps, which would otherwise be a large part
    # of a 10 us kernel.
    def step_eager(i):
        for t, (si, c) in enumerate(calls):
            call(si, c, i * len(calls) + t)

    for (si, c) in calls:  # eager first calls: one-time set-up happens outside capture
        call(si, c, 0)
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    for j in range(ncopy):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(gr, stream=cap):
                for t, (si, c) in enumerate(calls):
                    call(si, c, j * len(calls) + t)
        graphs.append(gr)
    torch.cuda.synchronize()

    # Settle: the device needs a few tenths of a second of sustained work to
    # reach its loaded clock (with a handful of warm-up steps the timed steps
    # ran 10-15% slower), so graph replays of the step run for SETTLE_S
    # seconds whatever --warmup says; then the W counted warm-up steps.
    t_settle = time.perf_counter()
    j = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(50):
            graphs[j % ncopy].replay()
            j += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % ncopy].replay()
        step_eager(i)
    torch.cuda.synchronize()
    log(f"settled for {time.perf_counter() - t_settle:.2f} s ({j} replays), warmup {args.warmup} steps done")

    # The timed region: K steps launched back to back on the current stream
    # (what a caller sees), bracketed by events and synchronisations.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step_eager(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    region_ms = t_start.elapsed_time(t_end)
    ms_per_step = region_ms / args.steps
    wbytes_step = sum(sets[si]["wbytes"] for si, _ in calls)
    value = wbytes_step / (ms_per_step * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (wall {wall:.3f} s), "
        f"{value:.1f} GB/s of weights")

    # the same steps replayed from HIP graphs (no host launch gaps)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % ncopy].replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms_per_step = e0.elapsed_time(e1) / args.steps

    n_launch = len(calls)
    alg_step = sum(sets[si]["wbytes"] + 2 * sets[si]["k"] * c + 2 * sets[si]["n"] * c
                   for si, c in calls)

    # per-configuration breakdown: a graph of ncopy launches of one call each
    per_call = {}
    for (si, c) in calls:
        s = sets[si]
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(gr, stream=cap):
                for j in range(ncopy):
                    call(si, c, j)
        for _ in range(20):
            gr.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        d = e0.elapsed_time(e1) / (50 * ncopy)
        alg = s["wbytes"] + 2 * s["k"] * c + 2 * s["n"] * c
        per_call[f"K{s['k']}_N{s['n']}_c{c}"] = {
            "us": round(d * 1e3, 2), "weight_GBs": round(s["wbytes"] / (d * 1e-3) / 1e9, 1),
            "alg_GBs": round(alg / (d * 1e-3) / 1e9, 1),
            "frac_hbm": round(alg / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "Mrows_per_s": round(s["n"] * c / (d * 1e-3) / 1e6, 1)}
    traffic, traffic_dram = read_traffic(os.path.join(ROOT, "gemm_wq_quantize_amd", "csrc", "gemv_w4.hip"))
    log("per launch:", json.dumps(per_call))
    # roofline of the kernel: algorithmic bytes of one launch over its average
    # duration, both averaged over the six configurations of a step
    avg_launch_ms = sum(v["us"] for v in per_call.values()) / len(per_call) * 1e-3
    achieved = (alg_step / n_launch) / (avg_launch_ms * 1e-3) / 1e9

    peaks = measured_peaks(g, torch, dev, alg_step // n_launch, log)

    rows = {"gemv_w4_decode": per_call}
    if not args.no_rows:
        which = {w.strip() for w in args.rows.split(",") if w.strip()}
        rows.update(secondary_rows(g, torch, np, wq_inputs, dev, log, which))
        for key in ("gemm_w4a16_8192", "gemm_w4a16_8192_group128"):
            if key in rows:
                rows[key]["frac_of_measured_mfma_loop"] = round(rows[key]["TFLOPs"] / peaks["mfma_bf16_TFLOPs"], 4)

    if args.calibrate_copy_mb:
        nb = args.calibrate_copy_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {nb} bytes done")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, wq_inputs, log)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4*bf16->f32",
        "data": "synthetic (seeded wq_inputs: codes U{0..15}, bf16 scales U(0.002,0.02), bf16 x N(0,1))",
        "config": {
            "workload": "decode W4A16 GEMV, K=5120,N=17280 and K=17280,N=5120, group 128, "
                        "zero 8, bf16 x and out, batch c in {1,2,4}; one step = the 6 calls",
            "weight_bytes_per_step": wbytes_step,
            "hbm_resident": "rotating weight copies > 256 MB Infinity Cache",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_gemv_w4_persist (c=1), k_gemv_w4_quad (c=2,4)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_dram_requests": traffic_dram,
            "alg_bytes_per_launch": round(alg_step / n_launch),
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "graph_replay_ms_per_step": round(graph_ms_per_step, 5),
            "frac_of_measured_read": round(achieved / peaks["hbm_read_GBs_same_bytes"], 4),
        },
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(result), flush=True)


def measured_peaks(g, torch, dev, launch_bytes, log):
    """What this device sustains, from the library's calibration kernels: a
    plain streaming read of one decode launch's byte count (rotating copies,
    so HBM serves it) and of 1 GiB, a bf16 matrix-core loop and an fp32 FMA
    loop, each timed from HIP graphs of back-to-back launches."""
    sink = torch.empty(g.wq_peak_read_sink_words(), dtype=torch.int32, device=dev)
    nb = (launch_bytes + 15) // 16 * 16
    nc = copies_for(nb, minimum=4)
    bufs = [torch.empty(nb, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(nc)]
    same = timed(torch, lambda i: g.wq_peak_read(bufs[i % nc], sink), 4 * nc)
    del bufs
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    gib = timed(torch, lambda i: g.wq_peak_read(big, sink), 4)
    del big
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wg_m, it_m = 8 * cus, 512
    msink = torch.empty(max(wg_m, 64 * cus) * 256, dtype=torch.float32, device=dev)
    mfma = timed(torch, lambda i: g.wq_peak_mfma_bf16(wg_m, it_m, msink), 4)
    wg_v, it_v = 64 * cus, 2048
    valu = timed(torch, lambda i: g.wq_peak_valu_fma(wg_v, it_v, msink), 4)
    out = {
        "hbm_read_GBs_same_bytes": round(nb / (same * 1e-3) / 1e9, 1),
        "read_bytes": nb,
        "read_us_same_bytes": round(same * 1e3, 2),
        "hbm_read_GBs_1GiB": round((1 << 30) / (gib * 1e-3) / 1e9, 1),
        "mfma_bf16_TFLOPs": round(wg_m * 4 * it_m * 8 * 32768 / (mfma * 1e-3) / 1e12, 1),
        "valu_fp32_fma_TFLOPs": round(wg_v * 256 * it_v * 8 * 2 / (valu * 1e-3) / 1e12, 1),
        "kernels": "wq_peak_read (1024 lanes per CU, 16-B loads, 4 in flight), wq_peak_mfma_bf16 "
                   "(8 independent 32x32x16 chains per wave, one wave per SIMD), wq_peak_valu_fma "
                   "(8 independent v_fma_f32 chains per lane, 64 workgroups per CU)",
    }
    log("measured peaks:", json.dumps(out))
    return out


def timed(torch, fn, iters):
    """Average ms per call of fn(i), i = 0..iters-1, captured in one HIP graph
    and replayed (launch gaps excluded)."""
    fn(0)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gr, stream=cap):
            for i in range(iters):
                fn(i)
    gr.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(3):
        gr.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (3 * iters)  # ms


def secondary_rows(g, torch, np, wq_inputs, dev, log, which):
    rows = {}
    if "small" in which:
        rows.update(small_batch_rows(g, torch, wq_inputs, dev, log))
    if "gemm" in which:
        rows.update(gemm_rows(g, torch, wq_inputs, dev, log))
    if "ternary" in which:
        rows.update(ternary_rows(g, torch, wq_inputs, dev, log))
    return rows


def small_batch_rows(g, torch, wq_inputs, dev, log):
    rows = {}
    # quantise + pack and the small-batch GEMV (bf16 group-128 scales)
    qrow, srow = {}, {}
    for (k, n) in wq_inputs.SMALL_BATCH_SHAPES:
        p = wq_inputs.small_batch_int4(k, n, cmax=32)
        w = torch.from_numpy(p.w_f16).view(torch.float16).to(dev)
        nc = copies_for(w.numel() * 2)
        ws = [w] + [w.clone() for _ in range(nc - 1)]
        pk = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((n, k // 128), dtype=torch.bfloat16, device=dev)
        ms = timed(torch, lambda i: g.wq_quantize_pack_int4(ws[i % nc], 128, 1, pk, sc), 20)
        qbytes = w.numel() * 2 + pk.numel() + sc.numel() * 2
        qrow[f"K{k}_N{n}"] = {"us": round(ms * 1e3, 2), "GBs": round(qbytes / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(qbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        wb = pk.numel() + sc.numel() * 2
        nc2 = copies_for(wb)
        cps = [(pk, sc)] + [(pk.clone(), sc.clone()) for _ in range(nc2 - 1)]
        x = torch.from_numpy(p.x_bits).view(torch.bfloat16).to(dev)
        out = torch.empty((32, n), dtype=torch.bfloat16, device=dev)
        for c in (8, 16, 32):
            ms = timed(torch, lambda i: g.wq_gemv_w4(cps[i % nc2][0], 1, cps[i % nc2][1], None, 8.0,
                                                      k, 128, x[:c], out[:c]), 50)
            # the products run on the matrix cores; the weight stream (plus x
            # and out) against HBM is the bound
            flops = 2.0 * n * k * c
            alg = wb + 2 * k * c + 2 * n * c
            srow[f"K{k}_N{n}_c{c}"] = {
                "us": round(ms * 1e3, 2), "weight_GBs": round(wb / (ms * 1e-3) / 1e9, 1),
                "alg_GBs": round(alg / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                "Mrows_per_s": round(n * c / (ms * 1e-3) / 1e6, 1)}
        del ws, cps
        torch.cuda.empty_cache()
    rows["quantize_pack_int4"] = qrow
    rows["gemv_w4_small_batch"] = srow
    log("quantise / small batch:", json.dumps(qrow), json.dumps(srow))
    return rows


def gemm_rows(g, torch, wq_inputs, dev, log):
    rows = {}
    # 8192^3 W4A16 GEMM
    q = wq_inputs.large_gemm(n_rows=1)
    a = torch.from_numpy(q.a_bits).view(torch.bfloat16).to(dev)
    b = torch.empty((q.n, q.k // 2), dtype=torch.uint8, device=dev)
    g.wq_pack_int4(torch.from_numpy(q.codes).to(dev), 1, b)
    sc = torch.from_numpy(q.scale_bits).view(torch.bfloat16).to(dev)
    c = torch.empty((q.m, q.n), dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda i: g.wq_gemm_w4a16(a, b, 1, sc, q.k, 8.0, c), 10)
    tf = 2.0 * q.m * q.n * q.k / (ms * 1e-3) / 1e12
    rows["gemm_w4a16_8192"] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1),
                               "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4)}
    log("gemm 8192^3:", json.dumps(rows["gemm_w4a16_8192"]))
    # the same product with group-128 bf16 scales (the quantiser's output
    # layout), drawn like the decode workload's scales
    qg = wq_inputs.grouped_gemm(8, q.n, q.k, 128)
    sg = torch.from_numpy(qg.scale_bits).view(torch.bfloat16).to(dev)
    ms = timed(torch, lambda i: g.wq_gemm_w4a16(a, b, 1, sg, 128, 8.0, c), 10)
    tf = 2.0 * q.m * q.n * q.k / (ms * 1e-3) / 1e12
    rows["gemm_w4a16_8192_group128"] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1),
                                        "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4)}
    log("gemm 8192^3, group 128:", json.dumps(rows["gemm_w4a16_8192_group128"]))
    del a, b, c, sg
    torch.cuda.empty_cache()
    return rows


def ternary_rows(g, torch, wq_inputs, dev, log):
    rows = {}
    # ternary GEMV, K=5120 N=17280
    t = wq_inputs.ternary_gemv(5120, 17280, cmax=8)
    wb = torch.empty((17280, 40, 28), dtype=torch.uint8, device=dev)
    g.wq_pack_ptq1_0(torch.from_numpy(t.trits).to(dev),
                     torch.from_numpy(t.d_bits).view(torch.int16).to(dev), wb)
    nc = copies_for(wb.numel())
    wcs = [wb] + [wb.clone() for _ in range(nc - 1)]
    xq = torch.empty((8, 160, 36), dtype=torch.uint8, device=dev)
    g.wq_quantize_q8_1(torch.from_numpy(t.x).to(dev), xq)
    y = torch.empty((8, 17280), dtype=torch.float32, device=dev)
    trow = {}
    for cc in (1, 4, 8):
        ms = timed(torch, lambda i: g.wq_gemv_ternary(wcs[i % nc], xq[:cc], 5120, y[:cc]), 50)
        trow[f"K5120_N17280_c{cc}"] = {
            "us": round(ms * 1e3, 2), "weight_GBs": round(wb.numel() / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(wb.numel() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "Mrows_per_s": round(17280 * cc / (ms * 1e-3) / 1e6, 1)}
    rows["gemv_ternary"] = trow
    log("ternary:", json.dumps(trow))
    # the same GEMV on PTQ1_1 superblocks (216 bytes per 1024 trits), with
    # block scales that have the exponent statistics of trained weights
    tc = wq_inputs.ternary_correlated_scales(5120, 17280, cmax=8)
    blk = torch.empty((17280, 40, 28), dtype=torch.uint8, device=dev)
    g.wq_pack_ptq1_0(torch.from_numpy(tc.trits).to(dev),
                     torch.from_numpy(tc.d_bits).view(torch.int16).to(dev), blk)
    sup, book, ei, ep = g.wq_ptq1_1_encode(blk.cpu().numpy())
    sup_d = torch.from_numpy(sup).to(dev)
    tabs = [torch.from_numpy(a).to(dev) for a in (book, ei, ep)]
    nc1 = copies_for(sup_d.numel())
    scs = [sup_d] + [sup_d.clone() for _ in range(nc1 - 1)]
    xq1 = torch.empty((8, 160, 36), dtype=torch.uint8, device=dev)
    g.wq_quantize_q8_1(torch.from_numpy(tc.x).to(dev), xq1)
    srow = {"escaped_superblocks": int(len(ei))}
    for cc in (1, 4, 8):
        ms = timed(torch, lambda i: g.wq_gemv_ternary_ptq1_1(scs[i % nc1], *tabs, xq1[:cc], 5120, y[:cc]), 50)
        srow[f"K5120_N17280_c{cc}"] = {
            "us": round(ms * 1e3, 2), "weight_GBs": round(sup_d.numel() / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(sup_d.numel() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "Mrows_per_s": round(17280 * cc / (ms * 1e-3) / 1e6, 1)}
    rows["gemv_ternary_ptq1_1"] = srow
    log("ternary ptq1_1:", json.dumps(srow))
    # 4096 activation columns: the matrix-core path (fp4 trits x fp8 pairs,
    # priced as 2 ops per useful MAC against the 5 POP/s int8 / fp8 peak;
    # the call includes unpacking both operands)
    gen = torch.Generator(device="cpu").manual_seed(0)
    mg = 4096
    xg = torch.empty((mg, 160, 36), dtype=torch.uint8, device=dev)
    g.wq_quantize_q8_1(torch.randn(mg, 5120, generator=gen).to(dev), xg)
    yg = torch.empty((mg, 17280), dtype=torch.float32, device=dev)
    ms = timed(torch, lambda i: g.wq_gemv_ternary(wcs[i % nc], xg, 5120, yg), 5)
    tops = 2.0 * mg * 17280 * 5120 / (ms * 1e-3) / 1e12
    rows["gemm_ternary_4096"] = {"ms": round(ms, 4), "TOPs": round(tops, 1),
                                 "frac_mfma_int8": round(tops / INT8_PEAK_TOPS, 4),
                                 "kernel": "k_unpack_ptq1_0_fp4 + k_unpack_q8_1_fp8 + k_gemm_ternary (v_mfma_scale_f32_32x32x64_f8f6f4)"}
    log("ternary gemm 4096 x 17280 x 5120:", json.dumps(rows["gemm_ternary_4096"]))
    # the same product on PTQ1_1 superblocks (unpacked by their own kernel)
    ms = timed(torch, lambda i: g.wq_gemv_ternary_ptq1_1(scs[i % nc1], *tabs, xg, 5120, yg), 5)
    tops = 2.0 * mg * 17280 * 5120 / (ms * 1e-3) / 1e12
    rows["gemm_ternary_ptq1_1_4096"] = {"ms": round(ms, 4), "TOPs": round(tops, 1),
                                        "frac_mfma_int8": round(tops / INT8_PEAK_TOPS, 4)}
    log("ternary gemm on ptq1_1 superblocks:", json.dumps(rows["gemm_ternary_ptq1_1_4096"]))
    del xg, yg, scs, sup_d
    return rows


def cpu_baseline(np, wq_inputs, log):
    """The oracle, untouched, on whole steps of the same workload (the 6
    GEMVs), repeated until at least 10 s of CPU time have been timed, with
    its BLAS pool set to the host cores this process may run on; plus the
    tiny int4 GEMV (256 x 512, one column) on one thread."""
    from oracle import int4 as o4
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # no pool control: the BLAS default (reported as is)
        threadpool_limits = None
    ctx = threadpool_limits(limits=threads) if threadpool_limits else _nullcontext()
    with ctx:
        out = _cpu_steps(np, o4, wq_inputs, log, threads)
    # the tiny per-row fp32 GEMV on one thread
    p = wq_inputs.tiny_int4()
    packed = o4.pack(p.codes, 0)
    ctx1 = threadpool_limits(limits=1) if threadpool_limits else _nullcontext()
    with ctx1:
        reps, t1 = 0, 0.0
        while t1 < 1.0:
            t0 = time.perf_counter()
            o4.gemv_w4(packed, 0, p.scales, p.zeros, 0.0, p.k, p.x)
            t1 += time.perf_counter() - t0
            reps += 1
    tiny_bytes = packed.nbytes + p.scales.nbytes + p.zeros.nbytes
    out["tiny_int4_gemv_1_thread"] = {"us_per_call": round(t1 / reps * 1e6, 1),
                                      "GBs": round(tiny_bytes * reps / t1 / 1e9, 4), "calls": reps}
    log(f"cpu oracle, tiny GEMV on 1 thread: {t1 / reps * 1e6:.1f} us per call")
    return out


class _nullcontext:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def _cpu_steps(np, o4, wq_inputs, log, threads):
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        model = "unknown"
    sets = []
    for (k, n) in wq_inputs.DECODE_SHAPES:
        p = wq_inputs.decode_int4(k, n, cmax=4)
        sets.append((o4.pack(p.codes, 1), p))
    total_bytes, total_s, steps = 0, 0.0, 0
    while total_s < 10.0:
        for packed, p in sets:
            for c in (1, 2, 4):
                t0 = time.perf_counter()
                o4.gemv_w4(packed, 1, p.scales, None, 8.0, 128, p.x[:c])
                total_s += time.perf_counter() - t0
                total_bytes += packed.nbytes + p.scale_bits.nbytes
        steps += 1
    v = total_bytes / total_s / 1e9
    log(f"cpu oracle: {steps} steps in {total_s:.2f} s, {v:.3f} GB/s, {threads} cores ({model})")
    return {"value": round(v, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu": model,
            "sample": f"{steps} full steps of the 6 decode GEMVs (both shapes, c = 1, 2, 4), "
                      f"{total_s:.1f} s"}


if __name__ == "__main__":
    main()
