"""Benchmark of the NVFP4 Newton–Schulz path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one ns_orthogonalize call (all of: orientation, clip, Frobenius
normalisation, and five NVFP4 NS steps of quantize X both ways, A = qX qX^T,
quantize A, B = bA + c qA qA^T, quantize B, X = aX + qB qX16, and the
write-out) on the 3072 x 8192 BF16 gradient workload, inputs resident in
HBM.  value = algorithmic TFLOP/s (symmetric products counted once).

The same JSON line carries:
  roofline      the dominant kernel of a step, launched in the iteration's
                order with HIP events around each launch on the stream it
                runs on, against the f16 MFMA dense peak;
  quant         the standalone quantizer + dequantizer on 2^28 BF16 values
                (16384 x 16384) in HBM GB/s against the 8 TB/s peak;
  bf16_ns       the same five steps in plain BF16 torch.matmul (hipBLASLt)
                on the same GPU, for a like-for-like speedup;
  cpu_baseline  the float64 oracle on the host cores, bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0     # MI355X dense f16/bf16 MFMA
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
QUANT_DESIGN_BYTES_PER_ELEM = (2 + 2 + 0.5 + 1 / 16) + (0.5 + 1 / 16 + 2)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--quant-steps", type=int, default=100)
    p.add_argument("--quant-warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--no-quant", action="store_true", help="skip the quantizer line")
    p.add_argument("--no-grouped", action="store_true",
                   help="skip the grouped batches (four 3072-wide blocks; the pages' d=4096/6144 blocks)")
    p.add_argument("--copy-probe", action="store_true",
                   help="finish with a plain 256 MiB device copy, the reference kernel that "
                        "scales the FETCH_SIZE / WRITE_SIZE counters of a profiled run")
    return p.parse_args()


def time_events(fn, reps, warm, stream):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps      # ms per call


def kernel_timings(ns, torch, dev, m, n, stream, reps=10):
    """The three products of an NS iteration launched through the C ABI on
    the bench stream, each on operands quantized as inside
    ns_orthogonalize.  Each product runs `reps` times back to back between
    one pair of HIP events, after a spin kernel that keeps the GPU busy
    while the host enqueues, so the interval holds the launches alone (a
    pair of events around every single launch would add the events' own
    processing, about 6 us, to each).  Returns {name: (average ms per
    launch, algorithmic flops per launch)}."""
    from synth import gaussian
    X = torch.from_numpy((gaussian(m, n, seed=77) / np.sqrt(m * n)).astype(np.float32)).to(dev)
    A = torch.empty((m, m), dtype=torch.float32, device=dev)
    Bm = torch.empty((m, m), dtype=torch.float32, device=dev)
    Xo = torch.empty_like(X)
    sym = m * (m + 1)
    flops = {"gemm_gram_xxT": sym * n, "gemm_gram_aaT": sym * m, "gemm_update_bx": 2 * m * m * n}
    qx = ns.nvfp4_quantize(X, ns.NVFP4_ROWS, stream=stream)
    qt = ns.nvfp4_quantize(X, ns.NVFP4_COLS, stream=stream)
    ws = {k: torch.empty(max(1, ns.nvfp4_gemm_workspace_bytes(*mnk)), dtype=torch.uint8, device=dev)
          for k, mnk in (("g1", (m, m, n, True)), ("g2", (m, m, m, True)), ("g3", (m, n, m, False)))}
    g1 = lambda: ns.nvfp4_gemm(qx, qx, m, m, n, symmetric=True, out=A, workspace=ws["g1"], stream=stream)
    g1()
    qa = ns.nvfp4_quantize(A, ns.NVFP4_ROWS, stream=stream)
    g2 = lambda: ns.nvfp4_gemm(qa, qa, m, m, m, symmetric=True, alpha=2.0315, beta=-4.775, addend=A,
                               out=Bm, workspace=ws["g2"], stream=stream)
    g2()
    qb = ns.nvfp4_quantize(Bm, ns.NVFP4_ROWS, stream=stream)
    g3 = lambda: ns.nvfp4_gemm(qb, qt, m, n, m, alpha=1.0, beta=3.4445, addend=X, out=Xo,
                               workspace=ws["g3"], stream=stream)
    out = {}
    for name, fn in (("gemm_gram_xxT", g1), ("gemm_gram_aaT", g2), ("gemm_update_bx", g3)):
        fn()
        fn()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(20_000_000)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        out[name] = (s, e)
    torch.cuda.synchronize()
    return {k: (s.elapsed_time(e) / reps, flops[k]) for k, (s, e) in out.items()}


def source_digest():
    """sha256 over the GEMM kernel sources; recorded HBM-traffic counters
    apply only to the kernel they were taken from."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "nvfp4_device.hpp"):
        with open(os.path.join(ROOT, "newton_schulz_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# HBM bytes per launch of the dominant kernel (X = a X + qB qX16^T at
# 3072 x 8192), from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE, each scaled by
# what the counter reads for a plain copy of known size; see profiles/.
DOMINANT_TRAFFIC = {"src_sha256": "363d1c41511f59121901871fb4283f57ea55485230a150b1c2893897923e7e5c",
                    "bytes_per_launch": 440327111}


def bf16_ns_ms(torch, G, coeffs, stream, reps=10):
    def run():
        X = G.float()
        X = (X / (X.norm() + 1e-7)).to(torch.bfloat16)
        for a, b, c in coeffs:
            A = torch.mm(X, X.t())
            B = b * A + c * torch.mm(A, A)
            X = a * X + torch.mm(B, X)
        return X
    return time_events(run, reps, 3, stream)


def grouped_line(ns, torch, synth, dev, stream, label, shapes, seed0, coeffs, clip_quantile,
                 reps=3, warm=1):
    """Grouped NS over a batch of BF16 gradients drawn on the device (the
    lowrank value model), against BF16 torch NS of the same batch."""
    from oracle.ns import ns_iteration_flops
    Gs = [synth.device_lowrank_bf16(r, c, seed0 + i, dev) for i, (r, c) in enumerate(shapes)]
    outs = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
    ws = torch.empty(ns.ns_grouped_workspace_bytes(shapes), dtype=torch.uint8, device=dev)
    if clip_quantile:
        run = lambda: ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clip_quantile=clip_quantile,
                                                     outs=outs, workspace=ws, stream=stream)
        clip_what = f"clip at the {clip_quantile} quantile of each |G| (on the device)"
    else:
        clips = [float(8.0 * torch.sqrt(torch.mean(g.double() ** 2))) for g in Gs]
        run = lambda: ns.ns_orthogonalize_grouped(Gs, coeffs, clips, outs=outs, workspace=ws,
                                                  stream=stream)
        clip_what = "clip 8 x RMS(G) per matrix"
    ms = time_events(run, reps, warm, stream)
    flops = sum(len(coeffs) * ns_iteration_flops(r, c) for r, c in shapes)

    def bf16_batch():
        for g in Gs:
            X = g.t() if g.shape[0] > g.shape[1] else g
            X = X.float()
            X = (X / (X.norm() + 1e-7)).to(torch.bfloat16)
            for a, b, c in coeffs:
                A = torch.mm(X, X.t())
                B = b * A + c * torch.mm(A, A)
                X = a * X + torch.mm(B, X)
    bms = time_events(bf16_batch, reps, warm, stream)
    del ws, outs, Gs
    return {"workload": label, "matrices": len(shapes), "ms": round(ms, 3),
            "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "algorithmic_tflop": round(flops / 1e12, 3), "clip": clip_what,
            "bf16_ms": round(bms, 3), "speedup_nvfp4_vs_bf16": round(bms / ms, 3)}


def cpu_baseline(G, clip, coeffs, m, n):
    from oracle import ns as N
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    G64 = G.astype(np.float64)
    done, t0 = 0, time.perf_counter()
    while True:
        N.ns_nvfp4(G64, coeffs[:1], clip=clip)
        done += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or done >= len(coeffs):
            break
    flops = done * N.ns_iteration_flops(m, n)
    return {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} NVFP4 NS step(s) of the 3072x8192 workload in float64 "
                      f"(numpy/BLAS), {el:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the NS path runs on a single GPU and has "
              "no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import newton_schulz_amd as ns
    import synth
    from oracle.ns import ns_iteration_flops

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    coeffs = [synth.QUINTIC] * synth.STEPS
    spec = synth.ns_workload("ns3072x8192")
    G, bits, clip = synth.ns_matrix(spec, 0)
    m, n = G.shape
    Gd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = torch.empty(ns.ns_workspace_bytes(m, n), dtype=torch.uint8, device=dev)
    step = lambda: ns.ns_orthogonalize(Gd, coeffs, clip, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(step, args.steps, 0, stream)
    wall = time.perf_counter() - t0
    flops = synth.STEPS * ns_iteration_flops(m, n)
    tflops = flops / (ms * 1e-3) / 1e12

    kt = kernel_timings(ns, torch, dev, m, n, stream)
    # share of one NS step: each GEMM runs once per iteration
    dom = max(kt, key=lambda k: kt[k][0])
    dms, dflops = kt[dom]
    achieved = dflops / (dms * 1e-3) / 1e12
    traffic = None
    if dom == "gemm_update_bx" and DOMINANT_TRAFFIC["src_sha256"] == source_digest():
        traffic = DOMINANT_TRAFFIC["bytes_per_launch"]
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
            "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per launch", "avg_launch_ms": round(dms, 4),
            "per_kernel_ms": {k: round(v[0], 4) for k, v in kt.items()}}

    line = {
        "metric": "NVFP4 Newton–Schulz TFLOP/s (% BF16 MFMA peak) + nvfp4_quant HBM GB/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "ns3072x8192: one 3072x8192 BF16 gradient (rank-32 signal "
                               "+ N(0,0.01^2) noise + 0.1% outliers x50, seed 4), clip 8xRMS, "
                               "5 NVFP4 NS steps with the quintic (3.4445,-4.775,2.0315)",
                   "m": m, "n": n, "ns_steps": synth.STEPS, "operands": "nvfp4 (e2m1 x e4m3/16 + f32)",
                   "accumulate": "f32", "frac_of_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        "roofline": roof,
        "wall_s_timed": round(wall, 3),
    }

    # the same step with the random Hadamard transform of every quantized
    # operand (one sign mask per NS step)
    masks = synth.rht_masks(synth.STEPS, seed=spec["seeds"][0])
    rstep = lambda: ns.ns_orthogonalize_rht(Gd, coeffs, masks, clip, out=out, workspace=ws,
                                            stream=stream)
    rms_ = time_events(rstep, args.steps, args.warmup, stream)
    line["ns_rht"] = {"ms": round(rms_, 4), "value": round(flops / (rms_ * 1e-3) / 1e12, 2),
                      "unit": "TFLOP/s",
                      "what": "ns_orthogonalize_rht: the same step with H_16^r on every "
                              "quantized operand (extra amax passes over the transformed tensors)"}

    # the same step with the clip taken on the device as the 0.99 quantile of
    # |G| (radix-selection passes over G before the normalisation: two for BF16)
    qstep_ = lambda: ns.ns_orthogonalize_ex(Gd, coeffs, clip_quantile=0.99, out=out, workspace=ws,
                                            stream=stream)
    qms_ = time_events(qstep_, args.steps, args.warmup, stream)
    qws_ = torch.empty(ns.ns_abs_quantile_workspace_bytes(), dtype=torch.uint8, device=dev)
    qout_ = torch.empty(1, dtype=torch.float32, device=dev)
    sel_ms = time_events(lambda: ns.ns_abs_quantile(Gd, 0.99, out=qout_, workspace=qws_, stream=stream),
                         20, 3, stream)
    line["ns_p99_clip"] = {"ms": round(qms_, 4), "value": round(flops / (qms_ * 1e-3) / 1e12, 2),
                           "unit": "TFLOP/s", "quantile_ms": round(sel_ms, 4),
                           "what": "ns_orthogonalize_ex with clip_quantile=0.99: the clip is the "
                                   "0.99 quantile of |G| found on the device (radix selection)"}

    # the same step with adaptive 4/6 block scaling on every quantization
    # (each block keeps the better of its M = 6 and M = 4 encodings)
    astep_ = lambda: ns.ns_orthogonalize_ex(Gd, coeffs, clip=clip, adaptive46=True, out=out,
                                            workspace=ws, stream=stream)
    ams_ = time_events(astep_, args.steps, args.warmup, stream)
    line["ns_46"] = {"ms": round(ams_, 4), "value": round(flops / (ams_ * 1e-3) / 1e12, 2),
                     "unit": "TFLOP/s",
                     "what": "ns_orthogonalize_ex with adaptive46: every quantization picks M = 4 "
                             "or 6 per block by squared error (two encodings per block)"}

    # BF16 torch NS of the same matrix, same GPU
    bms = bf16_ns_ms(torch, Gd, coeffs, stream)
    line["bf16_ns"] = {"ms": round(bms, 4), "speedup_nvfp4_vs_bf16": round(bms / ms, 3),
                       "what": "torch.mm in bf16 (hipBLASLt), full products, same 5 steps"}

    if not args.no_grouped:
        del ws
        torch.cuda.empty_cache()
        b4 = synth.ns_workload("ns4blocks")
        line["grouped"] = [
            grouped_line(ns, torch, synth, dev, stream,
                         "four blocks at width 3072: Q,K,V,O 3072^2, up 3072x8192, down 8192x3072 "
                         "(24 matrices), quintic x5", b4["shapes"], 5000, coeffs, 0.0),
            grouped_line(ns, torch, synth, dev, stream,
                         "the pages' four decoder blocks at d=4096 (d_ff 11008, 32 heads, 8 KV "
                         "heads; 28 matrices), quintic x5", synth.pages_block_shapes(4096), 6000,
                         coeffs, 0.99),
            grouped_line(ns, torch, synth, dev, stream,
                         "the pages' four decoder blocks at d=6144 (d_ff 13824, 48 heads, 8 KV "
                         "heads; 28 matrices), quintic x5", synth.pages_block_shapes(6144), 7000,
                         coeffs, 0.99),
        ]
        torch.cuda.empty_cache()
        ws = None

    if not args.no_quant:
        del ws
        qbits, _ = synth.quant_workload()
        xq = torch.from_numpy(qbits.view(np.int16)).view(torch.bfloat16).to(dev)
        rows, cols = xq.shape
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        sg = torch.empty(1, dtype=torch.float32, device=dev)
        qws = torch.empty(ns.nvfp4_quantize_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
        deq = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)

        def qstep():
            ns.nvfp4_quantize(xq, ns.NVFP4_ROWS, codes, scales, sg, workspace=qws, stream=stream)
            ns.nvfp4_dequantize(codes, scales, sg, rows, cols, ns.NVFP4_ROWS, ns.NS_BF16, out=deq,
                                stream=stream)
        qms = time_events(qstep, args.quant_steps, args.quant_warmup, stream)
        qbytes = QUANT_DESIGN_BYTES_PER_ELEM * rows * cols
        gbps = qbytes / (qms * 1e-3) / 1e9
        t_q = time_events(lambda: ns.nvfp4_quantize(xq, ns.NVFP4_ROWS, codes, scales, sg,
                                                    workspace=qws, stream=stream), 50, 5, stream)
        t_d = time_events(lambda: ns.nvfp4_dequantize(codes, scales, sg, rows, cols, ns.NVFP4_ROWS,
                                                      ns.NS_BF16, out=deq, stream=stream), 50, 5, stream)
        line["quant"] = {
            "metric": "nvfp4_quant HBM GB/s", "value": round(gbps, 1), "unit": "GB/s",
            "workload": "16384x16384 BF16 Student-t(3)*0.02 with 0.1% x50, quantize (amax pass + "
                        "encode) + dequantize to BF16, 1x16 blocks",
            "ms": round(qms, 4), "quantize_ms": round(t_q, 4), "dequantize_ms": round(t_d, 4),
            "design_bytes": int(qbytes),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None}}
        del xq, deq

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(G, clip, coeffs, m, n)
    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
