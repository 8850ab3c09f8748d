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
  accuracy      relative L2 error of plain NVFP4 NS and of its variants
                (transform, adaptive 4/6, p99 clip) against unquantized NS;
  cpu_baseline  the C++ oracle (float64 NS, exact quantizer, OpenMP) on the
                host cores: the four single-GPU workloads, a bounded sample
                of the largest.
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
    p.add_argument("--no-accuracy", action="store_true",
                   help="skip the accuracy table (NVFP4 variants against unquantized NS)")
    p.add_argument("--quant-only", action="store_true",
                   help="run only the standalone quantizer leg (for profiling its kernels)")
    p.add_argument("--gemm-only", action="store_true",
                   help="run only the three products of one NS iteration at 3072x8192, as in "
                        "the roofline leg (for profiling the GEMM kernels)")
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


def kernel_timings(ns, torch, dev, Gd, clip, coeffs, stream, reps=10):
    """The three products of an NS iteration launched through the C ABI on
    the bench stream, on the operands of the NS run itself: a two-step
    ns_orthogonalize call on the workload leaves its second step's X, qX,
    qX16, qA, qB and tensor scales in the workspace (ns_workspace_views).
    The update product runs in place (addend = out = X, beta = a), as in the
    iteration; the Gram products write the whole symmetric product (the
    iteration keeps only the upper triangle).  Each product runs `reps`
    times back to back between one pair of HIP events, after a spin kernel
    that keeps the GPU busy while the host enqueues, so the interval holds
    the launches alone (a pair of events around every single launch would
    add the events' own processing, about 6 us, to each).  Returns {name:
    (average ms per launch, algorithmic flops per launch)}."""
    m, n = Gd.shape
    wsn = torch.empty(ns.ns_workspace_bytes(m, n), dtype=torch.uint8, device=dev)
    out = torch.empty((m, n), dtype=torch.float32, device=dev)
    ns.ns_orthogonalize(Gd, coeffs[:2], clip, out=out, workspace=wsn, stream=stream)
    v = ns.ns_workspace_views(wsn, m, n)
    sg = v["sg"]
    qx = (*v["qX"], sg[0:1])
    qt = (*v["qX16"], sg[0:1])
    qa = (*v["qA"], sg[1:2])
    qb = (*v["qB"], sg[2:3])
    X = v["X"]
    a, b, c = coeffs[1]
    A = torch.empty((m, m), dtype=torch.float32, device=dev)
    Bm = torch.empty((m, m), dtype=torch.float32, device=dev)
    sym = m * (m + 1)
    flops = {"gemm_gram_xxT": sym * n, "gemm_gram_aaT": sym * m, "gemm_update_bx": 2 * m * m * n}
    ws = {k: torch.empty(max(1, ns.nvfp4_gemm_workspace_bytes(*mnk)), dtype=torch.uint8, device=dev)
          for k, mnk in (("g1", (m, m, n, True)), ("g2", (m, m, m, True)), ("g3", (m, n, m, False)))}
    g1 = lambda: ns.nvfp4_gemm(qx, qx, m, m, n, symmetric=True, out=A, workspace=ws["g1"], stream=stream)
    g1()          # the whole symmetric A: the addend of the next product
    g2 = lambda: ns.nvfp4_gemm(qa, qa, m, m, m, symmetric=True, alpha=c, beta=b, addend=A,
                               out=Bm, workspace=ws["g2"], stream=stream)
    g3 = lambda: ns.nvfp4_gemm(qb, qt, m, n, m, alpha=1.0, beta=a, addend=X, out=X,
                               workspace=ws["g3"], stream=stream)
    res = {}
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
        res[name] = (s, e)
    torch.cuda.synchronize()
    return {k: (s.elapsed_time(e) / reps, flops[k]) for k, (s, e) in res.items()}


def source_digest(files=("gemm.hip", "nvfp4_device.hpp")):
    """sha256 over the kernel sources' code (comments and blank lines left
    out); recorded HBM-traffic counters apply only to the code they were
    taken from."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "newton_schulz_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()


# HBM bytes per launch of the dominant kernel (X = a X + qB qX16^T at
# 3072 x 8192), from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE, each scaled by
# what the counter reads for a plain copy of known size; see profiles/.
DOMINANT_TRAFFIC = {"src_sha256": "75794f1efd41fced31aff27c81f9d13bb8e6609d5dcd98459d730eb955e4337e",
                    "bytes_per_launch": 440739011}
# Bytes of one quantize + dequantize pair of the 2^28 BF16 tensor (the
# maximum, encode and decode kernels) between the L2 caches and memory,
# measured the same way (Infinity Cache hits included).
QUANT_TRAFFIC = {"src_sha256": "7daac3cd0efa17fb7423ad5edf9acbee54c4b1352622e7e06f165cfd9ef83508",
                 "bytes_per_pair": 1914543616}
QUANT_UNIQUE_BYTES_PER_ELEM = (2 + 0.5 + 1 / 16) + (0.5 + 1 / 16 + 2)
# Of the design bytes, the Infinity Cache can serve the encode pass's re-read
# of the tensor's last 96 MiB (read last by the maximum pass, first by the
# encode pass; kCachedTailBytes in quant.hip) and the decode pass's read of
# the codes and scales the encode pass has just written.
QUANT_CACHED_TAIL_BYTES = 96 << 20


def iteration_flops(m, n):
    """Algorithmic flops of one NS step on an m x n matrix (the iterate is
    min(m, n) x max(m, n)): the two Gram products count their upper triangle
    with the diagonal, m(m+1)n and m(m+1)m, the update product 2 m^2 n."""
    m, n = min(m, n), max(m, n)
    return m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n


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
                 reps=3, warm=1, route=False):
    """Grouped NS over a batch of BF16 gradients drawn on the device (the
    lowrank value model), against BF16 torch NS of the same batch.  route:
    the pages' full route, the random Hadamard transform (one seeded 16-bit
    sign mask per step) and adaptive 4/6 on every quantization besides the
    quantile clip."""
    Gs = [synth.device_lowrank_bf16(r, c, seed0 + i, dev) for i, (r, c) in enumerate(shapes)]
    outs = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
    ws = torch.empty(ns.ns_grouped_workspace_bytes(shapes), dtype=torch.uint8, device=dev)
    if route:
        masks = [int(v) for v in np.random.default_rng(seed0).integers(0, 1 << 16, len(coeffs))]
        run = lambda: ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clip_quantile=clip_quantile,
                                                     rht_masks=masks, adaptive46=True, outs=outs,
                                                     workspace=ws, stream=stream)
        clip_what = (f"clip at the {clip_quantile} quantile of each |G| (on the device), random "
                     "Hadamard transform and adaptive 4/6 on every quantization")
    elif clip_quantile:
        run = lambda: ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clip_quantile=clip_quantile,
                                                     outs=outs, workspace=ws, stream=stream)
        clip_what = f"clip at the {clip_quantile} quantile of each |G| (on the device)"
    else:
        clips = [float(8.0 * torch.sqrt(torch.mean(g.double() ** 2))) for g in Gs]
        run = lambda: ns.ns_orthogonalize_grouped(Gs, coeffs, clips, outs=outs, workspace=ws,
                                                  stream=stream)
        clip_what = "clip 8 x RMS(G) per matrix"
    ms = time_events(run, reps, warm, stream)
    flops = sum(len(coeffs) * iteration_flops(r, c) for r, c in shapes)

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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, coeffs):
    """The C++ oracle (plain C++ NVFP4 quantizer and float64 NS loop, OpenMP
    over the host's cores) on the single-GPU workloads, each once: the
    256 x 512, 2048^2 and 3072 x 8192 NS in full (five steps) and the
    2^28-element quantize + dequantize; of the four-block batch (too long to
    run whole here) one matrix of the 3072^2 shape class, the other class
    (3072 x 8192 and its transpose) being the 3072 x 8192 workload, and the
    batch's time extrapolated from the two.  value = the 3072 x 8192 rate in
    algorithmic TFLOP/s."""
    from oracle import native as C
    res = {}
    for name in ("ns256x512", "ns2048", "ns3072x8192", "ns4blocks"):
        G, _, clip = synth.ns_matrix(synth.ns_workload(name), 0)
        G64 = G.astype(np.float64)
        t0 = time.perf_counter()
        C.ns_nvfp4(G64, coeffs, clip=clip)
        el = time.perf_counter() - t0
        m, n = G.shape
        key = name if name != "ns4blocks" else "ns4blocks_3072x3072"
        res[key] = {"steps": len(coeffs), "s": round(el, 3),
                    "tflops": round(len(coeffs) * iteration_flops(m, n) / el / 1e12, 5)}
    sq, big = res["ns4blocks_3072x3072"]["s"], res["ns3072x8192"]["s"]
    res["ns4blocks_estimate"] = {"s": round(16 * sq + 8 * big, 1),
                                 "how": "16 x the 3072^2 matrix + 8 x the 3072x8192 one "
                                        "(its transpose costs the same); not run"}
    _, qv = synth.quant_workload()
    t0 = time.perf_counter()
    C.dequantize_rows(C.quantize_rows(qv))
    el = time.perf_counter() - t0
    res["quant2p28"] = {"s": round(el, 3), "gbps": round(QUANT_DESIGN_BYTES_PER_ELEM * qv.size / el / 1e9, 2)}
    return {"value": res["ns3072x8192"]["tflops"], "unit": "TFLOP/s", "cores": C.threads(),
            "kind": "oracle",
            "sample": f"C++ oracle (float64 NS, exact-comparison quantizer, OpenMP, {C.threads()} "
                      f"threads on {os.cpu_count()} logical CPUs, {cpu_model()}), each workload once: "
                      f"3072x8192 NS {res['ns3072x8192']['s']} s (value is its rate), 256x512 NS "
                      f"{res['ns256x512']['s']} s, 2048^2 NS {res['ns2048']['s']} s, 2^28 BF16 "
                      f"quantize+dequantize {res['quant2p28']['s']} s, one 3072^2 matrix of the "
                      f"four-block batch {sq} s (whole batch estimated at "
                      f"{res['ns4blocks_estimate']['s']} s)",
            "per_workload": res}


def exact_ns_f64(torch, G, coeffs, clip):
    """Unquantized NS in float64 with torch on the GPU (the reference of the
    accuracy table): X_0 = clamp(G) / (||clamp(G)||_F + 1e-7) on G^T if m > n,
    then X <- a X + (b A + c A A) X with A = X X^T."""
    X = G.double()
    tr = X.shape[0] > X.shape[1]
    if tr:
        X = X.t().contiguous()
    if clip != float("inf"):
        X = X.clamp(-clip, clip)
    X = X / (torch.linalg.norm(X) + 1e-7)
    for a, b, c in coeffs:
        A = X @ X.t()
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.t() if tr else X


def accuracy_table(ns, torch, synth, dev, stream):
    """Relative L2 (Frobenius) error of the NVFP4 NS output against
    unquantized float64 NS of the same input, clip and coefficients: plain
    NVFP4, with the random Hadamard transform, with adaptive 4/6, with the
    on-device 0.99-quantile clip, and with all three; the quintic and the
    cubic, five steps, on the 256x512, 2048^2 and 3072x8192 workloads."""
    table = {}
    for name in ("ns256x512", "ns2048", "ns3072x8192"):
        spec = synth.ns_workload(name)
        G, bits, clip = synth.ns_matrix(spec, 0)
        if spec["dtype"] == "bf16":
            Gd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            Gd = torch.from_numpy(G).to(dev)
        masks = synth.rht_masks(synth.STEPS, seed=spec["seeds"][0])
        q99 = float(ns.ns_abs_quantile(Gd, 0.99, stream=stream).item())
        row = {}
        for sname, coeffs in (("quintic", [synth.QUINTIC] * synth.STEPS),
                              ("cubic", [(1.5, -0.5, 0.0)] * synth.STEPS)):
            ref = {c: exact_ns_f64(torch, Gd, coeffs, c) for c in {clip, q99}}
            runs = {"plain": dict(clip=clip), "rht": dict(clip=clip, rht_masks=masks),
                    "46": dict(clip=clip, adaptive46=True),
                    "p99": dict(clip_quantile=0.99),
                    "rht+46+p99": dict(clip_quantile=0.99, rht_masks=masks, adaptive46=True)}
            errs = {}
            for vname, kw in runs.items():
                out = ns.ns_orthogonalize_ex(Gd, coeffs, stream=stream, **kw).double()
                r = ref[q99] if "clip_quantile" in kw else ref[clip]
                errs[vname] = round(float(torch.linalg.norm(out - r) / torch.linalg.norm(r)), 4)
            row[sname] = errs
        table[name] = row
    return table


def copy_probe(torch, dev):
    """Three plain 256 MiB device copies: the reference kernel whose
    FETCH_SIZE / WRITE_SIZE readings scale those of a profiled run."""
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def quant_line(ns, torch, synth, dev, stream, args):
    """The standalone quantizer + dequantizer on the 2^28 BF16 tensor."""
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
    traffic = None
    if QUANT_TRAFFIC["src_sha256"] == source_digest(("quant.hip", "nvfp4_device.hpp")):
        traffic = QUANT_TRAFFIC["bytes_per_pair"]
    unique = QUANT_UNIQUE_BYTES_PER_ELEM * rows * cols
    cache_served = min(QUANT_CACHED_TAIL_BYTES, 2 * rows * cols) + (0.5 + 1 / 16) * rows * cols
    out = {
        "metric": "nvfp4_quant HBM GB/s", "value": round(gbps, 1), "unit": "GB/s",
        "bytes_basis": "design bytes, 7.125 B per element: the maximum pass reads the tensor, "
                       "the encode pass reads it again (a global maximum cannot be known in one "
                       "pass over a tensor twice the Infinity Cache) and writes codes and "
                       "scales, the decode pass reads those and writes BF16; L2 counters "
                       "measure the same bytes (traffic) but cannot tell Infinity Cache hits "
                       "from HBM: the encode pass re-reads the last 96 MiB and the decode pass "
                       "the fresh codes and scales from the cache where they hit, so HBM moves "
                       "between hbm_bytes_min and the design bytes",
        "hbm_bytes_min": int(qbytes - cache_served),
        "hbm_gbps_min": round((qbytes - cache_served) / (qms * 1e-3) / 1e9, 1),
        "workload": "16384x16384 BF16 Student-t(3)*0.02 with 0.1% x50, quantize (amax pass + "
                    "encode) + dequantize to BF16, 1x16 blocks",
        "ms": round(qms, 4), "quantize_ms": round(t_q, 4), "dequantize_ms": round(t_d, 4),
        "design_bytes": int(qbytes),
        "unique_bytes": int(unique), "unique_gbps": round(unique / (qms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_unit": "bytes the L2 caches exchange with memory (Infinity Cache "
                                     "or HBM) per quantize + dequantize pair"}}
    del xq, deq
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the NS path runs on a single GPU and has "
              "no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import newton_schulz_amd as ns
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.quant_only:
        # the standalone quantizer alone (for profiling its kernels)
        line = {"quant": quant_line(ns, torch, synth, dev, stream, args)}
        if args.copy_probe:
            copy_probe(torch, dev)
        print(json.dumps(line), flush=True)
        return
    coeffs = [synth.QUINTIC] * synth.STEPS
    spec = synth.ns_workload("ns3072x8192")
    G, bits, clip = synth.ns_matrix(spec, 0)
    m, n = G.shape
    Gd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if args.gemm_only:
        # the three products alone, 10 launches each (for profiling their kernels)
        kt = kernel_timings(ns, torch, dev, Gd, clip, coeffs, stream)
        if args.copy_probe:
            copy_probe(torch, dev)
        print(json.dumps({"gemm_ms": {k: round(v[0], 4) for k, v in kt.items()},
                          "gemm_tflops": {k: round(v[1] / (v[0] * 1e-3) / 1e12, 2)
                                          for k, v in kt.items()}}), flush=True)
        return
    out = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = torch.empty(ns.ns_workspace_bytes(m, n), dtype=torch.uint8, device=dev)
    step = lambda: ns.ns_orthogonalize(Gd, coeffs, clip, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(step, args.steps, 0, stream)
    wall = time.perf_counter() - t0
    flops = synth.STEPS * iteration_flops(m, n)
    tflops = flops / (ms * 1e-3) / 1e12

    # per-call spread: each call between its own pair of events (the events
    # add a few microseconds to each); ms_per_step above is the back-to-back mean
    per_call = []
    for _ in range(args.steps):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        step()
        s1.record(stream)
        per_call.append((s0, s1))
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) for a, b in per_call)

    kt = kernel_timings(ns, torch, dev, Gd, clip, coeffs, stream)
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
        "step_ms": {"median": round(float(np.median(per_call)), 4), "min": round(per_call[0], 4),
                    "max": round(per_call[-1], 4), "calls": len(per_call),
                    "how": "each call between its own pair of HIP events"},
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
                              "quantized operand (the products' epilogues fold the transformed maxima of their outputs)"}

    # the same step with the clip taken on the device as the 0.99 quantile of
    # |G| (a histogram selection over G before the normalisation: one pass for BF16)
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
                                   "0.99 quantile of |G| found on the device (one-pass histogram selection)"}

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

    # the square 2048^2 gradient (same value model, clip 8 x RMS), five steps
    G2, bits2, clip2 = synth.ns_matrix(synth.ns_workload("ns2048"), 0)
    G2d = torch.from_numpy(bits2.view(np.int16)).view(torch.bfloat16).to(dev)
    out2 = torch.empty(G2.shape, dtype=torch.float32, device=dev)
    ws2 = torch.empty(ns.ns_workspace_bytes(*G2.shape), dtype=torch.uint8, device=dev)
    s2 = lambda: ns.ns_orthogonalize(G2d, coeffs, clip2, out=out2, workspace=ws2, stream=stream)
    ms2 = time_events(s2, args.steps, args.warmup, stream)
    flops2 = synth.STEPS * iteration_flops(*G2.shape)
    bms2 = bf16_ns_ms(torch, G2d, coeffs, stream)
    line["ns2048"] = {"ms": round(ms2, 4), "value": round(flops2 / (ms2 * 1e-3) / 1e12, 2),
                      "unit": "TFLOP/s", "algorithmic_tflop": round(flops2 / 1e12, 4),
                      "bf16_ms": round(bms2, 4), "speedup_nvfp4_vs_bf16": round(bms2 / ms2, 3),
                      "what": "ns_orthogonalize on the 2048^2 BF16 gradient (rank-32 signal + "
                              "noise + 0.1% outliers x50, seed 3), clip 8 x RMS, quintic x5"}
    del out2, ws2

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
                         "the pages' four decoder blocks at d=4096, their full route (transform, "
                         "adaptive 4/6, p99 clip), quintic x5", synth.pages_block_shapes(4096),
                         6000, coeffs, 0.99, route=True),
            grouped_line(ns, torch, synth, dev, stream,
                         "the pages' four decoder blocks at d=6144 (d_ff 13824, 48 heads, 8 KV "
                         "heads; 28 matrices), quintic x5", synth.pages_block_shapes(6144), 7000,
                         coeffs, 0.99),
        ]
        torch.cuda.empty_cache()
        ws = None

    if not args.no_accuracy:
        line["accuracy"] = {
            "what": "relative L2 error of the NVFP4 NS output against unquantized float64 NS "
                    "(torch on the GPU) of the same input, clip and coefficients, five steps",
            "table": accuracy_table(ns, torch, synth, dev, stream)}

    if not args.no_quant:
        del ws
        line["quant"] = quant_line(ns, torch, synth, dev, stream, args)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(synth, coeffs)
    if args.copy_probe:
        copy_probe(torch, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
