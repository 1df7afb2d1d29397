"""Benchmark of the Q8_0 weight x activation product on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill: q8_quantize_act (bf16 2048 x 4096) + q8_gemm (M2048 N12288 K4096)
  decode : q8_quantize_act + q8_gemm at M=1 and at M=4 (N12288 K4096), and
           the same step fused, q8_gemm_act (quantise inside the decode kernel)
  (after the timed steps, apart from them: the 3-bit KV-cache codec,
           q8_kv3_encode / q8_kv3_decode, on one layer's K and V at 256K
           context, in "kv3"; block-sparse attention prefill, q8_attn_*, at
           64K tokens, in "attn")
  gated FFN step: q8_gemm_swiglu (gate+up product, silu(g)*u, Q8_0 for the
           down projection) at M2048 with I = 6144 hidden units (2I = 12288,
           the prefill weight's size), and at M=1 and M=4
Weights are packed once (not timed).  Packed weight copies are rotated from
step to step over more than the 256 MB MALL, so weights come from HBM.

value  = prefill throughput, 2*M*N*K / (quantise + GEMM time), in TOPS
         (int8 multiply-adds counted as 2 ops); times are the medians over the
         timed steps of per-launch event pairs.
roofline = the prefill GEMM kernel alone, timed with HIP events around each
         launch on the stream it runs on, against the 5.0 POP/s dense int8
         matrix-core peak.  "decode" carries the M=1 and M=4 kernels against
         8 TB/s HBM; a decode launch lasts ~10 us, about the cost of an event
         pair (and the small quantise launches are shorter than a Python
         call), so after the timed steps each decode call is captured 100
         times (weights rotated) into a HIP graph, the graph is replayed
         between one event pair, and the call's duration is that time / 100.
         The replayed output is checked bit for bit against an eager call.
cpu_baseline = the CPU oracle (oracle/q8ref.c, OpenMP) on the host cores,
         timed on a bounded sample of the same prefill product.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q8_0 GEMM TOPS @M=2048 (% int8 MFMA peak) + decode GEMV GB/s (% HBM)"
PEAK_INT8_TOPS = 5000.0          # MI355X dense int8 matrix-core peak, TOP/s
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--rotate", type=int, default=10,
                   help="packed weight copies cycled over (at least enough for 512 MB)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the benchmark, run device-to-device copies of MIB MiB "
                        "(a kernel of known traffic, to scale hardware byte counters)")
    p.add_argument("--workloads", action="store_true",
                   help="instead of the benchmark, time q8_quantize_act and q8_gemm on every "
                        "workload (tiny, decode, prefill, large up/down, the M512/M509 sweep), "
                        "one JSON line each")
    return p.parse_args()


def workloads_bench(reps=20):
    """Every workload's product (and its activation quantiser), seeded as in
    the parity tests: events around each of `reps` launches, median; packed
    weight copies rotated over at least 512 MB."""
    import numpy as np
    import torch

    import int8_block_scaled_amd as q8
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def median_us(call):
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            call(i)
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

    for layer in workloads.ALL_LAYERS:
        M, N, K = layer.M, layer.N, layer.K
        w = torch.from_numpy(workloads.weights(layer)).to(dev)
        qw, dw = q8.q8_quantize_act(w)
        del w
        blocks = torch.cat([dw.view(torch.uint8).view(N, K // 32, 2),
                            qw.view(torch.uint8).view(N, K // 32, 32)], dim=2).contiguous().view(-1)
        del qw, dw
        w_bytes = N * (K // 32) * 34
        copies = max(2, min(64, -(-(512 << 20) // w_bytes)))   # >= 512 MB where possible
        packs = [q8.q8_pack_weights(blocks, N, K) for _ in range(copies)]
        del blocks
        x = workloads.activations(layer)
        xt = (torch.from_numpy(x).to(dev) if x.dtype == np.float32
              else torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16))
        qa, da = q8.q8_quantize_act(xt)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        gemm_us = median_us(lambda i: q8.q8_gemm(qa, da, packs[i % copies], N, K, out=C))
        quant_us = median_us(lambda i: q8.q8_quantize_act(xt, q=qa, d=da))
        ops = 2.0 * M * N * K
        alg = w_bytes + M * (K // 32) * 34 + 4 * M * N
        tops = ops / (gemm_us * 1e-6) / 1e12
        gbs = alg / (gemm_us * 1e-6) / 1e9
        print(json.dumps({"workload": layer.name, "M": M, "N": N, "K": K,
                          "kernel": ("decode" if M <= 8 else
                                     "small-M matrix-core" if M <= 64 else "matrix-core tiles"),
                          "gemm_us": round(gemm_us, 2), "tops": round(tops, 1),
                          "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4),
                          "gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                          "quantize_us": round(quant_us, 2), "weight_copies": copies,
                          "timing": "events per launch, median of %d" % reps}), flush=True)
        del packs, xt, qa, da, C
        torch.cuda.empty_cache()


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))


def kernel_source_sha(name):
    path = os.path.join(ROOT, "int8_block_scaled_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(profile_name, source, per_launch_bytes_alg):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, profile_name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != kernel_source_sha(source):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.workloads:
        return workloads_bench()
    if args.gpus != 1:
        sys.exit("bench.py measures one GPU: the library has no multi-GPU path "
                 "(the product shards by N or M with no communication). "
                 "Run with --gpus 1.")

    import numpy as np
    import torch

    import int8_block_scaled_amd as q8
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pre, dec1, dec4 = workloads.PREFILL, workloads.DECODE_M1, workloads.DECODE_M4
    N, K = pre.N, pre.K
    assert (dec1.N, dec1.K) == (N, K)

    # ---- inputs (seeded, synthetic), weights quantised and packed on the GPU
    w = torch.from_numpy(workloads.weights(pre)).to(dev)
    qw, dw = q8.q8_quantize_act(w)
    del w
    blocks = torch.cat([dw.view(torch.uint8).view(N, K // 32, 2),
                        qw.view(torch.uint8).view(N, K // 32, 32)], dim=2).contiguous().view(-1)
    del qw, dw
    packed0 = q8.q8_pack_weights(blocks, N, K)
    # enough copies that the rotation spans at least 512 MB (twice the MALL)
    copies = max(args.rotate, -(-(512 << 20) // packed0.numel()))
    packs = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    # gate/up weight of I = N/2 hidden units: the same rows, read as gate
    # (first half) and up (second half)
    I = N // 2
    bl = blocks.view(N, -1)
    gu0 = q8.q8_pack_weights_gateup(bl[:I].contiguous().view(-1), bl[I:].contiguous().view(-1), I, K)
    gus = [gu0] + [gu0.clone() for _ in range(copies - 1)]
    del blocks, bl
    xp = torch.from_numpy(workloads.activations(pre).view(np.int16)).to(dev).view(torch.bfloat16)
    x4 = torch.from_numpy(workloads.activations(dec4).view(np.int16)).to(dev).view(torch.bfloat16)
    x1 = x4[:1]
    M = pre.M
    qa = torch.empty((M, K), dtype=torch.int8, device=dev)
    da = torch.empty((M, K // 32), dtype=torch.float16, device=dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    q4 = torch.empty((4, K), dtype=torch.int8, device=dev)
    d4 = torch.empty((4, K // 32), dtype=torch.float16, device=dev)
    q1 = torch.empty((1, K), dtype=torch.int8, device=dev)
    d1 = torch.empty((1, K // 32), dtype=torch.float16, device=dev)
    C4 = torch.empty((4, N), dtype=torch.float32, device=dev)
    C1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    qh = torch.empty((M, I), dtype=torch.int8, device=dev)
    dh = torch.empty((M, I // 32), dtype=torch.float16, device=dev)
    qh4 = torch.empty((4, I), dtype=torch.int8, device=dev)
    dh4 = torch.empty((4, I // 32), dtype=torch.float16, device=dev)
    qh1 = torch.empty((1, I), dtype=torch.int8, device=dev)
    dh1 = torch.empty((1, I // 32), dtype=torch.float16, device=dev)

    names = ["quant_prefill", "gemm_prefill", "quant_dec1", "gemv_dec1", "quant_dec4", "gemv_dec4",
             "fused_dec1", "fused_dec4", "swiglu_prefill", "swiglu_dec1", "swiglu_dec4"]

    def step(i, ev=None):
        wp = packs[i % len(packs)]
        calls = [
            lambda: q8.q8_quantize_act(xp, q=qa, d=da),
            lambda: q8.q8_gemm(qa, da, wp, N, K, out=C),
            lambda: q8.q8_quantize_act(x1, q=q1, d=d1),
            lambda: q8.q8_gemm(q1, d1, packs[(i + 3) % len(packs)], N, K, out=C1),
            lambda: q8.q8_quantize_act(x4, q=q4, d=d4),
            lambda: q8.q8_gemm(q4, d4, packs[(i + 5) % len(packs)], N, K, out=C4),
            lambda: q8.q8_gemm_act(x1, packs[(i + 2) % len(packs)], N, K, out=C1),
            lambda: q8.q8_gemm_act(x4, packs[(i + 6) % len(packs)], N, K, out=C4),
            lambda: q8.q8_gemm_swiglu(qa, da, gus[i % len(gus)], I, K, q=qh, d=dh),
            lambda: q8.q8_gemm_swiglu(q1, d1, gus[(i + 3) % len(gus)], I, K, q=qh1, d=dh1),
            lambda: q8.q8_gemm_swiglu(q4, d4, gus[(i + 5) % len(gus)], I, K, q=qh4, d=dh4),
        ]
        for j, c in enumerate(calls):
            if ev is not None:
                ev[j][0].record()
            c()
            if ev is not None:
                ev[j][1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in names]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # decode calls back to back in a HIP graph (see the module docstring)
    def block_us(call, out, reps=100):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                call(i)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                call(i)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        replayed = out.clone()
        call(reps - 1)                       # eager, same inputs as the graph's last call
        torch.cuda.synchronize()
        if not torch.equal(replayed.view(torch.int8), out.view(torch.int8)):
            raise RuntimeError("graph replay differs from the eager call")
        return e0.elapsed_time(e1) * 1e3 / reps

    P = len(packs)
    back = {
        "quant_dec1": block_us(lambda i: q8.q8_quantize_act(x1, q=q1, d=d1), q1),
        "quant_dec4": block_us(lambda i: q8.q8_quantize_act(x4, q=q4, d=d4), q4),
        "gemv_dec1": block_us(lambda i: q8.q8_gemm(q1, d1, packs[i % P], N, K, out=C1), C1),
        "gemv_dec4": block_us(lambda i: q8.q8_gemm(q4, d4, packs[i % P], N, K, out=C4), C4),
        "fused_dec1": block_us(lambda i: q8.q8_gemm_act(x1, packs[i % P], N, K, out=C1), C1),
        "fused_dec4": block_us(lambda i: q8.q8_gemm_act(x4, packs[i % P], N, K, out=C4), C4),
        "swiglu_dec1": block_us(lambda i: q8.q8_gemm_swiglu(q1, d1, gus[i % P], I, K, q=qh1, d=dh1),
                                qh1),
        "swiglu_dec4": block_us(lambda i: q8.q8_gemm_swiglu(q4, d4, gus[i % P], I, K, q=qh4, d=dh4),
                                qh4),
        "prefill": block_us(lambda i: (q8.q8_quantize_act(xp, q=qa, d=da),
                                       q8.q8_gemm(qa, da, packs[i % P], N, K, out=C)), C, reps=20),
    }

    dur = {n: np.array([events[i][j][0].elapsed_time(events[i][j][1]) for i in range(args.steps)])
           for j, n in enumerate(names)}                      # ms per launch
    # medians over the timed steps (p10 / p90 reported beside them)
    mean = {n: float(np.median(v)) for n, v in dur.items()}
    pct = {n: (float(np.percentile(v, 10)), float(np.percentile(v, 90))) for n, v in dur.items()}

    ops = 2.0 * M * N * K
    t_pre = (mean["quant_prefill"] + mean["gemm_prefill"]) * 1e-3
    # Context: the same pair replayed back to back from a HIP graph (20 pairs,
    # weights rotated), i.e. under sustained load with no gaps between them.
    sustained_tops = ops / (back["prefill"] * 1e-6) / 1e12
    value = ops / t_pre / 1e12
    gemm_tops = ops / (mean["gemm_prefill"] * 1e-3) / 1e12

    KB = K // 32
    w_bytes = N * KB * 34

    def gemv_bytes(m):
        return w_bytes + m * KB * 34 + 4 * m * N

    dec = {}
    for m, key in ((1, "gemv_dec1"), (4, "gemv_dec4")):
        us = back[key]
        fused_us = back[key.replace("gemv", "fused")]
        gbs = gemv_bytes(m) / (us * 1e-6) / 1e9
        dec["M%d" % m] = {"gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                          "kernel_us": round(us, 2),
                          "algorithmic_bytes": gemv_bytes(m),
                          "quantize_us": round(back[key.replace("gemv", "quant")], 2),
                          "two_call_us": round(us + back[key.replace("gemv", "quant")], 2),
                          "fused_us": round(fused_us, 2),
                          "fused_gbs": round((w_bytes + m * K * 2 + 4 * m * N)
                                             / (fused_us * 1e-6) / 1e9, 1),
                          "kernel_us_event_per_launch": round(mean[key] * 1e3, 2),
                          "traffic": measured_traffic("gemv_decode_M%d_traffic.json" % m,
                                                      "q8_gemv.hip", gemv_bytes(m)),
                          "fused_traffic": measured_traffic("fused_decode_M%d_traffic.json" % m,
                                                            "q8_gemv.hip", None)}

    roofline = {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TOPS", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                "traffic": measured_traffic("gemm_prefill_M2048_traffic.json", "q8_gemm.hip",
                                            None),
                "kernel": "gemm_q8_mfma_kernel", "kernel_us": round(mean["gemm_prefill"] * 1e3, 2),
                "kernel_us_p10_p90": [round(v * 1e3, 2) for v in pct["gemm_prefill"]],
                "timing": "median of %d launches, HIP events on the launch stream" % args.steps,
                "algorithmic_ops_per_launch": ops,
                # Two binary32 FMAs per output and block.  Measured on this
                # chip (probe, 4 waves per SIMD): an int8 MFMA plus 32
                # independent FMAs take 104 SIMD cycles, because the MFMA and
                # the vector instructions of its SIMD do not overlap; the
                # kernel's other 2.75 vector instructions per MFMA (counted)
                # add ~6 cycles at ~2.2 each, so at most 32/110 of the MFMA
                # peak per clock.  The clock is an assumption: 2.4 GHz in the
                # peak, 2.0-2.2 GHz measured (GRBM_GUI_ACTIVE over the
                # dispatch) while this kernel runs.
                "epilogue_ceiling_frac": {"per_clock": round(32 / 110, 3),
                                          "at_2.4GHz": round(32 / 110, 3),
                                          "at_2.1GHz": round(32 / 110 * 2.1 / 2.4, 3)}}

    sw_us = mean["swiglu_prefill"] * 1e3
    swiglu = {"workload": "M2048 I6144 K4096 (gate+up 12288 x 4096)",
              "kernel_us": round(sw_us, 2),
              "tops": round(2.0 * M * 2 * I * K / (sw_us * 1e-6) / 1e12, 1),
              "plain_gemm_same_shape_us": round(mean["gemm_prefill"] * 1e3, 2),
              "output_bytes": M * I + M * (I // 32) * 2,
              "plain_gemm_output_bytes": M * 2 * I * 4,
              "decode_M1_us": round(back["swiglu_dec1"], 2),
              "decode_M4_us": round(back["swiglu_dec4"], 2),
              "traffic": measured_traffic("swiglu_prefill_traffic.json", "q8_gemm.hip", None)}

    kv3 = kv3_bench(q8, workloads, torch, np, dev)
    attn = attn_bench(q8, workloads, torch, np, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds, qa, da, packs, N, K)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic (seeded N(0,1) bf16 activations, N(0,0.02) weights as Q8_0)",
        "config": {"workload": "prefill M2048 N12288 K4096 (+ decode M1 and M4, N12288 K4096)",
                   "M": M, "N": N, "K": K, "act_dtype": "bf16", "weights": "Q8_0",
                   "weight_copies_rotated": len(packs),
                   "gemm_only_tops": round(gemm_tops, 1),
                   "quantize_prefill_us": round(mean["quant_prefill"] * 1e3, 2),
                   "quantize_prefill_us_p10_p90": [round(v * 1e3, 2) for v in pct["quant_prefill"]],
                   "timing": "medians of %d steps (events per launch)" % args.steps,
                   "prefill_pair_us_sustained": round(back["prefill"], 2),
                   "prefill_tops_sustained": round(sustained_tops, 1)},
        "roofline": roofline,
        "decode": dec,
        "swiglu": swiglu,
        "kv3": kv3,
        "attn": attn,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def kv3_bench(q8, workloads, torch, np, dev, reps=20):
    """The 3-bit KV-cache codec on one layer's keys and values at 256K
    context: 262144 tokens x 4 KV heads x (K, V) = 2^21 rows of D = 256,
    bfloat16 (1.07 GB, far above the 256 MB MALL, so every launch streams
    from HBM).  Each launch is timed with an event pair on the stream it runs
    on; algorithmic bytes are the rows read plus the codes and scales written
    (encode), and the reverse (decode)."""
    R, D = 262144 * 8, 256
    x = workloads.kv_rows_device(R, D, 600, dev)
    codes = torch.empty((R, 3 * D // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((R,), dtype=torch.float32, device=dev)
    out = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def timed(call):
        for _ in range(3):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3   # us

    enc_us = timed(lambda: q8.q8_kv3_encode(x, codes=codes, scales=scales))
    dec_us = timed(lambda: q8.q8_kv3_decode(codes, scales, D, out=out))
    row_bytes_in, row_bytes_packed = 2 * D, 3 * D // 8 + 4
    alg = R * (row_bytes_in + row_bytes_packed)
    xf = x[:65536].float()
    err = (out[:65536].float() - xf).pow(2).sum() / xf.pow(2).sum()
    return {"workload": "one layer's K and V at 256K context: R %d rows x D %d, bf16 in/out" % (R, D),
            "encode_us": round(enc_us, 2), "encode_gbs": round(alg / (enc_us * 1e-6) / 1e9, 1),
            "encode_frac_hbm": round(alg / (enc_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "decode_us": round(dec_us, 2), "decode_gbs": round(alg / (dec_us * 1e-6) / 1e9, 1),
            "decode_frac_hbm": round(alg / (dec_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_launch": alg,
            "bits_per_element": 8.0 * row_bytes_packed / D,
            "compression_vs_bf16": round(row_bytes_in / row_bytes_packed, 3),
            "relative_mse_first_65536_rows": round(float(err), 5),
            "encode_traffic": measured_traffic("kv3_encode_traffic.json", "q8_kv3.hip", alg),
            "decode_traffic": measured_traffic("kv3_decode_traffic.json", "q8_kv3.hip", alg)}


PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 matrix cores


def attn_bench(q8, workloads, torch, np, dev, reps=10):
    """Block-sparse causal attention prefill: 64K tokens, 32 query heads over
    8 K/V heads, D = 128, 64 key blocks of 64 tokens per query block (block
    0, the diagonal and 62 selected; one list per K/V head).  Pooling, selection and the forward
    pass are timed with an event pair around each launch; the forward pass's
    algorithmic work is 4 D flops per attended (query, key) pair (two
    products), counted from the lists."""
    L, Hq, Hkv, D, k = 65536, 32, 8, 128, 64
    q, kk, v = workloads.attn_qkv_device(L, Hq, Hkv, D, 700, dev)
    NB = (L + 63) // 64
    pq = torch.empty((Hq, NB, D), dtype=torch.float32, device=dev)
    pk = torch.empty((Hkv, NB, D), dtype=torch.float32, device=dev)
    idx = torch.empty((Hkv, NB, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((Hkv, NB), dtype=torch.int32, device=dev)
    out = torch.empty((L, Hq * D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def timed(call):
        for _ in range(2):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3   # us

    pool_us = timed(lambda: (q8.q8_attn_pool(q, Hq, D, out=pq), q8.q8_attn_pool(kk, Hkv, D, out=pk)))
    sel_us = timed(lambda: q8.q8_attn_select(pq, pk, k, idx=idx, cnt=cnt))
    fwd_us = timed(lambda: q8.q8_attn_fwd(q, kk, v, Hq, Hkv, D, idx, cnt, out=out))
    c = np.repeat(cnt.cpu().numpy().astype(np.int64), Hq // Hkv, axis=0)   # per query head
    rows = np.full(NB, 64, dtype=np.int64)
    rows[-1] = L - 64 * (NB - 1)                       # queries of the last block
    # every listed block below the diagonal: rows x 64 keys; the diagonal:
    # the causal triangle
    pairs = int(((c - 1) * rows[None, :] * 64 + (rows * (rows + 1) // 2)[None, :]).sum())
    flops = 4.0 * D * pairs
    tflops = flops / (fwd_us * 1e-6) / 1e12
    return {"workload": "prefill L %d, %d query heads over %d K/V heads, D %d, %d blocks of 64 "
                        "per query block, bf16" % (L, Hq, Hkv, D, k),
            "fwd_us": round(fwd_us, 1), "fwd_tflops": round(tflops, 1),
            "fwd_frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flops": flops, "attended_pairs": int(pairs),
            "density": round(pairs / (Hq * L * (L + 1) / 2), 4),
            "pool_us": round(pool_us, 1), "select_us": round(sel_us, 1),
            "total_us": round(pool_us + sel_us + fwd_us, 1)}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds, qa_t, da_t, packs, N, K):
    """The oracle (plain C, OpenMP over rows) on a bounded row sample of the
    prefill product; rows are added until about ``seconds`` of CPU time."""
    import numpy as np
    import oracle

    orc = oracle.default()
    import torch

    qa = qa_t.cpu().numpy()
    da = da_t.cpu().view(torch.int16).numpy().view(np.uint16)
    # unpack the weights from the packed layout on the host (marshalling only)
    KB, NG = K // 32, (N + 63) // 64
    pk = packs[0].cpu().numpy()
    qplane = pk[:NG * KB * 2048].reshape(NG, KB, 2, 64, 16).view(np.int8)
    qw = np.ascontiguousarray(qplane.transpose(0, 3, 1, 2, 4).reshape(NG * 64, K)[:N])
    dw = np.ascontiguousarray(pk[NG * KB * 2048:].view(np.uint16).reshape(NG, KB, 64)
                              .transpose(0, 2, 1).reshape(NG * 64, KB)[:N])
    rows, elapsed, chunk = 0, 0.0, 4
    while elapsed < seconds and rows < qa.shape[0]:
        r1 = min(qa.shape[0], rows + chunk)
        t0 = time.perf_counter()
        orc.gemm(qa[rows:r1], da[rows:r1], qw, dw)
        elapsed += time.perf_counter() - t0
        rows = r1
        chunk = min(chunk * 2, 64)
    ops = 2.0 * rows * N * K
    return {"value": round(ops / elapsed / 1e12, 6), "unit": "TOPS", "cores": orc.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "prefill product rows 0..%d of 2048 (N12288 K4096), %.1f s" % (rows, elapsed)}


if __name__ == "__main__":
    main()
