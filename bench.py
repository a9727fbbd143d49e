#!/usr/bin/env python3
"""Benchmark of the BitNet b1.58 BitLinear forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: decode, M=1 token, K=2048, N=2048 (a d_model-2048
projection), bfloat16 activations, packed ternary weights.  One launch of the
decode kernel is far below HBM latency for a single 1 MiB matrix, so a step is
the batched decode forward over a pool of L distinct layers of that shape
(each with its own weights, activations and outputs; >= 1 GiB of packed
weights, several times the 256 MB last-level cache, so every byte comes from
HBM).  The metric is GB/s of algorithmic bytes (packed weights + activations +
outputs) against the 8 TB/s HBM3E peak.

--format radix3 streams the weights packed five per byte (1.6 bits) through
the same decode kernel; "weights_per_s" compares the two formats.  --format
lut contracts the same 2-bit weights through 81-entry LDS tables per block of
four activations (the CPU LUT scheme, as a comparison).

--workload ffn_block_decode_m8_d2048_f5632 / ffn_block_prefill_m2048_d4096_f11008
time the BitNet FFN block (BitLinear up -> ReLU^2 -> BitLinear down).

--workload ste_backward_m2048_k4096_n11008 times the STE backward (dX and dW)
of the 7B-like projection in bf16 TFLOP/s.

--workload prefill_ffn_m2048_k4096_n11008 (or the 8192x8192x28672 one) times
the prefill forward instead (activation quantiser + INT8-MFMA GEMM) and
reports INT8 TOPS (2*M*N*K per step) against the 5.0 POPS dense INT8 peak.

The default line carries both halves of the metric: after the decode step it
holds a "prefill" object with one entry per prefill workload (8192x8192x28672
and 2048x4096x11008): the whole prefill forward (activation quantiser +
INT8-MFMA GEMM) in INT8 TOPS, the GEMM alone ("kernel_ms") with its roofline
against the dense INT8 peak, and the CPU oracle beside it (--no-prefill leaves
them out).

Weight quantisation (absmean + ternarise + pack) runs once per weight matrix
before the timed region; it is timed separately and reported under
"weight_quantisation".

Every line also carries "attainable": what plain kernels reach on this GPU
(a 1 GiB streaming read, a streaming copy, back-to-back INT8 MFMAs on
registers) beside the published peaks that "roofline" uses (--no-peaks skips
them), and the CPU baseline names the host's CPU model.

Without --warmup / --steps, each timed section warms up for at least 0.3 s
under load (the GPU reaches its sustained state only after ~0.1-0.15 s of
continuous work) and times at least 0.25 s (and at least 50 steps); the line
reports the counts actually run.  Given on the command line, they are used
exactly.

Prints exactly one JSON line on stdout; progress goes to stderr.
--copy-calibration runs a plain 1 GiB device copy (for HBM counter scaling).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, TOPS
METRIC = "BitLinear fwd: decode GEMV GB/s (% HBM peak); prefill INT8 TOPS (% MFMA peak)"

DECODE_WORKLOADS = {"decode_m1_k2048_n2048": 0.02, "decode_ffn_up_m8_k2048_n5632": 0.02}
PREFILL_WORKLOADS = ("prefill_ffn_m2048_k4096_n11008", "prefill_ffn_m8192_k8192_n28672")

# HBM bytes per launch of the dominant kernel, read from rocprofv3 FETCH_SIZE and
# WRITE_SIZE counter runs and scaled by the same counters on a plain 1 GiB copy.
# Valid only while the kernel sources hash to `sources_sha` (else traffic = null).
TRAFFIC = {
    # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of the dominant launch (decode: the batched
    # launch; lut: the LUT kernel's launch; prefill: the GEMM launches of one call, summed) on
    # `bench.py --workload W [--format F] --steps 1 --warmup 1 --no-cpu-baseline`; scale
    # factors 2.0 (FETCH_SIZE) and 1.0 (WRITE_SIZE) from the 1 GiB copy of
    # `bench.py --copy-calibration` (524,300 KiB read, 1,048,576 KiB written).
    "decode_m1_k2048_n2048": {"sources_sha": "611c60b56dc85fee", "fetch_bytes": 1078214246, "write_bytes": 8393318},
    "decode_ffn_up_m8_k2048_n5632": {"sources_sha": "611c60b56dc85fee", "fetch_bytes": 1088587366, "write_bytes": 67223552},
    "decode_m1_k2048_n2048/radix3": {"sources_sha": "611c60b56dc85fee", "fetch_bytes": 1079871898, "write_bytes": 10330112},
    "decode_ffn_up_m8_k2048_n5632/radix3": {"sources_sha": "611c60b56dc85fee", "fetch_bytes": 1091135693, "write_bytes": 82722816},
    "decode_m1_k2048_n2048/lut": {"sources_sha": "6d4398590ebb1f5f", "fetch_bytes": 1076063744, "write_bytes": 8388608},
    "decode_ffn_up_m8_k2048_n5632/lut": {"sources_sha": "6d4398590ebb1f5f", "fetch_bytes": 1082523392, "write_bytes": 67223552},
    "prefill_ffn_m2048_k4096_n11008": {"sources_sha": "b4162daa313c2f73", "fetch_bytes": 117062656, "write_bytes": 90282240},
    "prefill_ffn_m8192_k8192_n28672": {"sources_sha": "b4162daa313c2f73", "fetch_bytes": 2116057216, "write_bytes": 939646976},
}

KERNEL_SOURCES = {
    "decode": ["decode.hip", "quant_act.hpp", "common.hpp"],
    "prefill": ["prefill.hip", "common.hpp"],
    "lut": ["lut.hip", "common.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "bitlinear_absmean_ternarise_bit_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kind: str):
    t = TRAFFIC.get(workload)
    if not t or t["sources_sha"] != sources_sha(kind):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


class Timer:
    """HIP events on the current stream (the stream every binding call launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


# Default warm-up and timed region, by time under load.  The GPU settles into
# its sustained state only after about 0.1-0.15 s of continuous load (decode
# streams ~3% faster after it; it falls back within a second of idling), so by
# default the untimed warm-up runs for at least SETTLE_S and the timed region
# for at least TIMED_S.  Explicit --warmup / --steps are used exactly as given.
SETTLE_S = 0.3
TIMED_S = 0.25
MIN_STEPS = 50
MIN_WARMUP = 5


def plan_steps(args, torch, step):
    """(warmup, steps) for this step function: the counts given on the command
    line, else derived from the duration of one step (timed after one call)."""
    if args.warmup is not None and args.steps is not None:
        return args.warmup, args.steps
    step()
    with Timer(torch) as t:
        step()
    est = max(t.ms * 1e-3, 1e-6)
    warmup = args.warmup if args.warmup is not None else min(100000, max(MIN_WARMUP, math.ceil(SETTLE_S / est)))
    steps = args.steps if args.steps is not None else min(100000, max(MIN_STEPS, math.ceil(TIMED_S / est)))
    return warmup, steps


def run_timed(args, torch, step, what: str):
    """Warm up, then time the step: (ms per step, warmup, steps)."""
    warmup, steps = plan_steps(args, torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {what}: warmup done ({warmup} steps)")
    with Timer(torch) as t:
        for _ in range(steps):
            step()
    ms = t.ms / steps
    log(f"[bench] {what}: timed {steps} steps, {ms * 1e3:.1f} us/step")
    return ms, warmup, steps


def sustained_obj(sus, units_per_step: float, unit: str, peak: float) -> dict:
    ms, warmup, steps = sus
    v = units_per_step / (ms * 1e-3)
    return {"value": round(v, 2), "unit": unit, "ms_per_step": round(ms, 6), "frac": round(v / peak, 4),
            "warmup": warmup, "steps": steps,
            "note": "the same step timed again after the line's own timed region, once the GPU has run it "
                    f"untimed for {SETTLE_S} s (the sustained state it reaches after ~0.15 s of load); "
                    "the line's value keeps the counts given on the command line"}


def sustained_after(args, torch, step, ms_step: float):
    """With explicit --warmup / --steps (timed exactly as given, above): the same
    step again after the default settling, as a second figure beside the line's
    value: untimed for at least SETTLE_S seconds, then timed for at least
    TIMED_S seconds.  None when the counts were already duration-based."""
    if args.warmup is None or args.steps is None:
        return None
    est = max(ms_step * 1e-3, 1e-6)
    warmup = min(100000, max(MIN_WARMUP, math.ceil(SETTLE_S / est)))
    steps = min(100000, max(MIN_STEPS, math.ceil(TIMED_S / est)))
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with Timer(torch) as t:
        for _ in range(steps):
            step()
    return t.ms / steps, warmup, steps


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def build_decode_pool(torch, bl, dev, workload: str, L: int, fmt: str = "2bit", keep=()):
    """The decode step's inputs: L layers of one workload shape, resident on the GPU.

    Layer 0 is the workload's seeded numpy draw; the other layers come from
    torch's seeded device generator (seed 1234) in the same distribution.  Weights
    are quantised on the GPU (``fmt`` "2bit" or "radix3"), in chunks of layers;
    the float32 weights of the layers in ``keep`` are returned on the host.
    Returns (P, X, packed, gamma, tq_ms, kept) with tq_ms the quantisation time.
    """
    import numpy as np
    from bitlinear_absmean_ternarise_bit_amd.workloads import make_workload

    sigma = DECODE_WORKLOADS[workload]
    P = make_workload(workload)
    M, K, N = P.M, P.K, P.N
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    X = torch.empty((L, M, K), dtype=torch.bfloat16, device=dev)
    X[0].copy_(torch.from_numpy(P.X_bf16_bits.view(np.int16)).view(torch.bfloat16))
    X[1:].copy_(torch.randn((L - 1, M, K), generator=g, device=dev).to(torch.bfloat16))
    if P.name == "decode_ffn_up_m8_k2048_n5632":  # same 1% outlier channels x20 in every layer
        ch = torch.from_numpy(P.notes["outlier_channels"]).to(dev)
        X[1:, :, ch] = (X[1:, :, ch].float() * 20.0).to(torch.bfloat16)
    if fmt == "radix3":
        packed = torch.empty((L, N, bl.r3_row_bytes(K)), dtype=torch.uint8, device=dev)
        quant = bl.quantize_weights_r3
    else:
        packed = torch.empty((L, N, bl.packed_words(K)), dtype=torch.int32, device=dev)
        quant = bl.quantize_weights
    gamma = torch.empty((L,), dtype=torch.float32, device=dev)
    ws = torch.empty((bl.abi.load().bitlinear_quantize_workspace_bytes(),), dtype=torch.uint8, device=dev)
    chunk = max(1, min(L, (1 << 32) // (4 * N * K)))
    Wc = torch.empty((chunk, N, K), dtype=torch.float32, device=dev)
    tq_ms = 0.0
    kept = {}
    for l0 in range(0, L, chunk):
        n = min(chunk, L - l0)
        Wc[:n].normal_(0.0, sigma, generator=g)
        if l0 == 0:
            Wc[0].copy_(torch.from_numpy(P.W))
        for l in keep:
            if l0 <= l < l0 + n:
                kept[l] = Wc[l - l0].cpu().numpy()
        with Timer(torch) as tq:
            for l in range(n):
                quant(Wc[l], out_packed=packed[l0 + l], out_gamma=gamma[l0 + l:l0 + l + 1], workspace=ws)
        tq_ms += tq.ms
    del Wc
    torch.cuda.empty_cache()
    return P, X, packed, gamma, tq_ms, kept


def bench_decode(args, torch, bl, dev):
    from bitlinear_absmean_ternarise_bit_amd.workloads import make_workload

    r3 = args.format == "radix3"
    lut = args.format == "lut"
    P0 = make_workload(args.workload)
    M, K, N = P0.M, P0.K, P0.N
    row_bytes = bl.r3_row_bytes(K) if r3 else bl.packed_words(K) * 4
    packed_bytes = N * row_bytes
    L = args.layers or max(8, -(-(1 << 30) // packed_bytes))  # >= 1 GiB of packed weights
    log(f"[bench] decode {args.workload} ({args.format}): M={M} K={K} N={N}, pool of {L} layers "
        f"({L * packed_bytes / 2**30:.2f} GiB packed)")
    # weights: quantisation is offline, not part of the step; timed separately
    P, X, packed, gamma, tq_ms, _ = build_decode_pool(torch, bl, dev, args.workload, L,
                                                      "radix3" if r3 else "2bit")
    Y = torch.empty((L, M, N), dtype=torch.float32, device=dev)
    wq_bytes = L * (4 * N * K + packed_bytes)
    log(f"[bench] weight quantisation of {L} layers: {tq_ms:.1f} ms")

    if lut:
        ws = torch.empty((bl.lut_workspace_bytes(L, M, K),), dtype=torch.uint8, device=dev)

        def step():
            bl.forward_lut(X, packed, gamma, K, out=Y, workspace=ws)

        def single(l, out):
            bl.forward_lut(X[l], packed[l], gamma[l:l + 1], K, out=out, workspace=ws)
    elif r3:
        def step():
            bl.forward_r3(X, packed, gamma, K, out=Y)

        def single(l, out):
            bl.forward_r3(X[l], packed[l], gamma[l:l + 1], K, out=out)
    else:
        def step():
            bl.forward_batched(X, packed, gamma, K, out=Y)

        def single(l, out):
            bl.forward(X[l], packed[l], gamma[l:l + 1], K, out=out)

    ms_step, warmup, steps = run_timed(args, torch, step, "decode")
    step_bytes = L * (packed_bytes + M * K * 2 + M * N * 4)
    sus = sustained_after(args, torch, step, ms_step)
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    gw_s = L * N * K / (ms_step * 1e-3) / 1e9
    log(f"[bench] decode: {gbps:.1f} GB/s, {gw_s:.1f} G weights/s")

    # one layer per call, rotating over the pool (cold weights): the latency-bound single call
    Y1 = torch.empty((M, N), dtype=torch.float32, device=dev)
    R = min(L, 256)
    for l in range(8):
        single(l, Y1)
    with Timer(torch) as t1:
        for l in range(R):
            single(l, Y1)
    single_us = t1.ms / R * 1e3
    graph_us = single_calls_in_graph(torch, dev, single, R, (M, N))
    layer_bytes = step_bytes // L

    out = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s",
        "ms_per_step": round(ms_step, 6), "warmup": warmup, "steps": steps,
        "dtype": "i8",
        "config": {"workload": f"{args.workload} x {L} layers per step (batched decode, cold weights)",
                   "M": M, "K": K, "N": N, "layers": L, "x_dtype": "bf16",
                   "weight_format": "radix-3, 5 weights per byte" if r3 else "2-bit",
                   "contraction": "81-entry LUTs in LDS (comparison variant)" if lut else "INT8 MFMA",
                   "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(args.workload + ("/radix3" if r3 else "/lut" if lut else ""),
                                            "lut" if lut else "decode"),
                     "kernel": ("lut_gemv_kernel (tables + lookups + rescale) after act_quant_kernel, two "
                                "launches per step" if lut else
                                "decode_kernel (fused quantise + GEMV + rescale), one launch per step")},
        "weights_per_s": {"value": round(gw_s, 2), "unit": "G weights/s",
                          "note": "N*K*layers per step / step time: compares weight formats"},
        **({"sustained": sustained_obj(sus, step_bytes / 1e9, "GB/s", HBM_PEAK_GBPS)} if sus else {}),
        "single_call": {"us": round(single_us, 2), "GBps": round(layer_bytes / (single_us * 1e-6) / 1e9, 2),
                        "us_graph": round(graph_us, 2),
                        "GBps_graph": round(layer_bytes / (graph_us * 1e-6) / 1e9, 2),
                        "note": "one layer per launch, cold weights: 'us' from a host loop of calls (bound by "
                                "the host's launch cost), 'us_graph' from the same calls replayed as one HIP "
                                "graph (its output checked against the eager call)"},
        "weight_quantisation": {"ms_per_matrix": round(tq_ms / L, 4),
                                "GBps": round(wq_bytes / (tq_ms * 1e-3) / 1e9, 2),
                                "bytes_per_matrix": wq_bytes // L,
                                "note": "absmean + ternarise + pack, offline, not in the step"},
    }
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(P, layer_bytes, args.cpu_seconds, lut)
    return out


def single_calls_in_graph(torch, dev, single, R, shape) -> float:
    """Microseconds per call of R single-layer calls (layers 0..R-1, each into
    its own output) captured in one HIP graph and replayed; the replayed
    outputs must equal the eager calls' bit for bit."""
    outs = torch.empty((R, *shape), dtype=torch.float32, device=dev)
    ref = torch.empty_like(outs)
    for l in range(R):
        single(l, ref[l])
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for l in range(4):
            single(l, outs[l])
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(R):
            single(l, outs[l])
    best = None
    for rep in range(4):
        outs.zero_()
        torch.cuda.synchronize()
        with Timer(torch) as t:
            graph.replay()
        if not torch.equal(outs, ref):
            raise RuntimeError("graph replay of the single-layer calls differs from the eager calls")
        if rep:
            best = t.ms if best is None else min(best, t.ms)
    del graph, outs, ref
    return best / R * 1e3


def cpu_baseline_decode(P, layer_bytes, seconds, lut=False):
    import oracle as O
    gamma, q, _ = O.quantize_weights(P.W)
    fwd = O.lut_forward if lut else O.forward_from_codes
    reps, t0 = 0, time.perf_counter()
    while True:
        fwd(P.X, q, gamma)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"[bench] cpu oracle: {reps} forwards of layer 0 in {el:.1f} s")
    out = {"value": round(reps * layer_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
           "kind": "oracle",
           "sample": f"layer 0 of the pool ({P.name}, seed 0): the oracle's forward from ternary "
                     f"codes (absmax quantise + {'LUT' if lut else 'exact'} contraction + rescale) "
                     f"repeated {reps} times"}
    if not lut:
        out["naive_loop"] = cpu_naive_loop(P, q)
    return out


def cpu_naive_loop(P, q, seconds=3.0):
    """The oracle's literal add / subtract / skip loop (pure Python, one core) on
    layer 0's first token, output channel after output channel, for a few seconds."""
    import oracle as O
    _, Xq, _ = O.absmax_quantize(P.X)
    xr = Xq[0].tolist()
    done, t0 = 0, time.perf_counter()
    while True:
        O.zero_gemm_dot(xr, q[done % q.shape[0]].tolist())
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"[bench] cpu naive loop: {done} outputs in {el:.1f} s")
    return {"value": round(done * P.K / el / 1e9, 6), "unit": "G weights/s", "cores": 1,
            "kind": "oracle naive add/subtract/skip loop",
            "sample": f"{done} outputs (token 0 against output channels 0..{min(done, q.shape[0]) - 1}, K={P.K})"}


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def bench_prefill(args, torch, bl, dev, workload=None):
    import numpy as np
    from bitlinear_absmean_ternarise_bit_amd.workloads import make_workload

    workload = workload or args.workload
    P = make_workload(workload)
    M, K, N = P.M, P.K, P.N
    log(f"[bench] prefill {workload}: M={M} K={K} N={N}")
    W = torch.from_numpy(P.W).to(dev)
    packed, gamma = bl.quantize_weights(W)  # first call loads the kernels: not timed
    ws_q = torch.empty((bl.abi.load().bitlinear_quantize_workspace_bytes(),), dtype=torch.uint8, device=dev)
    with Timer(torch) as tq:
        bl.quantize_weights(W, out_packed=packed, out_gamma=gamma, workspace=ws_q)
    del W
    torch.cuda.empty_cache()
    X = torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws_bytes = bl.abi.load().bitlinear_forward_workspace_bytes(M, K)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    def step():
        bl.forward(X, packed, gamma, K, out=Y, workspace=ws)

    ms_step, warmup, steps = run_timed(args, torch, step, f"prefill {workload}")
    ops = 2.0 * M * N * K
    tops = ops / (ms_step * 1e-3) / 1e12
    log(f"[bench] prefill {workload}: {tops:.1f} TOPS")

    # dominant kernel alone: the GEMM + rescale from precomputed codes, timed
    # over as many calls right after the step's own timed region
    Xq, ga, rs = bl.quantize_activations(X)
    for _ in range(2):
        bl.forward_quantized(Xq, ga, rs, packed, gamma, K, out=Y)
    with Timer(torch) as tg:
        for _ in range(steps):
            bl.forward_quantized(Xq, ga, rs, packed, gamma, K, out=Y)
    gemm_ms = tg.ms / steps
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    sus = sustained_after(args, torch, step, ms_step)
    sus_gemm = None
    if sus:
        # and the GEMM alone right after it, over as many calls
        with Timer(torch) as tg2:
            for _ in range(sus[2]):
                bl.forward_quantized(Xq, ga, rs, packed, gamma, K, out=Y)
        sus_gemm = tg2.ms / sus[2]
    step_bytes = N * bl.packed_words(K) * 4 + M * K * 2 + M * N * 4
    out = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS",
        "ms_per_step": round(ms_step, 6), "warmup": warmup, "steps": steps,
        "dtype": "i8",
        "config": {"workload": workload, "M": M, "K": K, "N": N, "x_dtype": "bf16",
                   "ops_per_step": ops, "bytes_per_step": step_bytes},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic_for(workload, "prefill"),
                     "kernel": "prefill_gemm_kernel (INT8 MFMA + fused rescale)",
                     "kernel_ms": round(gemm_ms, 6)},
        **({"sustained": dict(sustained_obj(sus, ops / 1e12, "TOPS", INT8_PEAK_TOPS),
                              kernel_ms=round(sus_gemm, 6),
                              achieved=round(ops / (sus_gemm * 1e-3) / 1e12, 2),
                              kernel_frac=round(ops / (sus_gemm * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              kernel="the GEMM alone (forward_quantized) right after, over as many calls")}
           if sus else {}),
        "weight_quantisation": {"ms_per_matrix": round(tq.ms, 4),
                                "GBps": round((4 * N * K + N * bl.packed_words(K) * 4) / (tq.ms * 1e-3) / 1e9, 2),
                                "note": "absmean + ternarise + pack, offline, not in the step"},
    }
    del X, Y, ws, Xq, ga, rs, packed
    torch.cuda.empty_cache()
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(P, args.cpu_seconds)
    return out


def prefill_objects(args, torch, bl, dev) -> dict:
    """The prefill half of the metric, carried in the default (decode) line:
    for each prefill workload, the whole forward (quantiser + GEMM) in TOPS,
    the GEMM alone (kernel_ms) with its roofline against the INT8 peak, and
    the CPU oracle beside it."""
    out = {}
    for w in PREFILL_WORKLOADS[::-1]:  # the largest first
        o = bench_prefill(args, torch, bl, dev, workload=w)
        cfg = o.pop("config")
        o.pop("metric")
        o = {"workload": w, "M": cfg["M"], "K": cfg["K"], "N": cfg["N"], "x_dtype": cfg["x_dtype"],
             "ops_per_step": cfg["ops_per_step"], **o}
        if "cpu_baseline" in o:
            o["cpu_baseline"].update(host_cpu())
        out[w] = o
    return out


def cpu_baseline_prefill(P, seconds):
    import numpy as np
    import oracle as O
    gamma, q, _ = O.quantize_weights(P.W)
    rows_per_rep = 32
    cols = np.arange(P.N)
    reps, t0 = 0, time.perf_counter()
    while True:
        r0 = (reps * rows_per_rep) % P.M
        O.sampled_forward(P.X, q, gamma, np.arange(r0, r0 + rows_per_rep), cols)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    ops = 2.0 * reps * rows_per_rep * P.N * P.K
    log(f"[bench] cpu oracle: {reps} x {rows_per_rep} tokens in {el:.1f} s")
    return {"value": round(ops / el / 1e12, 6), "unit": "TOPS", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} calls of {rows_per_rep} tokens x all {P.N} outputs of {P.name} "
                      f"({reps * rows_per_rep} token rows, cycling over its {P.M} tokens): "
                      f"the oracle's forward from ternary codes"}


# ---------------------------------------------------------------------------
# BitNet FFN block (BitLinear up -> ReLU^2 -> BitLinear down)
# ---------------------------------------------------------------------------

FFN_WORKLOADS = {"ffn_block_decode_m8_d2048_f5632": 0.02, "ffn_block_prefill_m2048_d4096_f11008": 0.015}


def bench_ffn(args, torch, bl, dev):
    import numpy as np
    from bitlinear_absmean_ternarise_bit_amd.workloads import make_ffn_workload

    P = make_ffn_workload(args.workload)
    sigma = FFN_WORKLOADS[args.workload]
    M, D, F, Do = P.M, P.D, P.F, P.D_out
    decode = bl.decode_fits(M, D, F) and bl.decode_fits(M, F, Do)
    wbytes = F * bl.packed_words(D) * 4 + Do * bl.packed_words(F) * 4
    L = (args.layers or max(8, -(-(1 << 30) // wbytes))) if decode else 1
    log(f"[bench] FFN block {args.workload}: M={M} D={D} F={F} D_out={Do}, {L} layer(s), "
        f"{'decode' if decode else 'prefill'} path")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    X = torch.empty((L, M, D), dtype=torch.bfloat16, device=dev)
    X[0].copy_(torch.from_numpy(P.X_bf16_bits.view(np.int16)).view(torch.bfloat16))
    if L > 1:
        X[1:].copy_(torch.randn((L - 1, M, D), generator=g, device=dev).to(torch.bfloat16))
        if "outlier_channels" in P.notes:
            ch = torch.from_numpy(P.notes["outlier_channels"]).to(dev)
            X[1:, :, ch] = (X[1:, :, ch].float() * 20.0).to(torch.bfloat16)
    pu = torch.empty((L, F, bl.packed_words(D)), dtype=torch.int32, device=dev)
    pd = torch.empty((L, Do, bl.packed_words(F)), dtype=torch.int32, device=dev)
    gu = torch.empty((L,), dtype=torch.float32, device=dev)
    gd = torch.empty((L,), dtype=torch.float32, device=dev)
    ws = torch.empty((bl.abi.load().bitlinear_quantize_workspace_bytes(),), dtype=torch.uint8, device=dev)
    Wu = torch.empty((F, D), dtype=torch.float32, device=dev)
    Wd = torch.empty((Do, F), dtype=torch.float32, device=dev)
    for l in range(L):
        if l == 0:
            Wu.copy_(torch.from_numpy(P.W_up))
            Wd.copy_(torch.from_numpy(P.W_down))
        else:
            Wu.normal_(0.0, sigma, generator=g)
            Wd.normal_(0.0, sigma, generator=g)
        bl.quantize_weights(Wu, out_packed=pu[l], out_gamma=gu[l:l + 1], workspace=ws)
        bl.quantize_weights(Wd, out_packed=pd[l], out_gamma=gd[l:l + 1], workspace=ws)
    del Wu, Wd
    Y = torch.empty((L, M, Do), dtype=torch.float32, device=dev)
    fws = torch.empty((bl.abi.load().bitlinear_ffn_workspace_bytes(L, M, D, F),), dtype=torch.uint8, device=dev)

    def step():
        bl.ffn_forward(X, (pu, gu), (pd, gd), out=Y, workspace=fws)

    ms_step, warmup, steps = run_timed(args, torch, step, "FFN block")
    ops = 2.0 * 2 * M * D * F * L
    tops = ops / (ms_step * 1e-3) / 1e12
    # algorithmic bytes: packed weights, X, the hidden layer written and read, Y
    step_bytes = L * (wbytes + M * D * 2 + 2 * M * F * 4 + M * Do * 4)
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"[bench] FFN block: {gbps:.1f} GB/s, {tops:.1f} TOPS")
    cfg = {"workload": args.workload + (f" x {L} layers per step (batched decode, cold weights)" if L > 1 else ""),
           "M": M, "D": D, "F": F, "D_out": Do, "layers": L, "x_dtype": "bf16", "path": "decode" if decode else "prefill",
           "bytes_per_step": step_bytes, "ops_per_step": ops}
    if decode:
        out = {"metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "ms_per_step": round(ms_step, 6),
               "warmup": warmup, "steps": steps, "dtype": "i8", "config": cfg,
               "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                            "kernel": "whole block: decode_kernel (up, ReLU^2 epilogue), activation quantiser over all hidden rows, decode_kernel (down, on those codes)"}}
    else:
        out = {"metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "ms_per_step": round(ms_step, 6),
               "warmup": warmup, "steps": steps, "dtype": "i8", "config": cfg,
               "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                            "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": None,
                            "kernel": "whole block: 2 x (activation quantiser + prefill GEMM)"}}
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_ffn(P, decode, step_bytes // L, args.cpu_seconds)
    return out


def cpu_baseline_ffn(P, decode, layer_bytes, seconds):
    import numpy as np
    import oracle as O
    g_up, q_up, _ = O.quantize_weights(P.W_up)
    g_dn, q_dn, _ = O.quantize_weights(P.W_down)
    rows = P.M if decode else 8
    reps, t0 = 0, time.perf_counter()
    while True:
        r0 = (reps * rows) % P.M
        O.ffn_from_codes(P.X[r0:r0 + rows], q_up, g_up, q_dn, g_dn)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"[bench] cpu oracle: {reps} blocks of {rows} tokens in {el:.1f} s")
    if decode:
        return {"value": round(reps * layer_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
                "kind": "oracle", "sample": f"layer 0 ({P.name}): the oracle's FFN block from ternary codes, "
                                            f"repeated {reps} times"}
    ops = 2.0 * 2 * rows * reps * P.D * P.F
    return {"value": round(ops / el / 1e12, 6), "unit": "TOPS", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps * rows} of {P.M} tokens of {P.name}: the oracle's FFN block from ternary codes, "
                      f"{rows} tokens per call"}


# ---------------------------------------------------------------------------
# STE backward (dX and dW of one BitLinear)
# ---------------------------------------------------------------------------

BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
BACKWARD_WORKLOADS = {"ste_backward_m2048_k4096_n11008": "prefill_ffn_m2048_k4096_n11008"}


def bench_backward(args, torch, bl, dev):
    import numpy as np
    from bitlinear_absmean_ternarise_bit_amd.workloads import make_workload

    P = make_workload(BACKWARD_WORKLOADS[args.workload])
    M, K, N = P.M, P.K, P.N
    log(f"[bench] STE backward {args.workload}: M={M} K={K} N={N} (dX and dW, bf16 gradients)")
    W = torch.from_numpy(P.W).to(dev)
    packed, gamma = bl.quantize_weights(W)
    X = torch.from_numpy(P.X_bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    Xq, ga, _ = bl.quantize_activations(X)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    dY = torch.randn((M, N), generator=g, device=dev).to(torch.bfloat16)
    packedT = torch.empty((K, bl.packed_words(N)), dtype=torch.int32, device=dev)
    mask = torch.empty((N, (K + 31) // 32), dtype=torch.int32, device=dev)
    bl.pack_transposed(W, gamma, out=packedT, mask_out=mask)  # warm
    with Timer(torch) as tp:
        bl.pack_transposed(W, gamma, out=packedT, mask_out=mask)
    ws = torch.empty((bl.abi.load().bitlinear_backward_workspace_bytes(M, N, K),), dtype=torch.uint8, device=dev)

    def step():
        bl.backward(dY, packedT, gamma, Xq, ga, mask, K, workspace=ws)

    ms_step, warmup, steps = run_timed(args, torch, step, "STE backward")
    flops = 2.0 * 2 * M * N * K
    tflops = flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] STE backward: {tflops:.1f} TFLOP/s")
    out = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms_step, 6),
           "warmup": warmup, "steps": steps,
           "dtype": "bf16",
           "config": {"workload": args.workload, "M": M, "K": K, "N": N, "flops_per_step": flops,
                      "note": "dX = gamma dY W_q and dW = (dY^T A_hat) * range mask, bf16 matrix cores"},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "bf16_gemm_nt_kernel x 2 + operand preparation, one step"},
           "pack_transposed": {"ms": round(tp.ms, 4),
                               "note": "codes of W^T and the range mask of W, once per weight update"}}
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(P, args.cpu_seconds)
    return out


def cpu_baseline_backward(P, seconds):
    import numpy as np
    import oracle as O
    from bitlinear_absmean_ternarise_bit_amd.workloads import f32_to_bf16_bits, bf16_bits_to_f32
    g, q, _ = O.quantize_weights(P.W)
    gA, Xq, _ = O.absmax_quantize(P.X)
    dY = bf16_bits_to_f32(f32_to_bf16_bits(np.random.default_rng(0).standard_normal((P.M, 64)).astype(np.float32)))
    rows = 8
    reps, t0 = 0, time.perf_counter()
    while True:
        r0 = (reps * rows) % P.M
        # dX for `rows` tokens (all N) and dW for 64 output channels (all M)
        dYr = bf16_bits_to_f32(f32_to_bf16_bits(np.random.default_rng(reps).standard_normal((rows, P.N))
                                                .astype(np.float32)))
        O.ste_backward(dYr, q, g, Xq[r0:r0 + rows], gA[r0:r0 + rows], P.W)
        O.ste_backward(dY, q[:64], g, Xq, gA, P.W[:64])
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    flops = reps * (2.0 * rows * P.N * P.K + 2.0 * 64 * P.M * P.K)
    log(f"[bench] cpu oracle: {reps} samples in {el:.1f} s")
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} x (dX of {rows} tokens + dW of 64 output channels) of {P.M}x{P.K}x{P.N}"}


# ---------------------------------------------------------------------------

def attainable_peaks(torch, bl, dev, read_blocks=(1024, 2048), mfma_iters: int = 20000) -> dict:
    """The chip's attainable rates for plain kernels, beside the published peaks:
    a 1 GiB streaming read (16-byte nontemporal loads, one contiguous slice per
    workgroup; the faster of 4 and 8 workgroups per CU), a 512 MiB -> 512 MiB
    streaming copy, and back-to-back INT8 and bf16 MFMAs on registers (two
    workgroups per CU)."""
    lib = bl.abi.load_probe()
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    out = torch.empty(max(read_blocks) * 256, dtype=torch.int32, device=dev)

    def timed(fn, reps=10):
        for _ in range(2):
            fn()
        with Timer(torch) as t:
            for _ in range(reps):
                fn()
        return t.ms / reps

    def call(name, st):
        bl.abi.check(name, st)

    ms_read = min(timed(lambda: call("bitlinear_probe_stream", lib.bitlinear_probe_stream(
        buf.data_ptr(), None, nbytes, b, out.data_ptr(), stream))) for b in read_blocks)
    half = buf.view(2, -1)
    ms_copy = min(timed(lambda: call("bitlinear_probe_stream", lib.bitlinear_probe_stream(
        half[0].data_ptr(), half[1].data_ptr(), nbytes // 2, b // 2, None, stream))) for b in read_blocks)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    mout = torch.empty(2 * cus * 256, dtype=torch.int32, device=dev)
    ms_mfma = timed(lambda: call("bitlinear_probe_mfma_i8", lib.bitlinear_probe_mfma_i8(
        mfma_iters, 2 * cus, mout.data_ptr(), stream)), reps=3)
    ops = 2 * cus * 4 * 8 * mfma_iters * 65536
    fout = torch.empty(2 * cus * 256, dtype=torch.float32, device=dev)
    ms_bf16 = timed(lambda: call("bitlinear_probe_mfma_bf16", lib.bitlinear_probe_mfma_bf16(
        mfma_iters, 2 * cus, fout.data_ptr(), stream)), reps=3)
    flops = 2 * cus * 4 * 8 * mfma_iters * 32768
    del buf, out, mout, fout
    return {"hbm_read_GBps": round(nbytes / ms_read / 1e6, 1),
            "hbm_copy_GBps": round(nbytes / ms_copy / 1e6, 1),
            "mfma_i8_TOPS": round(ops / ms_mfma / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops / ms_bf16 / 1e9, 1),
            "note": "plain kernels on this GPU: 1 GiB streaming read (the faster of 4 and 8 workgroups per CU); 512 MiB copy (GB/s of bytes read "
                    "+ written); independent v_mfma_i32_32x32x32_i8, and v_mfma_f32_32x32x16_bf16, on "
                    "registers"}


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        res = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for ln in res.stdout.splitlines():
            if ln.startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpu() -> dict:
    """What the CPU baseline ran on: the model, the logical CPUs the host
    offers (nproc) and those this process may use."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": cpu_model(), "nproc": os.cpu_count() or 1, "cpus_usable": usable}


def copy_calibration(torch, dev):
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    log("[bench] copy calibration: 3 x elementwise add of 1 GiB (1 GiB read + 1 GiB written each)")
    print(json.dumps({"copy_calibration_bytes_read": 1 << 30, "copy_calibration_bytes_written": 1 << 30}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help=f"timed steps (default: enough for {TIMED_S} s, at least {MIN_STEPS})")
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed warm-up steps (default: enough for {SETTLE_S} s under load, "
                         f"at least {MIN_WARMUP})")
    ap.add_argument("--workload", default="decode_m1_k2048_n2048",
                    choices=sorted(DECODE_WORKLOADS) + list(PREFILL_WORKLOADS) + sorted(FFN_WORKLOADS)
                    + sorted(BACKWARD_WORKLOADS))
    ap.add_argument("--layers", type=int, default=0, help="decode pool size (default: >= 1 GiB packed)")
    ap.add_argument("--format", default="2bit", choices=["2bit", "radix3", "lut"],
                    help="decode weight format: 2-bit codes or radix-3 (five weights per byte); "
                         "lut: 2-bit codes contracted through 81-entry tables (comparison)")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-prefill", dest="prefill", action="store_false",
                    help="decode workloads: leave out the prefill objects (both prefill workloads, "
                         "timed after the decode step) from the line")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the attainable-peak probes (streaming read and copy, register MFMAs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the BitLinear forward shards over tokens or output channels without changes to "
              "the kernel); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bitlinear_absmean_ternarise_bit_amd as bl

    dev = torch.device("cuda:0")
    bl.abi.load()
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    if args.format != "2bit" and args.workload not in DECODE_WORKLOADS:
        print("--format radix3 / lut apply to the decode workloads only", file=sys.stderr)
        sys.exit(2)
    if args.workload in BACKWARD_WORKLOADS:
        out = bench_backward(args, torch, bl, dev)
    elif args.workload in FFN_WORKLOADS:
        out = bench_ffn(args, torch, bl, dev)
    elif args.workload in DECODE_WORKLOADS:
        out = bench_decode(args, torch, bl, dev)
    else:
        out = bench_prefill(args, torch, bl, dev)
    line = {"metric": out.pop("metric"), "value": out.pop("value"), "unit": out.pop("unit"),
            "n_gpus": 1, "steps": out.pop("steps"), "warmup": out.pop("warmup"),
            "ms_per_step": out.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": out.pop("dtype"), "data": "synthetic (seeded)",
            "config": out.pop("config")}
    line.update(out)
    if "cpu_baseline" in line:
        line["cpu_baseline"].update(host_cpu())
    if args.prefill and args.workload in DECODE_WORKLOADS and args.format == "2bit":
        line["prefill"] = prefill_objects(args, torch, bl, dev)
    if args.peaks:
        line["attainable"] = attainable_peaks(torch, bl, dev)
    props = torch.cuda.get_device_properties(dev)
    line["device"] = torch.cuda.get_device_name(dev)
    line["device_cus"] = props.multi_processor_count
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
