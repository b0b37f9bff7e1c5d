#!/usr/bin/env python3
"""Benchmark of the GLA hot path on one MI355X.

Headline: chunked forward on the training-shape workload (B=8, H=16, T=2048,
d_k=d_v=128, bf16 q/k/v, fp32 log-gates, S0 = 0, fp32 o and S_T), reported as
tokens/s of one GLA layer with all 16 heads, with its HBM roofline and the
matrix-core utilisation. A second object reports the decode step on 1,280
sequences x 16 heads (fp32 state 1.34 GB updated in place, 100 chained
steps) as state GB/s against the HBM peak. The fp64 CPU oracle is timed on a
bounded sample of the headline workload as the CPU baseline.

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Three input sets rotate across steps so that q/k/v (201 MB per set) are not
served from the 256 MB last-level cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_linear_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, sources):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    if there are none or the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(kernel_key)
    if not rec or rec.get("source_hash") != kernel_source_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def time_launches(fn, steps, stream):
    """Run fn(i) for i in range(steps) on `stream` twice. The timed pass:
    back-to-back calls with nothing else enqueued, timed by the wall clock
    between synchronisations and by one HIP event pair recorded on that stream
    around all of them. Then a pass with an event pair around each call, for
    the per-call distribution (time_launches.last, sorted; each pair adds its
    own few microseconds of event overhead). Returns (wall seconds of the timed
    pass, mean GPU ms per call from the timed pass's event pair)."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e0.elapsed_time(e1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    time_launches.last = sorted(per)
    return wall, region_ms


def pair_error(x, ref, cu=None, state=False):
    """Largest normwise error, max |x - ref| / max |ref|, over (sequence, head)
    pairs: of a token-major tensor [B, T, H, ...] (packed spans cu[n] ..
    cu[n+1] when cu is given), or with state=True of [N, H, ...]."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if state:
        blocks = [(x[n, h], ref[n, h]) for n in range(x.shape[0]) for h in range(x.shape[1])]
    else:
        spans = ([(b, 0, x.shape[1]) for b in range(x.shape[0])] if cu is None else
                 [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)])
        blocks = [(x[b, s_:e, h], ref[b, s_:e, h]) for b, s_, e in spans if e > s_
                  for h in range(x.shape[2])]
    worst = 0.0
    for a, r in blocks:
        if not np.all(np.isfinite(a)):
            return float("inf")
        scale = np.abs(r).max()
        d = np.abs(a - r).max()
        worst = max(worst, float(d / scale if scale > 0 else d))
    return worst


def host_cores():
    """Cores this process may run on, and the machine's count."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"nproc": avail, "cpu_count": os.cpu_count()}


def percentiles_ms(per):
    """median, p10, p90 of per-launch times (ms), as bench.py reports them."""
    n = len(per)
    pick = lambda f: per[min(n - 1, int(f * (n - 1) + 0.5))]
    return {"median": round(pick(0.5), 5), "p10": round(pick(0.1), 5), "p90": round(pick(0.9), 5)}


def warm_up(fn, steps, seconds):
    """At least `steps` calls and at least `seconds` of wall time, so that the
    GPU clocks have settled before anything is timed."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < steps or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


# kernel that runs the headline forward at each chunk size, and the sources
# whose hash keys its committed counter record
# (bf16 inputs run every chunk size as 64-token chunks on one kernel)
FWD_KERNELS = {
    64: ("chunk_bf16_ws_kernel<float>",
         ["chunk_bf16_ws.hip", "bf16_blocks.h", "tile_loader.h", "gla_common.h"]),
}
FWD_KERNELS[128] = FWD_KERNELS[64]


def bench_forward(args):
    import numpy as np
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    w = synth.WORKLOADS["train_2k"]
    C = args.chunk
    dev = torch.device("cuda:0")
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    sets = []
    host_set0 = None
    for i in range(3):
        q, k, v, lg, S0, cu = synth.make_forward_inputs(w, seed=w.seed + 100 * i)
        if i == 0:
            host_set0 = (q, k, v, lg)
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
        sets.append((bf(q), bf(k), bf(v), torch.from_numpy(lg).to(dev)))
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step_at(c):
        def step(i):
            q, k, v, lg = sets[i % 3]
            gla.fwd_chunked(q, k, v, lg, None, None, chunk_size=c, o=o, S_T=S_T)
        return step

    step = step_at(C)
    n_warm = warm_up(step, args.warmup, args.warm_seconds)
    wall, kern_ms = time_launches(step, args.steps, stream)
    kern_pct = percentiles_ms(time_launches.last)
    ms_per_step = 1e3 * wall / args.steps
    tokens = B * T
    tok_heads = B * T * H
    # algorithmic bytes: q, k, v (bf16) + log-gates (fp32) + o (fp32) + S_T (fp32)
    alg_bytes = tok_heads * (2 * dk + 2 * dk + 2 * dv + 4 + 4 * dv) + B * H * dk * dv * 4
    # algorithmic flops of the chunked form at chunk C: causal intra-chunk scores
    # and P V, the state read Q S and the state update K^T V
    alg_flops = tok_heads * ((C + 1) * (dk + dv) + 4 * dk * dv)
    # the same with whole diagonal tiles (the dense-tile count)
    dense_tile_flops = tok_heads * (2 * C * (dk + dv) + 4 * dk * dv)
    # flops the matrix cores issue (whole 16x16 tiles, bf16 hi/lo splits, the
    # score tiles recomputed by each 64-column slice)
    n_chunks = B * H * (T // C)
    slices = dv // 64
    nm, ntile = C // 16, (C // 16) * (C // 16 + 1) // 2
    causal_pv = sum((16 * mi + 15) // 32 + 1 for mi in range(nm))
    mfma_per_chunk = slices * (ntile * (dk // 32)                        # scores
                               + 4 * (nm * (dk // 32) * 2                  # Q S hi/lo
                                      + causal_pv * 2                      # P V hi/lo
                                      + (dk // 16) * (C // 32) * 2))       # K^T V hi/lo
    issued_flops = n_chunks * mfma_per_chunk * 16 * 16 * 32 * 2
    achieved_gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
    kname, ksrc = FWD_KERNELS[C]
    traffic = measured_traffic("chunk_fwd_bf16_train_2k_c64", ksrc)  # one kernel, both sizes
    # the other chunk size, for reference (same inputs, same timing method)
    C2 = 128 if C == 64 else 64
    warm_up(step_at(C2), 10, 0.2)
    wall2, kern_ms2 = time_launches(step_at(C2), args.steps, stream)
    # the same forward writing o in bf16 (as a bf16 training stack would take it)
    o16 = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)

    def step_bf16_out(i):
        q, k, v, lg = sets[i % 3]
        gla.fwd_chunked(q, k, v, lg, None, None, chunk_size=C, o=o16, S_T=S_T,
                        out_dtype=torch.bfloat16)

    warm_up(step_bf16_out, 10, 0.2)
    wall3, kern_ms3 = time_launches(step_bf16_out, args.steps, stream)
    alg_bytes16 = alg_bytes - tok_heads * dv * 2
    # outputs of input set 0 at both chunk sizes, for the parity check
    outs = {}
    for c in (C, C2):
        step_at(c)(0)
        torch.cuda.synchronize()
        outs[c] = (o.cpu().numpy(), S_T.cpu().numpy())
    res = {
        "tokens": tokens,
        "ms_per_step": ms_per_step,
        "kernel_ms": kern_ms,
        "kernel_ms_pct": kern_pct,
        "value": tokens / (ms_per_step * 1e-3),
        "config": {"workload": "train_2k chunked forward", "B": B, "T": T, "H": H, "dk": dk,
                   "dv": dv, "chunk": C, "in_dtype": "bf16", "out_dtype": "f32", "S0": "zeros",
                   "global_batch": B, "seq_len": T, "input_sets_rotated": 3},
        "warmup_calls": n_warm,
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": alg_bytes, "kernel": kname},
        "other_chunk": {"chunk": C2, "kernel": FWD_KERNELS[C2][0],
                        "kernel_ms": round(kern_ms2, 5),
                        "tokens_per_s": round(tokens / (wall2 / args.steps), 1),
                        "hbm_frac": round(alg_bytes / (kern_ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "bf16_out": {"kernel_ms": round(kern_ms3, 5),
                     "tokens_per_s": round(tokens / (wall3 / args.steps), 1),
                     "algorithmic_bytes": alg_bytes16,
                     "hbm_frac": round(alg_bytes16 / (kern_ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "mfma": {"algorithmic_tflops": round(alg_flops / (kern_ms * 1e-3) / 1e12, 1),
                 "algorithmic_util": round(alg_flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "issued_tflops": round(issued_flops / (kern_ms * 1e-3) / 1e12, 1),
                 "issued_util": round(issued_flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "algorithmic_flops": alg_flops, "issued_flops": issued_flops,
                 "dense_tile_flops": dense_tile_flops, "chunk": C,
                 "dense_tile_util": round(dense_tile_flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "peak_tflops": BF16_PEAK_TFLOPS},
    }
    return res, host_set0, outs


def bench_backward(args):
    """The chunked backward on the training shape (dS_T = 0, S0 = 0)."""
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    w = synth.WORKLOADS["train_2k"]
    C = args.chunk
    dev = torch.device("cuda:0")
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, seed=w.seed)
    dO, _ = synth.make_backward_grads(w, B, T, H, B, seed=w.seed + 7, final_state=False)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    tq, tk, tv, tdo = bf(q), bf(k), bf(v), bf(dO)
    tlg = torch.from_numpy(lg).to(dev)
    ws = torch.empty(gla._lib.load().gla_bwd_chunked_workspace_size(B, T, H, dk, dv, B, C, 0,
                                                                      gla.GLA_BF16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        gla.bwd_chunked(tq, tk, tv, tlg, tdo, chunk_size=C, need_dS0=False, workspace=ws)

    warm_up(step, 3, min(args.warm_seconds, 0.5))
    steps = max(5, args.steps // 5)
    wall, kern_ms = time_launches(step, steps, stream)
    got = [x.cpu().numpy() for x in gla.bwd_chunked(tq, tk, tv, tlg, tdo, chunk_size=C,
                                                    need_dS0=False, workspace=ws)[:4]]
    bench_backward.parity_inputs = (q, k, v, lg, dO, got)
    tok_heads = B * T * H
    # read q, k, v, dO (bf16) and the gates once, write dq, dk, dv (fp32) and dg once
    alg_bytes = tok_heads * (2 * dk + 2 * dk + 2 * dv + 2 * dv + 4 + 4 * dk + 4 * dk + 4 * dv + 4)
    gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
    return {
        "metric": "chunked backward tokens/s",
        "value": round(B * T / (wall / steps), 1),
        "unit": "tokens/s",
        "ms_per_step": round(1e3 * wall / steps, 4),
        "kernel_ms": round(kern_ms, 4),
        "steps": steps,
        "config": {"workload": "train_2k chunked backward", "B": B, "T": T, "H": H, "dk": dk,
                   "dv": dv, "chunk": C, "in_dtype": "bf16", "grad_dtype": "f32",
                   "S0": "zeros", "dS_T": "zeros"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": alg_bytes,
                     "note": "whole gla_bwd_chunked call: three chunked-forward runs on "
                             "chunk_bf16_ws_kernel (dq with q.dq partials, dv and dk in "
                             "reversed time, dk with k.dk partials) and the gate scan"},
    }


def bench_decode(args):
    import numpy as np
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    D = synth.DECODE
    N, H, dk, dv, steps = D["N"], D["H"], D["dk"], D["dv"], D["steps"]
    dev = torch.device("cuda:0")
    S_host = synth.make_decode_state(N, H, dk, dv, seed=D["state_seed"])
    S = torch.from_numpy(S_host).to(dev)
    qs, ks, vs, gs = [], [], [], []
    host_steps = []  # the first steps' inputs, for the parity check and the oracle's time
    for s in range(steps):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=D["step_seed_base"] + s)
        if s < 3:
            host_steps.append((q, k, v, lg))
        qs.append(torch.from_numpy(q).to(torch.bfloat16).to(dev))
        ks.append(torch.from_numpy(k).to(torch.bfloat16).to(dev))
        vs.append(torch.from_numpy(v).to(torch.bfloat16).to(dev))
        gs.append(torch.from_numpy(lg).to(dev))
    o = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # the first step from the initial state, kept for the parity check (every pair)
    gla.decode_step(qs[0], ks[0], vs[0], gs[0], S, o=o)
    torch.cuda.synchronize()
    bench_decode.parity_inputs = (S_host, host_steps, o.cpu().numpy(), S.cpu().numpy())

    def step(i):
        gla.decode_step(qs[i % steps], ks[i % steps], vs[i % steps], gs[i % steps], S, o=o)

    warm_up(step, min(args.warmup, 10), min(args.warm_seconds, 0.5))
    wall, kern_ms = time_launches(step, steps, stream)
    pairs = N * H
    alg_bytes = pairs * (2 * dk * dv * 4 + 2 * dk + 2 * dk + 2 * dv + 4 + 4 * dv)
    gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic("decode_step_1280x16", ["decode.hip", "gla_common.h"])
    # the same chain against a serving pool: the 1,280 requests on random,
    # distinct slots of a 2,048-entry pool
    P = 2048
    del S
    pool = torch.empty((P, H, dk, dv), dtype=torch.float32, device=dev).normal_(0.0, 0.02)
    perm = np.random.default_rng(D["state_seed"]).permutation(P)[:N].astype(np.int32)
    slots = torch.from_numpy(perm).to(dev)
    # the streaming order over the pool (4 MiB blocks of entries at a stride,
    # slot order within a block): one small launch per step, shared by
    # every layer of the step (timed on its own below)
    order = gla.slot_order(slots, P, H * dk * dv * 4)

    def step_slots(i):
        gla.decode_step_slots(qs[i % steps], ks[i % steps], vs[i % steps], gs[i % steps], pool,
                              slots, o=o, order=order)

    def step_slots_given(i):  # the requests streamed in the batch's own (random) order
        gla.decode_step_slots(qs[i % steps], ks[i % steps], vs[i % steps], gs[i % steps], pool,
                              slots, o=o)

    warm_up(step_slots, 10, min(args.warm_seconds, 0.5))
    wall_s, kern_ms_s = time_launches(step_slots, steps, stream)
    gbs_s = alg_bytes / (kern_ms_s * 1e-3) / 1e9
    warm_up(step_slots_given, 10, 0.0)
    _, kern_ms_g = time_launches(step_slots_given, steps, stream)
    ord_buf = torch.empty_like(order)
    _, kern_ms_o = time_launches(
        lambda i: gla._lib.check(gla._lib.load().gla_decode_slot_order(
            slots.data_ptr(), N, P, H * dk * dv * 4, ord_buf.data_ptr(), stream.cuda_stream),
            "slot order"),
        steps, stream)
    return {
        "metric": "decode-step state HBM GB/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": 1e3 * wall / steps,
        "kernel_ms": kern_ms,
        "tokens_per_s": round(N / (wall / steps), 1),
        "config": {"workload": "decode 1280 sequences x 16 heads", "N": N, "H": H, "dk": dk,
                   "dv": dv, "chained_steps": steps, "in_dtype": "bf16", "state": "f32 in place"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": alg_bytes,
                     "kernel": "decode_step_kernel<128,128,bf16,float>"},
        "pool_slots": {"pool": P, "requests": N, "kernel_ms": round(kern_ms_s, 4),
                       "gbs": round(gbs_s, 1), "frac": round(gbs_s / HBM_PEAK_GBS, 4),
                       "entry": "gla_decode_step_slots with the gla_decode_slot_order order",
                       "order_kernel_ms": round(kern_ms_o, 4),
                       "given_order_kernel_ms": round(kern_ms_g, 4),
                       "given_order_frac": round(alg_bytes / (kern_ms_g * 1e-3) / 1e9
                                                 / HBM_PEAK_GBS, 4)},
    }


def _device_inputs(B, T, H, dk, dv, gate_bias, seed, dev):
    """Seeded device-side draws with the synthetic workloads' distributions
    (q, v ~ N(0, 1), k ~ N(0, 1/d_k), bf16; log-gates logsigmoid(N(0, 1) +
    gate_bias)), for shapes too large to draw on the host quickly."""
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn((B, T, H, dk), device=dev, generator=g).to(torch.bfloat16)
    k = (torch.randn((B, T, H, dk), device=dev, generator=g) / dk ** 0.5).to(torch.bfloat16)
    v = torch.randn((B, T, H, dv), device=dev, generator=g).to(torch.bfloat16)
    lg = torch.nn.functional.logsigmoid(torch.randn((B, T, H), device=dev, generator=g) + gate_bias)
    return q, k, v, lg


def bench_tiny(args):
    """The tiny fp32 workload (B=1, H=2, T=256, d=64, fp32 inputs and
    arithmetic, chunk 64): launch-latency bound, reported for information."""
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    w = synth.WORKLOADS["tiny_f32"]
    dev = torch.device("cuda:0")
    q, k, v, lg, _, _ = synth.make_forward_inputs(w)
    tq, tk, tv, tl = (torch.from_numpy(a).to(dev) for a in (q, k, v, lg))
    o = torch.empty((w.B, w.T, w.H, w.dv), device=dev)
    S_T = torch.empty((w.B, w.H, w.dk, w.dv), device=dev)
    fn = lambda i: gla.fwd_chunked(tq, tk, tv, tl, chunk_size=64, o=o, S_T=S_T)
    warm_up(fn, 20, min(args.warm_seconds, 0.2))
    steps = 200
    wall, kern_ms = time_launches(fn, steps, torch.cuda.current_stream(dev))
    return {"workload": "tiny_f32", "B": w.B, "T": w.T, "H": w.H, "d": w.dk,
            "call_us": round(1e6 * wall / steps, 2), "event_us": round(1e3 * kern_ms, 2),
            **{f"{k}_us": round(1e3 * v, 2) for k, v in percentiles_ms(time_launches.last).items()}}


def bench_prefill(args):
    """The 65,536-token prefill: B=1, H=32, d=128, bf16, S0 ~ N(0, 0.02^2), at
    both chunk sizes; the forward splits the sequence over the CUs (state
    pass, combine, output pass)."""
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    w = synth.WORKLOADS["prefill_64k"]
    dev = torch.device("cuda:0")
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q, k, v, lg = _device_inputs(B, T, H, dk, dv, w.gate_bias, w.seed, dev)
    S0 = torch.empty((B, H, dk, dv), device=dev).normal_(0.0, w.s0_std)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    S_T = torch.empty_like(S0)
    stream = torch.cuda.current_stream(dev)
    tok_heads = B * T * H
    alg = tok_heads * (2 * dk + 2 * dk + 2 * dv + 4 + 4 * dv) + 2 * B * H * dk * dv * 4
    out = {"config": {"workload": "prefill_64k", "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
                      "S0": "N(0, 0.02^2)"}, "algorithmic_bytes": alg}
    # a head sample (one per host core, spread over the heads) whose inputs and
    # outputs the oracle checks and whose oracle run is timed
    n_s = max(1, min(H, host_cores()["nproc"]))
    hs = list(range(0, H, H // n_s))[:n_s]
    hsel = lambda x: x[:, :, hs].float().cpu().numpy()
    sample = {"heads": hs, "inputs": (hsel(q), hsel(k), hsel(v), lg[:, :, hs].cpu().numpy(),
                                      S0[:, hs].cpu().numpy(), None), "outputs": {}}
    for C in (64, 128):
        ws = torch.empty(max(1, gla.workspace_size(B, T, H, dk, dv, B, C)), dtype=torch.uint8,
                         device=dev)
        fn = lambda i, C=C, ws=ws: gla.fwd_chunked(q, k, v, lg, S0, chunk_size=C, o=o, S_T=S_T,
                                                   workspace=ws)
        warm_up(fn, 3, min(args.warm_seconds, 0.3))
        steps = max(5, args.steps // 5)
        wall, call_ms = time_launches(fn, steps, stream)
        gbs = alg / (call_ms * 1e-3) / 1e9
        # the forward's segment rule: ceil(CUs / units) segments for a dense
        # batch with fewer (sequence, head, slice) units than CUs
        units = B * H * dv // 64
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        segs = 1 if units >= n_cu else -(-n_cu // units)
        out[f"c{C}"] = {"call_ms": round(call_ms, 4), "tokens_per_s": round(B * T / (wall / steps), 1),
                        "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                        "segments_per_sequence": segs, **percentiles_ms(time_launches.last)}
        sample["outputs"][C] = (o[:, :, hs].cpu().numpy(), S_T[:, hs].cpu().numpy())
    bench_prefill.sample = sample
    return out


def bench_varlen(args):
    """The packed 64-sequence batch (lengths i.i.d. uniform on [128, 8192],
    H=16, d=128, bf16, per-sequence S0), at both chunk sizes, against a dense
    batch of about the same token count; with the critical path in chunks."""
    import numpy as np
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    w = synth.WORKLOADS["varlen_64"]
    dev = torch.device("cuda:0")
    H, dk, dv = w.H, w.dk, w.dv
    lengths = synth.varlen_lengths(np.random.default_rng(w.seed), w.num_seqs, w.len_lo, w.len_hi)
    cu_h = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu_h[1:] = np.cumsum(lengths)
    total = int(cu_h[-1])
    cu = torch.from_numpy(cu_h).to(dev)
    q, k, v, lg = _device_inputs(1, total, H, dk, dv, w.gate_bias, w.seed, dev)
    N = len(lengths)
    S0 = torch.empty((N, H, dk, dv), device=dev).normal_(0.0, w.s0_std)
    S_T = torch.empty_like(S0)
    o = torch.empty((1, total, H, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = max(5, args.steps // 5)
    tok_heads = total * H
    alg = tok_heads * (2 * dk + 2 * dk + 2 * dv + 4 + 4 * dv) + 2 * N * H * dk * dv * 4
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {"config": {"workload": "varlen_64", "sequences": N, "tokens": total, "H": H,
                      "dk": dk, "dv": dv, "longest": int(lengths.max()),
                      "shortest": int(lengths.min())}, "algorithmic_bytes": alg}
    # dense comparison: T = 2048, B = tokens / 2048 rounded
    Bd = max(1, round(total / 2048))
    qd, kd, vd, lgd = (x[:, :Bd * 2048].reshape((Bd, 2048) + tuple(x.shape[2:])) for x in (q, k, v, lg))
    od = torch.empty((Bd, 2048, H, dv), dtype=torch.float32, device=dev)
    STd = torch.empty((Bd, H, dk, dv), device=dev)
    # a head sample over every sequence for the oracle (check and timing)
    hs = [0, H // 3, 2 * H // 3, H - 1]
    hsel = lambda x: x[:, :, hs].float().cpu().numpy()
    sample = {"heads": hs, "inputs": (hsel(q), hsel(k), hsel(v), lg[:, :, hs].cpu().numpy(),
                                      S0[:, hs].cpu().numpy(), cu_h), "outputs": {}}
    for C in (64, 128):
        ws = torch.empty(max(1, gla.workspace_size(1, total, H, dk, dv, N, C, True)),
                         dtype=torch.uint8, device=dev)
        fn = lambda i, C=C, ws=ws: gla.fwd_chunked(q, k, v, lg, S0, cu, chunk_size=C, o=o,
                                                   S_T=S_T, workspace=ws)
        warm_up(fn, 3, min(args.warm_seconds, 0.3))
        wall, call_ms = time_launches(fn, steps, stream)
        pct = percentiles_ms(time_launches.last)
        fd = lambda i, C=C: gla.fwd_chunked(qd, kd, vd, lgd, None, chunk_size=C, o=od, S_T=STd)
        warm_up(fd, 3, min(args.warm_seconds, 0.3))
        wall_d, _ = time_launches(fd, steps, stream)
        tps = total / (wall / steps)
        tps_d = Bd * 2048 / (wall_d / steps)
        gbs = alg / (call_ms * 1e-3) / 1e9
        # critical path: the longest work item in chunks (the forward splits a
        # packed batch's sequences at its per-CU share of the work) against
        # the chunk steps per CU of a perfectly balanced schedule
        slices = dv // 64
        share = max(C, -(-(total * H * slices // n_cu) // C) * C)
        seg = min(share, 65536)
        crit = int(-(-min(int(lengths.max()), seg) // C))
        balanced = sum(-(-int(L) // C) for L in lengths) * H * slices / n_cu
        out[f"c{C}"] = {"call_ms": round(call_ms, 4), "tokens_per_s": round(tps, 1),
                        "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                        "dense_same_tokens_tokens_per_s": round(tps_d, 1),
                        "efficiency_vs_dense": round(tps / tps_d, 4),
                        "critical_path_chunks": crit,
                        "balanced_chunks_per_cu": round(balanced, 1), **pct}
        # o holds this chunk size's result (the dense comparison writes od)
        sample["outputs"][C] = (o[:, :, hs].cpu().numpy(), S_T[:, hs].cpu().numpy())
    bench_varlen.sample = sample
    return out


def bench_laplace(args):
    """Laplace 3B's mixer shape (16 heads of d_k = 96, d_v = 192, fixed
    geometric decays): the fixed-decay forward on 8 x 2,048 tokens at both
    chunk sizes, the per-token-gate forward on the same decays, and the decode
    step on 1,280 sequences."""
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    w = synth.WORKLOADS["laplace_2k"]
    dev = torch.device("cuda:0")
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q, k, v, lg, _, _ = synth.make_forward_inputs(w)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    tq, tk, tv = bf(q), bf(k), bf(v)
    tlg = torch.from_numpy(lg).to(dev)
    lam = torch.from_numpy(synth.fixed_log_decays(H)).to(dev)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    tok_heads = B * T * H
    # q, k, v (bf16) + o (fp32) + S_T (fp32); the per-token form also reads its gates
    alg_fixed = tok_heads * (2 * dk + 2 * dk + 2 * dv + 4 * dv) + B * H * dk * dv * 4
    alg_gates = alg_fixed + tok_heads * 4
    steps = max(10, args.steps // 2)

    def timed(fn, alg_bytes):
        warm_up(fn, 5, min(args.warm_seconds, 0.3))
        wall, kern_ms = time_launches(fn, steps, stream)
        gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
        return {"kernel_ms": round(kern_ms, 5), "tokens_per_s": round(B * T / (wall / steps), 1),
                "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}

    fwd = {}
    lap_out = {}
    for C in (64, 128):
        fwd[f"fixed_decay_c{C}"] = timed(
            lambda i, C=C: gla.fwd_chunked_fixed_decay(tq, tk, tv, lam, chunk_size=C, o=o,
                                                       S_T=S_T), alg_fixed)
        lap_out[C] = (o.cpu().numpy(), S_T.cpu().numpy())
    bench_laplace.parity_inputs = ((q, k, v, lg), lap_out)
    fwd["token_gates_c64"] = timed(
        lambda i: gla.fwd_chunked(tq, tk, tv, tlg, chunk_size=64, o=o, S_T=S_T), alg_gates)

    # the backward on the same inputs (the decays as a per-token gate stream, dO
    # drawn like v, dS_T = 0); every run on the twelve-wavefront kernel, the dq
    # and dk runs' 192-dim keys as two 96-dim halves
    gen = torch.Generator(device=dev).manual_seed(w.seed + 4)
    tdo = torch.randn((B, T, H, dv), generator=gen, device=dev).to(torch.bfloat16)
    bws = torch.empty(gla._lib.load().gla_bwd_chunked_workspace_size(B, T, H, dk, dv, B, 64, 0,
                                                                     gla._lib.GLA_BF16),
                      dtype=torch.uint8, device=dev)
    alg_bwd = tok_heads * (2 * dk + 2 * dk + 2 * dv + 2 * dv + 4 + 4 * dk + 4 * dk + 4 * dv + 4)
    bwd = timed(lambda i: gla.bwd_chunked(tq, tk, tv, tlg, tdo, chunk_size=64, need_dS0=False,
                                          workspace=bws), alg_bwd)
    bwd.update({"algorithmic_bytes": alg_bwd, "chunk": 64,
                "kernels": "chunk_bf16_w8_kernel<96,6,float,false,false,false> (dq: the "
                           "192-dim keys as two 96-dim halves, head groups of two), "
                           "chunk_bf16_w8_kernel<96,6,float,false,true,false> (dv; dk: the "
                           "same split, time-reversed), gate kernels (halves summed with "
                           "the gate dots)"})
    del tdo, bws

    # the mixer epilogue on the forward's output: fp32 o, bf16 q, k, v and gate
    # stream in, bf16 z out (4 tiers of 4 heads)
    gate = bf(synth.make_epilogue_inputs(B * T, H, dk, dv, seed=w.seed + 2)[4]).view(B, T, H, dv)
    a, tier_w, tier = synth.make_epilogue_params(H, dk, dv, seed=w.seed + 3)
    ta = torch.from_numpy(a).to(dev)
    rms_w = gla.head_rms_weights(torch.from_numpy(tier_w).to(dev), torch.from_numpy(tier).to(dev))
    z = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    alg_epi = tok_heads * (4 * dv + 2 * dk + 2 * dk + 2 * dv + 2 * dv + 2 * dv)
    epi = timed(lambda i: gla.mixer_epilogue(o, tq, tk, tv, gate, ta, rms_w, 1e-6, z=z), alg_epi)
    epi.update({"algorithmic_bytes": alg_epi, "kernel": "mixer_epilogue_r16_kernel<96,192,float,bf16,bf16>",
                "traffic": measured_traffic("mixer_epilogue_laplace_2k", ["epilogue.hip", "gla_common.h"])})
    del tq, tk, tv, tlg, o, S_T, gate, z

    # decode: 1,280 sequences x 16 heads of 96 x 192 fp32 state, in place
    N, dsteps = 1280, 20
    S = torch.from_numpy(synth.make_decode_state(N, H, dk, dv, seed=w.seed + 1)).to(dev)
    lgd = lam.expand(N, H).contiguous()
    ins = []
    for s_ in range(dsteps):
        dq, dkk, dvv, _ = synth.make_decode_step_inputs(N, H, dk, dv, seed=w.seed + 10 + s_)
        ins.append((bf(dq), bf(dkk), bf(dvv)))
    od = torch.empty((N, H, dv), dtype=torch.float32, device=dev)

    def dstep(i):
        a, b_, c = ins[i % dsteps]
        gla.decode_step(a, b_, c, lgd, S, o=od)

    warm_up(dstep, 10, min(args.warm_seconds, 0.3))
    wall, kern_ms = time_launches(dstep, dsteps, stream)
    alg_dec = N * H * (2 * dk * dv * 4 + 2 * dk + 2 * dk + 2 * dv + 4 + 4 * dv)
    gbs = alg_dec / (kern_ms * 1e-3) / 1e9
    return {
        "config": {"workload": "laplace_2k forward and 1280-sequence decode", "B": B, "T": T,
                   "H": H, "dk": dk, "dv": dv, "in_dtype": "bf16", "out_dtype": "f32",
                   "decays": "fixed geometric schedule, half-lives 1 .. 2048 tokens"},
        "forward": fwd,
        "forward_kernel": "chunk_bf16_w8_kernel<96,6,float,false,false,false> "
                          "(both chunk sizes run as 64-token chunks)",
        "forward_algorithmic_bytes": alg_fixed,
        "backward": bwd,
        "epilogue": epi,
        "forward_traffic_c64": measured_traffic("chunk_fwd_bf16_laplace_2k_c64",
                                                ["chunk_bf16_w8.hip", "bf16_blocks.h",
                                                 "tile_loader.h", "gla_common.h"]),
        "decode": {"N": N, "kernel_ms": round(kern_ms, 5), "gbs": round(gbs, 1),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg_dec,
                   "traffic": measured_traffic("decode_step_laplace_1280x16",
                                               ["decode.hip", "gla_common.h"]),
                   "kernel": "decode_step_rows_kernel<96,192,192,8,bf16,float>"},
    }


def bench_decode_layers(args, layers=24, batches=(20, 1280)):
    """One decode step of a Laplace-shaped mixer stack (24 layers of 16 heads,
    96 x 192; per layer the slot-indexed decode against its own state pool and
    the mixer epilogue), run eagerly call by call and as one captured HIP
    graph, for a replica-sized batch of 20 sequences and for 1,280; then the
    same with the decode and the epilogue fused into one kernel per layer."""
    import torch

    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth

    H, dk, dv = 16, 96, 192
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    a, tier_w, tier = synth.make_epilogue_params(H, dk, dv, seed=77)
    ta = torch.from_numpy(a).to(dev)
    rms_w = gla.head_rms_weights(torch.from_numpy(tier_w).to(dev), torch.from_numpy(tier).to(dev))
    lam = torch.from_numpy(synth.fixed_log_decays(H)).to(dev)
    out = {"layers": layers, "config": {"H": H, "dk": dk, "dv": dv, "in_dtype": "bf16",
                                        "state": "f32 pool per layer", "z_dtype": "bf16"}}
    for N in batches:
        pools = [torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev).normal_(0.0, 0.02)
                 for _ in range(layers)]
        slots = torch.randperm(N, device=dev).to(torch.int32)
        qkv = [(torch.randn((N, H, dk), device=dev).to(bf),
                (torch.randn((N, H, dk), device=dev) / dk ** 0.5).to(bf),
                torch.randn((N, H, dv), device=dev).to(bf),
                torch.randn((N, H, dv), device=dev).to(bf)) for _ in range(layers)]
        lg = lam.expand(N, H).contiguous()
        o = [torch.empty((N, H, dv), dtype=torch.float32, device=dev) for _ in range(layers)]
        z = [torch.empty((N, H, dv), dtype=bf, device=dev) for _ in range(layers)]

        def step(i=0):
            order = gla.slot_order(slots, N, H * dk * dv * 4)  # once per step, for every layer
            for l in range(layers):
                q, k, v, g = qkv[l]
                gla.decode_step_slots(q, k, v, lg, pools[l], slots, o=o[l], order=order)
                gla.mixer_epilogue(o[l], q, k, v, g, ta, rms_w, 1e-6, z=z[l])

        warm_up(step, 3, min(args.warm_seconds, 0.3))
        steps = 20
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) / steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        replay = (time.perf_counter() - t0) / steps
        # the same step with the fused decode + epilogue: one kernel per layer
        def step_fused(i=0):
            order = gla.slot_order(slots, N, H * dk * dv * 4)
            for l in range(layers):
                q, k, v, g = qkv[l]
                gla.decode_mixer(q, k, v, lg, pools[l], g, ta, rms_w, 1e-6, slots=slots, z=z[l],
                                 order=order)

        warm_up(step_fused, 3, min(args.warm_seconds, 0.3))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step_fused(i)
        torch.cuda.synchronize()
        eager_f = (time.perf_counter() - t0) / steps
        graph_f = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_f):
            step_fused()
        for _ in range(3):
            graph_f.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graph_f.replay()
        torch.cuda.synchronize()
        replay_f = (time.perf_counter() - t0) / steps
        state_bytes = layers * N * H * dk * dv * 4 * 2
        out[f"N{N}"] = {"eager_ms": round(eager * 1e3, 4), "graph_ms": round(replay * 1e3, 4),
                        "tokens_per_s_graph": round(N / replay, 1),
                        "state_gbs_graph": round(state_bytes / replay / 1e9, 1),
                        "fused_eager_ms": round(eager_f * 1e3, 4),
                        "fused_graph_ms": round(replay_f * 1e3, 4),
                        "fused_tokens_per_s_graph": round(N / replay_f, 1),
                        "fused_state_gbs_graph": round(state_bytes / replay_f / 1e9, 1)}
        if N == 1280:  # HBM bytes per fused launch from the committed counter runs
            out[f"N{N}"]["fused_kernel"] = "decode_mixer_kernel<96,192,8,bf16,bf16>"
            out[f"N{N}"]["fused_algorithmic_bytes_per_layer"] = N * H * (
                2 * dk * dv * 4 + 2 * dk * 2 + 3 * dv * 2 + 4)
            out[f"N{N}"]["fused_traffic_per_layer"] = measured_traffic(
                "decode_mixer_laplace_1280x16", ["decode.hip", "gla_common.h"])
        del pools, qkv, o, z, graph, graph_f
        torch.cuda.empty_cache()
    return out


def cpu_baseline(host_set, target_s=10.0, min_wall=3.0):
    """Time the fp64 C oracle on a bounded sample of the headline workload:
    all 8 sequences over a subset of heads, sized to about target_s seconds."""
    import numpy as np

    from oracle import c_oracle

    q, k, v, lg = host_set
    B, T, H, dk = q.shape
    pick = lambda a, hs: np.ascontiguousarray(a[:, :, hs])
    # one core: one head of one sequence on one thread, repeated to about 1 s
    # (also the calibration of the all-core sample)
    one = (pick(q[:1], [0]), pick(k[:1], [0]), pick(v[:1], [0]), pick(lg[:1], [0]))
    n1, t_one = 0, 0.0
    while n1 == 0 or (t_one < 1.0 and n1 < 200):
        t0 = time.perf_counter()
        c_oracle.fwd(*one, nthreads=1)
        t_one += time.perf_counter() - t0
        n1 += 1
    t1 = t_one / n1
    _, _, cores = c_oracle.fwd(pick(q[:1], [0]), pick(k[:1], [0]), pick(v[:1], [0]),
                               pick(lg[:1], [0]), nthreads=0)
    n_heads = int(max(1, min(H, round(target_s * cores / max(t1, 1e-6) / B))))
    hs = list(range(n_heads))
    args = (pick(q, hs), pick(k, hs), pick(v, hs), pick(lg, hs))
    # when the sample is the whole workload and runs short, repeat it (up to
    # min_wall seconds) so that the rate is not one sub-second measurement
    reps, el = 0, 0.0
    while reps == 0 or (el < min_wall and reps < 50):
        t0 = time.perf_counter()
        _, _, used = c_oracle.fwd(*args, nthreads=0)
        el += time.perf_counter() - t0
        reps += 1
    tok_heads = B * T * n_heads
    return {"value": round(tok_heads * reps / el / H, 1), "unit": "tokens/s", "cores": used,
            "kind": "oracle",
            "sample": f"train_2k: all {B} sequences x {n_heads} of {H} heads x {T} tokens "
                      f"({tok_heads} token-heads) x {reps} runs, {el:.1f} s; value scaled to "
                      f"tokens/s of a {H}-head layer",
            "seconds": round(el, 2),
            "one_core_value": round(T / t1 / H, 1),
            "one_core_sample": f"one sequence x one head x {T} tokens on one thread, "
                               f"{n1} runs, {t_one:.2f} s"}


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def oracle_legs(fwd_outs, host_set, chunk):
    """The fp64 C oracle against the GPU results of the benchmarked configs
    (the largest normwise error over (sequence, head) pairs), and its own time
    on the same inputs as a CPU baseline per config. Every pair is checked for
    train_2k (both chunk sizes), the train_2k backward, laplace_2k and the
    first decode step (all 20,480 pairs); prefill_64k and varlen_64 on a head
    sample over every token (their inputs are drawn on the device)."""
    import numpy as np

    from oracle import c_oracle

    parity, cpu = {}, {}
    cores = host_cores()
    q, k, v, lg = host_set
    B, T, H, _ = q.shape
    (o_ref, S_ref, used), el = _timed(lambda: c_oracle.fwd(q, k, v, lg, None, None, nthreads=0))
    for c, (o, ST) in fwd_outs.items():
        parity[f"train_2k_c{c}"] = {"o": pair_error(o, o_ref), "S_T": pair_error(ST, S_ref, state=True),
                                    "pairs": B * H}
    cpu["train_2k_all_heads"] = {"value": round(B * T / el, 1), "unit": "tokens/s",
                                 "threads": used, "seconds": round(el, 2)}
    del o_ref, S_ref
    bi = getattr(bench_backward, "parity_inputs", None)
    if bi is not None:
        bq, bk, bv, blg, bdo, got = bi
        (ref, el) = _timed(lambda: c_oracle.bwd(bq, bk, bv, blg, bdo, None, None, None,
                                                 nthreads=0))
        parity[f"train_2k_backward_c{chunk}"] = {
            "dq": pair_error(got[0], ref[0]), "dk": pair_error(got[1], ref[1]),
            "dv": pair_error(got[2], ref[2]),
            "dlog_g": float(np.abs(got[3] - ref[3]).max() / np.abs(ref[3]).max()),
            "pairs": B * H, "note": "dlog_g normwise over the whole tensor"}
        cpu["train_2k_backward_all_heads"] = {"value": round(B * T / el, 1), "unit": "tokens/s",
                                              "threads": ref[5], "seconds": round(el, 2)}
        del ref, bi
        bench_backward.parity_inputs = None
    di = getattr(bench_decode, "parity_inputs", None)
    if di is not None:
        S0h, steps_in, o1, S1 = di
        S_ref = S0h.astype(np.float64)
        (res, el) = _timed(lambda: c_oracle.decode(*steps_in[0], S_ref, nthreads=0))
        N, Hd = S0h.shape[:2]
        parity["decode_step1"] = {"o": pair_error(o1, res[0], state=True),
                                  "S": pair_error(S1, S_ref, state=True), "pairs": N * Hd}
        times = [el]
        for st in steps_in[1:]:
            times.append(_timed(lambda st=st: c_oracle.decode(*st, S_ref, nthreads=0))[1])
        per = sum(times) / len(times)
        state_bytes = 2 * S0h.nbytes
        cpu["decode_1280x16"] = {"value": round(N / per, 1), "unit": "tokens/s",
                                 "state_gbs": round(state_bytes / per / 1e9, 2),
                                 "ms_per_step": round(1e3 * per, 1), "threads": res[1],
                                 "sample": f"all {N * Hd} (sequence, head) pairs, {len(times)} "
                                           f"chained steps (the benchmark chains 100)"}
        del S_ref, di
        bench_decode.parity_inputs = None
    for name, fn in (("prefill_64k", bench_prefill), ("varlen_64", bench_varlen)):
        smp = getattr(fn, "sample", None)
        if smp is None:
            continue
        sq, sk, sv, slg, sS0, cu = smp["inputs"]
        (res, el) = _timed(lambda: c_oracle.fwd(sq, sk, sv, slg, sS0, cu, nthreads=0))
        for c, (o, ST) in smp["outputs"].items():
            parity[f"{name}_c{c}"] = {"o": pair_error(o, res[0], cu),
                                      "S_T": pair_error(ST, res[1], state=True),
                                      "heads": smp["heads"]}
        ntok = sq.shape[1]
        H_full = {"prefill_64k": 32, "varlen_64": 16}[name]
        cpu[name] = {"value": round(ntok * len(smp["heads"]) / el / H_full, 1),
                     "unit": "tokens/s", "threads": res[2], "seconds": round(el, 2),
                     "sample": f"{len(smp['heads'])} of {H_full} heads x every token "
                               f"({ntok}); value scaled to tokens/s of a {H_full}-head layer"}
        del res, smp
        fn.sample = None
    li = getattr(bench_laplace, "parity_inputs", None)
    if li is not None:
        (lq, lk, lv, llg), outs = li
        (res, el) = _timed(lambda: c_oracle.fwd(lq, lk, lv, llg, None, None, nthreads=0))
        for c, (o, ST) in outs.items():
            parity[f"laplace_2k_c{c}"] = {"o": pair_error(o, res[0]),
                                          "S_T": pair_error(ST, res[1], state=True),
                                          "pairs": lq.shape[0] * lq.shape[2]}
        cpu["laplace_2k_all_heads"] = {"value": round(lq.shape[0] * lq.shape[1] / el, 1),
                                       "unit": "tokens/s", "threads": res[2],
                                       "seconds": round(el, 2)}
        del res, li
        bench_laplace.parity_inputs = None
    cpu.update(cores)
    return parity, cpu


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10,
                    help="minimum untimed calls before timing (see --warm-seconds)")
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="minimum wall time of the untimed warm-up, for the clocks to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-laplace", action="store_true")
    ap.add_argument("--no-decode-layers", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 65,536-token prefill and the packed varlen batch")
    ap.add_argument("--chunk", type=int, default=64, choices=[64, 128])
    ap.add_argument("--stream-reference", action="store_true",
                    help="only time two plain streams over the decode state's size (1.342 GB "
                         "fp32): a device copy and an in-place scale, as read+write GB/s")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the GLA kernels here are single-device and this "
              f"build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.stream_reference:
        from gated_linear_attention_amd import synth
        D = synth.DECODE
        n = D["N"] * D["H"] * D["dk"] * D["dv"]
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        res = {}
        for name, fn in (("copy", lambda i: b.copy_(a)), ("inplace_scale", lambda i: a.mul_(0.999))):
            warm_up(fn, 10, args.warm_seconds)
            wall, kern_ms = time_launches(fn, 50, torch.cuda.current_stream())
            res[name] = {"gbs": round(2 * n * 4 / (kern_ms * 1e-3) / 1e9, 1),
                         "kernel_ms": round(kern_ms, 4)}
        print(json.dumps({"stream_reference_bytes": 2 * n * 4, **res}), flush=True)
        return
    if args.copy_calibration:
        n = 512 * 1024 * 1024 // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 5}), flush=True)
        return

    log("forward: building inputs")
    fwd, host_set, fwd_outs = bench_forward(args)
    log(f"forward: {fwd['value']:.4g} tokens/s, kernel {fwd['kernel_ms']:.4f} ms")
    bwd = None
    if not args.no_backward:
        log("backward: building inputs")
        bwd = bench_backward(args)
        log(f"backward: {bwd['value']:.4g} tokens/s, call {bwd['kernel_ms']:.4f} ms")
    dec = None
    if not args.no_decode:
        log("decode: building inputs")
        dec = bench_decode(args)
        log(f"decode: {dec['value']} GB/s, kernel {dec['kernel_ms']:.4f} ms")
    lap = None
    if not args.no_laplace:
        log("laplace shape: building inputs")
        lap = bench_laplace(args)
        log(f"laplace: fwd {lap['forward']} decode {lap['decode']['gbs']} GB/s")
    tiny = bench_tiny(args)
    log(f"tiny_f32: {tiny}")
    pre = var = None
    if not args.no_long:
        log("prefill_64k: building inputs")
        pre = bench_prefill(args)
        log(f"prefill_64k: {pre}")
        log("varlen_64: building inputs")
        var = bench_varlen(args)
        log(f"varlen_64: {var}")
    layers = None
    if not args.no_decode_layers:
        log("decode layers: building pools")
        layers = bench_decode_layers(args)
        log(f"decode layers: {layers}")
    cpu = None
    log("parity: the fp64 oracle on the benchmarked configs")
    parity, per_config = oracle_legs(fwd_outs, host_set, args.chunk)
    log(f"parity: {parity}")
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle")
        cpu = cpu_baseline(host_set)
        cpu["gpu_over_cpu"] = round(fwd["value"] / cpu["value"], 1)
        cpu.update({"nproc": per_config["nproc"], "cpu_count": per_config["cpu_count"],
                    "per_config": {k_: v_ for k_, v_ in per_config.items()
                                   if k_ not in ("nproc", "cpu_count")}})
        log(f"cpu baseline: {cpu['value']} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "GLA chunked-fwd tokens/s + MFMA util; decode-step state HBM GB/s vs peak",
        "value": round(fwd["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fwd["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": fwd["config"],
        "kernel_ms": round(fwd["kernel_ms"], 5),
        "kernel_ms_pct": fwd["kernel_ms_pct"],
        "roofline": fwd["roofline"],
        "mfma": fwd["mfma"],
        "other_chunk": fwd["other_chunk"],
        "bf16_out": fwd["bf16_out"],
        "backward": bwd,
        "decode": dec,
        "tiny_f32": tiny,
        "prefill_64k": pre,
        "varlen_64": var,
        "laplace": lap,
        "decode_layers": layers,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
