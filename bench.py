"""Benchmark of the GDN hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A timed step is one chunked varlen prefill of the 4 x 4096-token workload
(h_k = 16, h_v = 32, d = 128, bf16 q/k/v, fp32 g/beta/state/output, width-4
conv + SiLU + q/k L2 norm, final recurrent and conv states written), inputs
resident in HBM.  `value` is prefill tokens/s.  The library records HIP
events on its stream around its two main kernels (gdn_prefill_varlen_timed),
so the roofline entry is for the dominant kernel, the cross-chunk carry, and
the chunk-local kernel is reported beside it.  The decode half of the metric
(256 slots x 32 value heads, d = 128, conv update, 512 MiB fp32 state pool
updated in place, 100 consecutive steps over 4 pools in rotation) is timed
separately and reported under "decode", and the multi-token (speculative)
decode of 4 tokens per slot under "decode_multi"; the same prefill with bf16
outputs under "prefill_bf16_out"; the packed varlen batch (60
sequences, h_v = 48) and a 32768-token sequence are timed under
"other_prefill_configs".  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 matrix cores
PREP_KERNEL = "prep_kernel"
CARRY_KERNEL = "carry_kernel"
DECODE_KERNEL = "decode_kernel"


def prefill_algorithmic(T, N, h_k, h_v, d, in_bytes=2, out_bytes=4, chunk=64):
    """Bytes: each input read once, outputs and final states written once.
    Flops per (token, value head): (4/G + 6) * chunk * d + 6 * d^2."""
    G = h_v // h_k
    C = 2 * h_k * d + h_v * d
    per_token = (2 * h_k * d + h_v * d) * in_bytes + 2 * h_v * 4 + h_v * d * out_bytes
    bytes_ = T * per_token + N * h_v * d * d * 4 + C * 4 * in_bytes + (N + 1) * 4 + N * C * 3 * in_bytes
    flops = T * h_v * ((4.0 / G + 6.0) * chunk * d + 6.0 * d * d)
    return bytes_, flops


def carry_algorithmic(T, h_v, d, chunk=64):
    """Flops of the cross-chunk kernel per call: per (token, value head) the
    three d x d state products K H, Q H and the update (2 d^2 each) and the
    two lower-triangular 64 x 64 products T R and P D (chunk + 1 MACs per
    column on average: (chunk + 1) d flops each)."""
    return T * h_v * (6.0 * d * d + 2.0 * (chunk + 1) * d)


def prep_bytes(T, N, h_k, h_v, d, in_bytes=2, chunk=64):
    """Bytes the chunk-local kernel must move: raw q and k (with the 3-row
    conv history per chunk), g and beta, and the chunk images it writes
    (split-fp16 K and Q; the 10 lower 16x16 blocks of T and P; 4 scalars per
    token), for the chunks of N equal sequences."""
    chunks = N * ((T // N + chunk - 1) // chunk)
    raw = (T + 3 * chunks) * 2 * h_k * d * in_bytes + T * h_v * 2 * 4
    images = chunks * (h_k * 2 * 2 * chunk * d * 2 + h_v * (2 * 2 * 320 * 8 * 2 + 4 * chunk * 4))
    return raw + images


def decode_algorithmic(N, h_k, h_v, d, in_bytes=2, out_bytes=4, conv=True):
    """State read + write, q/k/v/g/beta read, o written, and with the conv
    prologue the conv history read + written and the conv weights read;
    ~ (6 d^2 + O(d)) flops per (slot, head)."""
    state = N * h_v * d * d * 4
    C = 2 * h_k * d + h_v * d
    bytes_ = 2 * state + N * C * in_bytes + N * h_v * 2 * 4 + N * h_v * d * out_bytes
    if conv:
        bytes_ += 2 * N * C * 3 * in_bytes + C * 4 * in_bytes
    flops = N * h_v * 7.0 * d * d
    return bytes_, flops


def decode_multi_algorithmic(N, m, h_k, h_v, d, kept, in_bytes=2, out_bytes=4):
    """m tokens per slot: the state read once and written `kept` times (once
    per kept token state), per-token q/k/v/g/beta read and o written, the
    conv history read once and written `kept` times, conv weights read."""
    state = N * h_v * d * d * 4
    C = 2 * h_k * d + h_v * d
    return (state * (1 + kept) + N * m * (C * in_bytes + h_v * 2 * 4 + h_v * d * out_bytes)
            + N * C * 3 * in_bytes * (1 + kept) + C * 4 * in_bytes)


def extra_prefill(gdn, torch, dev, lengths, h_k, h_v, d, init_std, steps, seed):
    """Prefill throughput at another geometry, inputs drawn on the GPU with the
    distributions of the seeded workloads (q, k, v ~ N(0, 1) in bf16, conv taps
    0.5 N(0, 1), beta = sigmoid(N(0, 1)), g = -softplus(N(0, 1)), initial
    states init_std N(0, 1)); returns (us per call, tokens/s, prep us, carry us)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    T, N = int(sum(lengths)), len(lengths)
    bf = torch.bfloat16
    rn = lambda *shape: torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
    q, k = rn(T, h_k, d).to(bf), rn(T, h_k, d).to(bf)
    v = rn(T, h_v, d).to(bf)
    beta = torch.sigmoid(rn(T, h_v))
    g = -torch.nn.functional.softplus(rn(T, h_v))
    C = 2 * h_k * d + h_v * d
    w = (0.5 * rn(C, 4)).to(bf)
    h0 = init_std * rn(N, h_v, d, d) if init_std else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=dev)
    o = torch.empty((T, h_v, d), dtype=torch.float32, device=dev)
    fs = torch.empty((N, h_v, d, d), dtype=torch.float32, device=dev)
    prob = gdn.binding.make_problem(N, T, h_k, h_v, d, d, gdn.GDN_BF16, gdn.GDN_F32)
    ws = torch.empty(gdn.binding.gdn_prefill_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def call(e=None):
        gdn.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, initial_state=h0, out=o, final_state_out=fs,
                               output_conv_state=False, workspace=ws, validate=False, events=e)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    us = float(np.mean([e[0].elapsed_time(e[3]) for e in evs])) * 1e3
    prep = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    carry = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
    return us, T / (us * 1e-6), prep, carry


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel's sources changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "traffic.json")) as f:
            t = json.load(f)
        k = t[kernel]
        h = hashlib.sha256()
        for src in k["sources"]:
            with open(os.path.join(root, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] != k["src_sha256_16"]:
            return None
        return (k["fetch_kib"] * t["fetch_scale"] + k["write_kib"] * t["write_scale"]) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(x, nthreads):
    """The fp64 oracle on the same seeded inputs (all sequences, all heads), wall clock."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle
    oracle.build(force=False)
    g = x.geom
    dims = oracle.Dims(g.h_k, g.h_v, g.d_k, g.d_v, conv_width=4)
    t0 = time.perf_counter()
    oracle.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": x.total_tokens / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"whole workload ({x.num_seqs} x {x.total_tokens // x.num_seqs} tokens, all heads), "
                      f"fp64, one run of {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU reaches steady clocks only after ~100 prefill calls (~0.1 s) of
    # work; fewer warmup steps under-report the carry kernel by ~8%.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the other prefill geometries (packed varlen batch, long single sequence)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time the plain 1 GiB device-to-device copy (the measured HBM reference) even "
                         "with --no-decode")
    ap.add_argument("--no-copy-calibration", action="store_true",
                    help="skip the 1 GiB copy that the decode legs are compared with")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the recurrence shards by heads or sequences with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gateddeltanet_chunked_delta_amd as gdn
    from gateddeltanet_chunked_delta_amd.inputs import (Geometry, conv_state_pool, conv_weights, decode_inputs,
                                                        multi_decode_inputs, prefill_inputs, state_pool,
                                                        uniform_lengths)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    geom = Geometry(16, 32, 128, 128)
    B, Tseq = 4, 4096
    print(f"[bench] generating prefill inputs {B}x{Tseq} h_k=16 h_v=32 d=128 bf16", file=sys.stderr, flush=True)
    x = prefill_inputs(1, [Tseq] * B, geom, "bf16")
    bf = torch.bfloat16
    q = torch.from_numpy(x.q).to(dev, bf)
    k = torch.from_numpy(x.k).to(dev, bf)
    v = torch.from_numpy(x.v).to(dev, bf)
    g = torch.from_numpy(x.g).to(dev)
    beta = torch.from_numpy(x.beta).to(dev)
    w = torch.from_numpy(x.conv_w).to(dev, bf)
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(dev)
    T = x.total_tokens
    o = torch.empty((T, 32, 128), dtype=torch.float32, device=dev)
    fs = torch.empty((B, 32, 128, 128), dtype=torch.float32, device=dev)
    cso = torch.empty((B, geom.channels, 3), dtype=bf, device=dev)
    prob = gdn.binding.make_problem(B, T, 16, 32, 128, 128, gdn.GDN_BF16, gdn.GDN_F32)
    ws = torch.empty(gdn.binding.gdn_prefill_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        gdn.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, out=o, final_state_out=fs,
                               conv_state_out=cso, workspace=ws, validate=False, events=events)

    print("[bench] warmup", file=sys.stderr, flush=True)
    # HIP events recorded by the library on its stream around each stage:
    # [before prep_kernel, before carry_kernel, after it, after the last launch]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.warmup):
        step(evs[i % args.steps])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [e[0].elapsed_time(e[3]) for e in evs]
    prep_ms = [e[0].elapsed_time(e[1]) for e in evs]
    carry_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    avg_call_s = float(np.mean(call_ms)) / 1e3
    prep_s, carry_s = float(np.mean(prep_ms)) / 1e3, float(np.mean(carry_ms)) / 1e3
    pbytes, pflops = prefill_algorithmic(T, B, 16, 32, 128)
    cflops = carry_algorithmic(T, 32, 128)
    prbytes = prep_bytes(T, B, 16, 32, 128)
    print(f"[bench] prefill: {ms_step:.3f} ms/step wall, {avg_call_s * 1e3:.3f} ms/call, "
          f"prep_kernel {prep_s * 1e6:.1f} us, carry_kernel {carry_s * 1e6:.1f} us (events)",
          file=sys.stderr, flush=True)

    result = {
        "metric": "GDN prefill tokens/s (MFMA util); decode state-update HBM GB/s vs peak",
        "value": T / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked varlen prefill, 4 sequences x 4096 tokens, h_k=16, h_v=32, "
                               "d_k=d_v=128, bf16 q/k/v, fp32 g/beta/state/o, conv4+SiLU+L2, chunk 64",
                   "num_seqs": B, "seq_len": Tseq, "h_k": 16, "h_v": 32, "d": 128},
        # dominant kernel: the cross-chunk carry (dependent chain of matrix-core products)
        "roofline": {"bound": "mfma", "achieved": cflops / carry_s / 1e12, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": cflops / carry_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
                     "traffic": measured_traffic(CARRY_KERNEL), "kernel": CARRY_KERNEL,
                     "algorithmic_flops": cflops, "avg_launch_us": carry_s * 1e6},
        "kernels": {
            PREP_KERNEL: {"avg_launch_us": prep_s * 1e6, "bound": "hbm", "moved_bytes": prbytes,
                          "GB/s": prbytes / prep_s / 1e9, "frac": prbytes / prep_s / 1e9 / HBM_PEAK_GBS,
                          "traffic": measured_traffic(PREP_KERNEL)},
            CARRY_KERNEL: {"avg_launch_us": carry_s * 1e6, "bound": "mfma", "algorithmic_flops": cflops,
                           "TFLOP/s": cflops / carry_s / 1e12},
        },
        "call": {"avg_us": avg_call_s * 1e6, "algorithmic_bytes": pbytes, "GB/s": pbytes / avg_call_s / 1e9,
                 "hbm_frac": pbytes / avg_call_s / 1e9 / HBM_PEAK_GBS, "algorithmic_flops": pflops,
                 "TFLOP/s": pflops / avg_call_s / 1e12},
        "mfma_util": pflops / avg_call_s / (MFMA_F16_PEAK_TFLOPS * 1e12),
    }

    # The same workload with bf16 outputs (o rounded once, to nearest even)
    o16 = torch.empty((T, 32, 128), dtype=bf, device=dev)

    def step16(events=None):
        gdn.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, out=o16, final_state_out=fs,
                               conv_state_out=cso, workspace=ws, validate=False, events=events,
                               out_dtype=torch.bfloat16)

    for i in range(20):
        step16()
    torch.cuda.synchronize()
    for e in evs:
        step16(e)
    torch.cuda.synchronize()
    c16 = float(np.mean([e[0].elapsed_time(e[3]) for e in evs])) * 1e3
    b16, _ = prefill_algorithmic(T, B, 16, 32, 128, out_bytes=2)
    result["prefill_bf16_out"] = {"us_per_call": c16, "tokens_per_s": T / (c16 * 1e-6),
                                  "carry_kernel_us": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3,
                                  "algorithmic_bytes": b16, "GB/s": b16 / (c16 * 1e-6) / 1e9}
    print(f"[bench] prefill, bf16 o: {c16:.1f} us/call (events)", file=sys.stderr, flush=True)
    del o16

    if not args.no_decode:
        N = 256
        # Four pools in rotation: a pool comes back only after 1.5 GiB of other
        # state traffic, so no cache (256 MiB of last-level cache) holds it
        # between its steps, as in a model where every layer has its own pool.
        NPOOL = 4
        print(f"[bench] decode: 256 slots, {NPOOL} rotating 512 MiB pools", file=sys.stderr, flush=True)
        pools = [torch.from_numpy(state_pool(3, N, geom)).to(dev) for _ in range(1)]
        pools += [pools[0].clone() for _ in range(NPOOL - 1)]
        cpools = [torch.from_numpy(conv_state_pool(3, N, geom, "bf16")).to(dev, bf) for _ in range(1)]
        cpools += [cpools[0].clone() for _ in range(NPOOL - 1)]
        cw = torch.from_numpy(conv_weights(3, geom, "bf16")).to(dev, bf)
        nsteps = args.decode_steps
        dins = []
        for s in range(nsteps):
            d = decode_inputs(3, s, N, geom, "bf16")
            dins.append(tuple(torch.from_numpy(a).to(dev, dt) for a, dt in
                              ((d.q, bf), (d.k, bf), (d.v, bf), (d.g, torch.float32), (d.beta, torch.float32))))
        od = torch.empty((N, 32, 128), dtype=torch.float32, device=dev)

        def dstep(s):
            gdn.gdn_decode_step(*dins[s], pools[s % NPOOL], out=od, conv_weight=cw,
                                conv_state_pool=cpools[s % NPOOL], validate=False)

        for s in range(max(4 * NPOOL, 20)):
            dstep(s % nsteps)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(nsteps):
            dstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / nsteps
        dbytes, dflops = decode_algorithmic(N, 16, 32, 128)
        gbs = dbytes / (us * 1e-6) / 1e9
        result["decode"] = {"workload": "decode step, 256 slots x 32 value heads (16 key heads), d=128, "
                                        "bf16 q/k/v, conv4+SiLU+L2, fp32 512 MiB state pool in place, "
                                        f"{NPOOL} pools in rotation",
                            "steps": nsteps, "us_per_step": us, "GB/s": gbs,
                            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(DECODE_KERNEL),
                                         "kernel": DECODE_KERNEL,
                                         "algorithmic_bytes": dbytes}}
        print(f"[bench] decode: {us:.1f} us/step, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
        del pools, cpools, dins

        # Multi-token (speculative) decode: m = 4 tokens per slot in one call,
        # (a) keeping the state after every token in its own pool entry (2 GiB
        # pool of 4 entries per slot, for rollback), (b) only the final state,
        # in place.  Two pool sets in rotation (4 GiB of state traffic apart).
        m, NSET = 4, 2
        mins = []
        for c in range(8):
            d = multi_decode_inputs(3, c, N, m, geom, "bf16")
            mins.append(tuple(torch.from_numpy(a).to(dev, dt) for a, dt in
                              ((d.q, bf), (d.k, bf), (d.v, bf), (d.g, torch.float32), (d.beta, torch.float32))))
        om = torch.empty((N, m, 32, 128), dtype=torch.float32, device=dev)
        start = torch.from_numpy(state_pool(3, N, geom)).to(dev)
        cstart = torch.from_numpy(conv_state_pool(3, N, geom, "bf16")).to(dev, bf)
        idx = torch.arange(N * m, dtype=torch.int32, device=dev).reshape(N, m)
        mres = {"workload": f"{m} tokens per slot, 256 slots x 32 value heads (16 key heads), d=128, bf16 "
                            "q/k/v, conv4+SiLU+L2, fp32 state", "tokens_per_slot": m}
        for kept, name in ((m, "all_token_states_kept"), (1, "final_state_in_place")):
            P = N * m if kept == m else N
            mpools = [torch.zeros((P, 32, 128, 128), dtype=torch.float32, device=dev) for _ in range(NSET)]
            mcpools = [torch.zeros((P, geom.channels, 3), dtype=bf, device=dev) for _ in range(NSET)]
            for mp, mc in zip(mpools, mcpools):
                mp[idx[:, 0].long() if kept == m else slice(None)] = start
                mc[idx[:, 0].long() if kept == m else slice(None)] = cstart

            def mstep(c):
                gdn.gdn_decode_multi(*mins[c % len(mins)], mpools[c % NSET], out=om, conv_weight=cw,
                                     conv_state_pool=mcpools[c % NSET], state_indices=idx if kept == m else None,
                                     validate=False)

            for c in range(8):
                mstep(c)
            torch.cuda.synchronize()
            calls = 40
            e0.record(stream)
            for c in range(calls):
                mstep(c)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / calls
            mb = decode_multi_algorithmic(N, m, 16, 32, 128, kept)
            tkey = "decode_kernel_m4_all_states" if kept == m else "decode_kernel_m4_final_state"
            mres[name] = {"us_per_call": us, "tokens_per_s": N * m / (us * 1e-6), "algorithmic_bytes": mb,
                          "GB/s": mb / (us * 1e-6) / 1e9, "frac": mb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "traffic": measured_traffic(tkey)}
            print(f"[bench] decode x{m} ({name}): {us:.1f} us/call, {mb / (us * 1e-6) / 1e9:.0f} GB/s",
                  file=sys.stderr, flush=True)
            del mpools, mcpools
        result["decode_multi"] = mres

    if not args.no_extra_configs:
        extra = {}
        lens = uniform_lengths(2, 60, 1, 8192)
        print(f"[bench] packed varlen: 60 sequences, {int(lens.sum())} tokens, h_k=16 h_v=48", file=sys.stderr,
              flush=True)
        us, tps, pr, ca = extra_prefill(gdn, torch, dev, lens, 16, 48, 128, 0.02, 5, 2)
        extra["packed_varlen_60seq_hk16_hv48"] = {
            "workload": f"60 sequences, lengths uniform 1..8192 (seeded, {int(lens.sum())} tokens), h_k=16, "
                        "h_v=48, d=128, bf16 q/k/v, fp32 initial states 0.02 N(0,1), conv4+SiLU+L2",
            "us_per_call": us, "tokens_per_s": tps, "prep_kernel_us": pr, "carry_kernel_us": ca}
        print(f"[bench] packed varlen: {us:.0f} us/call, {tps / 1e6:.1f} M tokens/s", file=sys.stderr, flush=True)
        us, tps, pr, ca = extra_prefill(gdn, torch, dev, [32768], 16, 32, 128, 0.0, 5, 4)
        extra["single_sequence_32768_hk16_hv32"] = {
            "workload": "one sequence of 32768 tokens, h_k=16, h_v=32, d=128, bf16 q/k/v, zero initial state, "
                        "conv4+SiLU+L2 (a chain of 512 chunks)",
            "us_per_call": us, "tokens_per_s": tps, "prep_kernel_us": pr, "carry_kernel_us": ca}
        print(f"[bench] 32768-token sequence: {us:.0f} us/call, {tps / 1e6:.1f} M tokens/s", file=sys.stderr,
              flush=True)
        result["other_prefill_configs"] = extra

    if (args.copy_calibration or not args.no_decode) and not args.no_copy_calibration:
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        copy_gbs = 2 * nbytes / (us * 1e-6) / 1e9
        result["copy_calibration"] = {"bytes_read": nbytes, "bytes_written": nbytes, "us_per_copy": us,
                                      "GB/s": copy_gbs}
        # the decode legs against the measured copy as well as the datasheet peak
        if "decode" in result:
            result["decode"]["roofline"]["frac_of_measured_copy"] = result["decode"]["GB/s"] / copy_gbs
        for leg in result.get("decode_multi", {}).values():
            if isinstance(leg, dict):
                leg["frac_of_measured_copy"] = leg["GB/s"] / copy_gbs
        print(f"[bench] copy 1 GiB: {us:.1f} us, {2 * nbytes / (us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
        del src, dst

    if not args.no_cpu_baseline:
        n = len(os.sched_getaffinity(0))
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
        print(f"[bench] cpu baseline: fp64 oracle on {n} threads", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, n)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
