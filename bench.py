"""Benchmark of the GDN hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A timed step is one chunked varlen prefill of the 4 x 4096-token workload
(h_k = 16, h_v = 32, d = 128, bf16 q/k/v, fp32 g/beta/state/output, width-4
conv + SiLU + q/k L2 norm, final recurrent and conv states written), inputs
resident in HBM.  `value` is prefill tokens/s over the K timed steps.

Before the W warm-up steps the GPU is brought to its steady clocks by a fixed
stretch of untimed prefill calls (reported as "device_warmup"): without it the
first ~100 back-to-back calls run measurably slower.

Rooflines follow one rule: a kernel's (or a call's) floor is
max(algorithmic flops / matrix-core peak, algorithmic bytes / HBM peak), and
`frac` = floor / measured time against the roof that binds.  Algorithmic bytes
count each input read once and each output and final state written once, no
workspace; they are split between the two prefill kernels by who reads or
writes them (chunk-local kernel: q, k, g, beta; carry kernel: v, o, final
recurrent and conv states, initial states).  The library records HIP events on
its launch stream around each kernel (gdn_prefill_varlen_timed), so kernel
times are measured live; the events are created without the system-scope
fence (timing only), whose cache writeback at every record slowed each step.  `roofline` is the dominant kernel, the cross-chunk
carry; `call` is the whole prefill.  A plain streaming device copy (the
library's gdn_stream_copy) gives a measured HBM peak beside the datasheet's.

Other legs: the same prefill with bf16 outputs; the decode step (256 slots x 32
value heads, d = 128, conv update, 512 MiB fp32 state pool in place, 100
consecutive steps over 4 pools in rotation) and the 4-token decode; the packed
varlen batch (60 sequences, h_v = 48) and a 32768-token sequence; the fp64
oracle on the host cores (all threads and one, plus the decode step).  One
JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
PREP_KERNEL = "prep_kernel"
CARRY_KERNEL = "carry_kernel"
DECODE_KERNEL = "decode_kernel"
CHUNK = 64


class TimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence:
    recording it does no system-scope cache writeback and invalidation, which
    with default events (torch's) cost ~10 us per step and slowed the kernel
    after each record.  Results are read only after a full device
    synchronisation.  The HIP runtime is the instance already mapped in the
    process (the one torch and the library use).  `cuda_event` is the raw
    handle the library's timed entry point records."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        h = ctypes.c_void_p()
        err = self._runtime().hipEventCreateWithFlags(ctypes.byref(h), 0x20000000)  # hipEventDisableSystemFence
        if err != 0 or not h.value:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")
        self.cuda_event = h.value

    def record(self, stream):
        import ctypes
        err = self._runtime().hipEventRecord(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(stream.cuda_stream))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and completed)."""
        import ctypes
        ms = ctypes.c_float()
        err = self._runtime().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                  ctypes.c_void_p(end.cuda_event))
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return ms.value


def roofline(nbytes, flops, seconds, kernel=None):
    """The binding roof of work (bytes, flops) done in `seconds`."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    r = {"bound": "hbm" if t_hbm >= t_mfma else "mfma"}
    if r["bound"] == "hbm":
        r.update(achieved=nbytes / seconds / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        r.update(achieved=flops / seconds / 1e12, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s")
    r["frac"] = r["achieved"] / r["peak"]
    r.update(algorithmic_bytes=nbytes, algorithmic_flops=flops, floor_us=max(t_hbm, t_mfma) * 1e6,
             avg_us=seconds * 1e6, mfma_frac=flops / seconds / 1e12 / MFMA_BF16_PEAK_TFLOPS)
    if kernel:
        r["kernel"] = kernel
    return r


def prefill_work(lengths, h_k, h_v, d, in_bytes=2, out_bytes=4, initial_states=False, conv_state_out=True):
    """Algorithmic (bytes, flops) of one prefill call, split into the
    chunk-local kernel's and the carry kernel's shares.

    Flops per (token, value head): the Gram products K K^T and Q K^T shared by
    the G value heads of a key head (2 chunk d each), A, P (chunk d each per
    value head, folded into the (4/G + 6) chunk d of the textbook count), and
    the state-side work of the carry: three d x d products (K H, Q H and the
    update, 2 d^2 each) and T R, P D (2 (chunk + 1) d: lower-triangular 64 x 64
    products).  Total (4/G + 6) chunk d + 6 d^2."""
    lengths = np.asarray(lengths, dtype=np.int64)
    T, N = int(lengths.sum()), len(lengths)
    G = h_v // h_k
    C = 2 * h_k * d + h_v * d
    state = N * h_v * d * d * 4
    prep_b = T * (2 * h_k * d * in_bytes + 2 * h_v * 4)
    carry_b = T * (h_v * d * in_bytes + h_v * d * out_bytes) + state + C * 4 * in_bytes + (N + 1) * 4
    if initial_states:
        carry_b += state
    if conv_state_out:
        carry_b += N * C * 3 * in_bytes
    total_f = T * h_v * ((4.0 / G + 6.0) * CHUNK * d + 6.0 * d * d)
    carry_f = T * h_v * (6.0 * d * d + 2.0 * (CHUNK + 1) * d)
    return {"prep": (prep_b, total_f - carry_f), "carry": (carry_b, carry_f), "call": (prep_b + carry_b, total_f)}


def decode_algorithmic(N, h_k, h_v, d, in_bytes=2, out_bytes=4, conv=True, d_v=None):
    """State read + write, q/k/v/g/beta read, o written, and with the conv
    prologue the conv history read + written and the conv weights read;
    ~ 7 d_k d_v flops per (slot, head).  d is d_k; d_v defaults to it."""
    dv = d if d_v is None else d_v
    state = N * h_v * d * dv * 4
    C = 2 * h_k * d + h_v * dv
    bytes_ = 2 * state + N * C * in_bytes + N * h_v * 2 * 4 + N * h_v * dv * out_bytes
    if conv:
        bytes_ += 2 * N * C * 3 * in_bytes + C * 4 * in_bytes
    return bytes_, N * h_v * 7.0 * d * dv


def decode_multi_algorithmic(N, m, h_k, h_v, d, kept, in_bytes=2, out_bytes=4, d_v=None):
    """m tokens per slot: the state read once and written `kept` times (once
    per kept token state), per-token q/k/v/g/beta read and o written, the
    conv history read once and written `kept` times, conv weights read.  d is
    d_k; d_v defaults to it."""
    dv = d if d_v is None else d_v
    state = N * h_v * d * dv * 4
    C = 2 * h_k * d + h_v * dv
    return (state * (1 + kept) + N * m * (C * in_bytes + h_v * 2 * 4 + h_v * dv * out_bytes)
            + N * C * 3 * in_bytes * (1 + kept) + C * 4 * in_bytes)


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


def extra_prefill(gdn, torch, dev, lengths, h_k, h_v, d, init_std, steps, seed, segment_chunks=0):
    """Prefill at another geometry, inputs drawn on the GPU with the
    distributions of the seeded workloads (q, k, v ~ N(0, 1) in bf16, conv taps
    0.5 N(0, 1), beta = sigmoid(N(0, 1)), g = -softplus(N(0, 1)), initial
    states init_std N(0, 1)); mean event times over `steps` calls."""
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
    prob = gdn.binding.make_problem(N, T, h_k, h_v, d, d, gdn.GDN_BF16, gdn.GDN_F32, segment_chunks=segment_chunks)
    ws = torch.empty(gdn.binding.gdn_prefill_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    evs = [[TimingEvent() for _ in range(4)] for _ in range(steps)]

    def call(e=None):
        gdn.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, initial_state=h0, out=o, final_state_out=fs,
                               output_conv_state=False, workspace=ws, validate=False, events=e,
                               segment_chunks=segment_chunks)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    us = float(np.mean([e[0].elapsed_time(e[3]) for e in evs])) * 1e3
    prep = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    carry = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
    work = prefill_work(lengths, h_k, h_v, d, initial_states=init_std is not None and init_std > 0,
                        conv_state_out=False)
    r = {"us_per_call": us, "tokens_per_s": T / (us * 1e-6), "prep_kernel_us": prep, "carry_kernel_us": carry,
         "roofline": roofline(*work["call"], us * 1e-6),
         "carry_roofline": roofline(*work["carry"], carry * 1e-6, CARRY_KERNEL)}
    if segment_chunks:
        r["segment_chunks"] = segment_chunks
        r["combine_and_correct_us"] = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e3
    return r


def stream_copy_peak(gdn, torch, dev, stream):
    """Best read + write bandwidth of the library's streaming copy of 1 GiB
    over a few grid sizes (the measured HBM peak)."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    e0, e1 = TimingEvent(), TimingEvent()
    best = None
    for per_cu in (2, 4, 8, 16):
        blocks = per_cu * cus
        for _ in range(3):
            gdn.binding.gdn_stream_copy(dst, src, blocks)
        torch.cuda.synchronize()
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            gdn.binding.gdn_stream_copy(dst, src, blocks)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = 2 * nbytes / (us * 1e-6) / 1e9
        if best is None or gbs > best["GB/s"]:
            best = {"bytes_read": nbytes, "bytes_written": nbytes, "us_per_copy": us, "GB/s": gbs,
                    "workgroups": blocks, "kernel": "stream_copy_kernel (16-byte nontemporal loads and stores)"}
    assert bool((dst == 1.0).all()), "stream copy produced wrong data"
    del src, dst
    return best


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo, no child process)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baselines(x, geom, nthreads):
    """The fp64 oracle on the host cores: the whole prefill workload on every
    thread, one of its sequences on one thread, and two decode steps of the
    256-slot workload on every thread (wall clock; bounded samples)."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle
    from gateddeltanet_chunked_delta_amd.inputs import conv_state_pool, conv_weights, decode_inputs, state_pool
    oracle.build(force=False)
    dims = oracle.Dims(geom.h_k, geom.h_v, geom.d_k, geom.d_v, conv_width=4)
    t0 = time.perf_counter()
    oracle.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, nthreads=nthreads)
    dt = time.perf_counter() - t0
    L = int(x.cu_seqlens[1])
    t0 = time.perf_counter()
    oracle.prefill(dims, x.cu_seqlens[:2], x.q[:L], x.k[:L], x.v[:L], x.g[:L], x.beta[:L], x.conv_w, nthreads=1)
    dt1 = time.perf_counter() - t0
    N, steps = 256, 2
    pool = state_pool(3, N, geom).astype(np.float64)
    cpool = conv_state_pool(3, N, geom, "bf16").astype(np.float64)
    cw = conv_weights(3, geom, "bf16")
    ins = [decode_inputs(3, s, N, geom, "bf16") for s in range(steps)]
    idx = np.arange(N)
    t0 = time.perf_counter()
    for d in ins:
        oracle.decode(dims, d.q, d.k, d.v, d.g, d.beta, pool, idx, cw, None, cpool, nthreads=nthreads)
    ddt = (time.perf_counter() - t0) / steps
    dbytes, _ = decode_algorithmic(N, geom.h_k, geom.h_v, geom.d_k)
    return {"value": x.total_tokens / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"whole prefill workload ({x.num_seqs} x {L} tokens, all heads, conv + SiLU + L2), fp64, "
                      f"one run of {dt:.2f} s on {nthreads} threads",
            "cpu_model": cpu_model(),
            "one_core": {"value": L / dt1, "unit": "tokens/s", "cores": 1,
                         "sample": f"one sequence of {L} tokens, all heads, one run of {dt1:.2f} s"},
            "decode": {"value": dbytes / ddt / 1e9, "unit": "GB/s", "cores": nthreads,
                       "sample": f"{steps} decode steps of 256 slots x 32 value heads with the conv update, fp64 "
                                 f"state, {ddt * 1e3:.1f} ms per step; GB/s of the GPU step's algorithmic bytes "
                                 "(fp32 state) so the two rates compare"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--device-warmup-ms", type=float, default=400.0,
                    help="untimed prefill calls before the warm-up steps, until this much wall time has passed "
                         "(brings the GPU to its steady clocks)")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the other prefill geometries (packed varlen batch, long single sequence)")
    ap.add_argument("--no-copy-peak", action="store_true", help="skip the streaming-copy HBM reference")
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

    # HIP events recorded by the library on its stream around each stage:
    # [before prep_kernel, before carry_kernel, after it, after the last launch]
    evs = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    print("[bench] device warm-up", file=sys.stderr, flush=True)
    dw_calls, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.device_warmup_ms:
        for _ in range(10):
            step()
        dw_calls += 10
        torch.cuda.synchronize()
    dw_ms = (time.perf_counter() - t0) * 1e3
    print(f"[bench] warmup ({args.warmup} steps)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(evs[i % args.steps])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_us = [e[0].elapsed_time(e[3]) * 1e3 for e in evs]
    prep_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    carry_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    call_s, prep_s, carry_s = (float(np.mean(x)) / 1e6 for x in (call_us, prep_us, carry_us))
    ms_step = wall * 1e3 / args.steps
    work = prefill_work([Tseq] * B, 16, 32, 128)
    print(f"[bench] prefill: {ms_step:.3f} ms/step wall, {call_s * 1e3:.3f} ms/call, "
          f"prep_kernel {prep_s * 1e6:.1f} us, carry_kernel {carry_s * 1e6:.1f} us (events)",
          file=sys.stderr, flush=True)

    carry_roof = roofline(*work["carry"], carry_s, CARRY_KERNEL)
    carry_roof["traffic"] = measured_traffic(CARRY_KERNEL)
    prep_roof = roofline(*work["prep"], prep_s, PREP_KERNEL)
    prep_roof["traffic"] = measured_traffic(PREP_KERNEL)
    call_roof = roofline(*work["call"], call_s)
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
        "device_warmup": {"calls": dw_calls, "ms": dw_ms,
                          "note": "untimed prefill calls before the warm-up steps, to reach steady GPU clocks"},
        "roofline": carry_roof,
        "kernels": {PREP_KERNEL: prep_roof, CARRY_KERNEL: carry_roof},
        "call": call_roof,
        "mfma_util": call_roof["mfma_frac"],
        # per-call HIP event times over the timed steps (the rooflines use the means)
        "event_stats_us": {name: {"mean": float(np.mean(x)), "median": float(np.median(x)),
                                  "min": float(np.min(x)), "max": float(np.max(x)), "n": len(x)}
                           for name, x in (("call", call_us), (PREP_KERNEL, prep_us), (CARRY_KERNEL, carry_us))},
    }

    # The same workload with bf16 outputs (o rounded once, to nearest even)
    o16 = torch.empty((T, 32, 128), dtype=bf, device=dev)

    def step16(events=None):
        gdn.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, out=o16, final_state_out=fs,
                               conv_state_out=cso, workspace=ws, validate=False, events=events,
                               out_dtype=torch.bfloat16)

    # the same clock warm-up as the fp32 leg (a fixed number of calls left the
    # clocks ramping after the host work between the legs)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < max(args.device_warmup_ms, 1.0):
        for _ in range(10):
            step16()
        torch.cuda.synchronize()
    for e in evs:
        step16(e)
    torch.cuda.synchronize()
    c16 = float(np.mean([e[0].elapsed_time(e[3]) for e in evs])) / 1e3
    w16 = prefill_work([Tseq] * B, 16, 32, 128, out_bytes=2)
    result["prefill_bf16_out"] = {"us_per_call": c16 * 1e6, "tokens_per_s": T / c16,
                                  "carry_kernel_us": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3,
                                  "roofline": roofline(*w16["call"], c16)}
    print(f"[bench] prefill, bf16 o: {c16 * 1e6:.1f} us/call (events)", file=sys.stderr, flush=True)
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
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        for s in range(nsteps):
            dstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / nsteps
        dbytes, dflops = decode_algorithmic(N, 16, 32, 128)
        droof = roofline(dbytes, dflops, us * 1e-6, DECODE_KERNEL)
        droof["traffic"] = measured_traffic(DECODE_KERNEL)
        result["decode"] = {"workload": "decode step, 256 slots x 32 value heads (16 key heads), d=128, "
                                        "bf16 q/k/v, conv4+SiLU+L2, fp32 512 MiB state pool in place, "
                                        f"{NPOOL} pools in rotation",
                            "steps": nsteps, "us_per_step": us, "GB/s": dbytes / (us * 1e-6) / 1e9,
                            "roofline": droof}
        print(f"[bench] decode: {us:.1f} us/step, {dbytes / (us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr,
              flush=True)
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
        oms = {torch.float32: torch.empty((N, m, 32, 128), dtype=torch.float32, device=dev),
               torch.bfloat16: torch.empty((N, m, 32, 128), dtype=bf, device=dev)}
        start = torch.from_numpy(state_pool(3, N, geom)).to(dev)
        cstart = torch.from_numpy(conv_state_pool(3, N, geom, "bf16")).to(dev, bf)
        idx = torch.arange(N * m, dtype=torch.int32, device=dev).reshape(N, m)
        mres = {"workload": f"{m} tokens per slot, 256 slots x 32 value heads (16 key heads), d=128, bf16 "
                            "q/k/v, conv4+SiLU+L2, fp32 state", "tokens_per_slot": m}
        for kept, name, odt in ((m, "all_token_states_kept", torch.float32),
                                (1, "final_state_in_place", torch.float32),
                                (1, "final_state_in_place_bf16_out", bf)):
            P = N * m if kept == m else N
            mpools = [torch.zeros((P, 32, 128, 128), dtype=torch.float32, device=dev) for _ in range(NSET)]
            mcpools = [torch.zeros((P, geom.channels, 3), dtype=bf, device=dev) for _ in range(NSET)]
            for mp, mc in zip(mpools, mcpools):
                mp[idx[:, 0].long() if kept == m else slice(None)] = start
                mc[idx[:, 0].long() if kept == m else slice(None)] = cstart

            def mstep(c):
                gdn.gdn_decode_multi(*mins[c % len(mins)], mpools[c % NSET], out=oms[odt], conv_weight=cw,
                                     conv_state_pool=mcpools[c % NSET], state_indices=idx if kept == m else None,
                                     validate=False, out_dtype=odt)

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
            mb = decode_multi_algorithmic(N, m, 16, 32, 128, kept, out_bytes=2 if odt == bf else 4)
            mres[name] = {"us_per_call": us, "tokens_per_s": N * m / (us * 1e-6),
                          "roofline": roofline(mb, N * m * 32 * 7.0 * 128 * 128, us * 1e-6, DECODE_KERNEL)}
            # counters were taken on the fp32-output instances only
            mres[name]["roofline"]["traffic"] = None if odt == bf else measured_traffic(
                "decode_kernel_m4_all_states" if kept == m else "decode_kernel_m4_final_state")
            print(f"[bench] decode x{m} ({name}): {us:.1f} us/call, {mb / (us * 1e-6) / 1e9:.0f} GB/s",
                  file=sys.stderr, flush=True)
            del mpools, mcpools
        result["decode_multi"] = mres

        # The other head dims: one step and a 4-token final-state call each
        # (256 slots, 16 key / 32 value heads, bf16 q/k/v, conv, fp32 o, two
        # pools in rotation)
        hres = {}
        for dk, dv in ((128, 64), (64, 128), (64, 64)):
            gm = Geometry(16, 32, dk, dv)
            hpools = [torch.from_numpy(state_pool(3, N, gm)).to(dev)]
            hpools.append(hpools[0].clone())
            hcpools = [torch.from_numpy(conv_state_pool(3, N, gm, "bf16")).to(dev, bf) for _ in range(2)]
            hcw = torch.from_numpy(conv_weights(3, gm, "bf16")).to(dev, bf)
            leg = {}
            for mm in (1, 4):
                hins = []
                for c in range(4):
                    d = decode_inputs(3, c, N, gm, "bf16") if mm == 1 else multi_decode_inputs(3, c, N, mm, gm, "bf16")
                    hins.append(tuple(torch.from_numpy(a).to(dev, dt) for a, dt in
                                      ((d.q, bf), (d.k, bf), (d.v, bf), (d.g, torch.float32), (d.beta, torch.float32))))
                ho = torch.empty(((N, 32, dv) if mm == 1 else (N, mm, 32, dv)), dtype=torch.float32, device=dev)
                call = gdn.gdn_decode_step if mm == 1 else gdn.gdn_decode_multi

                def hstep(c):
                    call(*hins[c % 4], hpools[c % 2], out=ho, conv_weight=hcw, conv_state_pool=hcpools[c % 2],
                         validate=False)

                for c in range(8):
                    hstep(c)
                torch.cuda.synchronize()
                calls = 40
                e0.record(stream)
                for c in range(calls):
                    hstep(c)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / calls
                if mm == 1:
                    hb, hf = decode_algorithmic(N, 16, 32, dk, d_v=dv)
                else:
                    hb = decode_multi_algorithmic(N, mm, 16, 32, dk, 1, d_v=dv)
                    hf = N * mm * 32 * 7.0 * dk * dv
                leg["step" if mm == 1 else f"x{mm}_final_state"] = {
                    "us_per_call": us, "roofline": roofline(hb, hf, us * 1e-6, DECODE_KERNEL)}
                leg["step" if mm == 1 else f"x{mm}_final_state"]["roofline"]["traffic"] = None
                print(f"[bench] decode d_k={dk} d_v={dv} m={mm}: {us:.1f} us/call, "
                      f"{hb / (us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
            hres[f"dk{dk}_dv{dv}"] = leg
            del hpools, hcpools
        result["decode_head_dims"] = hres

    if not args.no_extra_configs:
        extra = {}
        lens = uniform_lengths(2, 60, 1, 8192)
        print(f"[bench] packed varlen: 60 sequences, {int(lens.sum())} tokens, h_k=16 h_v=48", file=sys.stderr,
              flush=True)
        r = extra_prefill(gdn, torch, dev, lens, 16, 48, 128, 0.02, 5, 2)
        r["workload"] = (f"60 sequences, lengths uniform 1..8192 (seeded, {int(lens.sum())} tokens), h_k=16, "
                         "h_v=48, d=128, bf16 q/k/v, fp32 initial states 0.02 N(0,1), conv4+SiLU+L2")
        extra["packed_varlen_60seq_hk16_hv48"] = r
        print(f"[bench] packed varlen: {r['us_per_call']:.0f} us/call, {r['tokens_per_s'] / 1e6:.1f} M tokens/s",
              file=sys.stderr, flush=True)
        r = extra_prefill(gdn, torch, dev, [32768], 16, 32, 128, 0.0, 5, 4)
        r["workload"] = ("one sequence of 32768 tokens, h_k=16, h_v=32, d=128, bf16 q/k/v, zero initial state, "
                         "conv4+SiLU+L2 (a chain of 512 chunks)")
        extra["single_sequence_32768_hk16_hv32"] = r
        print(f"[bench] 32768-token sequence: {r['us_per_call']:.0f} us/call, "
              f"{r['tokens_per_s'] / 1e6:.1f} M tokens/s", file=sys.stderr, flush=True)
        r = extra_prefill(gdn, torch, dev, [32768], 16, 32, 128, 0.0, 5, 4, segment_chunks=256)
        r["workload"] = ("the same 32768-token sequence with the segment split (segment_chunks = 256: two "
                         "segments of 256 chunks run in parallel, then combined and corrected)")
        extra["single_sequence_32768_hk16_hv32_split256"] = r
        print(f"[bench] 32768-token sequence, split: {r['us_per_call']:.0f} us/call (carry {r['carry_kernel_us']:.0f},"
              f" combine+correct {r['combine_and_correct_us']:.0f}), {r['tokens_per_s'] / 1e6:.1f} M tokens/s",
              file=sys.stderr, flush=True)
        result["other_prefill_configs"] = extra

    if not args.no_copy_peak:
        peak = stream_copy_peak(gdn, torch, dev, stream)
        result["measured_hbm_peak"] = peak
        mp = peak["GB/s"]
        # fractions of every HBM-bound figure against the measured peak too
        for r in [result["roofline"], result["kernels"][PREP_KERNEL], result["call"],
                  result["prefill_bf16_out"]["roofline"]] + \
                ([result["decode"]["roofline"]] if "decode" in result else []) + \
                [leg["roofline"] for leg in result.get("decode_multi", {}).values() if isinstance(leg, dict)] + \
                [c["roofline"] for leg in result.get("decode_head_dims", {}).values() for c in leg.values()] + \
                [leg[key] for leg in result.get("other_prefill_configs", {}).values()
                 for key in ("roofline", "carry_roofline")]:
            if r["bound"] == "hbm":
                r["frac_of_measured_peak"] = r["achieved"] / mp
        print(f"[bench] stream copy 1 GiB: {peak['us_per_copy']:.1f} us, {mp:.0f} GB/s "
              f"({peak['workgroups']} workgroups)", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        n = len(os.sched_getaffinity(0))
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
        print(f"[bench] cpu baseline: fp64 oracle on {n} threads and on 1", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baselines(x, geom, n)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
