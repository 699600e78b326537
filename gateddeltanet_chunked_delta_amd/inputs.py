"""Seeded synthetic inputs for the GDN layer core.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  The same draws feed the GPU library and the fp64 oracle.

Recipe (one numpy ``Generator(PCG64)`` per sequence, keyed by
``(workload_id, seq_id)``, so a sequence's values do not depend on what else
is in the batch):
  * raw q|k|v channels ``x [len, C]`` ~ N(0, 1), ``C = 2 h_k d_k + h_v d_v``;
  * ``b_raw [len, h_v]`` ~ N(0, 1) then ``a_raw [len, h_v]`` ~ N(0, 1);
  * ``beta = sigmoid(b_raw)``, ``g = -softplus(a_raw)`` (fp64, stored fp32);
  * conv weights ``[C, 4]`` = 0.5 * N(0, 1) from key ``(workload_id, 1000)``;
  * initial states 0.02 * N(0, 1) per sequence from ``(workload_id, seq_id, 7)``.
bf16 inputs are the fp32 draws rounded to nearest-even; the values handed to
both sides are identical (an fp32 array holding exactly representable bf16
values plus its bf16 bit pattern).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


def _workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n)), 16))


@dataclass(frozen=True)
class Geometry:
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_width: int = 4

    @property
    def channels(self) -> int:
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v


def _bf16_round_inplace(x: np.ndarray, block: int = 1 << 18) -> np.ndarray:
    """Round a contiguous fp32 array to bf16 values (ties to even) in place, in
    cache-sized blocks."""
    u = x.reshape(-1).view(np.uint32)
    lsb = np.empty(min(block, u.size), dtype=np.uint32)
    for i in range(0, u.size, block):
        b = u[i:i + block]
        if not np.all(np.isfinite(b.view(np.float32))):
            raise ValueError("bf16_round expects finite values")
        t = lsb[:b.size]
        np.right_shift(b, 16, out=t)
        np.bitwise_and(t, np.uint32(1), out=t)
        b += np.uint32(0x7FFF)  # no wrap: finite fp32 bit patterns stay below 0xFF800000
        b += t
        b &= np.uint32(0xFFFF0000)
    return x


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    return _bf16_round_inplace(np.array(x, dtype=np.float32, order="C", copy=True))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def sequence_draw(workload_id: int, seq_id: int, length: int, geom: Geometry, dtype: str):
    """Raw channels, g and beta of one sequence: (x [len, C] f32, g, beta [len, h_v] f32)."""
    r = _rng(workload_id, seq_id)
    x = r.standard_normal((length, geom.channels), dtype=np.float32)
    b_raw = r.standard_normal((length, geom.h_v))
    a_raw = r.standard_normal((length, geom.h_v))
    if dtype == "bf16":
        x = _bf16_round_inplace(x)
    beta = _sigmoid(b_raw).astype(np.float32)
    g = (-_softplus(a_raw)).astype(np.float32)
    return x, g, beta


def conv_weights(workload_id: int, geom: Geometry, dtype: str) -> np.ndarray:
    w = (0.5 * _rng(workload_id, 1000).standard_normal((geom.channels, geom.conv_width))).astype(np.float32)
    return bf16_round(w) if dtype == "bf16" else w


def conv_bias(workload_id: int, geom: Geometry, dtype: str) -> np.ndarray:
    """Conv bias [C] = 0.5 * N(0, 1) from key (workload_id, 1001)."""
    b = (0.5 * _rng(workload_id, 1001).standard_normal(geom.channels)).astype(np.float32)
    return bf16_round(b) if dtype == "bf16" else b


def gate_logits(workload_id: int, rows: int, h_v: int) -> np.ndarray:
    """Raw write-strength gates b [rows, h_v] = 2 N(0, 1) (fp32), key (workload_id, 1002)."""
    return (2.0 * _rng(workload_id, 1002).standard_normal((rows, h_v))).astype(np.float32)


def state_draw(workload_id: int, seq_id: int, geom: Geometry, std: float = 0.02) -> np.ndarray:
    r = _rng(workload_id, seq_id, 7)
    return (std * r.standard_normal((geom.h_v, geom.d_k, geom.d_v))).astype(np.float32)


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n sequence lengths drawn uniformly from lo..hi inclusive."""
    return _rng(seed, 99).integers(lo, hi + 1, size=n).astype(np.int64)


@dataclass
class PrefillInputs:
    geom: Geometry
    dtype: str                  # "bf16" or "f32": dtype of q, k, v and conv weights
    cu_seqlens: np.ndarray      # int64 [N+1]
    q: np.ndarray               # f32 [T, h_k, d_k] (values exact in dtype)
    k: np.ndarray               # f32 [T, h_k, d_k]
    v: np.ndarray               # f32 [T, h_v, d_v]
    g: np.ndarray               # f32 [T, h_v]
    beta: np.ndarray            # f32 [T, h_v]
    conv_w: np.ndarray | None   # [C, W] (values exact in dtype) or None
    initial_state: np.ndarray | None  # f32 [N, h_v, d_k, d_v] or None
    conv_state_in: np.ndarray | None  # [N, C, W-1] (values exact in dtype) or None

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def prefill_inputs(workload_id: int, lengths, geom: Geometry, dtype: str, *,
                   seq_ids=None, conv: bool = True, initial_state_std: float | None = None,
                   conv_state: bool = False) -> PrefillInputs:
    """Packed varlen prefill inputs for sequences ``seq_ids`` (default 0..N-1)."""
    lengths = [int(x) for x in lengths]
    if seq_ids is None:
        seq_ids = list(range(len(lengths)))
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    nq, nv = geom.h_k * geom.d_k, geom.h_v * geom.d_v
    q = np.empty((T, geom.h_k, geom.d_k), np.float32)
    k = np.empty((T, geom.h_k, geom.d_k), np.float32)
    v = np.empty((T, geom.h_v, geom.d_v), np.float32)
    g = np.empty((T, geom.h_v), np.float32)
    beta = np.empty((T, geom.h_v), np.float32)
    def fill(n):
        sid, L = seq_ids[n], lengths[n]
        x, gg, bb = sequence_draw(workload_id, sid, L, geom, dtype)
        s = slice(cu[n], cu[n + 1])
        q[s] = x[:, :nq].reshape(L, geom.h_k, geom.d_k)
        k[s] = x[:, nq:2 * nq].reshape(L, geom.h_k, geom.d_k)
        v[s] = x[:, 2 * nq:].reshape(L, geom.h_v, geom.d_v)
        g[s] = gg
        beta[s] = bb

    # Sequences are independent draws (one generator each), so they are
    # filled by a thread pool; numpy releases the GIL in these loops.
    workers = min(len(lengths), _workers())
    if workers > 1 and T * geom.channels > (1 << 22):
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(len(lengths))))
    else:
        for n in range(len(lengths)):
            fill(n)
    conv_w = conv_weights(workload_id, geom, dtype) if conv else None
    init = None
    if initial_state_std is not None:
        init = np.stack([state_draw(workload_id, sid, geom, initial_state_std) for sid in seq_ids]) \
            if len(seq_ids) else np.zeros((0, geom.h_v, geom.d_k, geom.d_v), np.float32)
    csi = None
    if conv_state:
        csi = np.stack([_rng(workload_id, sid, 11).standard_normal((geom.channels, geom.conv_width - 1),
                                                                   dtype=np.float32)
                        for sid in seq_ids])
        if dtype == "bf16":
            csi = bf16_round(csi)
    return PrefillInputs(geom, dtype, cu, q, k, v, g, beta, conv_w, init, csi)


@dataclass
class DecodeInputs:
    geom: Geometry
    dtype: str
    q: np.ndarray      # f32 [N, h_k, d_k]
    k: np.ndarray      # f32 [N, h_k, d_k]
    v: np.ndarray      # f32 [N, h_v, d_v]
    g: np.ndarray      # f32 [N, h_v]
    beta: np.ndarray   # f32 [N, h_v]


def decode_inputs(workload_id: int, step: int, n: int, geom: Geometry, dtype: str) -> DecodeInputs:
    """One decode step's inputs for n slots, seeded by (workload_id, step)."""
    r = _rng(workload_id, 1_000_000 + step)
    x = r.standard_normal((n, geom.channels), dtype=np.float32)
    b_raw = r.standard_normal((n, geom.h_v))
    a_raw = r.standard_normal((n, geom.h_v))
    if dtype == "bf16":
        x = bf16_round(x)
    nq = geom.h_k * geom.d_k
    return DecodeInputs(geom, dtype,
                        np.ascontiguousarray(x[:, :nq].reshape(n, geom.h_k, geom.d_k)),
                        np.ascontiguousarray(x[:, nq:2 * nq].reshape(n, geom.h_k, geom.d_k)),
                        np.ascontiguousarray(x[:, 2 * nq:].reshape(n, geom.h_v, geom.d_v)),
                        (-_softplus(a_raw)).astype(np.float32),
                        _sigmoid(b_raw).astype(np.float32))


def multi_decode_inputs(workload_id: int, call: int, n: int, m: int, geom: Geometry, dtype: str) -> DecodeInputs:
    """m tokens per slot for n slots (arrays [n, m, ...]); token j of call c is
    drawn like decode step 64 c + j, so a slot's tokens are the same whatever
    m-token calls they are issued in."""
    steps = [decode_inputs(workload_id, 64 * call + j, n, geom, dtype) for j in range(m)]
    stack = lambda f: np.ascontiguousarray(np.stack([getattr(s, f) for s in steps], axis=1))
    return DecodeInputs(geom, dtype, stack("q"), stack("k"), stack("v"), stack("g"), stack("beta"))


def state_pool(workload_id: int, pool: int, geom: Geometry, std: float = 0.02) -> np.ndarray:
    """fp32 state pool [pool, h_v, d_k, d_v] ~ std * N(0, 1)."""
    r = _rng(workload_id, 2_000_000)
    return (std * r.standard_normal((pool, geom.h_v, geom.d_k, geom.d_v), dtype=np.float32))


def conv_state_pool(workload_id: int, pool: int, geom: Geometry, dtype: str) -> np.ndarray:
    r = _rng(workload_id, 3_000_000)
    x = r.standard_normal((pool, geom.channels, geom.conv_width - 1), dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x
