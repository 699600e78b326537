"""fp64 CPU oracle for the GatedDeltaNet gated delta-rule -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product library never calls it and shares no
code with it.  The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64); this
module only builds that file with gcc and marshals numpy arrays through ctypes.

Array conventions (all numpy float64, C-contiguous, time-first, packed by
``cu_seqlens``): q, k ``[T, h_k, d_k]``; v ``[T, h_v, d_v]``; g, beta
``[T, h_v]``; o ``[T, h_v, d_v]``; states ``[N, h_v, d_k, d_v]`` (the stored
state is the transpose of the math state S); conv weight ``[C, W]``, bias
``[C]``, conv states ``[N, C, W-1]`` with ``C = 2 h_k d_k + h_v d_v``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c with gcc (fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
    return _lib


class _Dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int64), ("total_tokens", ctypes.c_int64),
                ("h_k", ctypes.c_int64), ("h_v", ctypes.c_int64),
                ("d_k", ctypes.c_int64), ("d_v", ctypes.c_int64),
                ("conv_width", ctypes.c_int64), ("qk_l2norm", ctypes.c_int64),
                ("l2_eps", ctypes.c_double), ("scale", ctypes.c_double)]


@dataclass
class Dims:
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_width: int = 4
    qk_l2norm: bool = True
    l2_eps: float = 1e-6
    scale: float | None = None  # None -> d_k ** -0.5

    @property
    def channels(self) -> int:
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v

    def c_struct(self, num_seqs: int, total_tokens: int) -> _Dims:
        s = self.d_k ** -0.5 if self.scale is None else self.scale
        return _Dims(num_seqs, total_tokens, self.h_k, self.h_v, self.d_k, self.d_v,
                     self.conv_width, int(bool(self.qk_l2norm)), self.l2_eps, s)


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def prologue(dims: Dims, cu_seqlens, q_raw, k_raw, v_raw, conv_w=None, conv_b=None,
             conv_state_in=None, want_conv_state=True, nthreads=0):
    """Conv1d + SiLU + per-head q/k L2 norm. Returns (q, k, v, conv_state_out)."""
    lib = _load()
    if dims.conv_width > 0 and conv_w is None:
        raise ValueError("conv_width > 0 needs conv_w")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N, T = len(cu) - 1, int(cu[-1])
    q_raw, k_raw, v_raw = _f64(q_raw), _f64(k_raw), _f64(v_raw)
    q = np.empty_like(q_raw); k = np.empty_like(k_raw); v = np.empty_like(v_raw)
    cso = None
    if want_conv_state and dims.conv_width > 1:
        cso = np.zeros((N, dims.channels, dims.conv_width - 1))
    d = dims.c_struct(N, T)
    lib.gdn_oracle_prologue(ctypes.byref(d), _p(cu), _p(q_raw), _p(k_raw), _p(v_raw),
                            _p(_f64(conv_w)), _p(_f64(conv_b)), _p(_f64(conv_state_in)), _p(cso),
                            _p(q), _p(k), _p(v), ctypes.c_int(nthreads))
    return q, k, v, cso


def recurrent(dims: Dims, cu_seqlens, q, k, v, g, beta, initial_state=None, nthreads=0):
    """Step-by-step recurrence on post-prologue q/k/v. Returns (o, final_state)."""
    lib = _load()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N, T = len(cu) - 1, int(cu[-1])
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    o = np.zeros((T, dims.h_v, dims.d_v))
    fs = np.zeros((N, dims.h_v, dims.d_k, dims.d_v))
    d = dims.c_struct(N, T)
    lib.gdn_oracle_recurrent(ctypes.byref(d), _p(cu), _p(q), _p(k), _p(v), _p(g), _p(beta),
                             _p(_f64(initial_state)), _p(o), _p(fs), ctypes.c_int(nthreads))
    return o, fs


def chunked(dims: Dims, cu_seqlens, q, k, v, g, beta, initial_state=None, chunk=64, nthreads=0):
    """Independent chunked (WY/UT) fp64 form. Returns (o, final_state)."""
    lib = _load()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N, T = len(cu) - 1, int(cu[-1])
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    o = np.zeros((T, dims.h_v, dims.d_v))
    fs = np.zeros((N, dims.h_v, dims.d_k, dims.d_v))
    d = dims.c_struct(N, T)
    lib.gdn_oracle_chunked(ctypes.byref(d), _p(cu), ctypes.c_int64(chunk), _p(q), _p(k), _p(v),
                           _p(g), _p(beta), _p(_f64(initial_state)), _p(o), _p(fs),
                           ctypes.c_int(nthreads))
    return o, fs


def prefill(dims: Dims, cu_seqlens, q_raw, k_raw, v_raw, g, beta, conv_w=None, conv_b=None,
            conv_state_in=None, initial_state=None, nthreads=0):
    """Whole prefill layer core: prologue then the sequential recurrence.

    Returns (o, final_state, conv_state_out)."""
    q, k, v, cso = prologue(dims, cu_seqlens, q_raw, k_raw, v_raw, conv_w, conv_b,
                            conv_state_in, nthreads=nthreads)
    o, fs = recurrent(dims, cu_seqlens, q, k, v, g, beta, initial_state, nthreads=nthreads)
    return o, fs, cso


def decode(dims: Dims, q_raw, k_raw, v_raw, g, beta, state_pool, state_indices=None,
           conv_w=None, conv_b=None, conv_state_pool=None, nthreads=0):
    """One decode step. ``state_pool`` and ``conv_state_pool`` are updated IN PLACE
    (float64 arrays).  Returns o ``[N, h_v, d_v]`` (rows of skipped slots are 0)."""
    lib = _load()
    if dims.conv_width > 0 and (conv_w is None or conv_state_pool is None):
        raise ValueError("conv_width > 0 needs conv_w and conv_state_pool")
    q_raw, k_raw, v_raw, g, beta = map(_f64, (q_raw, k_raw, v_raw, g, beta))
    N = q_raw.shape[0]
    assert state_pool.dtype == np.float64 and state_pool.flags["C_CONTIGUOUS"]
    if conv_state_pool is not None:
        assert conv_state_pool.dtype == np.float64 and conv_state_pool.flags["C_CONTIGUOUS"]
    idx = None if state_indices is None else np.ascontiguousarray(state_indices, dtype=np.int64)
    o = np.zeros((N, dims.h_v, dims.d_v))
    d = dims.c_struct(N, N)
    lib.gdn_oracle_decode(ctypes.byref(d), _p(q_raw), _p(k_raw), _p(v_raw), _p(g), _p(beta),
                          _p(_f64(conv_w)), _p(_f64(conv_b)), _p(conv_state_pool),
                          _p(state_pool), _p(idx), _p(o), ctypes.c_int(nthreads))
    return o


def decode_multi(dims: Dims, q_raw, k_raw, v_raw, g, beta, state_pool, state_indices=None,
                 num_accepted=None, conv_w=None, conv_b=None, conv_state_pool=None, nthreads=0):
    """m decode tokens per slot, in order (multi-token / speculative decode).

    The definition is m single-token decode steps per slot ("[Feature] Add
    batch invariance support to GDN_ATTN backend", commit messages: separate
    spec and non-spec decode over the state pool), with the pool bookkeeping
    of the library's m-token call: slot n starts from entry
    ``state_indices[n, num_accepted[n] - 1]`` (entry n without indices) and
    the state and conv history after token j are copied to entry
    ``state_indices[n, j]`` when it is >= 0 (entry n after the last token
    without indices); a start entry of -1 skips the slot.
    q_raw, k_raw ``[N, m, h_k, d_k]``; v_raw ``[N, m, h_v, d_v]``; g, beta
    ``[N, m, h_v]``.  Pools (float64) are updated IN PLACE.  Returns o
    ``[N, m, h_v, d_v]`` (rows of skipped slots are 0)."""
    q_raw, k_raw, v_raw, g, beta = map(_f64, (q_raw, k_raw, v_raw, g, beta))
    N, m = q_raw.shape[0], q_raw.shape[1]
    conv = dims.conv_width > 0
    acc = np.ones(N, dtype=np.int64) if num_accepted is None else np.asarray(num_accepted, dtype=np.int64)
    if state_indices is None:
        start = np.arange(N)
        dest = np.full((N, m), -1, dtype=np.int64)
        dest[:, m - 1] = np.arange(N)
    else:
        idx = np.asarray(state_indices, dtype=np.int64).reshape(N, m)
        start = idx[np.arange(N), acc - 1]
        dest = idx
    # the running state of every slot, gathered from its start entry
    live = start >= 0
    work = np.zeros((N,) + state_pool.shape[1:])
    work[live] = state_pool[start[live]]
    cwork = None
    if conv:
        cwork = np.zeros((N,) + conv_state_pool.shape[1:])
        cwork[live] = conv_state_pool[start[live]]
    sel = np.where(live, np.arange(N), -1)
    o = np.zeros((N, m, dims.h_v, dims.d_v))
    for j in range(m):
        o[:, j] = decode(dims, q_raw[:, j], k_raw[:, j], v_raw[:, j], g[:, j], beta[:, j], work, sel,
                         conv_w, conv_b, cwork, nthreads=nthreads)
        for n in range(N):
            if live[n] and dest[n, j] >= 0:
                state_pool[dest[n, j]] = work[n]
                if conv:
                    conv_state_pool[dest[n, j]] = cwork[n]
    return o
