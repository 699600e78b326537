"""ctypes binding of libgdn.so: argument checks and marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/gdn.h).  PyTorch supplies device memory and streams: the kernels go to
torch's current stream or a given torch.cuda.Stream, on which the call's
temporaries and default outputs are allocated too.
There is no fallback: if libgdn.so is missing or a call fails, this module
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
_STATUS = {0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_DTYPE",
           -4: "GDN_ERR_UNSUPPORTED", -5: "GDN_ERR_WORKSPACE", -6: "GDN_ERR_HIP", -7: "GDN_ERR_ALIAS",
           -8: "GDN_ERR_SCRATCH"}
EXPORTED = ("gdn_prefill_workspace_bytes", "gdn_prefill_varlen", "gdn_prefill_varlen_timed",
            "gdn_prefill_varlen_noalloc", "gdn_prefill_varlen_pooled", "gdn_decode_step", "gdn_decode_multi",
            "gdn_stream_copy", "gdn_status_string")
# Size of the static workspace behind gdn_prefill_varlen_noalloc (GDN_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 128 << 20


class GdnProblem(ctypes.Structure):
    """Mirror of gdn_problem in include/gdn.h."""
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("qk_l2norm", ctypes.c_int32),
                ("l2_eps", ctypes.c_float), ("conv_width", ctypes.c_int32),
                ("beta_logits", ctypes.c_int32), ("segment_chunks", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({status_string(status)})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads libgdn.so (built in-tree by build.py); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gateddeltanet_chunked_delta_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, c64 = ctypes.c_void_p, ctypes.c_size_t
        lib.gdn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(GdnProblem)]
        lib.gdn_prefill_workspace_bytes.restype = c64
        lib.gdn_prefill_varlen.argtypes = [ctypes.POINTER(GdnProblem)] + [vp] * 14 + [c64, vp]
        lib.gdn_prefill_varlen.restype = ctypes.c_int
        lib.gdn_prefill_varlen_timed.argtypes = [ctypes.POINTER(GdnProblem)] + [vp] * 14 + [c64, vp,
                                                                                           ctypes.POINTER(vp)]
        lib.gdn_prefill_varlen_timed.restype = ctypes.c_int
        lib.gdn_prefill_varlen_noalloc.argtypes = [ctypes.POINTER(GdnProblem)] + [vp] * 14
        lib.gdn_prefill_varlen_noalloc.restype = ctypes.c_int
        lib.gdn_prefill_varlen_pooled.argtypes = [ctypes.POINTER(GdnProblem)] + [vp] * 14 + [c64, vp]
        lib.gdn_prefill_varlen_pooled.restype = ctypes.c_int
        lib.gdn_decode_step.argtypes = [ctypes.POINTER(GdnProblem)] + [vp] * 11 + [vp]
        lib.gdn_decode_step.restype = ctypes.c_int
        lib.gdn_decode_multi.argtypes = [ctypes.POINTER(GdnProblem), ctypes.c_int32] + [vp] * 13
        lib.gdn_decode_multi.restype = ctypes.c_int
        lib.gdn_stream_copy.argtypes = [vp, vp, c64, ctypes.c_int32, vp]
        lib.gdn_stream_copy.restype = ctypes.c_int
        lib.gdn_status_string.argtypes = [ctypes.c_int]
        lib.gdn_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def _dtype_code(dt: torch.dtype, what: str) -> int:
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise ValueError(f"{what}: dtype {dt} not supported (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _resolve_stream(stream, dev):
    """The stream the kernels go to: torch's current stream of `dev`, or the
    given torch.cuda.Stream (a raw handle is refused: the temporaries of a
    call must be allocated on the stream that uses them)."""
    if stream is None:
        return torch.cuda.current_stream(dev)
    if not isinstance(stream, torch.cuda.Stream):
        raise ValueError("stream must be a torch.cuda.Stream (or None for the current stream)")
    if stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the inputs on {dev}")
    return stream


def _hold_for(s, dev, tensors):
    """On a stream other than the current one, mark every tensor the kernels
    use as in use by that stream, so that the caching allocator does not hand
    its memory to other work before the kernels are done with it."""
    if s != torch.cuda.current_stream(dev):
        for t in tensors:
            if isinstance(t, torch.Tensor) and t.is_cuda:
                t.record_stream(s)


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_problem(num_seqs, total_tokens, h_k, h_v, d_k, d_v, qkv_dtype, out_dtype, scale=None,
                 qk_l2norm=True, l2_eps=1e-6, conv_width=4, beta_logits=False, segment_chunks=0) -> GdnProblem:
    return GdnProblem(int(num_seqs), int(total_tokens), int(h_k), int(h_v), int(d_k), int(d_v),
                      int(qkv_dtype), int(out_dtype), float(0.0 if scale is None else scale),
                      int(bool(qk_l2norm)), float(l2_eps), int(conv_width), int(bool(beta_logits)),
                      int(segment_chunks))


def gdn_prefill_workspace_bytes(problem: GdnProblem) -> int:
    return int(load().gdn_prefill_workspace_bytes(ctypes.byref(problem)))


def _validate_cu(cu_host: torch.Tensor, T: int):
    if cu_host.numel() < 1 or int(cu_host[0]) != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if int(cu_host[-1]) != T:
        raise ValueError(f"cu_seqlens[-1] = {int(cu_host[-1])} != total tokens {T}")
    if bool((cu_host[1:] < cu_host[:-1]).any()):
        raise ValueError("cu_seqlens must be non-decreasing")


def gdn_prefill_varlen(q, k, v, g, beta, cu_seqlens=None, *, conv_weight=None, conv_bias=None,
                       conv_state=None, initial_state=None, output_final_state=True,
                       output_conv_state=True, use_qk_l2norm=True, scale=None, l2_eps=1e-6,
                       out_dtype=torch.float32, validate=True, out=None, final_state_out=None,
                       conv_state_out=None, workspace=None, stream=None, events=None, beta_logits=False,
                       noalloc=False, segment_chunks=0):
    """Chunked varlen prefill (C ABI ``gdn_prefill_varlen``).

    q, k: ``[T, h_k, d_k]`` (or ``[B, T, h_k, d_k]`` with equal lengths and no
    cu_seqlens); v: ``[T, h_v, d_v]``; g, beta: ``[T, h_v]`` fp32; cu_seqlens:
    int32 ``[N+1]`` on the device (or a CPU tensor / list, copied).  Returns
    ``(o, final_state or None, conv_state_out or None)``.  With ``events`` (four
    ``torch.cuda.Event(enable_timing=True)``, or objects holding a HIP event
    handle in ``cuda_event``) the call goes through ``gdn_prefill_varlen_timed``,
    which records them around its stages.
    ``segment_chunks > 0`` turns on the segment split of sequences longer than
    that many 64-token chunks (see ``gdn_problem.segment_chunks``).
    With ``noalloc=True`` the call goes through ``gdn_prefill_varlen_noalloc``
    (no workspace; the library's static scratch).  ``stream``: a
    ``torch.cuda.Stream`` or None (the current stream); temporaries and
    default outputs are allocated on it.
    """
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("with cu_seqlens, q/k/v must be packed [T, H, D] (no batch dimension)")
        B, Tb = q.shape[0], q.shape[1]
        q, k, v = q.reshape(B * Tb, *q.shape[2:]), k.reshape(B * Tb, *k.shape[2:]), v.reshape(B * Tb, *v.shape[2:])
        g, beta = g.reshape(B * Tb, -1), beta.reshape(B * Tb, -1)
        cu_seqlens = torch.arange(0, (B + 1) * Tb, Tb, dtype=torch.int32)
    if q.dim() != 3:
        raise ValueError("q must be [T, h_k, d_k] (time-first, packed)")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    s = _resolve_stream(stream, dev)
    T, h_k, d_k = q.shape
    if v.dim() != 3 or v.shape[0] != T:
        raise ValueError("v must be [T, h_v, d_v]")
    h_v, d_v = v.shape[1], v.shape[2]
    qdt = q.dtype
    qcode = _dtype_code(qdt, "q")
    ocode = _dtype_code(out_dtype, "out_dtype")
    _check(q, "q", (T, h_k, d_k), qdt, dev)
    _check(k, "k", (T, h_k, d_k), qdt, dev)
    _check(v, "v", (T, h_v, d_v), qdt, dev)
    _check(g, "g", (T, h_v), torch.float32, dev)
    _check(beta, "beta", (T, h_v), torch.float32, dev)
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32)
    if not isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = torch.tensor(list(cu_seqlens), dtype=torch.int32)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    if validate:
        _validate_cu(cu_seqlens.cpu(), T)
    with torch.cuda.stream(s):
        if cu_seqlens.device != dev:
            cu_seqlens = cu_seqlens.to(dev)
        cu_seqlens = cu_seqlens.contiguous()
    N = cu_seqlens.numel() - 1
    C = 2 * h_k * d_k + h_v * d_v
    conv_width = 4 if conv_weight is not None else 0
    if conv_weight is not None:
        _check(conv_weight, "conv_weight", (C, 4), qdt, dev)
        _check(conv_bias, "conv_bias", (C,), qdt, dev)
        _check(conv_state, "conv_state", (N, C, 3), qdt, dev)
    elif conv_bias is not None or conv_state is not None:
        raise ValueError("conv_bias/conv_state given without conv_weight")
    _check(initial_state, "initial_state", (N, h_v, d_k, d_v), torch.float32, dev)

    with torch.cuda.stream(s):
        o = out if out is not None else torch.empty((T, h_v, d_v), dtype=out_dtype, device=dev)
        fs = None
        if output_final_state:
            fs = final_state_out if final_state_out is not None else torch.empty((N, h_v, d_k, d_v), dtype=torch.float32, device=dev)
        cso = None
        if output_conv_state and conv_width:
            cso = conv_state_out if conv_state_out is not None else torch.empty((N, C, 3), dtype=qdt, device=dev)
    _check(o, "out", (T, h_v, d_v), out_dtype, dev)
    _check(fs, "final_state_out", (N, h_v, d_k, d_v), torch.float32, dev)
    _check(cso, "conv_state_out", (N, C, 3), qdt, dev)
    prob = make_problem(N, T, h_k, h_v, d_k, d_v, qcode, ocode, scale, use_qk_l2norm, l2_eps, conv_width,
                        beta_logits, segment_chunks)
    if noalloc:
        if workspace is not None or events is not None:
            raise ValueError("noalloc takes neither a workspace nor events")
        _hold_for(s, dev, (q, k, v, g, beta, cu_seqlens, conv_weight, conv_bias, conv_state, cso, initial_state,
                           o, fs))
        st = load().gdn_prefill_varlen_noalloc(
            ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
            _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(cso), _ptr(initial_state), _ptr(o),
            _ptr(fs), ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise GdnError(st, "gdn_prefill_varlen_noalloc")
        return o, fs, cso
    ws_bytes = gdn_prefill_workspace_bytes(prob)
    if workspace is None:
        with torch.cuda.stream(s):
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    _hold_for(s, dev, (q, k, v, g, beta, cu_seqlens, conv_weight, conv_bias, conv_state, cso, initial_state, o, fs,
                       workspace))
    args = (ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(cu_seqlens), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state),
            _ptr(cso), _ptr(initial_state), _ptr(o), _ptr(fs), _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(s.cuda_stream))
    if events is None:
        st = load().gdn_prefill_varlen(*args)
    else:
        if len(events) != 4:
            raise ValueError("events must be four torch.cuda.Event")
        handles = []
        for e in events:
            if e.cuda_event == 0:  # torch creates the event at its first record
                e.record()
            handles.append(e.cuda_event)
        arr = (ctypes.c_void_p * 4)(*handles)
        st = load().gdn_prefill_varlen_timed(*args, arr)
    if st != 0:
        raise GdnError(st, "gdn_prefill_varlen")
    return o, fs, cso



def gdn_prefill_varlen_noalloc(q, k, v, g, beta, cu_seqlens=None, **kw):
    """Chunked varlen prefill through the C ABI ``gdn_prefill_varlen_noalloc``:
    the same arguments and results as :func:`gdn_prefill_varlen` (no
    ``workspace`` or ``events``); the library uses its static scratch, so the
    C call allocates nothing (pass ``out``, ``final_state_out`` and
    ``conv_state_out`` to keep this wrapper from allocating outputs)."""
    return gdn_prefill_varlen(q, k, v, g, beta, cu_seqlens, noalloc=True, **kw)

def gdn_stream_copy(dst, src, blocks, stream=None):
    """Device copy of src into dst (same byte size) by the library's streaming
    copy kernel (C ABI ``gdn_stream_copy``), a bandwidth reference."""
    if dst.device != src.device or dst.device.type != "cuda":
        raise ValueError("dst and src must be on the same GPU")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("dst and src must be contiguous buffers of the same size")
    s = _resolve_stream(stream, src.device)
    _hold_for(s, src.device, (dst, src))
    st = load().gdn_stream_copy(_ptr(dst), _ptr(src), ctypes.c_size_t(nbytes), ctypes.c_int32(blocks),
                                ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_stream_copy")


def _check_indices(state_indices, N, P, Pc, dev, validate):
    """state_indices: int32 [N] on dev, each -1 or a distinct entry below P (and Pc)."""
    if state_indices is None:
        if validate and (N > P or (Pc is not None and N > Pc)):
            raise ValueError("without state_indices the pools need at least N entries")
        return
    _check(state_indices, "state_indices", (N,), torch.int32, dev)
    if validate and N:
        idx = state_indices.cpu()
        used = idx[idx >= 0]
        if bool((idx < -1).any()) or bool((used >= P).any()) or (Pc is not None and bool((used >= Pc).any())):
            raise ValueError("state_indices out of range")
        if used.numel() != torch.unique(used).numel():
            raise ValueError("state_indices must be distinct")


def gdn_prefill_varlen_pooled(q, k, v, g, beta, cu_seqlens, state_pool, *, state_indices=None,
                              has_initial_state=None, conv_weight=None, conv_bias=None, conv_state_pool=None,
                              use_qk_l2norm=True, scale=None, l2_eps=1e-6, out_dtype=torch.float32,
                              validate=True, out=None, workspace=None, stream=None, beta_logits=False,
                              segment_chunks=0):
    """Chunked varlen prefill over pooled states, in place (C ABI
    ``gdn_prefill_varlen_pooled``).

    q, k: ``[T, h_k, d_k]``; v: ``[T, h_v, d_v]``; g, beta: ``[T, h_v]`` fp32;
    cu_seqlens: int32 ``[N+1]`` (device, or CPU tensor / list, copied);
    state_pool: fp32 ``[P, h_v, d_k, d_v]``; conv_state_pool: ``[P, C, 3]``
    (with conv_weight); state_indices: int32 ``[N]`` or None (entry n), -1 =
    no entry; has_initial_state: int32 ``[N]`` or None (all 1).  Sequence n
    starts from entry state_indices[n] (zero if -1 or has_initial_state[n] = 0)
    and leaves its final states there.  Returns o.
    """
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be packed [T, H, D]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    T, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    qdt = q.dtype
    qcode = _dtype_code(qdt, "q")
    ocode = _dtype_code(out_dtype, "out_dtype")
    _check(q, "q", (T, h_k, d_k), qdt, dev)
    _check(k, "k", (T, h_k, d_k), qdt, dev)
    _check(v, "v", (T, h_v, d_v), qdt, dev)
    _check(g, "g", (T, h_v), torch.float32, dev)
    _check(beta, "beta", (T, h_v), torch.float32, dev)
    if not isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = torch.tensor(list(cu_seqlens), dtype=torch.int32)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    if validate:
        _validate_cu(cu_seqlens.cpu(), T)
    s = _resolve_stream(stream, dev)
    with torch.cuda.stream(s):
        cu_seqlens = cu_seqlens.to(dev).contiguous()
    N = cu_seqlens.numel() - 1
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [P, h_v, d_k, d_v]")
    P = state_pool.shape[0]
    _check(state_pool, "state_pool", (P, h_v, d_k, d_v), torch.float32, dev)
    C = 2 * h_k * d_k + h_v * d_v
    conv_width = 4 if conv_weight is not None else 0
    Pc = None
    if conv_weight is not None:
        _check(conv_weight, "conv_weight", (C, 4), qdt, dev)
        _check(conv_bias, "conv_bias", (C,), qdt, dev)
        if conv_state_pool is None or conv_state_pool.dim() != 3:
            raise ValueError("conv_weight needs conv_state_pool [P, C, 3]")
        Pc = conv_state_pool.shape[0]
        _check(conv_state_pool, "conv_state_pool", (Pc, C, 3), qdt, dev)
    elif conv_bias is not None or conv_state_pool is not None:
        raise ValueError("conv_bias/conv_state_pool given without conv_weight")
    _check_indices(state_indices, N, P, Pc, dev, validate)
    if has_initial_state is not None:
        _check(has_initial_state, "has_initial_state", (N,), torch.int32, dev)
    with torch.cuda.stream(s):
        o = out if out is not None else torch.empty((T, h_v, d_v), dtype=out_dtype, device=dev)
    _check(o, "out", (T, h_v, d_v), out_dtype, dev)
    prob = make_problem(N, T, h_k, h_v, d_k, d_v, qcode, ocode, scale, use_qk_l2norm, l2_eps, conv_width,
                        beta_logits, segment_chunks)
    ws_bytes = gdn_prefill_workspace_bytes(prob)
    if workspace is None:
        with torch.cuda.stream(s):
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    _hold_for(s, dev, (q, k, v, g, beta, cu_seqlens, conv_weight, conv_bias, conv_state_pool, state_pool,
                       state_indices, has_initial_state, o, workspace))
    st = load().gdn_prefill_varlen_pooled(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
        _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state_pool), _ptr(state_pool), _ptr(state_indices),
        _ptr(has_initial_state), _ptr(o), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
        ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_prefill_varlen_pooled")
    return o


def gdn_decode_step(q, k, v, g, beta, state_pool, *, state_indices=None, conv_weight=None,
                    conv_bias=None, conv_state_pool=None, use_qk_l2norm=True, scale=None, l2_eps=1e-6,
                    out_dtype=torch.float32, validate=True, out=None, stream=None, beta_logits=False):
    """One decode step over a state pool, in place (C ABI ``gdn_decode_step``).

    q, k: ``[N, h_k, d_k]``; v: ``[N, h_v, d_v]``; g, beta: ``[N, h_v]`` fp32;
    state_pool: fp32 ``[P, h_v, d_k, d_v]`` (updated in place); state_indices:
    int32 ``[N]`` or None (slot n uses entry n); -1 skips a slot.  Returns o.
    """
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [N, H, D]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    N, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    qdt = q.dtype
    qcode = _dtype_code(qdt, "q")
    ocode = _dtype_code(out_dtype, "out_dtype")
    _check(q, "q", (N, h_k, d_k), qdt, dev)
    _check(k, "k", (N, h_k, d_k), qdt, dev)
    _check(v, "v", (N, h_v, d_v), qdt, dev)
    _check(g, "g", (N, h_v), torch.float32, dev)
    _check(beta, "beta", (N, h_v), torch.float32, dev)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [P, h_v, d_k, d_v]")
    P = state_pool.shape[0]
    _check(state_pool, "state_pool", (P, h_v, d_k, d_v), torch.float32, dev)
    C = 2 * h_k * d_k + h_v * d_v
    conv_width = 4 if conv_weight is not None else 0
    if conv_weight is not None:
        _check(conv_weight, "conv_weight", (C, 4), qdt, dev)
        _check(conv_bias, "conv_bias", (C,), qdt, dev)
        if conv_state_pool is None:
            raise ValueError("conv_weight needs conv_state_pool")
        if conv_state_pool.dim() != 3:
            raise ValueError("conv_state_pool must be [P, C, 3]")
        _check(conv_state_pool, "conv_state_pool", (conv_state_pool.shape[0], C, 3), qdt, dev)
    _check_indices(state_indices, N, P, conv_state_pool.shape[0] if conv_width else None, dev, validate)
    s = _resolve_stream(stream, dev)
    with torch.cuda.stream(s):
        o = out if out is not None else torch.empty((N, h_v, d_v), dtype=out_dtype, device=dev)
    _check(o, "out", (N, h_v, d_v), out_dtype, dev)
    prob = make_problem(N, N, h_k, h_v, d_k, d_v, qcode, ocode, scale, use_qk_l2norm, l2_eps, conv_width,
                        beta_logits)
    _hold_for(s, dev, (q, k, v, g, beta, conv_weight, conv_bias, conv_state_pool, state_pool, state_indices, o))
    st = load().gdn_decode_step(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state_pool), _ptr(state_pool),
                                _ptr(state_indices), _ptr(o), ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_decode_step")
    return o


def gdn_decode_multi(q, k, v, g, beta, state_pool, *, state_indices=None, num_accepted=None,
                     conv_weight=None, conv_bias=None, conv_state_pool=None, use_qk_l2norm=True, scale=None,
                     l2_eps=1e-6, out_dtype=torch.float32, validate=True, out=None, stream=None,
                     beta_logits=False):
    """m tokens per slot in one call (C ABI ``gdn_decode_multi``).

    q, k: ``[N, m, h_k, d_k]``; v: ``[N, m, h_v, d_v]``; g, beta: ``[N, m, h_v]``
    fp32; state_pool: fp32 ``[P, h_v, d_k, d_v]``; state_indices: int32
    ``[N, m]`` or None; num_accepted: int32 ``[N]`` (1..m) or None.  Slot n
    reads entry ``state_indices[n, num_accepted[n] - 1]`` and writes the state
    (and conv history) after token j to ``state_indices[n, j]`` (-1: not
    written); without indices entry n is read and receives the state after the
    last token.  Returns o ``[N, m, h_v, d_v]``.
    """
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [N, m, H, D]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    N, m, h_k, d_k = q.shape
    h_v, d_v = v.shape[2], v.shape[3]
    qdt = q.dtype
    qcode = _dtype_code(qdt, "q")
    ocode = _dtype_code(out_dtype, "out_dtype")
    _check(q, "q", (N, m, h_k, d_k), qdt, dev)
    _check(k, "k", (N, m, h_k, d_k), qdt, dev)
    _check(v, "v", (N, m, h_v, d_v), qdt, dev)
    _check(g, "g", (N, m, h_v), torch.float32, dev)
    _check(beta, "beta", (N, m, h_v), torch.float32, dev)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [P, h_v, d_k, d_v]")
    P = state_pool.shape[0]
    _check(state_pool, "state_pool", (P, h_v, d_k, d_v), torch.float32, dev)
    C = 2 * h_k * d_k + h_v * d_v
    conv_width = 4 if conv_weight is not None else 0
    Pc = None
    if conv_weight is not None:
        _check(conv_weight, "conv_weight", (C, 4), qdt, dev)
        _check(conv_bias, "conv_bias", (C,), qdt, dev)
        if conv_state_pool is None:
            raise ValueError("conv_weight needs conv_state_pool")
        if conv_state_pool.dim() != 3:
            raise ValueError("conv_state_pool must be [P, C, 3]")
        Pc = conv_state_pool.shape[0]
        _check(conv_state_pool, "conv_state_pool", (Pc, C, 3), qdt, dev)
    if state_indices is None:
        if validate and (N > P or (Pc is not None and N > Pc)):
            raise ValueError("without state_indices the pools need at least N entries")
    else:
        _check(state_indices, "state_indices", (N, m), torch.int32, dev)
        if validate and N:
            idx = state_indices.cpu()
            used = idx[idx >= 0]
            if bool((idx < -1).any()) or bool((used >= P).any()) or (Pc is not None and bool((used >= Pc).any())):
                raise ValueError("state_indices out of range")
            # entries may repeat inside a slot's row, never across slots
            for n in range(N):
                mine = set(idx[n][idx[n] >= 0].tolist())
                others = idx[torch.arange(N) != n]
                if mine and bool(torch.isin(others, torch.tensor(sorted(mine), dtype=torch.int32)).any()):
                    raise ValueError("state_indices of different slots must be distinct")
    if num_accepted is not None:
        _check(num_accepted, "num_accepted", (N,), torch.int32, dev)
        if validate and N:
            acc = num_accepted.cpu()
            if bool((acc < 1).any()) or bool((acc > m).any()):
                raise ValueError("num_accepted must lie in 1..m")
    s = _resolve_stream(stream, dev)
    with torch.cuda.stream(s):
        o = out if out is not None else torch.empty((N, m, h_v, d_v), dtype=out_dtype, device=dev)
    _check(o, "out", (N, m, h_v, d_v), out_dtype, dev)
    prob = make_problem(N, N * m, h_k, h_v, d_k, d_v, qcode, ocode, scale, use_qk_l2norm, l2_eps, conv_width,
                        beta_logits)
    _hold_for(s, dev, (q, k, v, g, beta, conv_weight, conv_bias, conv_state_pool, state_pool, state_indices,
                       num_accepted, o))
    st = load().gdn_decode_multi(ctypes.byref(prob), ctypes.c_int32(m), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                 _ptr(beta), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state_pool),
                                 _ptr(state_pool), _ptr(state_indices), _ptr(num_accepted), _ptr(o),
                                 ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_decode_multi")
    return o
