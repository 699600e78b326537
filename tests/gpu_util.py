"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, run the oracle on the same values, and
measure the error the way the tolerance is stated (max |delta| / rms(ref))."""
from __future__ import annotations

import numpy as np
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, PrefillInputs

# max|gpu - oracle| / rms(oracle), for outputs and final states
TOL = {"f32": 1e-4, "bf16": 1e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-300))


def canary(shape, dtype):
    """A device tensor whose bytes are all 0xFF (NaN in fp32 and bf16): an
    output element the kernels fail to write stays NaN."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF)
    return t


def canary_outputs(x: PrefillInputs, out_dtype=torch.float32, conv=True, segment_chunks=0):
    """NaN-canary o, final states, conv states and workspace for a prefill of x."""
    g = x.geom
    N, T = x.num_seqs, x.total_tokens
    o = canary((T, g.h_v, g.d_v), out_dtype)
    fs = canary((N, g.h_v, g.d_k, g.d_v), torch.float32)
    cso = canary((N, g.channels, 3), TORCH_DT[x.dtype]) if conv else None
    prob = binding.make_problem(N, T, g.h_k, g.h_v, g.d_k, g.d_v, 1, 0, segment_chunks=segment_chunks)
    ws = canary((max(binding.gdn_prefill_workspace_bytes(prob), 1),), torch.uint8)
    return o, fs, cso, ws


def gpu_prefill(x: PrefillInputs, *, use_initial=True, use_conv_state=True, out_dtype=torch.float32,
                conv=True, scale=None, qk_l2norm=True, noalloc=False, segment_chunks=0):
    """The HIP prefill of x with every output and the workspace pre-filled
    with NaN bytes; asserts that every o row and final state was written."""
    dt = TORCH_DT[x.dtype]
    conv = conv and x.conv_w is not None
    o, fs, cso, ws = canary_outputs(x, out_dtype, conv, segment_chunks)
    res = binding.gdn_prefill_varlen(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta),
        torch.from_numpy(x.cu_seqlens.astype(np.int32)),
        conv_weight=dev(x.conv_w, dt) if conv else None,
        conv_state=dev(x.conv_state_in, dt) if (conv and use_conv_state and x.conv_state_in is not None) else None,
        initial_state=dev(x.initial_state) if (use_initial and x.initial_state is not None) else None,
        out_dtype=out_dtype, scale=scale, use_qk_l2norm=qk_l2norm, out=o, final_state_out=fs,
        conv_state_out=cso, workspace=None if noalloc else ws, noalloc=noalloc, segment_chunks=segment_chunks)
    torch.cuda.synchronize()
    o, fs, cso = res
    o, fs = o.float().cpu().numpy(), fs.cpu().numpy()
    assert np.all(np.isfinite(o)), "o has unwritten (NaN canary) or non-finite elements"
    assert np.all(np.isfinite(fs)), "final states have unwritten (NaN canary) or non-finite elements"
    return o, fs, None if cso is None else cso.float().cpu().numpy()


def oracle_prefill(oracle, x: PrefillInputs, *, use_initial=True, use_conv_state=True, conv=True, scale=None,
                   qk_l2norm=True, nthreads=0):
    g = x.geom
    dims = oracle.Dims(g.h_k, g.h_v, g.d_k, g.d_v, conv_width=4 if (conv and x.conv_w is not None) else 0,
                       qk_l2norm=qk_l2norm, scale=scale)
    return oracle.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta,
                          x.conv_w if dims.conv_width else None, None,
                          x.conv_state_in if (dims.conv_width and use_conv_state) else None,
                          x.initial_state if use_initial else None, nthreads=nthreads)


def head_slice(x: PrefillInputs, n: int, hk: int) -> PrefillInputs:
    """Sequence n restricted to key head hk and its G value heads (with the
    matching conv channels), so the oracle can check one unit of a large run."""
    g = x.geom
    G = g.h_v // g.h_k
    s = slice(int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1]))
    L = s.stop - s.start
    hv = slice(hk * G, (hk + 1) * G)
    geom = Geometry(1, G, g.d_k, g.d_v, g.conv_width)
    conv_w = None
    if x.conv_w is not None:
        nq = g.h_k * g.d_k
        rows = np.concatenate([np.arange(hk * g.d_k, (hk + 1) * g.d_k),
                               nq + np.arange(hk * g.d_k, (hk + 1) * g.d_k),
                               2 * nq + np.arange(hk * G * g.d_v, (hk + 1) * G * g.d_v)])
        conv_w = np.ascontiguousarray(x.conv_w[rows])
        csi = None if x.conv_state_in is None else np.ascontiguousarray(x.conv_state_in[n:n + 1][:, rows])
    else:
        csi = None
    return PrefillInputs(geom, x.dtype, np.array([0, L], dtype=np.int64),
                         np.ascontiguousarray(x.q[s, hk:hk + 1]), np.ascontiguousarray(x.k[s, hk:hk + 1]),
                         np.ascontiguousarray(x.v[s, hv]), np.ascontiguousarray(x.g[s, hv]),
                         np.ascontiguousarray(x.beta[s, hv]), conv_w,
                         None if x.initial_state is None else np.ascontiguousarray(x.initial_state[n:n + 1, hv]),
                         csi)
