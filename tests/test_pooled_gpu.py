"""GPU tests of gdn_prefill_varlen_pooled: prefill whose recurrent and conv
states live in pools addressed by state_indices (with has_initial_state).

* Bitwise: the pooled call equals gdn_prefill_varlen on the states gathered
  from the pool entries (zero for index -1 or has_initial_state 0), writes the
  final states into exactly those entries, and leaves every other entry alone.
* Oracle parity of the same run (max|delta| / rms within the dtype's bound).
* Continuation: a sequence prefilled in two pooled calls split at a multiple
  of 64 tokens equals one call, bit for bit.
* Mixed batch: length-1 sequences continuing from their entries (decode
  tokens) next to new prefills, against the oracle.
* Pool entries past element 2^31 give the bits of a compact pool.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, conv_state_pool, prefill_inputs, state_pool
from tests.gpu_util import TOL, TORCH_DT, dev, rel_err

pytestmark = pytest.mark.gpu


def _gather(pool, idx, has, n_seq):
    out = np.zeros((n_seq,) + pool.shape[1:], dtype=pool.dtype)
    for n in range(n_seq):
        if idx[n] >= 0 and has[n]:
            out[n] = pool[idx[n]]
    return out


@pytest.mark.parametrize("dtype,d_k,d_v", [("bf16", 128, 128), ("f32", 128, 128), ("bf16", 128, 64),
                                           ("f32", 64, 128)])
def test_pooled_matches_gathered_states(oracle_mod, dtype, d_k, d_v):
    geom = Geometry(2, 4, d_k, d_v)
    lengths = [70, 1, 130, 64, 5]
    idx = np.array([5, -1, 0, 3, 6], dtype=np.int32)
    has = np.array([1, 1, 0, 1, 1], dtype=np.int32)
    P = 7
    dt = TORCH_DT[dtype]
    x = prefill_inputs(60, lengths, geom, dtype)
    pool_np = state_pool(60, P, geom)
    cpool_np = conv_state_pool(60, P, geom, dtype)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta))
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32))
    w = dev(x.conv_w, dt)
    o = binding.gdn_prefill_varlen_pooled(*args, cu, pool, state_indices=dev(idx, torch.int32),
                                          has_initial_state=dev(has, torch.int32), conv_weight=w,
                                          conv_state_pool=cpool)
    h0 = _gather(pool_np, idx, has, len(lengths))
    cs0 = _gather(cpool_np, idx, has, len(lengths))
    o_ref, fs_ref, cso_ref = binding.gdn_prefill_varlen(*args, cu, conv_weight=w, conv_state=dev(cs0, dt),
                                                        initial_state=dev(h0))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    pool_after, cpool_after = pool.cpu().numpy(), cpool.float().cpu().numpy()
    for n, i in enumerate(idx):
        if i >= 0:
            assert np.array_equal(pool_after[i], fs_ref[n].cpu().numpy())
            assert np.array_equal(cpool_after[i], cso_ref[n].float().cpu().numpy())
    for i in sorted(set(range(P)) - set(int(j) for j in idx if j >= 0)):
        assert np.array_equal(pool_after[i], pool_np[i])
        assert np.array_equal(cpool_after[i], cpool_np[i])
    dims = oracle_mod.Dims(2, 4, d_k, d_v, conv_width=4)
    ro, rfs, _ = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, None, cs0, h0)
    eo = rel_err(o.float().cpu().numpy(), ro)
    used = [n for n in range(len(lengths)) if idx[n] >= 0]
    ef = rel_err(np.stack([pool_after[idx[n]] for n in used]), rfs[used])
    print(f"  rel err o={eo:.3e} final_state={ef:.3e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("d_k,d_v", [(128, 128), (64, 128), (128, 64)])
def test_pooled_continuation_bitwise(d_k, d_v):
    """200 tokens in one pooled call == 128 + 72 tokens in two (entry 2 carries the state)."""
    geom = Geometry(2, 4, d_k, d_v)
    dt = TORCH_DT["bf16"]
    x = prefill_inputs(61, [200], geom, "bf16")
    q, k, v, g, b = dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta)
    w = dev(x.conv_w, dt)
    P = 4
    pool0, cpool0 = dev(state_pool(61, P, geom)), dev(conv_state_pool(61, P, geom, "bf16"), dt)
    idx = dev(np.array([2], dtype=np.int32), torch.int32)
    pa, ca = pool0.clone(), cpool0.clone()
    oa = binding.gdn_prefill_varlen_pooled(q, k, v, g, b, [0, 200], pa, state_indices=idx, conv_weight=w,
                                           conv_state_pool=ca)
    pb, cb = pool0.clone(), cpool0.clone()
    s1, s2 = slice(0, 128), slice(128, 200)
    o1 = binding.gdn_prefill_varlen_pooled(q[s1].contiguous(), k[s1].contiguous(), v[s1].contiguous(),
                                           g[s1].contiguous(), b[s1].contiguous(), [0, 128], pb, state_indices=idx,
                                           conv_weight=w, conv_state_pool=cb)
    o2 = binding.gdn_prefill_varlen_pooled(q[s2].contiguous(), k[s2].contiguous(), v[s2].contiguous(),
                                           g[s2].contiguous(), b[s2].contiguous(), [0, 72], pb, state_indices=idx,
                                           conv_weight=w, conv_state_pool=cb)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2]), oa)
    assert torch.equal(pb, pa) and torch.equal(cb, ca)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pooled_mixed_prefill_and_decode(oracle_mod, dtype):
    """Sequences of 1 token continuing from entries 4 and 1 (decode tokens),
    beside a new 150-token prefill into entry 0 and a 64-token one into entry
    3, in one call."""
    geom = Geometry(2, 6, 64, 64)
    lengths = [1, 150, 1, 64]
    idx = np.array([4, 0, 1, 3], dtype=np.int32)
    has = np.array([1, 0, 1, 0], dtype=np.int32)
    P = 5
    dt = TORCH_DT[dtype]
    x = prefill_inputs(62, lengths, geom, dtype)
    pool_np = state_pool(62, P, geom)
    cpool_np = conv_state_pool(62, P, geom, dtype)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    o = binding.gdn_prefill_varlen_pooled(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), torch.from_numpy(x.cu_seqlens.astype(np.int32)),
        pool, state_indices=dev(idx, torch.int32), has_initial_state=dev(has, torch.int32),
        conv_weight=dev(x.conv_w, dt), conv_state_pool=cpool)
    torch.cuda.synchronize()
    h0, cs0 = _gather(pool_np, idx, has, 4), _gather(cpool_np, idx, has, 4)
    dims = oracle_mod.Dims(2, 6, 64, 64, conv_width=4)
    ro, rfs, rcso = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, None, cs0, h0)
    eo = rel_err(o.float().cpu().numpy(), ro)
    pa, ca = pool.cpu().numpy(), cpool.float().cpu().numpy()
    ef = rel_err(pa[idx], rfs)
    print(f"  rel err o={eo:.3e} final_state={ef:.3e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
    assert np.array_equal(ca[idx], rcso.astype(np.float32))
    assert np.array_equal(pa[2], pool_np[2])


def test_pooled_entries_beyond_32_bits():
    """Pooled prefill over a 4200-entry pool (h_v = 32, d = 128: entry 4096
    starts at element 2^31): sequences reading and writing entries past that
    point give bit for bit the outputs, final states and conv states of the same
    call on a compact pool holding those entries."""
    geom = Geometry(16, 32, 128, 128)
    P = 4200
    lengths = [70, 1, 130, 3]
    big = np.array([4199, 4097, -1, 100], dtype=np.int32)
    small = np.array([0, 1, -1, 3], dtype=np.int32)
    dt = torch.bfloat16
    x = prefill_inputs(62, lengths, geom, "bf16")
    pool_np = state_pool(62, len(lengths), geom)
    cpool_np = conv_state_pool(62, len(lengths), geom, "bf16")
    pool_big = torch.zeros((P, 32, 128, 128), dtype=torch.float32, device="cuda")
    cpool_big = torch.zeros((P, geom.channels, 3), dtype=dt, device="cuda")
    for n in range(len(lengths)):
        if big[n] >= 0:
            pool_big[int(big[n])] = dev(pool_np[n])
            cpool_big[int(big[n])] = dev(cpool_np[n], dt)
    pool_small, cpool_small = dev(pool_np), dev(cpool_np, dt)
    args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta))
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32))
    w = dev(x.conv_w, dt)
    o_big = binding.gdn_prefill_varlen_pooled(*args, cu, pool_big, state_indices=dev(big, torch.int32),
                                              conv_weight=w, conv_state_pool=cpool_big)
    o_small = binding.gdn_prefill_varlen_pooled(*args, cu, pool_small, state_indices=dev(small, torch.int32),
                                                conv_weight=w, conv_state_pool=cpool_small)
    torch.cuda.synchronize()
    assert torch.equal(o_big, o_small)
    for n in range(len(lengths)):
        if big[n] >= 0:
            assert torch.equal(pool_big[int(big[n])], pool_small[int(small[n])])
            assert torch.equal(cpool_big[int(big[n])], cpool_small[int(small[n])])
