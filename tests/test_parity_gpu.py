"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max|gpu - oracle| / rms(oracle) <= 1e-4 for fp32 inputs and <= 1e-2 for
bf16 inputs, on outputs and on final states; conv states (raw values moved)
bit-exact.  Sizes span several 64-token chunks with ragged tails; the full
prefill workload (4 x 4096 tokens, 16 key / 32 value heads, d = 128, bf16) is
compared with the oracle on the whole output and every final state, and the
256-slot decode over 100 consecutive steps on sampled slots.  Prefill outputs
and workspace start as NaN bytes (tests.gpu_util.gpu_prefill), so an element
the kernels do not write fails.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import (Geometry, bf16_round, conv_bias, conv_state_pool, conv_weights,
                                                    decode_inputs, gate_logits, prefill_inputs, state_pool,
                                                    uniform_lengths)
from tests.gpu_util import TOL, TORCH_DT, dev, gpu_prefill, head_slice, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


def _check_prefill(oracle, x, **kw):
    o, fs, cso = gpu_prefill(x, **kw)
    kw.pop("out_dtype", None)
    ro, rfs, rcso = oracle_prefill(oracle, x, **kw)
    eo, ef = rel_err(o, ro), rel_err(fs, rfs)
    print(f"  rel err o={eo:.3e} final_state={ef:.3e} (tol {TOL[x.dtype]:.0e})", flush=True)
    assert np.all(np.isfinite(o))
    assert eo <= TOL[x.dtype] and ef <= TOL[x.dtype]
    if rcso is not None and cso is not None:
        assert np.array_equal(cso, rcso)
    return o, fs


def test_single_sequence_fp32_T256(oracle_mod):
    """1 x 256 tokens, 4 heads, d = 64, fp32, conv + SiLU + L2, zero state."""
    x = prefill_inputs(0, [256], Geometry(4, 4, 64, 64), "f32")
    _check_prefill(oracle_mod, x)


@pytest.mark.parametrize("d", [128, 64])
def test_ragged_bf16(oracle_mod, d):
    lengths = [1, 63, 64, 65, 200, 3, 130, 0, 2]
    x = prefill_inputs(10 + d, lengths, Geometry(2, 4, d, d), "bf16", initial_state_std=0.02, conv_state=True)
    _check_prefill(oracle_mod, x)


def test_ragged_fp32_gqa3(oracle_mod):
    x = prefill_inputs(20, [5, 64, 129, 70, 1], Geometry(2, 6, 64, 64), "f32", initial_state_std=0.02,
                       conv_state=True)
    _check_prefill(oracle_mod, x)


def test_ragged_fp32_d128(oracle_mod):
    x = prefill_inputs(24, [3, 64, 100], Geometry(1, 2, 128, 128), "f32", initial_state_std=0.02,
                       conv_state=True)
    _check_prefill(oracle_mod, x)


def test_fp32_without_conv(oracle_mod):
    x = prefill_inputs(21, [100, 37], Geometry(1, 2, 64, 64), "f32", initial_state_std=0.02)
    _check_prefill(oracle_mod, x, conv=False)


def test_fp32_without_l2norm(oracle_mod):
    """qk_l2norm = 0 with inputs already scaled to unit-size heads."""
    x = prefill_inputs(22, [90], Geometry(1, 1, 64, 64), "f32", initial_state_std=0.02)
    x.q /= np.linalg.norm(x.q, axis=-1, keepdims=True)
    x.k /= np.linalg.norm(x.k, axis=-1, keepdims=True)
    _check_prefill(oracle_mod, x, conv=False, qk_l2norm=False)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_conv_bias(oracle_mod, dtype, d):
    """Conv with a bias, ragged sequences (interior and boundary chunks),
    carried conv states and initial states."""
    geom = Geometry(2, 4, d, d)
    x = prefill_inputs(25, [1, 64, 200, 130, 3], geom, dtype, initial_state_std=0.02, conv_state=True)
    bias = conv_bias(25, geom, dtype)
    dt = TORCH_DT[dtype]
    o, fs, cso = binding.gdn_prefill_varlen(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), torch.from_numpy(x.cu_seqlens.astype(np.int32)),
        conv_weight=dev(x.conv_w, dt), conv_bias=dev(bias, dt), conv_state=dev(x.conv_state_in, dt),
        initial_state=dev(x.initial_state))
    torch.cuda.synchronize()
    dims = oracle_mod.Dims(2, 4, d, d, conv_width=4)
    ro, rfs, rcso = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, bias,
                                       x.conv_state_in, x.initial_state)
    eo, ef = rel_err(o.cpu().numpy(), ro), rel_err(fs.cpu().numpy(), rfs)
    print(f"  rel err o={eo:.3e} final_state={ef:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
    assert np.array_equal(cso.float().cpu().numpy(), rcso)


def _sigmoid64(b):
    return 1.0 / (1.0 + np.exp(-b.astype(np.float64)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_beta_logits_prefill(oracle_mod, dtype):
    """beta_logits = 1: the beta input holds raw gates b (2 N(0, 1), some
    saturating) and the kernels use sigmoid(b); the oracle gets sigmoid(b)."""
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(26, [70, 130, 3], geom, dtype, initial_state_std=0.02, conv_state=True)
    b = gate_logits(26, x.total_tokens, geom.h_v)
    b[0, 0], b[1, 1] = 60.0, -60.0
    x.beta = b
    dt = TORCH_DT[dtype]
    o, fs, _ = binding.gdn_prefill_varlen(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(b), torch.from_numpy(x.cu_seqlens.astype(np.int32)),
        conv_weight=dev(x.conv_w, dt), conv_state=dev(x.conv_state_in, dt), initial_state=dev(x.initial_state),
        beta_logits=True)
    torch.cuda.synchronize()
    dims = oracle_mod.Dims(2, 4, 128, 128, conv_width=4)
    ro, rfs, _ = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, _sigmoid64(b), x.conv_w, None,
                                    x.conv_state_in, x.initial_state)
    eo, ef = rel_err(o.cpu().numpy(), ro), rel_err(fs.cpu().numpy(), rfs)
    print(f"  rel err o={eo:.3e} final_state={ef:.3e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


def test_bf16_inputs_beyond_fp16_range(oracle_mod):
    """bf16 inputs use split-bf16 products, which keep fp32's range: v and the
    initial states scaled by 2^22 (state entries far above fp16's 65504) still
    meet the bar."""
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(27, [150, 40], geom, "bf16", initial_state_std=0.02)
    x.v *= 2.0 ** 22           # exact in bf16
    x.initial_state *= 2.0 ** 22
    o, fs = _check_prefill(oracle_mod, x)
    print(f"  max|final state| = {np.max(np.abs(fs)):.3e}, max|o| = {np.max(np.abs(o)):.3e}", flush=True)
    assert np.max(np.abs(fs)) > 65504.0


def test_fp32_inputs_beyond_fp16_range(oracle_mod):
    """fp32 inputs take fp32 matrix-core products, which keep fp32's range and
    precision: v and the initial states scaled by 2^20 (state entries far above
    fp16's 65504) still meet the fp32 bar."""
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(28, [150, 40], geom, "f32", initial_state_std=0.02, conv_state=True)
    x.v *= 2.0 ** 20
    x.initial_state *= 2.0 ** 20
    x.conv_state_in[:, 2 * geom.h_k * geom.d_k:] *= 2.0 ** 20  # the v channels' history
    o, fs = _check_prefill(oracle_mod, x)
    print(f"  max|final state| = {np.max(np.abs(fs)):.3e}, max|o| = {np.max(np.abs(o)):.3e}", flush=True)
    assert np.max(np.abs(fs)) > 65504.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d_k,d_v", [(128, 64), (64, 128)])
def test_mixed_head_dims(oracle_mod, dtype, d_k, d_v):
    """d_k != d_v (the state is (v_heads, k_head_dim, v_head_dim)): ragged
    sequences, GQA 2, conv with carried conv states and initial states."""
    x = prefill_inputs(29 + d_k // 64, [1, 63, 200, 64, 130, 0], Geometry(2, 4, d_k, d_v), dtype,
                       initial_state_std=0.02, conv_state=True)
    _check_prefill(oracle_mod, x)


def test_side_stream_prefill_is_safe():
    """A call on a side stream allocates its temporaries there; memory
    allocated and written on the current stream right after the call cannot
    reuse them while the kernels still run, so the result is bit-identical to
    the same call on the current stream."""
    x = prefill_inputs(46, [700, 300], Geometry(4, 8, 128, 128), "bf16", initial_state_std=0.02, conv_state=True)
    ref_o, ref_fs, ref_cso = gpu_prefill(x)
    dt = TORCH_DT["bf16"]
    args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta))
    w, cs, h0 = dev(x.conv_w, dt), dev(x.conv_state_in, dt), dev(x.initial_state)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, fs, cso = binding.gdn_prefill_varlen(*args, x.cu_seqlens.astype(np.int32).tolist(), conv_weight=w,
                                            conv_state=cs, initial_state=h0, stream=side)
    # churn the current stream's allocations while the side stream runs
    junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(16)]
    del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(o.cpu().numpy(), ref_o)
    assert np.array_equal(fs.cpu().numpy(), ref_fs)
    assert np.array_equal(cso.float().cpu().numpy(), ref_cso)


def test_stream_must_be_a_torch_stream():
    x = prefill_inputs(47, [10], Geometry(1, 1, 64, 64), "bf16")
    with pytest.raises(ValueError):
        binding.gdn_prefill_varlen(dev(x.q, torch.bfloat16), dev(x.k, torch.bfloat16), dev(x.v, torch.bfloat16),
                                   dev(x.g), dev(x.beta), [0, 10], stream=torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("h_k,h_v,d,dtype", [(1, 8, 128, "bf16"), (2, 10, 64, "f32"), (2, 16, 128, "bf16")])
def test_large_gqa_groups(oracle_mod, h_k, h_v, d, dtype):
    """8, 5 (odd) and 8 value heads per key head: the chunk-local kernel takes
    the group's value heads two at a time, the carry one workgroup per
    (value head, slice)."""
    x = prefill_inputs(27 + h_v, [100, 64, 1, 150], Geometry(h_k, h_v, d, d), dtype, initial_state_std=0.02,
                       conv_state=True)
    _check_prefill(oracle_mod, x)


def test_custom_scale(oracle_mod):
    x = prefill_inputs(23, [70], Geometry(2, 2, 128, 128), "bf16")
    _check_prefill(oracle_mod, x, scale=0.5)


def test_short_sequence_many_heads_is_time_first(oracle_mod):
    """T = 12 with 32 value heads (fewer tokens than heads): one layout, no heuristic."""
    x = prefill_inputs(30, [12], Geometry(16, 32, 128, 128), "bf16")
    _check_prefill(oracle_mod, x)


def test_29_packed_sequences(oracle_mod):
    lengths = uniform_lengths(31, 29, 1, 300)
    x = prefill_inputs(31, lengths, Geometry(2, 4, 128, 128), "bf16", initial_state_std=0.02, conv_state=True)
    _check_prefill(oracle_mod, x)


def test_bf16_output(oracle_mod):
    """bf16 o is the kernel's fp32 o rounded to nearest even at the store (bit
    for bit), so |o_bf16 - oracle| <= tol rms(oracle) + half a bf16 ulp (2^-8 |o|)."""
    x = prefill_inputs(32, [150, 40], Geometry(2, 4, 128, 128), "bf16", initial_state_std=0.02)
    o16, f16, _ = gpu_prefill(x, out_dtype=torch.bfloat16)
    o32, f32, _ = gpu_prefill(x)
    assert np.array_equal(o16, bf16_round(o32))
    assert np.array_equal(f16, f32)
    ro, _, _ = oracle_prefill(oracle_mod, x)
    rms = np.sqrt(np.mean(ro ** 2))
    assert np.all(np.abs(o16 - ro) <= TOL["bf16"] * rms + 2.0 ** -8 * np.abs(o32))


def test_many_short_ragged_sequences(oracle_mod):
    """600 sequences of 1..130 tokens (about 900 chunks, most with a ragged
    tail): more (chunk, key head) units than the chunk-local kernel has
    resident workgroups, so each workgroup walks several units of different
    sequences; the whole run is compared with the oracle."""
    geom = Geometry(1, 2, 64, 64)
    lengths = uniform_lengths(44, 600, 1, 130)
    x = prefill_inputs(44, lengths, geom, "bf16", initial_state_std=0.02, conv_state=True)
    _check_prefill(oracle_mod, x)


@pytest.mark.parametrize("n_seqs", [512, 513])
def test_map_paths_at_the_boundary(oracle_mod, n_seqs):
    """512 sequences take the one-workgroup map kernel, 513 the three map
    kernels (chunk map, order, slot descriptors); both against the oracle."""
    lengths = uniform_lengths(45 + n_seqs, n_seqs, 0, 70)
    x = prefill_inputs(45, lengths, Geometry(1, 1, 64, 64), "bf16", initial_state_std=0.02, conv_state=True)
    _check_prefill(oracle_mod, x)


def test_full_prefill_4x4096_whole(oracle_mod):
    """4 x 4096 tokens, h_k = 16, h_v = 32, d = 128, bf16, conv + SiLU + L2 (the
    benchmark's workload and launch): the whole output, every final state and
    every conv state against the oracle; worst sequence reported."""
    geom = Geometry(16, 32, 128, 128)
    x = prefill_inputs(1, [4096] * 4, geom, "bf16")
    o, fs, cso = gpu_prefill(x)
    ro, rfs, rcso = oracle_prefill(oracle_mod, x)
    eo, ef = rel_err(o, ro), rel_err(fs, rfs)
    per_seq = [rel_err(o[4096 * n:4096 * (n + 1)], ro[4096 * n:4096 * (n + 1)]) for n in range(4)]
    print(f"  whole: rel err o={eo:.3e} final={ef:.3e}; worst sequence o={max(per_seq):.3e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    assert np.array_equal(cso, rcso)


# ---------------------------------------------------------------- invariants

def test_beta0_g0_keeps_state_bitwise():
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(40, [70, 130], geom, "bf16", initial_state_std=0.02)
    x.beta[:] = 0.0
    x.g[:] = 0.0
    _, fs, _ = gpu_prefill(x)
    assert np.array_equal(fs, x.initial_state)


def test_run_to_run_bitwise():
    x = prefill_inputs(41, [300, 5, 64], Geometry(2, 4, 128, 128), "bf16", initial_state_std=0.02)
    o1, f1, _ = gpu_prefill(x)
    o2, f2, _ = gpu_prefill(x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_batch_invariance_bitwise():
    """Target sequences give bit-identical outputs and final states alone and
    packed at different positions among seeded filler sequences."""
    geom = Geometry(2, 4, 128, 128)
    targets = [(500, 300), (501, 64), (502, 1)]  # (seq id, length)
    alone = {}
    for sid, L in targets:
        x = prefill_inputs(42, [L], geom, "bf16", seq_ids=[sid], initial_state_std=0.02)
        o, fs, _ = gpu_prefill(x)
        alone[sid] = (o, fs[0])
    rng = np.random.default_rng(42)
    for batch in (4, 9):
        fill = uniform_lengths(42 + batch, batch, 1, 400)
        ids = list(range(batch))
        pos = sorted(rng.choice(batch + len(targets), size=len(targets), replace=False))
        lengths, seq_ids = list(fill), list(ids)
        for (sid, L), p in zip(targets, pos):
            lengths.insert(p, L)
            seq_ids.insert(p, sid)
        x = prefill_inputs(42, lengths, geom, "bf16", seq_ids=seq_ids, initial_state_std=0.02)
        o, fs, _ = gpu_prefill(x)
        for sid, _ in targets:
            n = seq_ids.index(sid)
            s = slice(int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1]))
            assert np.array_equal(o[s], alone[sid][0]), (batch, sid)
            assert np.array_equal(fs[n], alone[sid][1]), (batch, sid)


@pytest.mark.parametrize("split", [64, 128])
def test_split_and_resume_bitwise_at_64_multiples(split):
    """Prefill of 300 tokens equals prefill of the first `split` tokens then of
    the rest from the carried recurrent and conv states, bit for bit."""
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(43, [300], geom, "bf16", initial_state_std=0.02, conv_state=True)
    dt = TORCH_DT["bf16"]
    q, k, v, g, b = dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta)
    w, cs, h0 = dev(x.conv_w, dt), dev(x.conv_state_in, dt), dev(x.initial_state)
    o, fs, cso = binding.gdn_prefill_varlen(q, k, v, g, b, [0, 300], conv_weight=w, conv_state=cs, initial_state=h0)
    a = slice(0, split)
    c = slice(split, 300)
    o1, f1, c1 = binding.gdn_prefill_varlen(q[a].contiguous(), k[a].contiguous(), v[a].contiguous(),
                                            g[a].contiguous(), b[a].contiguous(), [0, split], conv_weight=w,
                                            conv_state=cs, initial_state=h0)
    o2, f2, c2 = binding.gdn_prefill_varlen(q[c].contiguous(), k[c].contiguous(), v[c].contiguous(),
                                            g[c].contiguous(), b[c].contiguous(), [0, 300 - split], conv_weight=w,
                                            conv_state=c1, initial_state=f1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2]), o)
    assert torch.equal(f2, fs)
    assert torch.equal(c2, cso)


@pytest.mark.parametrize("segment_chunks", [0, 1])
def test_in_place_state_and_conv_state(segment_chunks):
    """final_state may alias initial_state and conv_state_out conv_state_in,
    also with the segment split (the 700-token sequence as 11 one-chunk
    segments run side by side: the conv history must be read before the
    final conv state replaces it)."""
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(44, [700, 7], geom, "bf16", initial_state_std=0.02, conv_state=True)
    dt = TORCH_DT["bf16"]
    args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), x.cu_seqlens.astype(np.int32).tolist())
    w = dev(x.conv_w, dt)
    h0, cs = dev(x.initial_state), dev(x.conv_state_in, dt)
    o, fs, cso = binding.gdn_prefill_varlen(*args, conv_weight=w, conv_state=cs.clone(), initial_state=h0.clone(),
                                            segment_chunks=segment_chunks)
    o2, fs2, cso2 = binding.gdn_prefill_varlen(*args, conv_weight=w, conv_state=cs, initial_state=h0,
                                               final_state_out=h0, conv_state_out=cs, segment_chunks=segment_chunks)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fs, h0) and torch.equal(cso, cs)


def test_empty_and_zero_length():
    geom = Geometry(2, 4, 128, 128)
    x = prefill_inputs(45, [0, 0], geom, "bf16", initial_state_std=0.02)
    o, fs, _ = gpu_prefill(x)
    assert o.shape == (0, 4, 128)
    assert np.array_equal(fs, x.initial_state)


# -------------------------------------------------------------------- decode

@pytest.mark.parametrize("conv", [False, True])
def test_decode_256_slots_100_steps(oracle_mod, conv):
    """256 slots x 32 value heads (16 key heads), d = 128, bf16 inputs, the fp32
    pool of 512 MiB updated in place for 100 consecutive steps with fresh
    seeded inputs (with and without the conv update of a conv pool); sampled
    slots' outputs at every step and their states after steps 50 and 100
    against the fp64 oracle run through the same 100 steps."""
    geom = Geometry(16, 32, 128, 128)
    N, steps = 256, 100
    pool = dev(state_pool(3, N, geom))
    sample = [0, 77, 255]
    ref_pool = pool[sample].double().cpu().numpy().copy()
    cw_np = conv_weights(3, geom, "bf16") if conv else None
    cpool = dev(conv_state_pool(3, N, geom, "bf16"), torch.bfloat16) if conv else None
    ref_cpool = cpool[sample].double().cpu().numpy().copy() if conv else None
    cw = dev(cw_np, torch.bfloat16) if conv else None
    dims = oracle_mod.Dims(16, 32, 128, 128, conv_width=4 if conv else 0)
    worst = 0.0
    for s in range(steps):
        d = decode_inputs(3, s, N, geom, "bf16")
        o = binding.gdn_decode_step(dev(d.q, torch.bfloat16), dev(d.k, torch.bfloat16), dev(d.v, torch.bfloat16),
                                    dev(d.g), dev(d.beta), pool, conv_weight=cw, conv_state_pool=cpool)
        ro = oracle_mod.decode(dims, d.q[sample], d.k[sample], d.v[sample], d.g[sample], d.beta[sample], ref_pool,
                               np.arange(len(sample)), cw_np, None, ref_cpool)
        e = rel_err(o[sample].cpu().numpy(), ro)
        worst = max(worst, e)
        assert e <= TOL["bf16"], (s, e)
        if s + 1 in (50, steps):
            ef = rel_err(pool[sample].cpu().numpy(), ref_pool)
            print(f"  after step {s + 1}: worst o rel err so far {worst:.3e}, states {ef:.3e}", flush=True)
            assert ef <= TOL["bf16"]
            if conv:
                assert np.array_equal(cpool[sample].float().cpu().numpy(), ref_cpool.astype(np.float32))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_decode_conv_and_indices(oracle_mod, dtype, d):
    """Conv update from the conv pool, a permuted index map and a skipped slot."""
    geom = Geometry(2, 4, d, d)
    P, N = 7, 5
    dt = TORCH_DT[dtype]
    pool_np = state_pool(50, P, geom)
    cpool_np = conv_state_pool(50, P, geom, dtype)
    w_np = conv_weights(50, geom, dtype)
    idx = np.array([3, -1, 0, 6, 2], dtype=np.int32)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    ref_pool, ref_cpool = pool_np.astype(np.float64), cpool_np.astype(np.float64)
    dims = oracle_mod.Dims(2, 4, d, d, conv_width=4)
    for s in range(3):
        x = decode_inputs(50, s, N, geom, dtype)
        o = binding.gdn_decode_step(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), pool,
                                    state_indices=dev(idx, torch.int32), conv_weight=dev(w_np, dt),
                                    conv_state_pool=cpool)
        ro = oracle_mod.decode(dims, x.q, x.k, x.v, x.g, x.beta, ref_pool, idx.astype(np.int64), w_np, None,
                               ref_cpool)
        used = idx >= 0
        assert rel_err(o.cpu().numpy()[used], ro[used]) <= TOL[dtype]
    assert rel_err(pool.cpu().numpy(), ref_pool) <= TOL[dtype]
    assert np.array_equal(cpool.float().cpu().numpy(), ref_cpool.astype(np.float32))
    assert np.array_equal(pool[1].cpu().numpy(), pool_np[1])  # untouched entries


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_conv_bias(oracle_mod, dtype):
    """Decode with a conv bias, two steps, in place."""
    geom = Geometry(2, 4, 128, 128)
    P = 4
    dt = TORCH_DT[dtype]
    pool_np = state_pool(51, P, geom)
    cpool_np = conv_state_pool(51, P, geom, dtype)
    w_np, b_np = conv_weights(51, geom, dtype), conv_bias(51, geom, dtype)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    ref_pool, ref_cpool = pool_np.astype(np.float64), cpool_np.astype(np.float64)
    dims = oracle_mod.Dims(2, 4, 128, 128, conv_width=4)
    idx = np.arange(P, dtype=np.int64)
    for s in range(2):
        x = decode_inputs(51, s, P, geom, dtype)
        o = binding.gdn_decode_step(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), pool,
                                    conv_weight=dev(w_np, dt), conv_bias=dev(b_np, dt), conv_state_pool=cpool)
        ro = oracle_mod.decode(dims, x.q, x.k, x.v, x.g, x.beta, ref_pool, idx, w_np, b_np, ref_cpool)
        assert rel_err(o.cpu().numpy(), ro) <= TOL[dtype]
    assert rel_err(pool.cpu().numpy(), ref_pool) <= TOL[dtype]
    assert np.array_equal(cpool.float().cpu().numpy(), ref_cpool.astype(np.float32))


def test_decode_beta_logits(oracle_mod):
    """Decode with raw gates b in the beta input (beta_logits = 1)."""
    geom = Geometry(2, 4, 128, 128)
    P = 3
    pool_np = state_pool(52, P, geom)
    pool = dev(pool_np)
    ref_pool = pool_np.astype(np.float64)
    dims = oracle_mod.Dims(2, 4, 128, 128, conv_width=0)
    x = decode_inputs(52, 0, P, geom, "bf16")
    b = gate_logits(52, P, geom.h_v)
    o = binding.gdn_decode_step(dev(x.q, torch.bfloat16), dev(x.k, torch.bfloat16), dev(x.v, torch.bfloat16),
                                dev(x.g), dev(b), pool, beta_logits=True)
    ro = oracle_mod.decode(dims, x.q, x.k, x.v, x.g, _sigmoid64(b), ref_pool, np.arange(P, dtype=np.int64))
    assert rel_err(o.cpu().numpy(), ro) <= TOL["bf16"]
    assert rel_err(pool.cpu().numpy(), ref_pool) <= TOL["bf16"]


@pytest.mark.parametrize("h_k,h_v,d_k,d_v", [(3, 3, 64, 64), (2, 6, 128, 64), (1, 4, 64, 128), (1, 8, 128, 128),
                                             (2, 10, 64, 64)])
def test_decode_gqa_groups(oracle_mod, h_k, h_v, d_k, d_v):
    """Value heads per key head 1, 3 and 4 (one workgroup serves the group and
    shifts its conv history), with d_k != d_v, conv and an index map."""
    geom = Geometry(h_k, h_v, d_k, d_v)
    P, N = 6, 4
    dt = torch.bfloat16
    pool_np = state_pool(53, P, geom)
    cpool_np = conv_state_pool(53, P, geom, "bf16")
    w_np = conv_weights(53, geom, "bf16")
    idx = np.array([5, 1, -1, 2], dtype=np.int32)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    ref_pool, ref_cpool = pool_np.astype(np.float64), cpool_np.astype(np.float64)
    dims = oracle_mod.Dims(h_k, h_v, d_k, d_v, conv_width=4)
    for s in range(2):
        x = decode_inputs(53, s, N, geom, "bf16")
        o = binding.gdn_decode_step(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), pool,
                                    state_indices=dev(idx, torch.int32), conv_weight=dev(w_np, dt),
                                    conv_state_pool=cpool)
        ro = oracle_mod.decode(dims, x.q, x.k, x.v, x.g, x.beta, ref_pool, idx.astype(np.int64), w_np, None,
                               ref_cpool)
        used = idx >= 0
        assert rel_err(o.cpu().numpy()[used], ro[used]) <= TOL["bf16"]
    assert rel_err(pool.cpu().numpy(), ref_pool) <= TOL["bf16"]
    assert np.array_equal(cpool.float().cpu().numpy(), ref_cpool.astype(np.float32))
    for e in (0, 3, 4):  # entries no index names stay untouched
        assert np.array_equal(pool[e].cpu().numpy(), pool_np[e])


def test_decode_steps_match_prefill(oracle_mod):
    """T decode steps from a pooled state equal one prefill of the T tokens (tolerance)."""
    geom = Geometry(2, 4, 128, 128)
    T = 40
    x = prefill_inputs(51, [T], geom, "bf16", initial_state_std=0.02, conv_state=True)
    o_pre, fs_pre, cso_pre = gpu_prefill(x)
    dt = torch.bfloat16
    pool = dev(x.initial_state)
    cpool = dev(x.conv_state_in, dt)
    w = dev(x.conv_w, dt)
    outs = []
    for t in range(T):
        outs.append(binding.gdn_decode_step(dev(x.q[t:t + 1], dt), dev(x.k[t:t + 1], dt), dev(x.v[t:t + 1], dt),
                                            dev(x.g[t:t + 1]), dev(x.beta[t:t + 1]), pool, conv_weight=w,
                                            conv_state_pool=cpool))
    o_dec = torch.cat(outs).cpu().numpy()
    assert rel_err(o_dec, o_pre) <= TOL["bf16"]
    assert rel_err(pool.cpu().numpy(), fs_pre) <= TOL["bf16"]
    assert np.array_equal(cpool.float().cpu().numpy(), cso_pre)


@pytest.mark.parametrize("d_k,d_v", [(128, 128), (128, 64), (64, 64)])
def test_decode_batch_invariance_bitwise(d_k, d_v):
    """A slot's output and state do not depend on which other slots share the call."""
    geom = Geometry(16, 32, d_k, d_v)
    N = 64
    pool0 = dev(state_pool(52, N, geom))
    x = decode_inputs(52, 0, N, geom, "bf16")
    dt = torch.bfloat16
    pa = pool0.clone()
    oa = binding.gdn_decode_step(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), pa)
    sub = [5, 40]
    pb = pool0.clone()
    ob = binding.gdn_decode_step(dev(x.q[sub], dt), dev(x.k[sub], dt), dev(x.v[sub], dt), dev(x.g[sub]),
                                 dev(x.beta[sub]), pb, state_indices=dev(np.array(sub, np.int32), torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(oa[sub], ob)
    assert torch.equal(pa[sub], pb[sub])
