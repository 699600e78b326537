"""GPU tests of the segment split (gdn_problem.segment_chunks > 0): a long
sequence runs as parallel segments, each after the first from zero state
beside d_k identity columns, then the start states are chained through the
segments' transitions and the outputs corrected by one product with them.

* Oracle parity (the same fp64 recurrence; the split changes rounding only):
  ragged sequences some of which split into 2-4 segments and some not, with
  initial recurrent and conv states, bf16 and fp32 inputs, d_k = d_v and
  d_k != d_v; outputs and workspace start as NaN bytes.
* Batch invariance with the split on: target sequences alone and packed
  among fillers give bit-identical outputs and final states (the split
  depends on each sequence's length alone).
* bf16 outputs are the split's fp32 outputs rounded once (bit for bit).
* Pooled states with the split (continuation from an entry, final states
  written back).
* The 32768-token sequence (h_k = 16, h_v = 32, d = 128, bf16) split into
  two segments of 256 chunks: the whole output and final state against the
  oracle.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, bf16_round, conv_state_pool, prefill_inputs, state_pool
from tests.gpu_util import TOL, TORCH_DT, dev, gpu_prefill, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


def _segments(length, seg):
    nch = -(-length // 64)
    return -(-nch // seg) if nch > seg else 1


@pytest.mark.parametrize("dtype,d_k,d_v", [("bf16", 128, 128), ("f32", 64, 64), ("bf16", 64, 128),
                                           ("f32", 128, 64)])
def test_split_matches_oracle(oracle_mod, dtype, d_k, d_v):
    seg = 3
    lengths = [700, 1, 192, 193, 0, 450, 64]  # 11, 1, 3, 4, 0, 8, 1 chunks
    assert [_segments(L, seg) for L in lengths] == [4, 1, 1, 2, 1, 3, 1]
    x = prefill_inputs(80 + d_k + d_v, lengths, Geometry(2, 4, d_k, d_v), dtype, initial_state_std=0.02,
                       conv_state=True)
    o, fs, cso = gpu_prefill(x, segment_chunks=seg)
    ro, rfs, rcso = oracle_prefill(oracle_mod, x)
    eo, ef = rel_err(o, ro), rel_err(fs, rfs)
    print(f"  split: rel err o={eo:.3e} final_state={ef:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
    assert np.array_equal(cso, rcso)
    # sequences that are not split give the bits of the unsplit call
    o0, fs0, _ = gpu_prefill(x)
    cu = x.cu_seqlens
    for n, L in enumerate(lengths):
        if _segments(L, seg) == 1:
            assert np.array_equal(o[cu[n]:cu[n + 1]], o0[cu[n]:cu[n + 1]]), n
            assert np.array_equal(fs[n], fs0[n]), n


def test_split_gqa_beta_logits_and_scale(oracle_mod):
    x = prefill_inputs(85, [520, 90, 1000], Geometry(1, 3, 128, 128), "bf16", initial_state_std=0.02,
                       conv_state=True)
    o, fs, _ = gpu_prefill(x, segment_chunks=2, scale=0.07)
    ro, rfs, _ = oracle_prefill(oracle_mod, x, scale=0.07)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(fs, rfs) <= TOL["bf16"]


def test_split_batch_invariance_bitwise():
    geom = Geometry(2, 4, 128, 128)
    targets = [(900, 1300), (901, 200), (902, 640)]  # (sequence id, length): 21, 4 and 10 chunks
    seg = 4
    alone = {}
    for sid, L in targets:
        x = prefill_inputs(86, [L], geom, "bf16", seq_ids=[sid], initial_state_std=0.02)
        o, fs, _ = gpu_prefill(x, segment_chunks=seg)
        alone[sid] = (o, fs[0])
    rng = np.random.default_rng(86)
    for batch in (3, 7):
        lengths = [int(v) for v in rng.integers(1, 900, size=batch)]
        seq_ids = list(range(batch))
        for (sid, L), pos in zip(targets, sorted(rng.choice(batch + 3, size=3, replace=False))):
            lengths.insert(pos, L)
            seq_ids.insert(pos, sid)
        x = prefill_inputs(86, lengths, geom, "bf16", seq_ids=seq_ids, initial_state_std=0.02)
        o, fs, _ = gpu_prefill(x, segment_chunks=seg)
        for sid, _ in targets:
            n = seq_ids.index(sid)
            s = slice(int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1]))
            assert np.array_equal(o[s], alone[sid][0]), (batch, sid)
            assert np.array_equal(fs[n], alone[sid][1]), (batch, sid)


def test_split_bf16_output_is_rounded_once():
    x = prefill_inputs(87, [900, 130], Geometry(2, 4, 128, 128), "bf16", initial_state_std=0.02)
    o16, f16, _ = gpu_prefill(x, out_dtype=torch.bfloat16, segment_chunks=3)
    o32, f32, _ = gpu_prefill(x, segment_chunks=3)
    assert np.array_equal(o16, bf16_round(o32))
    assert np.array_equal(f16, f32)


def test_split_pooled(oracle_mod):
    geom = Geometry(2, 4, 128, 128)
    lengths = [800, 5, 300]
    idx = np.array([2, -1, 0], dtype=np.int32)
    P = 3
    dt = TORCH_DT["bf16"]
    x = prefill_inputs(88, lengths, geom, "bf16")
    pool_np, cpool_np = state_pool(88, P, geom), conv_state_pool(88, P, geom, "bf16")
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    o = binding.gdn_prefill_varlen_pooled(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), torch.from_numpy(x.cu_seqlens.astype(np.int32)),
        pool, state_indices=dev(idx, torch.int32), conv_weight=dev(x.conv_w, dt), conv_state_pool=cpool,
        segment_chunks=4)
    torch.cuda.synchronize()
    h0 = np.stack([pool_np[i] if i >= 0 else np.zeros_like(pool_np[0]) for i in idx])
    cs0 = np.stack([cpool_np[i] if i >= 0 else np.zeros_like(cpool_np[0]) for i in idx])
    dims = oracle_mod.Dims(2, 4, 128, 128, conv_width=4)
    ro, rfs, rcso = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, None, cs0, h0)
    assert rel_err(o.cpu().numpy(), ro) <= TOL["bf16"]
    pa = pool.cpu().numpy()
    assert rel_err(pa[[2, 0]], rfs[[0, 2]]) <= TOL["bf16"]
    assert np.array_equal(cpool.float().cpu().numpy()[[2, 0]], rcso[[0, 2]].astype(np.float32))
    assert np.array_equal(pa[1], pool_np[1])  # entry 1 untouched


def test_split_long_sequence_32768_whole(oracle_mod):
    """One sequence of 32768 tokens (512 chunks) with segment_chunks = 256: two
    segments of 256 chunks.  Whole output and final state vs the oracle."""
    geom = Geometry(16, 32, 128, 128)
    x = prefill_inputs(42, [32768], geom, "bf16", initial_state_std=0.02)
    o, fs, _ = gpu_prefill(x, segment_chunks=256)
    ro, rfs, _ = oracle_prefill(oracle_mod, x)
    eo, ef = rel_err(o, ro), rel_err(fs, rfs)
    print(f"  32768 tokens, 2 segments: rel err o={eo:.3e} final={ef:.3e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
