"""GPU parity at the full sizes of the packed varlen and batch-invariance
workloads, in the launch configuration the benchmark uses (one call of
gdn_prefill_varlen over the whole packed batch).

* Packed varlen prefill: 60 sequences with lengths drawn uniformly from
  1..8192, h_k = 16, h_v = 48 (3 value heads per key head), d = 128, bf16
  q/k/v, fp32 g/beta, per-sequence initial states ~ 0.02 N(0, 1).  Sampled
  (sequence, key head) units are recomputed by the oracle alone.
* Batch invariance: 8 fixed target sequences of 2048 tokens (h_k = 16,
  h_v = 32, d = 128, bf16) alone, packed together, and at random positions
  inside a packed batch of 60 with filler sequences of length 1..8192: their
  outputs and final states must be bit-identical across all batchings.
* Long context: one sequence of 32768 tokens at the same geometry, sampled
  against the oracle.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, prefill_inputs, uniform_lengths
from tests.gpu_util import TOL, dev, head_slice, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _run(x):
    """One prefill call over the whole packed batch; device tensors back."""
    o, fs, _ = binding.gdn_prefill_varlen(
        dev(x.q, BF), dev(x.k, BF), dev(x.v, BF), dev(x.g), dev(x.beta),
        torch.from_numpy(x.cu_seqlens.astype(np.int32)), conv_weight=dev(x.conv_w, BF),
        initial_state=None if x.initial_state is None else dev(x.initial_state), output_conv_state=False)
    torch.cuda.synchronize()
    return o, fs


def _check_units(oracle_mod, x, o, fs, units, label):
    G = x.geom.h_v // x.geom.h_k
    for n, hk in units:
        xs = head_slice(x, n, hk)
        ro, rfs, _ = oracle_prefill(oracle_mod, xs)
        s = slice(int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1]))
        hv = slice(G * hk, G * hk + G)
        eo = rel_err(o[s, hv].float().cpu().numpy(), ro)
        ef = rel_err(fs[n, hv].cpu().numpy(), rfs[0])
        print(f"  {label}: seq {n} (len {s.stop - s.start}) key head {hk}: rel err o={eo:.3e} final={ef:.3e}",
              flush=True)
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_packed_varlen_60_sequences_hv48(oracle_mod):
    geom = Geometry(16, 48, 128, 128)
    lengths = uniform_lengths(20, 60, 1, 8192)
    x = prefill_inputs(20, lengths, geom, "bf16", initial_state_std=0.02)
    print(f"  {x.total_tokens} tokens, lengths {int(lengths.min())}..{int(lengths.max())}", flush=True)
    o, fs = _run(x)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(fs).all())
    longest, shortest = int(np.argmax(lengths)), int(np.argmin(lengths))
    _check_units(oracle_mod, x, o, fs, [(longest, 0), (shortest, 15), (30, 7)], "60 packed")


def test_batch_invariance_targets_across_batchings(oracle_mod):
    geom = Geometry(16, 32, 128, 128)
    rng = np.random.default_rng(41)
    targets = list(range(8))                      # sequence ids of the 8 targets
    fill_ids = list(range(100, 152))              # 52 fillers
    fill_len = uniform_lengths(41, 52, 1, 8192)
    # batch of 60: targets at random positions among the fillers
    order60 = rng.permutation(60)
    ids60 = [(targets + fill_ids)[i] for i in order60]
    lens60 = [2048 if i < 8 else int(fill_len[i - 8]) for i in order60]
    order8 = rng.permutation(8)
    ids8 = [targets[i] for i in order8]

    def target_results(ids, lens):
        x = prefill_inputs(41, lens, geom, "bf16", seq_ids=ids, initial_state_std=0.02)
        o, fs = _run(x)
        out = {}
        for pos, sid in enumerate(ids):
            if sid in targets:
                s = slice(int(x.cu_seqlens[pos]), int(x.cu_seqlens[pos + 1]))
                out[sid] = (o[s].clone(), fs[pos].clone())
        return out, x

    alone = {}
    for sid in targets:
        r, x1 = target_results([sid], [2048])
        alone.update(r)
        if sid == 0:
            x_alone0, o0, fs0 = x1, r[0][0], r[0][1]
    in8, _ = target_results(ids8, [2048] * 8)
    in60, _ = target_results(ids60, lens60)
    for sid in targets:
        for other, name in ((in8, "8"), (in60, "60")):
            assert torch.equal(alone[sid][0], other[sid][0]), f"target {sid}: o differs in the batch of {name}"
            assert torch.equal(alone[sid][1], other[sid][1]), f"target {sid}: final state differs in the batch of {name}"
    _check_units(oracle_mod, x_alone0, o0, fs0[None], [(0, 3)], "target alone")


def test_long_sequence_32768(oracle_mod):
    geom = Geometry(16, 32, 128, 128)
    x = prefill_inputs(42, [32768], geom, "bf16", initial_state_std=0.02)
    o, fs = _run(x)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(fs).all())
    _check_units(oracle_mod, x, o, fs, [(0, 5)], "32768 tokens")
