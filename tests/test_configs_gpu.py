"""GPU parity at the full sizes of the packed varlen and batch-invariance
workloads, in the launch configuration the benchmark uses (one call of
gdn_prefill_varlen over the whole packed batch).

* Packed varlen prefill: 60 sequences with lengths drawn uniformly from
  1..8192, h_k = 16, h_v = 48 (3 value heads per key head), d = 128, bf16
  q/k/v, fp32 g/beta, per-sequence initial states ~ 0.02 N(0, 1).  Every
  sequence is checked against the oracle on one key head (and its 3 value
  heads), the key head rotating with the sequence index.
* Batch invariance: 8 fixed target sequences of 2048 tokens (h_k = 16,
  h_v = 32, d = 128, bf16) alone, packed together, and at random positions
  inside a packed batch of 60 with filler sequences of length 1..8192: their
  outputs and final states must be bit-identical across all batchings.
* Long context: one sequence of 32768 tokens at the same geometry, the whole
  output and final state against the oracle.
* Offsets past 32 bits: a short sequence packed after 540,032 tokens, whose
  output rows start beyond element 2^31 of o, against the oracle and against
  a call that holds it alone (bitwise).
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, prefill_inputs, uniform_lengths
from tests.gpu_util import TOL, canary_outputs, dev, head_slice, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _run(x):
    """One prefill call over the whole packed batch, outputs and workspace
    pre-filled with NaN bytes; device tensors back."""
    o0, fs0, _, ws = canary_outputs(x, conv=False)
    o, fs, _ = binding.gdn_prefill_varlen(
        dev(x.q, BF), dev(x.k, BF), dev(x.v, BF), dev(x.g), dev(x.beta),
        torch.from_numpy(x.cu_seqlens.astype(np.int32)), conv_weight=dev(x.conv_w, BF),
        initial_state=None if x.initial_state is None else dev(x.initial_state), output_conv_state=False,
        out=o0, final_state_out=fs0, workspace=ws)
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
    _check_units(oracle_mod, x, o, fs, [(n, n % 16) for n in range(60)], "60 packed")


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
    ro, rfs, _ = oracle_prefill(oracle_mod, x)
    eo, ef = rel_err(o.cpu().numpy(), ro), rel_err(fs.cpu().numpy(), rfs)
    print(f"  32768 tokens, whole: rel err o={eo:.3e} final={ef:.3e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_offsets_beyond_32_bits(oracle_mod):
    """A 100-token sequence packed after one of 540,032 tokens (h_k = 16, h_v =
    32, d = 128, bf16): its output rows start at element 2.2e9 (> 2^31) of o and
    its K|Q image at byte 8.8e9, so every offset past 32 bits is exercised.  The
    short sequence (with initial recurrent and conv states) must match the
    oracle and be bit-identical to a call that holds it alone; the long one's
    outputs and final state must be finite.  The long sequence's inputs are
    drawn on the device (q, k, v ~ N(0, 1) in bf16, beta = sigmoid(N(0, 1)),
    g = -softplus(N(0, 1))); ~36 GB of device memory."""
    geom = Geometry(16, 32, 128, 128)
    long_len = 540_032
    xs = prefill_inputs(61, [100], geom, "bf16", initial_state_std=0.02, conv_state=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(61)
    rn = lambda *shape: torch.randn(*shape, generator=gen, device="cuda", dtype=torch.float32)
    T = long_len + 100
    q = torch.empty((T, 16, 128), dtype=BF, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, 32, 128), dtype=BF, device="cuda")
    g = torch.empty((T, 32), dtype=torch.float32, device="cuda")
    beta = torch.empty_like(g)
    for lo in range(0, long_len, 1 << 16):
        hi = min(lo + (1 << 16), long_len)
        q[lo:hi], k[lo:hi], v[lo:hi] = rn(hi - lo, 16, 128), rn(hi - lo, 16, 128), rn(hi - lo, 32, 128)
        g[lo:hi] = -torch.nn.functional.softplus(rn(hi - lo, 32))
        beta[lo:hi] = torch.sigmoid(rn(hi - lo, 32))
    q[long_len:], k[long_len:], v[long_len:] = dev(xs.q, BF), dev(xs.k, BF), dev(xs.v, BF)
    g[long_len:], beta[long_len:] = dev(xs.g), dev(xs.beta)
    C = geom.channels
    h0 = torch.zeros((2, 32, 128, 128), dtype=torch.float32, device="cuda")
    h0[1] = dev(xs.initial_state[0])
    cs0 = torch.zeros((2, C, 3), dtype=BF, device="cuda")
    cs0[1] = dev(xs.conv_state_in[0], BF)
    w = dev(xs.conv_w, BF)
    cu = torch.tensor([0, long_len, T], dtype=torch.int32)

    o, fs, cso = binding.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, conv_state=cs0, initial_state=h0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o[:long_len]).all()) and bool(torch.isfinite(fs[0]).all())
    o_tail, fs_tail, cso_tail = o[long_len:].cpu().numpy(), fs[1].cpu().numpy(), cso[1].float().cpu().numpy()
    del o, fs, q, k, v, g, beta
    torch.cuda.empty_cache()

    o1, fs1, cso1 = binding.gdn_prefill_varlen(
        dev(xs.q, BF), dev(xs.k, BF), dev(xs.v, BF), dev(xs.g), dev(xs.beta),
        torch.from_numpy(xs.cu_seqlens.astype(np.int32)), conv_weight=w,
        conv_state=dev(xs.conv_state_in, BF), initial_state=dev(xs.initial_state))
    torch.cuda.synchronize()
    assert np.array_equal(o_tail, o1.cpu().numpy())
    assert np.array_equal(fs_tail, fs1[0].cpu().numpy())
    assert np.array_equal(cso_tail, cso1[0].float().cpu().numpy())

    ro, rfs, rcso = oracle_prefill(oracle_mod, xs)
    eo, ef = rel_err(o_tail, ro), rel_err(fs_tail, rfs[0])
    print(f"  tail sequence at token {long_len}: rel err o={eo:.3e} final={ef:.3e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    assert np.array_equal(cso_tail, rcso[0])
