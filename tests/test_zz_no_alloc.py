"""GPU test of gdn_prefill_varlen_noalloc, the prefill entry point that takes no
workspace and allocates nothing (its workspace is the library's static device
scratch).

Two calls in a row through the C ABI, the second on a smaller problem (so the
second reads scratch memory the first left behind), without and with the
segment split: each must give, bit for bit, the outputs, final states and
conv states of gdn_prefill_varlen with a caller workspace on the same inputs,
and meet the oracle's bar.  A problem
whose workspace exceeds the scratch is refused with GDN_ERR_SCRATCH.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, prefill_inputs
from tests.gpu_util import TOL, TORCH_DT, canary_outputs, dev, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


def _call(x, noalloc, segment_chunks=0):
    dt = TORCH_DT[x.dtype]
    o, fs, cso, ws = canary_outputs(x, segment_chunks=segment_chunks)
    binding.gdn_prefill_varlen(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta),
        torch.from_numpy(x.cu_seqlens.astype(np.int32)), conv_weight=dev(x.conv_w, dt),
        conv_state=dev(x.conv_state_in, dt), initial_state=dev(x.initial_state), out=o, final_state_out=fs,
        conv_state_out=cso, workspace=None if noalloc else ws, noalloc=noalloc, segment_chunks=segment_chunks)
    torch.cuda.synchronize()
    return o.cpu().numpy(), fs.cpu().numpy(), cso.float().cpu().numpy()


def test_noalloc_matches_workspace_entry_point(oracle_mod):
    geom = Geometry(4, 8, 128, 128)
    big = prefill_inputs(70, [700, 1, 64, 300, 129], geom, "bf16", initial_state_std=0.02, conv_state=True)
    small = prefill_inputs(71, [90, 3], geom, "bf16", initial_state_std=0.02, conv_state=True)
    assert binding.gdn_prefill_workspace_bytes(binding.make_problem(5, big.total_tokens, 4, 8, 128, 128, 1, 0)) \
        <= binding.NOALLOC_SCRATCH_BYTES
    for x in (big, small):
        na = _call(x, noalloc=True)
        ws = _call(x, noalloc=False)
        for a, b in zip(na, ws):
            assert np.array_equal(a, b)
        ro, rfs, rcso = oracle_prefill(oracle_mod, x)
        eo, ef = rel_err(na[0], ro), rel_err(na[1], rfs)
        print(f"  {x.total_tokens} tokens: rel err o={eo:.3e} final={ef:.3e}", flush=True)
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
        assert np.array_equal(na[2], rcso)


def test_noalloc_fp32_mixed_dims(oracle_mod):
    x = prefill_inputs(72, [150, 40, 0, 64], Geometry(2, 4, 64, 128), "f32", initial_state_std=0.02,
                       conv_state=True)
    na = _call(x, noalloc=True)
    ws = _call(x, noalloc=False)
    for a, b in zip(na, ws):
        assert np.array_equal(a, b)
    ro, rfs, _ = oracle_prefill(oracle_mod, x)
    assert rel_err(na[0], ro) <= TOL["f32"] and rel_err(na[1], rfs) <= TOL["f32"]


def test_noalloc_with_segment_split(oracle_mod):
    # the split's chain map and segment buffers live in the scratch too; the
    # second, smaller call splits differently (4 then 2 chunks per segment)
    geom = Geometry(2, 4, 128, 128)
    first = prefill_inputs(73, [900, 50, 0], geom, "bf16", initial_state_std=0.02, conv_state=True)
    second = prefill_inputs(74, [300], geom, "bf16", initial_state_std=0.02, conv_state=True)
    for x, seg in ((first, 4), (second, 2)):
        na = _call(x, noalloc=True, segment_chunks=seg)
        ws = _call(x, noalloc=False, segment_chunks=seg)
        for a, b in zip(na, ws):
            assert np.array_equal(a, b)
        ro, rfs, rcso = oracle_prefill(oracle_mod, x)
        eo, ef = rel_err(na[0], ro), rel_err(na[1], rfs)
        print(f"  {x.total_tokens} tokens, {seg} chunks per segment: rel err o={eo:.3e} final={ef:.3e}", flush=True)
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
        assert np.array_equal(na[2], rcso)


def test_noalloc_refuses_problems_beyond_the_scratch():
    T = 8192
    bf = torch.bfloat16
    q = torch.zeros((T, 16, 128), dtype=bf, device="cuda")
    v = torch.zeros((T, 32, 128), dtype=bf, device="cuda")
    g = torch.zeros((T, 32), device="cuda")
    prob = binding.make_problem(1, T, 16, 32, 128, 128, 1, 0)
    assert binding.gdn_prefill_workspace_bytes(prob) > binding.NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.GdnError) as e:
        binding.gdn_prefill_varlen_noalloc(q, q.clone(), v, g, g.clone(), [0, T])
    assert e.value.status == -8
