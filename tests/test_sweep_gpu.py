"""GPU parity over a seeded sweep of prefill configurations.

Each case draws its geometry and options from its own seed: key heads 1..4,
group size 1..4, d_k and d_v each in {64, 128}, bf16 or fp32 inputs, 1..6 sequences whose
lengths mix the chunk edges (0, 1, 63, 64, 65, 127, 128, 129) with random
lengths up to 400, conv on or off, with or without initial recurrent and conv
states, raw gate logits or beta, and the default or a custom scale.  The HIP
path (through the C ABI) is compared with the fp64 oracle on the whole output,
the final states (max|delta| / rms <= 1e-4 for fp32 inputs, 1e-2 for bf16) and
the conv states (bit-exact).  Outputs and workspace start as NaN bytes, so an
element the kernels do not write fails the comparison.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, gate_logits, prefill_inputs
from tests.gpu_util import TOL, TORCH_DT, canary_outputs, dev, rel_err

pytestmark = pytest.mark.gpu

EDGE_LENGTHS = [0, 1, 2, 3, 63, 64, 65, 127, 128, 129]
CASES = 32


def draw_case(i: int) -> dict:
    r = np.random.default_rng([7919, i])
    h_k = int(r.integers(1, 5))
    G = int(r.integers(1, 5))
    d = int(r.choice([64, 128]))
    n = int(r.integers(1, 7))
    lengths = [int(r.choice(EDGE_LENGTHS)) if r.random() < 0.5 else int(r.integers(1, 401)) for _ in range(n)]
    conv = bool(r.random() < 0.75)
    c = dict(dtype=str(r.choice(["bf16", "f32"])), lengths=lengths, conv=conv, initial=bool(r.random() < 0.6),
             conv_state=conv and bool(r.random() < 0.6), logits=bool(r.random() < 0.3),
             scale=float(r.choice([0.0, 0.05])))
    d_v = int(r.choice([64, 128]))  # drawn last, so the earlier draws of a case keep their values
    c["geom"] = Geometry(h_k, h_k * G, d, d_v)
    return c


@pytest.mark.parametrize("case", range(CASES))
def test_prefill_sweep(oracle_mod, case):
    c = draw_case(case)
    print(f"  case {case}: {c}", flush=True)
    geom, dtype = c["geom"], c["dtype"]
    x = prefill_inputs(5000 + case, c["lengths"], geom, dtype, conv=c["conv"],
                       initial_state_std=0.02 if c["initial"] else None, conv_state=c["conv_state"])
    beta_in = gate_logits(5000 + case, x.total_tokens, geom.h_v) if c["logits"] else x.beta
    scale = c["scale"] if c["scale"] > 0 else None

    dt = TORCH_DT[dtype]
    o0, fs0, cso0, ws = canary_outputs(x, conv=c["conv"])
    o, fs, cso = binding.gdn_prefill_varlen(
        dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(beta_in),
        torch.from_numpy(x.cu_seqlens.astype(np.int32)),
        conv_weight=dev(x.conv_w, dt) if c["conv"] else None,
        conv_state=dev(x.conv_state_in, dt) if c["conv_state"] else None,
        initial_state=dev(x.initial_state) if c["initial"] else None,
        scale=scale, beta_logits=c["logits"], out=o0, final_state_out=fs0, conv_state_out=cso0, workspace=ws)
    torch.cuda.synchronize()

    # with raw logits the oracle takes beta = sigmoid(b) in fp64
    beta_ref = 1.0 / (1.0 + np.exp(-beta_in.astype(np.float64))) if c["logits"] else x.beta
    dims = oracle_mod.Dims(geom.h_k, geom.h_v, geom.d_k, geom.d_v, conv_width=4 if c["conv"] else 0, scale=scale)
    ro, rfs, rcso = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, beta_ref,
                                       x.conv_w if c["conv"] else None, None,
                                       x.conv_state_in if c["conv_state"] else None,
                                       x.initial_state if c["initial"] else None)
    o = o.float().cpu().numpy()
    eo, ef = rel_err(o, ro), rel_err(fs.cpu().numpy(), rfs)
    print(f"  rel err o={eo:.3e} final_state={ef:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert o.shape == ro.shape and np.all(np.isfinite(o)) and bool(torch.isfinite(fs).all())
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
    if c["conv"]:
        assert np.array_equal(cso.float().cpu().numpy(), rcso)
