"""Writes tests/golden/oracle_tiny.json from the fp64 oracle alone.

The pages print no numeric example of the recurrence, so this file holds no
page values; it is a regression lock on the oracle for a tiny seeded case
(2 sequences of 10 and 5 tokens, h_k=1, h_v=2, d_k=d_v=8, fp32 inputs, conv
width 4, q/k L2-normalised, initial states 0.02*N(0,1)).  Run:
    python -m tests.golden.make_golden
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def compute(oracle):
    from gateddeltanet_chunked_delta_amd.inputs import Geometry, prefill_inputs
    geom = Geometry(1, 2, 8, 8)
    x = prefill_inputs(424242, [10, 5], geom, "f32", initial_state_std=0.02, conv_state=True)
    dims = oracle.Dims(1, 2, 8, 8, conv_width=4, qk_l2norm=True)
    o, fs, cso = oracle.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, x.beta, x.conv_w, None,
                                x.conv_state_in, x.initial_state)
    return {"o": o.tolist(), "final_state": fs.tolist(), "conv_state_out": cso.tolist()}


if __name__ == "__main__":
    import oracle
    out = {"source": "fp64 oracle (oracle/gdn_oracle.c), tests/golden/make_golden.py",
           "values": compute(oracle)}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json"), "w") as f:
        json.dump(out, f)
    print("wrote oracle_tiny.json")
