"""The C ABI calls inside a captured HIP graph (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream (no allocation,
no memset, no synchronisation), so a prefill and a decode step can be captured
once and replayed.  Each replay is checked bit for bit against the same call
made eagerly, with eager work (output clears, new input values copied into the
captured buffers) between the replays.
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import (Geometry, conv_state_pool, conv_weights, decode_inputs,
                                                    prefill_inputs, state_pool)
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


@pytest.mark.parametrize("mode", ["workspace", "noalloc", "segment_split"])
def test_prefill_graph_replays_match_eager(mode):
    """Captured prefill with a caller workspace, with the library's static
    scratch (the allocation-free entry point), and with the segment split
    (its chain map and combine kernels in the graph)."""
    geom = Geometry(2, 4, 128, 128)
    lengths = [70, 130, 3, 64]
    xs = [prefill_inputs(80 + i, lengths, geom, "bf16", initial_state_std=0.02, conv_state=True) for i in range(3)]
    x = xs[0]
    N, T = len(lengths), x.total_tokens
    q, k, v = dev(x.q, BF), dev(x.k, BF), dev(x.v, BF)
    g, beta = dev(x.g), dev(x.beta)
    w, cs, h0 = dev(x.conv_w, BF), dev(x.conv_state_in, BF), dev(x.initial_state)
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32)).cuda()
    seg = 1 if mode == "segment_split" else 0  # one chunk per segment: every multi-chunk sequence splits
    prob = binding.make_problem(N, T, 2, 4, 128, 128, 1, 0, segment_chunks=seg)
    ws = None if mode == "noalloc" else torch.empty(binding.gdn_prefill_workspace_bytes(prob), dtype=torch.uint8,
                                                     device="cuda")
    o = torch.empty((T, 4, 128), device="cuda")
    fs = torch.empty((N, 4, 128, 128), device="cuda")
    cso = torch.empty((N, geom.channels, 3), dtype=BF, device="cuda")

    def call(out, fso, csout):
        binding.gdn_prefill_varlen(q, k, v, g, beta, cu, conv_weight=w, conv_state=cs, initial_state=h0, out=out,
                                   final_state_out=fso, conv_state_out=csout, workspace=ws, validate=False,
                                   noalloc=mode == "noalloc", segment_chunks=seg)

    def load(xi):
        for dst, src, dt in ((q, xi.q, BF), (k, xi.k, BF), (v, xi.v, BF), (g, xi.g, torch.float32),
                             (beta, xi.beta, torch.float32), (cs, xi.conv_state_in, BF),
                             (h0, xi.initial_state, torch.float32)):
            dst.copy_(dev(src, dt))

    # eager references for the three input sets
    refs = []
    for xi in xs:
        load(xi)
        ro, rf, rc = torch.empty_like(o), torch.empty_like(fs), torch.empty_like(cso)
        call(ro, rf, rc)
        torch.cuda.synchronize()
        refs.append((ro, rf, rc))

    load(xs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(o, fs, cso)  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o, fs, cso)
    for rep in range(6):
        i = rep % 3
        load(xs[i])
        o.zero_()
        fs.zero_()
        cso.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ro, rf, rc = refs[i]
        assert torch.equal(o, ro), f"replay {rep}: o"
        assert torch.equal(fs, rf), f"replay {rep}: final state"
        assert torch.equal(cso, rc), f"replay {rep}: conv state"


def test_decode_graph_replays_match_eager():
    """A captured decode step (state and conv pools updated in place) replayed
    five times equals five eager steps, bit for bit, after every step."""
    geom = Geometry(16, 32, 128, 128)
    N, P = 64, 80
    pool_np = state_pool(81, P, geom)
    cpool_np = conv_state_pool(81, P, geom, "bf16")
    w = dev(conv_weights(81, geom, "bf16"), BF)
    idx = dev(np.random.default_rng(81).permutation(P)[:N].astype(np.int32), torch.int32)
    x = decode_inputs(81, 0, N, geom, "bf16")
    q, k, v, g, beta = dev(x.q, BF), dev(x.k, BF), dev(x.v, BF), dev(x.g), dev(x.beta)
    pool_e, cpool_e = dev(pool_np), dev(cpool_np, BF)
    pool_g, cpool_g = dev(pool_np), dev(cpool_np, BF)
    o_e = torch.empty((N, 32, 128), device="cuda")
    o_g = torch.empty_like(o_e)

    def step(pool, cpool, out):
        binding.gdn_decode_step(q, k, v, g, beta, pool, state_indices=idx, conv_weight=w, conv_state_pool=cpool,
                                out=out, validate=False)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    scratch_pool, scratch_cpool = pool_g.clone(), cpool_g.clone()
    with torch.cuda.stream(side):
        step(scratch_pool, scratch_cpool, o_g)  # warm-up outside the graph, on copies
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(pool_g, cpool_g, o_g)
    # capture records the work without running it: the pools are untouched
    assert torch.equal(pool_g, pool_e) and torch.equal(cpool_g, cpool_e)
    for rep in range(5):
        step(pool_e, cpool_e, o_e)
        o_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {rep}: o"
        assert torch.equal(pool_g, pool_e), f"replay {rep}: state pool"
        assert torch.equal(cpool_g, cpool_e), f"replay {rep}: conv pool"
