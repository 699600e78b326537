"""GPU parity over seeded combinations of the entry points' options.

Prefill: each case draws its geometry (key heads 1..4, group size 1..4, d_k
and d_v each 64 or 128), bf16 or fp32 inputs, 1..6 sequences mixing the chunk
edges with lengths up to 1300, conv on or off with or without carried conv
state, initial states, raw gate logits, a custom scale, the segment split (0,
1, 2, 3 or 5 chunks per segment) and the entry point: with a workspace,
allocation-free, or over a state pool (permuted entries, some new sequences,
some without an entry).  Decode: single steps with skipped slots and m-token
calls (m up to 8) with accepted counts and unwritten entries, fp32 or bf16
outputs.  Everything is
compared with the fp64 oracle (max|delta| / rms within the dtype's bound; conv
states bit-exact; pool entries no sequence owns untouched).
"""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import Geometry, conv_state_pool, gate_logits, prefill_inputs, state_pool
from tests.gpu_util import TOL, TORCH_DT, canary, dev, rel_err

pytestmark = pytest.mark.gpu

EDGE = [0, 1, 2, 3, 63, 64, 65, 127, 128, 129, 191, 192, 193]


def _prefill_case(i):
    r = np.random.default_rng([4243, i])
    h_k, G = int(r.integers(1, 5)), int(r.integers(1, 5))
    c = dict(geom=Geometry(h_k, h_k * G, int(r.choice([64, 128])), int(r.choice([64, 128]))),
             dtype=str(r.choice(["bf16", "f32"])))
    c["lengths"] = [int(r.choice(EDGE)) if r.random() < 0.5 else int(r.integers(1, 1301))
                    for _ in range(int(r.integers(1, 7)))]
    c["conv"] = bool(r.random() < 0.8)
    c["initial"] = bool(r.random() < 0.6)
    c["conv_state"] = c["conv"] and bool(r.random() < 0.6)
    c["logits"] = bool(r.random() < 0.3)
    c["scale"] = 0.07 if r.random() < 0.3 else None
    c["segment_chunks"] = int(r.choice([0, 1, 2, 3, 5]))
    c["path"] = str(r.choice(["workspace", "noalloc", "pooled"]))
    c["rng"] = r
    return c


@pytest.mark.parametrize("case", range(48))
def test_prefill_combination(oracle_mod, case):
    c = _prefill_case(case)
    r, geom, dtype, path, seg = c["rng"], c["geom"], c["dtype"], c["path"], c["segment_chunks"]
    print(f"  case {case}: { {k: v for k, v in c.items() if k != 'rng'} }", flush=True)
    x = prefill_inputs(9500 + case, c["lengths"], geom, dtype, conv=c["conv"],
                       initial_state_std=0.02 if c["initial"] else None, conv_state=c["conv_state"])
    dt = TORCH_DT[dtype]
    N, T = x.num_seqs, x.total_tokens
    beta_in = gate_logits(9500 + case, T, geom.h_v) if c["logits"] else x.beta
    beta_ref = 1.0 / (1.0 + np.exp(-beta_in.astype(np.float64))) if c["logits"] else x.beta
    if path == "noalloc":
        prob = binding.make_problem(N, T, geom.h_k, geom.h_v, geom.d_k, geom.d_v, 1 if dtype == "bf16" else 0, 0,
                                    segment_chunks=seg)
        if binding.gdn_prefill_workspace_bytes(prob) > binding.NOALLOC_SCRATCH_BYTES:
            path = "workspace"
    args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(beta_in))
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32))
    w = dev(x.conv_w, dt) if c["conv"] else None
    owned = np.ones(N, dtype=bool)  # sequences whose final states are written somewhere
    if path == "pooled":
        P = N + 3
        idx = r.permutation(P)[:N].astype(np.int32)
        has = (r.random(N) < 0.8).astype(np.int32)
        if N > 1 and r.random() < 0.3:
            idx[int(r.integers(0, N))] = -1
        owned = idx >= 0
        pool_np = state_pool(9600 + case, P, geom)
        cpool_np = conv_state_pool(9600 + case, P, geom, dtype)
        pool, cpool = dev(pool_np), dev(cpool_np, dt)
        o = binding.gdn_prefill_varlen_pooled(*args, cu, pool, state_indices=dev(idx, torch.int32),
                                              has_initial_state=dev(has, torch.int32), conv_weight=w,
                                              conv_state_pool=cpool if c["conv"] else None, scale=c["scale"],
                                              beta_logits=c["logits"], segment_chunks=seg)
        torch.cuda.synchronize()
        h0 = np.zeros((N, geom.h_v, geom.d_k, geom.d_v), np.float32)
        cs0 = np.zeros((N, geom.channels, 3), np.float32)
        for n in range(N):
            if idx[n] >= 0 and has[n]:
                h0[n], cs0[n] = pool_np[idx[n]], cpool_np[idx[n]]
        o = o.float().cpu().numpy()
        pool_after, cpool_after = pool.cpu().numpy(), cpool.float().cpu().numpy()
        fs = np.stack([pool_after[i] if i >= 0 else np.zeros_like(pool_after[0]) for i in idx])
        cso = np.stack([cpool_after[i] if i >= 0 else np.zeros_like(cpool_after[0]) for i in idx])
        for e in sorted(set(range(P)) - set(idx.tolist())):
            assert np.array_equal(pool_after[e], pool_np[e]), f"pool entry {e} changed"
            assert np.array_equal(cpool_after[e], cpool_np[e]), f"conv pool entry {e} changed"
        use_h0, use_cs0 = h0, (cs0 if c["conv"] else None)
    else:
        o0 = canary((T, geom.h_v, geom.d_v), torch.float32)
        fs0 = canary((N, geom.h_v, geom.d_k, geom.d_v), torch.float32)
        cso0 = canary((N, geom.channels, 3), dt) if c["conv"] else None
        o, fs, cso = binding.gdn_prefill_varlen(
            *args, cu, conv_weight=w, conv_state=dev(x.conv_state_in, dt) if c["conv_state"] else None,
            initial_state=dev(x.initial_state) if c["initial"] else None, scale=c["scale"], beta_logits=c["logits"],
            out=o0, final_state_out=fs0, conv_state_out=cso0, noalloc=path == "noalloc", segment_chunks=seg)
        torch.cuda.synchronize()
        o, fs = o.cpu().numpy(), fs.cpu().numpy()
        cso = cso.float().cpu().numpy() if c["conv"] else None
        use_h0 = x.initial_state if c["initial"] else None
        use_cs0 = x.conv_state_in if c["conv_state"] else None
    dims = oracle_mod.Dims(geom.h_k, geom.h_v, geom.d_k, geom.d_v, conv_width=4 if c["conv"] else 0, scale=c["scale"])
    ro, rfs, rcso = oracle_mod.prefill(dims, x.cu_seqlens, x.q, x.k, x.v, x.g, beta_ref,
                                       x.conv_w if c["conv"] else None, None, use_cs0, use_h0)
    eo, ef = rel_err(o, ro), rel_err(fs[owned], rfs[owned])
    print(f"  path {path}: rel err o={eo:.3e} final={ef:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(fs))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
    if c["conv"]:
        assert np.array_equal(cso[owned], rcso[owned])


@pytest.mark.parametrize("case", range(24))
def test_decode_combination(oracle_mod, case):
    r = np.random.default_rng([778, case])
    h_k, G = int(r.integers(1, 5)), int(r.integers(1, 5))
    d_k, d_v = int(r.choice([64, 128])), int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f32"]))
    N, m = int(r.integers(1, 40)), int(r.integers(1, 9))
    conv, logits = bool(r.random() < 0.8), bool(r.random() < 0.3)
    single = m == 1 and bool(r.random() < 0.5)
    out = str(r.choice(["f32", "bf16"]))
    print(f"  case {case}: h_k={h_k} G={G} d_k={d_k} d_v={d_v} {dtype} N={N} m={m} conv={conv} "
          f"logits={logits} single={single} out={out}", flush=True)
    geom = Geometry(h_k, h_k * G, d_k, d_v)
    hv, C, dt = geom.h_v, geom.channels, TORCH_DT[dtype]

    def draw(*shape):
        a = r.standard_normal(shape).astype(np.float32)
        return torch.from_numpy(a).to(torch.bfloat16).float().numpy() if dtype == "bf16" else a

    q, k, v = draw(N, m, h_k, d_k), draw(N, m, h_k, d_k), draw(N, m, hv, d_v)
    g = (-np.log1p(np.exp(r.standard_normal((N, m, hv))))).astype(np.float32)
    braw = r.standard_normal((N, m, hv)).astype(np.float32)
    beta = braw if logits else (1.0 / (1.0 + np.exp(-braw.astype(np.float64)))).astype(np.float32)
    beta_ref = 1.0 / (1.0 + np.exp(-braw.astype(np.float64))) if logits else beta
    w = 0.5 * draw(C, 4) if conv else None
    P = N * m + 5
    pool_np = (0.02 * r.standard_normal((P, hv, d_k, d_v))).astype(np.float32)
    cpool_np = draw(P, C, 3)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    rpool, rcpool = pool_np.astype(np.float64), cpool_np.astype(np.float64)
    dims = oracle_mod.Dims(h_k, hv, d_k, d_v, conv_width=4 if conv else 0)
    wt = dev(w, dt) if conv else None
    if single:
        idx = r.permutation(P)[:N].astype(np.int32)
        if N > 1:
            idx[int(r.integers(0, N))] = -1
        o = binding.gdn_decode_step(dev(q[:, 0], dt), dev(k[:, 0], dt), dev(v[:, 0], dt), dev(g[:, 0]),
                                    dev(beta[:, 0]), pool, state_indices=dev(idx, torch.int32), conv_weight=wt,
                                    conv_state_pool=cpool if conv else None, beta_logits=logits,
                                    out_dtype=TORCH_DT[out])
        torch.cuda.synchronize()
        ro = oracle_mod.decode(dims, q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta_ref[:, 0], rpool, idx,
                               w if conv else None, None, rcpool if conv else None)
        live = idx >= 0
        o, ro = o.float().cpu().numpy()[live], ro[live]
    else:
        idx = r.permutation(P)[:N * m].astype(np.int32).reshape(N, m)
        acc = r.integers(1, m + 1, N).astype(np.int32)
        for n in range(N):
            for j in range(m):
                if j != acc[n] - 1 and r.random() < 0.2:
                    idx[n, j] = -1
        o = binding.gdn_decode_multi(dev(q, dt), dev(k, dt), dev(v, dt), dev(g), dev(beta), pool,
                                     state_indices=dev(idx, torch.int32), num_accepted=dev(acc, torch.int32),
                                     conv_weight=wt, conv_state_pool=cpool if conv else None, beta_logits=logits,
                                     out_dtype=TORCH_DT[out])
        torch.cuda.synchronize()
        ro = oracle_mod.decode_multi(dims, q, k, v, g, beta_ref, rpool, idx, acc, w if conv else None, None,
                                     rcpool if conv else None)
        o = o.float().cpu().numpy()
    eo, ep = rel_err(o, ro), rel_err(pool.cpu().numpy(), rpool)
    print(f"  rel err o={eo:.3e} pool={ep:.3e}", flush=True)
    assert np.all(np.isfinite(o))
    if out == "bf16":
        # bf16 o is the fp32 result rounded once: within one bf16 ulp of the oracle beyond the dtype's bound
        assert np.all(np.abs(o - ro) <= np.abs(ro) * 2.0 ** -8 + TOL[dtype] * np.sqrt(np.mean(ro ** 2)))
    else:
        assert eo <= TOL[dtype]
    assert ep <= TOL[dtype]
    if conv:
        assert np.array_equal(cpool.float().cpu().numpy(), rcpool.astype(np.float32))
