"""Multi-token (speculative) decode through the C ABI (gdn_decode_multi):
parity with the fp64 oracle, the pool bookkeeping for rollback
(num_accepted), and bit-identity with single-token decode steps."""
import numpy as np
import pytest
import torch

from gateddeltanet_chunked_delta_amd import binding
from gateddeltanet_chunked_delta_amd.inputs import (Geometry, conv_state_pool, conv_weights, decode_inputs,
                                                    multi_decode_inputs, prefill_inputs, state_pool)
from tests.gpu_util import TOL, TORCH_DT, dev, rel_err

pytestmark = pytest.mark.gpu


def _multi(x, dt, pool, **kw):
    return binding.gdn_decode_multi(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta), pool, **kw)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("bf16", 64), ("f32", 64)])
def test_decode_multi_vs_oracle_with_rollback(oracle_mod, dtype, d):
    """Two 4-token calls over a pool with per-token entries: the second call
    resumes each slot from the entry of its last accepted token.  Covers a
    skipped slot, -1 (unkept) entries, an entry written twice in one call and
    a slot whose read entry is also written."""
    geom = Geometry(2, 4, d, d)
    N, m, P = 5, 4, 24
    dt = TORCH_DT[dtype]
    pool_np = state_pool(60, P, geom)
    cpool_np = conv_state_pool(60, P, geom, dtype)
    w_np = conv_weights(60, geom, dtype)
    idx = np.array([[0, 1, 2, 3], [4, 5, -1, 7], [-1, -1, -1, -1], [12, 13, 14, 12], [16, 17, 18, 19]],
                   dtype=np.int32)
    pool, cpool = dev(pool_np), dev(cpool_np, dt)
    ref_pool, ref_cpool = pool_np.astype(np.float64), cpool_np.astype(np.float64)
    dims = oracle_mod.Dims(2, 4, d, d, conv_width=4)
    for call, acc in enumerate(([1, 2, 1, 1, 3], [3, 2, 1, 4, 1])):
        x = multi_decode_inputs(60, call, N, m, geom, dtype)
        acc_np = np.array(acc, dtype=np.int32)
        o = _multi(x, dt, pool, state_indices=dev(idx, torch.int32), num_accepted=dev(acc_np, torch.int32),
                   conv_weight=dev(w_np, dt), conv_state_pool=cpool)
        ro = oracle_mod.decode_multi(dims, x.q, x.k, x.v, x.g, x.beta, ref_pool, idx, acc_np, w_np, None,
                                     ref_cpool)
        live = np.array([r[a - 1] >= 0 for r, a in zip(idx, acc)])
        e = rel_err(o.cpu().numpy()[live], ro[live])
        print(f"  call {call}: rel err o={e:.3e}", flush=True)
        assert e <= TOL[dtype]
    used = sorted({int(e) for e in idx.ravel() if e >= 0})
    got = pool.cpu().numpy()
    assert rel_err(got[used], ref_pool[used]) <= TOL[dtype]
    assert np.array_equal(cpool.float().cpu().numpy(), ref_cpool.astype(np.float32))
    untouched = [e for e in range(P) if e not in used]
    assert np.array_equal(got[untouched], pool_np[untouched])


@pytest.mark.parametrize("dtype,beta_logits,d_k,d_v,out", [
    ("bf16", False, 128, 128, "f32"), ("bf16", True, 128, 128, "f32"), ("f32", False, 128, 128, "f32"),
    ("f32", True, 128, 128, "f32"), ("bf16", False, 128, 128, "bf16"), ("bf16", False, 128, 64, "f32"),
    ("f32", True, 128, 64, "bf16"), ("bf16", False, 64, 128, "bf16"), ("bf16", True, 64, 64, "f32"),
    ("f32", False, 64, 64, "bf16")])
def test_decode_multi_bitwise_equals_single_steps(dtype, beta_logits, d_k, d_v, out):
    """m tokens in one call == m single-token gdn_decode_step calls, bit for
    bit (outputs, recurrent states and conv states), at each head size (the
    64-column instances sum their partials by quarter-waves) and output
    dtype."""
    geom = Geometry(2, 4, d_k, d_v)
    N, m = 6, 5
    dt, odt = TORCH_DT[dtype], TORCH_DT[out]
    pool_a = dev(state_pool(61, N, geom))
    pool_b = pool_a.clone()
    cpool_a = dev(conv_state_pool(61, N, geom, dtype), dt)
    cpool_b = cpool_a.clone()
    w = dev(conv_weights(61, geom, dtype), dt)
    x = multi_decode_inputs(61, 0, N, m, geom, dtype)
    o_multi = _multi(x, dt, pool_a, conv_weight=w, conv_state_pool=cpool_a, beta_logits=beta_logits,
                     out_dtype=odt)
    for j in range(m):
        o_j = binding.gdn_decode_step(dev(x.q[:, j], dt), dev(x.k[:, j], dt), dev(x.v[:, j], dt), dev(x.g[:, j]),
                                      dev(x.beta[:, j]), pool_b, conv_weight=w, conv_state_pool=cpool_b,
                                      beta_logits=beta_logits, out_dtype=odt)
        assert torch.equal(o_multi[:, j], o_j), j
    assert torch.equal(pool_a, pool_b)
    assert torch.equal(cpool_a, cpool_b)


def test_decode_multi_one_token_is_decode_step():
    geom = Geometry(2, 4, 128, 128)
    N = 7
    pool_a = dev(state_pool(62, N, geom))
    pool_b = pool_a.clone()
    x = multi_decode_inputs(62, 0, N, 1, geom, "bf16")
    idx = torch.tensor([[6], [5], [4], [-1], [2], [1], [0]], dtype=torch.int32, device="cuda")
    o_multi = _multi(x, torch.bfloat16, pool_a, state_indices=idx)
    o_step = binding.gdn_decode_step(dev(x.q[:, 0], torch.bfloat16), dev(x.k[:, 0], torch.bfloat16),
                                     dev(x.v[:, 0], torch.bfloat16), dev(x.g[:, 0]), dev(x.beta[:, 0]), pool_b,
                                     state_indices=idx[:, 0].contiguous())
    live = idx[:, 0] >= 0
    assert torch.equal(o_multi[live, 0], o_step[live])
    assert torch.equal(pool_a, pool_b)


def test_decode_multi_256_slots_sampled(oracle_mod):
    """256 slots x 32 value heads (16 key heads), d = 128, bf16 inputs, 4
    speculative tokens per slot with every token's state kept (a 2 GiB pool of
    1024 entries), conv on; sampled slots vs the oracle."""
    geom = Geometry(16, 32, 128, 128)
    N, m = 256, 4
    P = N * m
    start = state_pool(63, N, geom)
    pool = torch.zeros((P, 32, 128, 128), dtype=torch.float32, device="cuda")
    idx = np.arange(P, dtype=np.int32).reshape(N, m)
    pool[idx[:, 0].astype(np.int64)] = dev(start)
    cstart = conv_state_pool(63, N, geom, "bf16")
    cpool = torch.zeros((P, geom.channels, 3), dtype=torch.bfloat16, device="cuda")
    cpool[idx[:, 0].astype(np.int64)] = dev(cstart, torch.bfloat16)
    w_np = conv_weights(63, geom, "bf16")
    x = multi_decode_inputs(63, 0, N, m, geom, "bf16")
    o = _multi(x, torch.bfloat16, pool, state_indices=dev(idx, torch.int32), conv_weight=dev(w_np, torch.bfloat16),
               conv_state_pool=cpool)
    torch.cuda.synchronize()
    sample = [0, 77, 255]
    dims = oracle_mod.Dims(16, 32, 128, 128, conv_width=4)
    ref_pool = np.zeros((len(sample) * m, 32, 128, 128))
    ref_cpool = np.zeros((len(sample) * m, geom.channels, 3))
    sidx = np.arange(len(sample) * m).reshape(len(sample), m)
    ref_pool[sidx[:, 0]] = start[sample]
    ref_cpool[sidx[:, 0]] = cstart[sample]
    ro = oracle_mod.decode_multi(dims, x.q[sample], x.k[sample], x.v[sample], x.g[sample], x.beta[sample], ref_pool,
                                 sidx, None, w_np, None, ref_cpool)
    e = rel_err(o[sample].cpu().numpy(), ro)
    es = rel_err(pool[idx[sample].ravel().astype(np.int64)].cpu().numpy(), ref_pool)
    print(f"  rel err o={e:.3e} states={es:.3e}", flush=True)
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.array_equal(cpool[idx[sample].ravel().astype(np.int64)].float().cpu().numpy(),
                          ref_cpool.astype(np.float32))


@pytest.mark.parametrize("dtype,d,out", [("f32", 64, "f32"), ("bf16", 128, "bf16")])
def test_decode_multi_eight_tokens_without_conv(oracle_mod, dtype, d, out):
    """The largest m (8), no conv prologue, raw gates (sigmoid in the kernel),
    fp32 or bf16 outputs; every token's state kept."""
    geom = Geometry(2, 4, d, d)
    N, m = 3, 8
    dt = TORCH_DT[dtype]
    P = N * m
    pool_np = np.zeros((P, 4, d, d), dtype=np.float32)
    idx = np.arange(P, dtype=np.int32).reshape(N, m)
    pool_np[idx[:, 0]] = state_pool(64, N, geom)
    pool = dev(pool_np)
    ref_pool = pool_np.astype(np.float64)
    x = multi_decode_inputs(64, 0, N, m, geom, dtype)
    b_raw = np.log(x.beta / (1.0 - x.beta)).astype(np.float32)  # raw gates with sigmoid(b) ~ beta
    beta_used = 1.0 / (1.0 + np.exp(-b_raw.astype(np.float64)))
    o = binding.gdn_decode_multi(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(b_raw), pool,
                                 state_indices=dev(idx, torch.int32), beta_logits=True,
                                 out_dtype=TORCH_DT[out])
    dims = oracle_mod.Dims(2, 4, d, d, conv_width=0)
    ro = oracle_mod.decode_multi(dims, x.q, x.k, x.v, x.g, beta_used, ref_pool, idx)
    got = o.float().cpu().numpy()
    if out == "bf16":
        # bf16 o is the fp32 result rounded once: within one bf16 ulp of the oracle
        assert np.all(np.abs(got - ro) <= np.abs(ro) * 2.0 ** -8 + 1e-2 * np.sqrt(np.mean(ro ** 2)))
    else:
        assert rel_err(got, ro) <= TOL[dtype]
    assert rel_err(pool.cpu().numpy(), ref_pool) <= TOL[dtype]


def test_decode_multi_binding_validation():
    """Host-side checks of the Python binding: num_accepted outside 1..m and an
    entry shared by two slots are refused before any launch; a slot may reuse
    its own entry."""
    geom = Geometry(1, 2, 64, 64)
    N, m = 2, 3
    x = multi_decode_inputs(65, 0, N, m, geom, "bf16")
    bf = torch.bfloat16
    args = (dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.g), dev(x.beta))
    pool = torch.zeros((8, 2, 64, 64), dtype=torch.float32, device="cuda")
    ok = torch.tensor([[0, 1, 0], [2, 3, -1]], dtype=torch.int32, device="cuda")
    binding.gdn_decode_multi(*args, pool, state_indices=ok)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        binding.gdn_decode_multi(*args, pool, state_indices=ok,
                                 num_accepted=torch.tensor([1, 4], dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        binding.gdn_decode_multi(*args, pool, state_indices=ok,
                                 num_accepted=torch.tensor([0, 1], dtype=torch.int32, device="cuda"))
    shared = torch.tensor([[0, 1, 2], [2, 3, 4]], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        binding.gdn_decode_multi(*args, pool, state_indices=shared)
    with pytest.raises(ValueError):
        binding.gdn_decode_multi(*args, pool, state_indices=torch.tensor([[0, 1, 8], [2, 3, 4]], dtype=torch.int32,
                                                                         device="cuda"))


def test_pooled_prefill_then_speculative_decode(oracle_mod):
    """A serving flow over one pool: a pooled prefill of a prompt per slot, then
    two 3-token decode calls keeping every token's state; after the first call
    slot 0 accepts 2 tokens and slot 1 all 3, and the second call resumes from
    those entries.  The outputs and final states equal the oracle's prefill of
    each slot's accepted token stream (the prompt, then the accepted tokens)."""
    geom = Geometry(2, 4, 128, 128)
    dt = torch.bfloat16
    lengths = [70, 129]
    N, m = 2, 3
    P = 1 + N * m  # entry 0 unused, slot n uses entries 1 + n m .. n m + m
    x = prefill_inputs(66, lengths, geom, "bf16", initial_state_std=0.02, conv_state=True)
    w_np = x.conv_w
    pool = torch.zeros((P, 4, 128, 128), dtype=torch.float32, device="cuda")
    cpool = torch.zeros((P, geom.channels, 3), dtype=dt, device="cuda")
    idx = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.int32)
    start = idx[:, 0].astype(np.int64)
    pool[start] = dev(x.initial_state)
    cpool[start] = dev(x.conv_state_in, dt)
    binding.gdn_prefill_varlen_pooled(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta),
                                      torch.from_numpy(x.cu_seqlens.astype(np.int32)).cuda(), pool,
                                      state_indices=dev(idx[:, 0].copy(), torch.int32), conv_weight=dev(w_np, dt),
                                      conv_state_pool=cpool)
    calls = [multi_decode_inputs(66, c, N, m, geom, "bf16") for c in range(2)]
    accepted = [np.array([1, 1], dtype=np.int32), np.array([2, 3], dtype=np.int32)]  # read entry per call
    outs = []
    for c in range(2):
        y = calls[c]
        outs.append(binding.gdn_decode_multi(dev(y.q, dt), dev(y.k, dt), dev(y.v, dt), dev(y.g), dev(y.beta), pool,
                                             state_indices=dev(idx, torch.int32),
                                             num_accepted=dev(accepted[c], torch.int32),
                                             conv_weight=dev(w_np, dt), conv_state_pool=cpool).cpu().numpy())
    # each slot's stream: prompt, the accepted tokens of call 0, then all of call 1
    keep0 = accepted[1]  # tokens of call 0 the second call builds on
    cu = x.cu_seqlens
    dims = oracle_mod.Dims(2, 4, 128, 128, conv_width=4)
    for n in range(N):
        s0 = slice(int(cu[n]), int(cu[n + 1]))
        a = int(keep0[n])
        cat = lambda f, pre: np.concatenate([pre[s0], getattr(calls[0], f)[n, :a], getattr(calls[1], f)[n]])
        q = cat("q", x.q); k = cat("k", x.k); v = cat("v", x.v); g = cat("g", x.g); b = cat("beta", x.beta)
        L = q.shape[0]
        ro, rfs, rcs = oracle_mod.prefill(dims, np.array([0, L]), q, k, v, g, b, w_np, None,
                                          x.conv_state_in[n:n + 1], x.initial_state[n:n + 1])
        lp = lengths[n]
        e1 = rel_err(outs[1][n], ro[lp + a:])
        e0 = rel_err(outs[0][n, :a], ro[lp:lp + a])
        es = rel_err(pool[int(idx[n, m - 1])].cpu().numpy(), rfs[0])
        print(f"  slot {n}: rel err call0 o={e0:.3e} call1 o={e1:.3e} state={es:.3e}", flush=True)
        assert e0 <= TOL["bf16"] and e1 <= TOL["bf16"] and es <= TOL["bf16"]
        assert np.array_equal(cpool[int(idx[n, m - 1])].float().cpu().numpy(), rcs[0])


def test_decode_pool_entries_beyond_32_bits(oracle_mod):
    """Decode over a 4200-entry state pool (h_v = 32, d = 128: 8.8 GB, entry
    4096 starts at element 2^31): slots whose entries lie past that point, a
    skipped slot and a low entry.  Two single-token steps with the conv update
    are checked against the oracle; those steps and then a 3-token call (each
    token's state to its own high entry, resume from the accepted one) must
    give bit for bit what the same calls give on a compact 6-entry pool."""
    geom = Geometry(16, 32, 128, 128)
    P, N, m = 4200, 6, 3
    dt = torch.bfloat16
    big = np.array([4199, 4097, -1, 4098, 100, 4150], dtype=np.int32)
    small = np.array([0, 1, -1, 3, 4, 5], dtype=np.int32)
    pool_np = state_pool(70, N, geom)
    cpool_np = conv_state_pool(70, N, geom, "bf16")
    w = dev(conv_weights(70, geom, "bf16"), dt)
    pool_big = torch.zeros((P, 32, 128, 128), dtype=torch.float32, device="cuda")
    cpool_big = torch.zeros((P, geom.channels, 3), dtype=dt, device="cuda")
    for i in range(N):
        if big[i] >= 0:
            pool_big[int(big[i])] = dev(pool_np[i])
            cpool_big[int(big[i])] = dev(cpool_np[i], dt)
    pool_small, cpool_small = dev(pool_np), dev(cpool_np, dt)
    ref_pool, ref_cpool = pool_np.astype(np.float64), cpool_np.astype(np.float64)
    dims = oracle_mod.Dims(16, 32, 128, 128, conv_width=4)
    used = big >= 0

    for s in range(2):
        x = decode_inputs(70, s, N, geom, "bf16")
        args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta))
        o_big = binding.gdn_decode_step(*args, pool_big, state_indices=dev(big, torch.int32), conv_weight=w,
                                        conv_state_pool=cpool_big)
        o_small = binding.gdn_decode_step(*args, pool_small, state_indices=dev(small, torch.int32), conv_weight=w,
                                          conv_state_pool=cpool_small)
        ro = oracle_mod.decode(dims, x.q, x.k, x.v, x.g, x.beta, ref_pool, small.astype(np.int64),
                               conv_weights(70, geom, "bf16"), None, ref_cpool)
        torch.cuda.synchronize()
        ob, osm = o_big.cpu().numpy(), o_small.cpu().numpy()
        assert np.array_equal(ob[used], osm[used])
        e = rel_err(ob[used], ro[used])
        print(f"  step {s}: rel err o={e:.3e}", flush=True)
        assert e <= TOL["bf16"]
    for i in range(N):
        if big[i] >= 0:
            assert np.array_equal(pool_big[int(big[i])].cpu().numpy(), pool_small[i].cpu().numpy())
            assert np.array_equal(cpool_big[int(big[i])].float().cpu().numpy(), cpool_small[i].float().cpu().numpy())
    assert rel_err(pool_small.cpu().numpy()[used], ref_pool[used]) <= TOL["bf16"]

    # 3 tokens per slot: token j's state to entry 4100 + 3 i + j (compact: 6 + 3 i + j),
    # read from the entry the single steps left
    pool_small = torch.cat([pool_small, torch.zeros((3 * N, 32, 128, 128), device="cuda")])
    cpool_small = torch.cat([cpool_small, torch.zeros((3 * N, geom.channels, 3), dtype=dt, device="cuda")])
    rows_big = np.stack([[big[i]] + [4100 + 3 * i + j for j in range(m - 1)] for i in range(N)]).astype(np.int32)
    rows_small = np.stack([[small[i]] + [6 + 3 * i + j for j in range(m - 1)] for i in range(N)]).astype(np.int32)
    rows_big[2, :], rows_small[2, :] = -1, -1
    acc = np.ones(N, dtype=np.int32)
    x = multi_decode_inputs(70, 0, N, m, geom, "bf16")
    o_big = _multi(x, dt, pool_big, state_indices=dev(rows_big, torch.int32), num_accepted=dev(acc, torch.int32),
                   conv_weight=w, conv_state_pool=cpool_big)
    o_small = _multi(x, dt, pool_small, state_indices=dev(rows_small, torch.int32),
                     num_accepted=dev(acc, torch.int32), conv_weight=w, conv_state_pool=cpool_small)
    torch.cuda.synchronize()
    assert np.array_equal(o_big.cpu().numpy()[used], o_small.cpu().numpy()[used])
    for i in range(N):
        for j in range(m):
            if rows_big[i, j] >= 0:
                assert np.array_equal(pool_big[int(rows_big[i, j])].cpu().numpy(),
                                      pool_small[int(rows_small[i, j])].cpu().numpy())


@pytest.mark.parametrize("case", range(12))
def test_decode_multi_sweep(oracle_mod, case):
    """Seeded sweep: key heads 1-3, group 1-4, d_k and d_v in {64, 128}
    independently, bf16 or fp32, 1-8 tokens per slot, conv on or off, slots
    that keep every token's state, only some or none, and a skipped slot; two
    calls, the second resuming from each slot's accepted token, against the
    oracle."""
    r = np.random.default_rng([4242, case])
    h_k, G = int(r.integers(1, 4)), int(r.integers(1, 5))
    d_k, d_v = int(r.choice([64, 128])), int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f32"]))
    m, N = int(r.integers(1, 9)), int(r.integers(1, 7))
    conv = bool(r.random() < 0.7)
    geom = Geometry(h_k, h_k * G, d_k, d_v)
    print(f"  case {case}: {geom} {dtype} m={m} N={N} conv={conv}", flush=True)
    P = N * m + 2
    dt = TORCH_DT[dtype]
    pool_np = state_pool(90 + case, P, geom)
    cpool_np = conv_state_pool(90 + case, P, geom, dtype) if conv else None
    w_np = conv_weights(90 + case, geom, dtype) if conv else None
    # slot n owns entries n*m .. n*m + m - 1; some tokens are not kept (-1), the
    # last slot is skipped when there are several
    idx = np.arange(N * m, dtype=np.int32).reshape(N, m)
    drop = r.random((N, m)) < 0.3
    drop[:, 0] = False
    idx[drop] = -1
    if N > 1:
        idx[N - 1, :] = -1
    pool = dev(pool_np)
    cpool = dev(cpool_np, dt) if conv else None
    ref_pool = pool_np.astype(np.float64)
    ref_cpool = cpool_np.astype(np.float64) if conv else None
    dims = oracle_mod.Dims(h_k, h_k * G, d_k, d_v, conv_width=4 if conv else 0)
    for call in range(2):
        # accepted counts point at kept entries (the read entry must exist)
        acc_np = np.array([max([j + 1 for j in range(m) if idx[n, j] >= 0] or [1]) if call else
                           int(r.integers(1, m + 1)) for n in range(N)], dtype=np.int32)
        for n in range(N):
            while acc_np[n] > 1 and idx[n, acc_np[n] - 1] < 0:
                acc_np[n] -= 1
        x = multi_decode_inputs(90 + case, call, N, m, geom, dtype)
        o = _multi(x, dt, pool, state_indices=dev(idx, torch.int32), num_accepted=dev(acc_np, torch.int32),
                   conv_weight=dev(w_np, dt) if conv else None, conv_state_pool=cpool)
        ro = oracle_mod.decode_multi(dims, x.q, x.k, x.v, x.g, x.beta, ref_pool, idx, acc_np, w_np, None,
                                     ref_cpool)
        live = np.array([row[a - 1] >= 0 for row, a in zip(idx, acc_np)])
        if live.any():
            e = rel_err(o.cpu().numpy()[live], ro[live])
            print(f"  call {call}: rel err o={e:.3e}", flush=True)
            assert e <= TOL[dtype]
    used = sorted({int(e) for e in idx.ravel() if e >= 0})
    assert rel_err(pool.cpu().numpy()[used], ref_pool[used]) <= TOL[dtype]
    if conv:
        assert np.array_equal(cpool.float().cpu().numpy(), ref_cpool.astype(np.float32))
