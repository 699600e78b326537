"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

The pages print no numeric example of the recurrence, so every pin here is a
closed form, an invariant, a hand-worked example or a special case that
reduces to a library routine (numpy / torch CPU).  Each is chosen so that a
plausible slip in the oracle (a dropped decay, a wrong sign, a transposed
state, a wrong conv orientation, an output read before the update, a wrong
GQA map) fails at least one of them.

Update rule under test ("Qwen3.5-27B GPTQ Garbage Inference -- Root Cause
Analysis", section "Why abliteration failed on Qwen3.5", item 3, with dv read
as the delta-rule error): S_t = e^{g_t} S_{t-1} + beta_t (v_t - e^{g_t}
S_{t-1} k_t) k_t^T, o_t = scale * S_t q_t.  Stored state H = S^T.
"""
import numpy as np
import pytest
import torch

pytestmark = []


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _dims(oracle, h_k=2, h_v=2, d_k=8, d_v=6, conv=0, norm=False, scale=None):
    return oracle.Dims(h_k, h_v, d_k, d_v, conv_width=conv, qk_l2norm=norm, scale=scale)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _both(oracle, dims, cu, q, k, v, g, b, s0):
    """Run the recurrent and the independent chunked form."""
    return (oracle.recurrent(dims, cu, q, k, v, g, b, s0),
            oracle.chunked(dims, cu, q, k, v, g, b, s0, chunk=4))


def test_hand_worked_example(oracle_mod):
    """Two steps worked by hand with exact numbers (d_k = d_v = 2, scale 1).

    S0 = [[1,0],[0,2]].  Step 1: k=(1,0), v=(3,1), q=(0,1), e^g=1/2, beta=1/2:
      e^g S0 = [[.5,0],[0,1]], p = (.5,0), d = .5*(2.5,1) = (1.25,.5),
      S1 = [[1.75,0],[.5,1]], o1 = S1 q = (0,1).
    Step 2: k=(.6,.8), v=(1,-1), q=(1,0), g=0, beta=1:
      p = S1 k = (1.05,1.1), d = (-.05,-2.1),
      S2 = S1 + d k^T = [[1.72,-.04],[-.76,-.68]], o2 = (1.72,-.76).
    """
    o = oracle_mod
    dims = o.Dims(1, 1, 2, 2, conv_width=0, qk_l2norm=False, scale=1.0)
    cu = _cu([2])
    q = np.array([[[0.0, 1.0]], [[1.0, 0.0]]])
    k = np.array([[[1.0, 0.0]], [[0.6, 0.8]]])
    v = np.array([[[3.0, 1.0]], [[1.0, -1.0]]])
    g = np.array([[np.log(0.5)], [0.0]])
    b = np.array([[0.5], [1.0]])
    S0 = np.array([[1.0, 0.0], [0.0, 2.0]])
    H0 = S0.T[None, None].copy()
    S2 = np.array([[1.72, -0.04], [-0.76, -0.68]])
    for out, fs in _both(o, dims, cu, q, k, v, g, b, H0):
        np.testing.assert_allclose(out[0, 0], [0.0, 1.0], atol=1e-14)
        np.testing.assert_allclose(out[1, 0], [1.72, -0.76], atol=1e-14)
        np.testing.assert_allclose(fs[0, 0], S2.T, atol=1e-14)


def test_beta0_g0_keeps_state_and_reads_it(oracle_mod):
    """beta=0, g=0: S_t = S0 exactly; o_t = d_k^{-1/2} S0 q_t (numpy matmul)."""
    o = oracle_mod
    rng = np.random.default_rng(1)
    dims = _dims(o, 2, 4, 8, 6)
    cu = _cu([5, 9])
    T = 14
    q, k = _rand(rng, T, 2, 8), _rand(rng, T, 2, 8)
    v = _rand(rng, T, 4, 6)
    g, b = np.zeros((T, 4)), np.zeros((T, 4))
    H0 = _rand(rng, 2, 4, 8, 6)
    for out, fs in _both(o, dims, cu, q, k, v, g, b, H0):
        assert np.array_equal(fs, H0)
        for n in range(2):
            for t in range(cu[n], cu[n + 1]):
                for h in range(4):
                    expect = (H0[n, h].T @ q[t, h // 2]) / np.sqrt(8)
                    np.testing.assert_allclose(out[t, h], expect, rtol=1e-13, atol=1e-14)


def test_delta_rule_projection(oracle_mod):
    """beta=1 and unit k: the updated state maps k_t exactly to v_t, for any g, S0."""
    o = oracle_mod
    rng = np.random.default_rng(2)
    dims = _dims(o, 1, 1, 6, 5)
    T = 7
    q = _rand(rng, T, 1, 6)
    k = _unit_rows(_rand(rng, T, 1, 6))
    v = _rand(rng, T, 1, 5)
    g = -np.abs(_rand(rng, T, 1))
    b = np.ones((T, 1))
    H0 = _rand(rng, 1, 1, 6, 5)
    for t in range(1, T + 1):
        cu = _cu([t])
        for _, fs in _both(o, dims, cu, q[:t], k[:t], v[:t], g[:t], b[:t], H0):
            S_t = fs[0, 0].T
            np.testing.assert_allclose(S_t @ k[t - 1, 0], v[t - 1, 0], atol=1e-12)


def test_full_decay_forgets(oracle_mod):
    """g -> -inf (e^g underflows to 0): S_t = beta_t v_t k_t^T, o_t = scale beta_t (k_t.q_t) v_t."""
    o = oracle_mod
    rng = np.random.default_rng(3)
    dims = _dims(o, 1, 2, 5, 4)
    T = 6
    q, k = _rand(rng, T, 1, 5), _rand(rng, T, 1, 5)
    v = _rand(rng, T, 2, 4)
    g = np.full((T, 2), -1e4)
    b = rng.uniform(0.1, 0.9, (T, 2))
    H0 = _rand(rng, 1, 2, 5, 4)
    (out, fs), (outc, fsc) = _both(o, dims, _cu([T]), q, k, v, g, b, H0)
    for h in range(2):
        for t in range(T):
            expect = b[t, h] * (k[t, 0] @ q[t, 0]) * v[t, h] / np.sqrt(5)
            np.testing.assert_allclose(out[t, h], expect, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(outc[t, h], expect, rtol=1e-12, atol=1e-14)
        S_T = b[-1, h] * np.outer(v[-1, h], k[-1, 0])
        np.testing.assert_allclose(fs[0, h], S_T.T, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(fsc[0, h], S_T.T, rtol=1e-12, atol=1e-14)


def test_beta0_is_pure_decay(oracle_mod):
    """beta=0: S_T = e^{sum g} S0 and o_t = scale e^{gam_t} S0 q_t."""
    o = oracle_mod
    rng = np.random.default_rng(4)
    dims = _dims(o, 1, 1, 4, 3)
    T = 9
    q, k = _rand(rng, T, 1, 4), _rand(rng, T, 1, 4)
    v = _rand(rng, T, 1, 3)
    g = -rng.uniform(0.0, 0.5, (T, 1))
    b = np.zeros((T, 1))
    H0 = _rand(rng, 1, 1, 4, 3)
    for out, fs in _both(o, dims, _cu([T]), q, k, v, g, b, H0):
        np.testing.assert_allclose(fs[0, 0], np.exp(g.sum()) * H0[0, 0], rtol=1e-12)
        gam = np.cumsum(g[:, 0])
        for t in range(T):
            np.testing.assert_allclose(out[t, 0], np.exp(gam[t]) * (H0[0, 0].T @ q[t, 0]) / 2.0,
                                       rtol=1e-12, atol=1e-15)


def test_orthonormal_keys_store_and_recall(oracle_mod):
    """Orthonormal keys, beta=1, g=0, S0=0: S_T = sum_t v_t k_t^T; querying with
    k_j returns scale * v_j."""
    o = oracle_mod
    rng = np.random.default_rng(5)
    dk, dv, T = 8, 5, 6
    dims = _dims(o, 1, 1, dk, dv)
    Qm, _ = np.linalg.qr(_rand(rng, dk, dk))
    k = Qm[:T][:, None, :]
    v = _rand(rng, T, 1, dv)
    q = np.concatenate([_rand(rng, T - 1, 1, dk), k[2:3]])  # last query asks for key 2
    g, b = np.zeros((T, 1)), np.ones((T, 1))
    for out, fs in _both(o, dims, _cu([T]), q, k, v, g, b, None):
        S = sum(np.outer(v[t, 0], k[t, 0]) for t in range(T))
        np.testing.assert_allclose(fs[0, 0], S.T, atol=1e-12)
        np.testing.assert_allclose(out[-1, 0], v[2, 0] / np.sqrt(dk), atol=1e-12)


def test_linear_in_values_and_initial_state(oracle_mod):
    o = oracle_mod
    rng = np.random.default_rng(6)
    dims = _dims(o, 1, 2, 6, 4)
    T = 11
    q, k = _rand(rng, T, 1, 6), _rand(rng, T, 1, 6)
    g, b = -rng.uniform(0, 1, (T, 2)), rng.uniform(0, 1, (T, 2))
    V1, V2 = _rand(rng, T, 2, 4), _rand(rng, T, 2, 4)
    S1, S2 = _rand(rng, 1, 2, 6, 4), _rand(rng, 1, 2, 6, 4)
    a1, a2 = 0.7, -1.3
    cu = _cu([T])
    for f in (o.recurrent, o.chunked):
        o1, f1 = f(dims, cu, q, k, V1, g, b, S1)
        o2, f2 = f(dims, cu, q, k, V2, g, b, S2)
        o3, f3 = f(dims, cu, q, k, a1 * V1 + a2 * V2, g, b, a1 * S1 + a2 * S2)
        np.testing.assert_allclose(o3, a1 * o1 + a2 * o2, atol=1e-12)
        np.testing.assert_allclose(f3, a1 * f1 + a2 * f2, atol=1e-12)


@pytest.mark.parametrize("chunk", [64, 16, 7])
def test_chunked_equals_recurrent(oracle_mod, chunk):
    """The independent chunked algebra equals the step-by-step recurrence (fp64)."""
    o = oracle_mod
    rng = np.random.default_rng(7 + chunk)
    dims = _dims(o, 2, 4, 16, 12, norm=False)
    lengths = [1, 63, 64, 65, 130, 300, 0, 17]
    cu = _cu(lengths)
    T = int(cu[-1])
    q = _unit_rows(_rand(rng, T, 2, 16))
    k = _unit_rows(_rand(rng, T, 2, 16))
    v = _rand(rng, T, 4, 12)
    g = -np.logaddexp(0, _rand(rng, T, 4))
    b = 1 / (1 + np.exp(-_rand(rng, T, 4)))
    H0 = 0.02 * _rand(rng, len(lengths), 4, 16, 12)
    o_r, f_r = o.recurrent(dims, cu, q, k, v, g, b, H0)
    o_c, f_c = o.chunked(dims, cu, q, k, v, g, b, H0, chunk=chunk)
    assert np.max(np.abs(o_c - o_r)) <= 1e-10 * np.sqrt(np.mean(o_r ** 2))
    assert np.max(np.abs(f_c - f_r)) <= 1e-10 * np.sqrt(np.mean(f_r ** 2))
    # length-0 sequence: final state is the initial state
    assert np.array_equal(f_r[6], H0[6]) and np.array_equal(f_c[6], H0[6])


def test_chunked_strong_decay(oracle_mod):
    """Very negative g inside a chunk (cumulative decay ~ -1000) stays finite."""
    o = oracle_mod
    rng = np.random.default_rng(8)
    dims = _dims(o, 1, 1, 8, 8)
    T = 100
    q, k = _unit_rows(_rand(rng, T, 1, 8)), _unit_rows(_rand(rng, T, 1, 8))
    v = _rand(rng, T, 1, 8)
    g = -rng.uniform(5, 20, (T, 1))
    b = rng.uniform(0, 1, (T, 1))
    o_r, f_r = o.recurrent(dims, _cu([T]), q, k, v, g, b, None)
    o_c, f_c = o.chunked(dims, _cu([T]), q, k, v, g, b, None, chunk=64)
    assert np.all(np.isfinite(o_c))
    np.testing.assert_allclose(o_c, o_r, atol=1e-12)
    np.testing.assert_allclose(f_c, f_r, atol=1e-12)


def _prefill_case(rng, dims, lengths, with_state=True, with_conv_state=True):
    cu = _cu(lengths)
    T = int(cu[-1])
    N = len(lengths)
    C = dims.channels
    return dict(
        cu=cu,
        q=_rand(rng, T, dims.h_k, dims.d_k), k=_rand(rng, T, dims.h_k, dims.d_k),
        v=_rand(rng, T, dims.h_v, dims.d_v),
        g=-np.logaddexp(0, _rand(rng, T, dims.h_v)), b=1 / (1 + np.exp(-_rand(rng, T, dims.h_v))),
        w=0.5 * _rand(rng, C, 4), bias=_rand(rng, C),
        cs=_rand(rng, N, C, 3) if with_conv_state else None,
        H0=0.02 * _rand(rng, N, dims.h_v, dims.d_k, dims.d_v) if with_state else None)


def test_packed_equals_per_sequence(oracle_mod):
    """Packing sequences with cu_seqlens changes nothing: bit-exact per sequence."""
    o = oracle_mod
    rng = np.random.default_rng(9)
    dims = o.Dims(2, 4, 8, 8, conv_width=4, qk_l2norm=True)
    lengths = [5, 1, 70, 2, 0, 33]
    c = _prefill_case(rng, dims, lengths)
    out, fs, cso = o.prefill(dims, c["cu"], c["q"], c["k"], c["v"], c["g"], c["b"], c["w"], c["bias"],
                             c["cs"], c["H0"])
    cu = c["cu"]
    for n in range(len(lengths)):
        s = slice(cu[n], cu[n + 1])
        o1, f1, cs1 = o.prefill(dims, _cu([lengths[n]]), c["q"][s], c["k"][s], c["v"][s], c["g"][s],
                                c["b"][s], c["w"], c["bias"], c["cs"][n:n + 1], c["H0"][n:n + 1])
        assert np.array_equal(out[s], o1)
        assert np.array_equal(fs[n], f1[0])
        assert np.array_equal(cso[n], cs1[0])


def test_split_and_resume_equals_one_shot(oracle_mod):
    """Prefill of a+b tokens equals prefill of a, then of b from the carried
    recurrent and conv states (state carry across prefill chunks)."""
    o = oracle_mod
    rng = np.random.default_rng(10)
    dims = o.Dims(1, 2, 8, 8, conv_width=4, qk_l2norm=True)
    c = _prefill_case(rng, dims, [100])
    full, fs, cso = o.prefill(dims, c["cu"], c["q"], c["k"], c["v"], c["g"], c["b"], c["w"], None,
                              c["cs"], c["H0"])
    for a in (1, 2, 64, 77):
        s1, s2 = slice(0, a), slice(a, 100)
        o1, f1, c1 = o.prefill(dims, _cu([a]), c["q"][s1], c["k"][s1], c["v"][s1], c["g"][s1], c["b"][s1],
                               c["w"], None, c["cs"], c["H0"])
        o2, f2, c2 = o.prefill(dims, _cu([100 - a]), c["q"][s2], c["k"][s2], c["v"][s2], c["g"][s2],
                               c["b"][s2], c["w"], None, c1, f1)
        np.testing.assert_allclose(np.concatenate([o1, o2]), full, rtol=0, atol=1e-13)
        np.testing.assert_allclose(f2, fs, rtol=0, atol=1e-13)
        assert np.array_equal(c2, cso)


def test_decode_steps_equal_prefill(oracle_mod):
    """T single-token decode steps (state and conv state updated in place) equal
    one prefill of the same T tokens."""
    o = oracle_mod
    rng = np.random.default_rng(11)
    dims = o.Dims(2, 4, 8, 8, conv_width=4, qk_l2norm=True)
    T = 9
    c = _prefill_case(rng, dims, [T])
    full, fs, cso = o.prefill(dims, c["cu"], c["q"], c["k"], c["v"], c["g"], c["b"], c["w"], c["bias"],
                              c["cs"], c["H0"])
    pool = np.zeros((3, 4, 8, 8))
    pool[2] = c["H0"][0]
    cpool = np.zeros((3, dims.channels, 3))
    cpool[2] = c["cs"][0]
    for t in range(T):
        od = o.decode(dims, c["q"][t:t + 1], c["k"][t:t + 1], c["v"][t:t + 1], c["g"][t:t + 1],
                      c["b"][t:t + 1], pool, np.array([2]), c["w"], c["bias"], cpool)
        np.testing.assert_allclose(od[0], full[t], rtol=0, atol=1e-14)
    np.testing.assert_allclose(pool[2], fs[0], rtol=0, atol=1e-14)
    assert np.array_equal(cpool[2], cso[0])
    assert not pool[:2].any() and not cpool[:2].any()


def test_decode_skips_negative_index(oracle_mod):
    o = oracle_mod
    rng = np.random.default_rng(12)
    dims = o.Dims(1, 1, 4, 4, conv_width=0, qk_l2norm=True)
    pool = _rand(rng, 2, 1, 4, 4)
    before = pool.copy()
    od = o.decode(dims, _rand(rng, 2, 1, 4), _rand(rng, 2, 1, 4), _rand(rng, 2, 1, 4),
                  -np.ones((2, 1)), 0.5 * np.ones((2, 1)), pool, np.array([-1, 0]))
    assert np.array_equal(pool[1], before[1]) and not np.array_equal(pool[0], before[0])
    assert not od[0].any() and od[1].any()


def test_decode_multi_equals_prefill_prefixes(oracle_mod):
    """m tokens per slot in one multi-token decode: token j's output and the
    state kept after it equal a prefill of the slot's first j + 1 tokens from
    the start entry (the prefill recurrence is separate code from the decode
    step); num_accepted picks the start entry; a -1 start skips the slot."""
    o = oracle_mod
    rng = np.random.default_rng(21)
    dims = o.Dims(2, 4, 8, 8, conv_width=4, qk_l2norm=True)
    N, m, P = 3, 4, 16
    C = dims.channels
    pool0 = 0.05 * _rand(rng, P, 4, 8, 8)
    cpool0 = _rand(rng, P, C, 3)
    q, k = _rand(rng, N, m, 2, 8), _rand(rng, N, m, 2, 8)
    v = _rand(rng, N, m, 4, 8)
    g, b = -rng.uniform(0, 2, (N, m, 4)), rng.uniform(0, 1, (N, m, 4))
    w, bias = 0.5 * _rand(rng, C, 4), 0.1 * _rand(rng, C)
    idx = np.array([[3, 4, -1, 6], [-1, -1, -1, -1], [9, 10, 11, 12]])
    acc = np.array([2, 1, 1])  # slot 0 resumes from entry 4, slot 2 from entry 9
    pool, cpool = pool0.copy(), cpool0.copy()
    od = o.decode_multi(dims, q, k, v, g, b, pool, idx, acc, w, bias, cpool)
    for n, start in ((0, 4), (2, 9)):
        for j in range(m):
            ref_o, ref_s, ref_c = o.prefill(dims, _cu([j + 1]), q[n, :j + 1], k[n, :j + 1], v[n, :j + 1],
                                            g[n, :j + 1], b[n, :j + 1], w, bias, cpool0[start:start + 1],
                                            pool0[start:start + 1])
            np.testing.assert_allclose(od[n, j], ref_o[j], rtol=0, atol=1e-13)
            if idx[n, j] >= 0:
                np.testing.assert_allclose(pool[idx[n, j]], ref_s[0], rtol=0, atol=1e-13)
                assert np.array_equal(cpool[idx[n, j]], ref_c[0])
    assert not od[1].any()
    untouched = [e for e in range(P) if e not in (3, 4, 6, 9, 10, 11, 12)]
    assert np.array_equal(pool[untouched], pool0[untouched]) and np.array_equal(cpool[untouched], cpool0[untouched])
    assert np.array_equal(pool[5], pool0[5])
    # without indices: entry n is read and receives the state after the last token
    pool2, cpool2 = pool0.copy(), cpool0.copy()
    od2 = o.decode_multi(dims, q, k, v, g, b, pool2, None, None, w, bias, cpool2)
    for n in range(N):
        ref_o, ref_s, ref_c = o.prefill(dims, _cu([m]), q[n], k[n], v[n], g[n], b[n], w, bias,
                                        cpool0[n:n + 1], pool0[n:n + 1])
        np.testing.assert_allclose(od2[n], ref_o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(pool2[n], ref_s[0], rtol=0, atol=1e-13)
        assert np.array_equal(cpool2[n], ref_c[0])
    assert np.array_equal(pool2[N:], pool0[N:])


def test_dv_permutation_permutes_rows(oracle_mod):
    """Rows of S (the d_v coordinates) evolve independently."""
    o = oracle_mod
    rng = np.random.default_rng(13)
    dims = _dims(o, 1, 1, 6, 7, norm=True)
    T = 20
    q, k, v = _rand(rng, T, 1, 6), _rand(rng, T, 1, 6), _rand(rng, T, 1, 7)
    g, b = -rng.uniform(0, 1, (T, 1)), rng.uniform(0, 1, (T, 1))
    H0 = _rand(rng, 1, 1, 6, 7)
    perm = rng.permutation(7)
    for f in (o.recurrent, o.chunked):
        o1, f1 = f(dims, _cu([T]), q, k, v, g, b, H0)
        o2, f2 = f(dims, _cu([T]), q, k, v[..., perm], g, b, H0[..., perm])
        np.testing.assert_allclose(o2, o1[..., perm], atol=1e-13)
        np.testing.assert_allclose(f2, f1[..., perm], atol=1e-13)


def test_conv_identity_tap(oracle_mod):
    """w = e_3 (only the newest tap), no bias: conv is the identity before SiLU."""
    o = oracle_mod
    rng = np.random.default_rng(14)
    dims = o.Dims(1, 1, 4, 4, conv_width=4, qk_l2norm=False)
    T = 6
    q, k, v = _rand(rng, T, 1, 4), _rand(rng, T, 1, 4), _rand(rng, T, 1, 4)
    w = np.zeros((dims.channels, 4))
    w[:, 3] = 1.0
    qo, ko, vo, _ = o.prologue(dims, _cu([T]), q, k, v, w, None, _rand(rng, 1, dims.channels, 3))
    silu = lambda x: x / (1 + np.exp(-x))
    np.testing.assert_allclose(qo, silu(q), rtol=1e-15)
    np.testing.assert_allclose(ko, silu(k), rtol=1e-15)
    np.testing.assert_allclose(vo, silu(v), rtol=1e-15)


@pytest.mark.parametrize("lengths", [[7, 1, 2, 12], [3]])
def test_conv_matches_torch_conv1d(oracle_mod, lengths):
    """General weights, bias and carried history against torch's grouped conv1d
    over [history, x] with no padding, then SiLU; the new conv state is the last
    three raw inputs (causal conv of the GDN prologue)."""
    o = oracle_mod
    rng = np.random.default_rng(15)
    dims = o.Dims(2, 2, 4, 3, conv_width=4, qk_l2norm=False)
    C = dims.channels
    cu = _cu(lengths)
    T = int(cu[-1])
    q, k, v = _rand(rng, T, 2, 4), _rand(rng, T, 2, 4), _rand(rng, T, 2, 3)
    w, bias = 0.5 * _rand(rng, C, 4), _rand(rng, C)
    hist = _rand(rng, len(lengths), C, 3)
    qo, ko, vo, cso = o.prologue(dims, cu, q, k, v, w, bias, hist)
    x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    got = np.concatenate([qo.reshape(T, -1), ko.reshape(T, -1), vo.reshape(T, -1)], axis=1)
    for n in range(len(lengths)):
        xs = torch.from_numpy(np.concatenate([hist[n], x[cu[n]:cu[n + 1]].T], axis=1))[None]
        y = torch.nn.functional.conv1d(xs, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias),
                                       padding=0, groups=C)
        ref = torch.nn.functional.silu(y)[0].numpy().T
        np.testing.assert_allclose(got[cu[n]:cu[n + 1]], ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(cso[n], xs[0, :, -3:].numpy())


def test_conv_zero_history_at_sequence_start(oracle_mod):
    """Without a conv state, history is zero at every sequence start: no leakage
    from the previous packed sequence."""
    o = oracle_mod
    rng = np.random.default_rng(16)
    dims = o.Dims(1, 1, 4, 4, conv_width=4, qk_l2norm=True)
    c = _prefill_case(rng, dims, [5, 6], with_state=False, with_conv_state=False)
    q1, k1, v1, _ = o.prologue(dims, c["cu"], c["q"], c["k"], c["v"], c["w"], None, None)
    s = slice(5, 11)
    q2, k2, v2, _ = o.prologue(dims, _cu([6]), c["q"][s], c["k"][s], c["v"][s], c["w"], None,
                               np.zeros((1, dims.channels, 3)))
    assert np.array_equal(q1[s], q2) and np.array_equal(k1[s], k2) and np.array_equal(v1[s], v2)


def test_l2norm_gives_unit_heads(oracle_mod):
    o = oracle_mod
    rng = np.random.default_rng(17)
    dims = o.Dims(3, 3, 16, 4, conv_width=0, qk_l2norm=True)
    T = 5
    qo, ko, vo, _ = o.prologue(dims, _cu([T]), 10 * _rand(rng, T, 3, 16), _rand(rng, T, 3, 16),
                               _rand(rng, T, 3, 4))
    np.testing.assert_allclose(np.linalg.norm(qo, axis=-1), 1.0, atol=1e-8)
    np.testing.assert_allclose(np.linalg.norm(ko, axis=-1), 1.0, atol=1e-6)


def test_gqa_equals_repeated_heads(oracle_mod):
    """GQA (value head h reads key head h // G) equals multi-head attention on
    q/k repeated per value head (repeat_interleave); G = 1 is plain multi-head."""
    o = oracle_mod
    rng = np.random.default_rng(18)
    T, hk, hv, d = 30, 2, 6, 8
    q, k = _rand(rng, T, hk, d), _rand(rng, T, hk, d)
    v = _rand(rng, T, hv, d)
    g, b = -rng.uniform(0, 1, (T, hv)), rng.uniform(0, 1, (T, hv))
    H0 = _rand(rng, 1, hv, d, d)
    gqa = o.Dims(hk, hv, d, d, conv_width=0, qk_l2norm=True)
    mha = o.Dims(hv, hv, d, d, conv_width=0, qk_l2norm=True)
    qr, kr = np.repeat(q, hv // hk, axis=1), np.repeat(k, hv // hk, axis=1)
    qn, kn, _, _ = o.prologue(gqa, _cu([T]), q, k, v)
    qrn, krn, _, _ = o.prologue(mha, _cu([T]), qr, kr, v)
    for f in (o.recurrent, o.chunked):
        o1, f1 = f(gqa, _cu([T]), qn, kn, v, g, b, H0)
        o2, f2 = f(mha, _cu([T]), qrn, krn, v, g, b, H0)
        assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_golden_regression(oracle_mod):
    """Oracle outputs on a tiny fixed case, stored by tests/golden/make_golden.py
    (which calls only the oracle).  Guards against unannounced changes."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    with open(path) as f:
        gold = json.load(f)
    from tests.golden.make_golden import compute
    cur = compute(oracle_mod)
    for key in gold["values"]:
        np.testing.assert_allclose(np.array(cur[key]), np.array(gold["values"][key]), rtol=1e-12, atol=1e-15)
