"""Host-side checks of the C ABI (no GPU): exports, struct layout, and the
argument errors that must be returned before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from gateddeltanet_chunked_delta_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from gateddeltanet_chunked_delta_amd.build import build
        build()
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gdn_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_problem_struct_layout_matches_c(tmp_path):
    """ctypes mirror of gdn_problem has the C compiler's size and offsets."""
    fields = [f[0] for f in binding.GdnProblem._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'printf("{f} %zu\\n", offsetof(gdn_problem, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "gdn.h"\nint main(void){{\n'
                   f'printf("size %zu\\n", sizeof(gdn_problem));\n{body}\nreturn 0;}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True,
                                                   check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(binding.GdnProblem)
    for f in fields:
        assert int(got[f]) == getattr(binding.GdnProblem, f).offset, f


def test_status_strings(lib):
    for code in range(-8, 1):
        s = binding.status_string(code)
        assert s and s != "unknown status"
    assert binding.status_string(-99) == "unknown status"


# Fake, 256-byte aligned device addresses: validation never dereferences them,
# and every call below must fail validation before any HIP call.
def _fake(i):
    return ctypes.c_void_p(0x10000000 + i * 0x1000000)


def _prefill(lib, prob, q=1, k=2, v=3, g=4, b=5, cu=6, cw=None, cb=None, csi=None, cso=None, h0=None,
             o=7, fs=None, ws=8, ws_bytes=1 << 20):
    f = lambda x: None if x is None else (_fake(x) if isinstance(x, int) else x)
    return lib.gdn_prefill_varlen(ctypes.byref(prob), f(q), f(k), f(v), f(g), f(b), f(cu), f(cw), f(cb), f(csi),
                                  f(cso), f(h0), f(o), f(fs), f(ws), ctypes.c_size_t(ws_bytes), None)


def _prob(**kw):
    base = dict(num_seqs=2, total_tokens=100, h_k=2, h_v=4, d_k=128, d_v=128, qkv_dtype=1, out_dtype=0,
                scale=None, qk_l2norm=True, l2_eps=1e-6, conv_width=4)
    base.update(kw)
    return binding.make_problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(h_v=3), -2),                # h_v % h_k != 0
    (dict(h_k=0), -2),
    (dict(num_seqs=-1), -2),
    (dict(total_tokens=-5), -2),
    (dict(qkv_dtype=7), -3),
    (dict(out_dtype=2), -3),
    (dict(d_k=96, d_v=96), -4),       # no kernel for d = 96
    (dict(d_k=128, d_v=96), -4),      # no kernel for d_v = 96
    (dict(d_k=32, d_v=64), -4),       # nor for d_k = 32
    (dict(conv_width=3), -4),
    (dict(num_seqs=0, total_tokens=5), -2),
])
def test_prefill_rejects_bad_problem(lib, kw, code):
    assert _prefill(lib, _prob(**kw), cw=9) == code


def test_prefill_rejects_bad_flag(lib):
    prob = _prob()
    prob.qk_l2norm = 2
    assert _prefill(lib, prob, cw=9) == -2
    prob = _prob()
    prob.l2_eps = -1.0
    assert _prefill(lib, prob, cw=9) == -2
    prob = _prob()
    prob.beta_logits = 2
    assert _prefill(lib, prob, cw=9) == -2


def _noalloc(lib, prob, q=1, k=2, v=3, g=4, b=5, cu=6, cw=None, cb=None, csi=None, cso=None, h0=None, o=7,
             fs=None):
    f = lambda x: None if x is None else (_fake(x) if isinstance(x, int) else x)
    return lib.gdn_prefill_varlen_noalloc(ctypes.byref(prob), f(q), f(k), f(v), f(g), f(b), f(cu), f(cw), f(cb),
                                          f(csi), f(cso), f(h0), f(o), f(fs), None)


def test_noalloc_rejects_before_any_hip_call(lib):
    """The allocation-free prefill validates like gdn_prefill_varlen and
    refuses problems whose workspace exceeds its static scratch."""
    assert lib.gdn_prefill_varlen_noalloc(None, *([None] * 14)) == -1
    assert _noalloc(lib, _prob(h_v=3), cw=9) == -2
    assert _noalloc(lib, _prob(d_k=96, d_v=96), cw=9) == -4
    assert _noalloc(lib, _prob(), cw=None) == -1
    assert _noalloc(lib, _prob(conv_width=0), o=1) == -7                 # o == q
    # the workspace need grows with the tokens: find a size just past the scratch
    big = _prob(num_seqs=4, total_tokens=4 * 4096, h_k=16, h_v=32, conv_width=0)
    assert binding.gdn_prefill_workspace_bytes(big) > binding.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, big) == -8
    assert binding.status_string(-8) != "unknown status"


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES


def test_prefill_null_problem(lib):
    assert lib.gdn_prefill_varlen(None, *([None] * 14), ctypes.c_size_t(0), None) == -1


def test_prefill_null_pointers(lib):
    prob = _prob()
    assert _prefill(lib, prob, cw=None) == -1           # conv_width 4 needs conv_w
    assert _prefill(lib, prob, cw=9, q=None) == -1
    assert _prefill(lib, prob, cw=9, o=None) == -1
    assert _prefill(lib, prob, cw=9, cu=None) == -1


def test_prefill_workspace(lib):
    prob = _prob(conv_width=0)
    need = binding.gdn_prefill_workspace_bytes(prob)
    assert need >= 2 * 4 and need % 256 == 0
    assert _prefill(lib, prob, ws=None) == -5
    assert _prefill(lib, prob, ws_bytes=need - 1) == -5
    assert binding.gdn_prefill_workspace_bytes(_prob(num_seqs=0, total_tokens=0)) == 0


def test_prefill_workspace_size_formula(lib):
    """(T + 63 N) / 64 chunk slots of 512 d_k h_k + 21504 h_v + 16 bytes, plus the
    256-byte aligned order and chunk-base arrays, as the header states."""
    for N, T, h_k, h_v, d in [(4, 16384, 16, 32, 128), (60, 250000, 16, 48, 128), (3, 7, 2, 6, 64), (1, 0, 1, 1, 64)]:
        need = binding.gdn_prefill_workspace_bytes(_prob(num_seqs=N, total_tokens=T, h_k=h_k, h_v=h_v, d_k=d, d_v=d))
        slots = (T + 63 * N) // 64
        body = slots * (512 * d * h_k + 21504 * h_v + 16)
        assert body <= need <= body + 5 * 256 + 8 * (N + 1) + 256, (N, T, need, body)


def test_prefill_timed_needs_four_events(lib):
    prob = _prob(conv_width=0)
    f = lambda x: None if x is None else _fake(x)
    args = [ctypes.byref(prob)] + [f(i) for i in (1, 2, 3, 4, 5, 6)] + [None] * 3 + [None, None, f(7), None, f(8),
                                                                                    ctypes.c_size_t(1 << 30), None]
    assert lib.gdn_prefill_varlen_timed(*args, None) == -1
    ev = (ctypes.c_void_p * 4)(_fake(20).value, _fake(21).value, None, _fake(23).value)
    assert lib.gdn_prefill_varlen_timed(*args, ev) == -1
    ev = (ctypes.c_void_p * 4)(*[_fake(20 + i).value for i in range(4)])
    assert lib.gdn_prefill_varlen_timed(*args[:1], None, *args[2:], ev) == -1  # q missing: no event recorded


def test_prefill_alias_and_alignment(lib):
    prob = _prob(conv_width=0)
    assert _prefill(lib, prob, o=1) == -7                       # o == q
    assert _prefill(lib, prob, fs=3) == -7                      # final state over v
    assert _prefill(lib, prob, o=ctypes.c_void_p(0x10000000 + 8 * 0x1000000 + 4)) == -4  # misaligned o


def test_prefill_empty_batch_is_a_no_op(lib):
    prob = _prob(num_seqs=0, total_tokens=0, conv_width=0)
    assert _prefill(lib, prob, q=None, k=None, v=None, g=None, b=None, cu=None, o=None, ws=None, ws_bytes=0) == 0


def _decode(lib, prob, q=1, k=2, v=3, g=4, b=5, cw=None, cb=None, cs=None, pool=6, idx=None, o=7):
    f = lambda x: None if x is None else (_fake(x) if isinstance(x, int) else x)
    return lib.gdn_decode_step(ctypes.byref(prob), f(q), f(k), f(v), f(g), f(b), f(cw), f(cb), f(cs), f(pool),
                               f(idx), f(o), None)


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, _prob(num_seqs=4, total_tokens=5, conv_width=0)) == -2   # total_tokens != N
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4, conv_width=0), pool=None) == -1
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4), cw=9, cs=None) == -1  # conv needs its pool
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4, conv_width=0, d_k=32)) == -4
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4, conv_width=0, qkv_dtype=5)) == -3
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4, conv_width=0), o=1) == -7
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4, conv_width=0), o=6) == -7  # o == state pool
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4, conv_width=0), v=6) == -7  # v over the state pool
    big = _prob(num_seqs=1 << 24, total_tokens=1 << 24, conv_width=0, h_k=256, h_v=256)
    assert _decode(lib, big) == -2                                                   # grid of 2^32 workgroups
    assert _decode(lib, _prob(num_seqs=4, total_tokens=4), cw=9, cs=2) == -7         # k over the conv pool
    assert _decode(lib, _prob(num_seqs=0, total_tokens=0, conv_width=0), q=None, k=None, v=None, g=None,
                   b=None, pool=None, o=None) == 0


def _multi(lib, prob, m, q=1, k=2, v=3, g=4, b=5, cw=None, cb=None, cs=None, pool=6, idx=None, acc=None, o=7):
    f = lambda x: None if x is None else (_fake(x) if isinstance(x, int) else x)
    return lib.gdn_decode_multi(ctypes.byref(prob), ctypes.c_int32(m), f(q), f(k), f(v), f(g), f(b), f(cw), f(cb),
                                f(cs), f(pool), f(idx), f(acc), f(o), None)


def test_decode_multi_rejects_bad_arguments(lib):
    ok = dict(num_seqs=4, total_tokens=12, conv_width=0)
    assert _multi(lib, _prob(**ok), 0) == -2                                 # m < 1
    assert _multi(lib, _prob(num_seqs=4, total_tokens=36, conv_width=0), 9) == -4  # m above 8
    assert _multi(lib, _prob(num_seqs=4, total_tokens=11, conv_width=0), 3) == -2  # total_tokens != N m
    assert _multi(lib, _prob(**ok), 3, pool=None) == -1
    assert _multi(lib, _prob(num_seqs=4, total_tokens=12), 3, cw=9, cs=None) == -1
    assert _multi(lib, _prob(**ok), 3, o=1) == -7                            # o == q
    assert _multi(lib, _prob(**ok), 3, o=6) == -7                            # o == state pool
    assert _multi(lib, _prob(**ok), 3, o=10, acc=10) == -7                   # o over num_accepted
    assert _multi(lib, _prob(**ok), 3, acc=ctypes.c_void_p(0x10000000 + 12 * 0x1000000 + 2)) == -4
    assert _multi(lib, _prob(num_seqs=0, total_tokens=0, conv_width=0), 3, q=None, k=None, v=None, g=None,
                  b=None, pool=None, o=None) == 0


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 1, 64)
    with pytest.raises(ValueError):
        binding.gdn_prefill_varlen(x, x, x, torch.zeros(4, 1), torch.zeros(4, 1), [0, 4])
    with pytest.raises(ValueError):
        binding.gdn_decode_step(x, x, x, torch.zeros(4, 1), torch.zeros(4, 1), torch.zeros(4, 1, 64, 64))


def _pooled(lib, prob, q=1, k=2, v=3, g=4, b=5, cu=6, cw=None, cb=None, cpool=None, pool=9, idx=None, hi=None,
            o=7, ws=8, ws_bytes=1 << 20):
    f = lambda x: None if x is None else (_fake(x) if isinstance(x, int) else x)
    return lib.gdn_prefill_varlen_pooled(ctypes.byref(prob), f(q), f(k), f(v), f(g), f(b), f(cu), f(cw), f(cb),
                                         f(cpool), f(pool), f(idx), f(hi), f(o), f(ws), ctypes.c_size_t(ws_bytes),
                                         None)


def test_pooled_prefill_rejects_bad_arguments(lib):
    assert _pooled(lib, _prob(h_v=3), cw=10, cpool=11) == -2
    assert _pooled(lib, _prob(conv_width=0), pool=None) == -1              # the state pool is required
    assert _pooled(lib, _prob(), cw=10, cpool=None) == -1                   # conv needs its pool
    assert _pooled(lib, _prob(), cw=None, cpool=11) == -1                   # conv needs its weights
    assert _pooled(lib, _prob(conv_width=0), cu=None) == -1
    assert _pooled(lib, _prob(conv_width=0, d_k=96, d_v=96)) == -4
    assert _pooled(lib, _prob(conv_width=0), ws=None) == -5
    assert _pooled(lib, _prob(conv_width=0), o=1) == -7                     # o == q
    assert _pooled(lib, _prob(conv_width=0), o=9) == -7                     # o == state pool
    assert _pooled(lib, _prob(conv_width=0), ws=9) == -7                    # workspace == state pool
    assert _pooled(lib, _prob(), cw=10, cpool=9) == -7                      # conv pool == state pool
    assert _pooled(lib, _prob(conv_width=0), idx=ctypes.c_void_p(0x10000000 + 12 * 0x1000000 + 2)) == -4
    assert _pooled(lib, _prob(num_seqs=0, total_tokens=0, conv_width=0), q=None, k=None, v=None, g=None, b=None,
                   cu=None, pool=None, o=None, ws=None, ws_bytes=0) == 0
