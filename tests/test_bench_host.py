"""Host logic of bench.py (CPU): the algorithmic work counts, the roofline
rule, the traffic lookup and the one-GPU guard.

The expected byte and flop counts are written out from the workload
definitions (4 sequences x 4096 tokens, h_k = 16, h_v = 32, d = 128, bf16 in,
fp32 g/beta/o/states; 256 decode slots) so that a change to the counting
functions shows up here.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_call_bytes_and_flops():
    w = bench.prefill_work([4096] * 4, 16, 32, 128)
    T, N, hk, hv, d = 16384, 4, 16, 32, 128
    C = 2 * hk * d + hv * d
    qkv = T * (2 * hk * d + hv * d) * 2
    gb = T * hv * 2 * 4
    o = T * hv * d * 4
    state = N * hv * d * d * 4
    conv = N * C * 3 * 2 + C * 4 * 2
    expect_bytes = qkv + gb + o + state + conv + (N + 1) * 4
    assert w["call"][0] == expect_bytes
    assert abs(w["call"][0] / 1e6 - 549.7) < 0.1  # the figure the design notes quote
    G = hv // hk
    assert w["call"][1] == T * hv * ((4 / G + 6) * 64 * d + 6 * d * d)
    # the shares add up to the call
    assert w["prep"][0] + w["carry"][0] == w["call"][0]
    assert w["prep"][1] + w["carry"][1] == w["call"][1]
    # the chunk-local share is q, k, g and beta
    assert w["prep"][0] == T * (2 * hk * d * 2 + 2 * hv * 4)


def test_prefill_bf16_output_bytes():
    w32 = bench.prefill_work([4096] * 4, 16, 32, 128)
    w16 = bench.prefill_work([4096] * 4, 16, 32, 128, out_bytes=2)
    assert w32["call"][0] - w16["call"][0] == 16384 * 32 * 128 * 2


def test_decode_step_bytes():
    b, f = bench.decode_algorithmic(256, 16, 32, 128)
    state = 256 * 32 * 128 * 128 * 4
    C = 2 * 16 * 128 + 32 * 128
    expect = 2 * state + 256 * C * 2 + 256 * 32 * 8 + 256 * 32 * 128 * 4 + 2 * 256 * C * 3 * 2 + C * 4 * 2
    assert b == expect
    # without the conv prologue: the state, q/k/v, g/beta and o only
    b0, _ = bench.decode_algorithmic(256, 16, 32, 128, conv=False)
    assert b0 == 2 * state + 256 * C * 2 + 256 * 32 * 8 + 256 * 32 * 128 * 4
    assert f == 256 * 32 * 7.0 * 128 * 128


def test_decode_bytes_with_unequal_head_dims():
    b, f = bench.decode_algorithmic(256, 16, 32, 128, d_v=64)
    state = 256 * 32 * 128 * 64 * 4
    C = 2 * 16 * 128 + 32 * 64
    assert b == 2 * state + 256 * C * 2 + 256 * 32 * 8 + 256 * 32 * 64 * 4 + 2 * 256 * C * 3 * 2 + C * 4 * 2
    assert f == 256 * 32 * 7.0 * 128 * 64
    # d_v defaults to d_k
    assert bench.decode_algorithmic(8, 2, 4, 64) == bench.decode_algorithmic(8, 2, 4, 64, d_v=64)
    one = bench.decode_multi_algorithmic(256, 4, 16, 32, 64, kept=1, d_v=128)
    assert one == (256 * 32 * 64 * 128 * 4 * 2 + 256 * 4 * ((2 * 16 * 64 + 32 * 128) * 2 + 32 * 8 + 32 * 128 * 4)
                   + 256 * (2 * 16 * 64 + 32 * 128) * 3 * 2 * 2 + (2 * 16 * 64 + 32 * 128) * 4 * 2)


def test_multi_decode_bytes_count_kept_states():
    one = bench.decode_multi_algorithmic(256, 4, 16, 32, 128, kept=1)
    four = bench.decode_multi_algorithmic(256, 4, 16, 32, 128, kept=4)
    state = 256 * 32 * 128 * 128 * 4
    C = 2 * 16 * 128 + 32 * 128
    assert four - one == 3 * state + 3 * 256 * C * 3 * 2


def test_multi_decode_bf16_output_bytes():
    f32 = bench.decode_multi_algorithmic(256, 4, 16, 32, 128, kept=1)
    b16 = bench.decode_multi_algorithmic(256, 4, 16, 32, 128, kept=1, out_bytes=2)
    assert f32 - b16 == 256 * 4 * 32 * 128 * 2


def test_roofline_takes_the_binding_roof():
    # HBM-bound work: 8 GB in 2 ms -> 4 TB/s = half of the 8 TB/s peak
    r = bench.roofline(8e9, 1e12, 2e-3, "k")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["kernel"] == "k"
    assert abs(r["achieved"] - 4000.0) < 1e-6 and abs(r["frac"] - 0.5) < 1e-12
    assert abs(r["floor_us"] - 1000.0) < 1e-6
    # flop-bound work: 2.5 PFLOP in 2 s -> 1.25 PFLOP/s = half of the bf16 peak
    r = bench.roofline(1e9, 2.5e15, 2.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - 0.5) < 1e-12 and abs(r["mfma_frac"] - 0.5) < 1e-12
    # frac is the floor over the measured time under either roof
    for nbytes, flops, sec in ((5.5e8, 8.6e10, 4.3e-4), (1e6, 1e13, 1e-2)):
        r = bench.roofline(nbytes, flops, sec)
        assert abs(r["frac"] - r["floor_us"] / r["avg_us"]) < 1e-9


def test_measured_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    # the committed table: known kernels either match their sources or report None
    for k in (bench.PREP_KERNEL, bench.CARRY_KERNEL, bench.DECODE_KERNEL):
        t = bench.measured_traffic(k)
        assert t is None or t > 0
    # a table whose hash does not match the sources reports None
    root = tmp_path
    (root / "profiles").mkdir()
    src = root / "k.hip"
    src.write_text("kernel")
    table = {"fetch_scale": 2.0, "write_scale": 1.0,
             "k": {"sources": ["k.hip"], "src_sha256_16": "0" * 16, "fetch_kib": 1.0, "write_kib": 1.0}}
    (root / "profiles" / "traffic.json").write_text(json.dumps(table))
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(root / "bench.py"))
    assert bench.measured_traffic("k") is None
    import hashlib
    table["k"]["src_sha256_16"] = hashlib.sha256(b"kernel").hexdigest()[:16]
    (root / "profiles" / "traffic.json").write_text(json.dumps(table))
    assert bench.measured_traffic("k") == (1.0 * 2.0 + 1.0 * 1.0) * 1024.0
    assert bench.measured_traffic("missing") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
