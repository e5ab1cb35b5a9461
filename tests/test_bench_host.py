"""Host-side logic of bench.py: the work and byte counts its rates divide
by, the measured-traffic lookup, and the one-GPU contract. No GPU needed."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod   # the CPU leg's process pool pickles its functions by name
    spec.loader.exec_module(mod)
    return mod


def test_prefill_dense_flops(bench):
    # 4 d per unmasked (query, key) pair: causal N (N + 1) / 2 pairs per head
    N = 131072
    assert bench.prefill_dense_flops(1, 8, N, 128) == 4 * 128 * 8 * N * (N + 1) // 2
    assert bench.prefill_dense_flops(1, 8, N, 128) == 35184640524288
    assert bench.prefill_dense_flops(2, 3, 100, 64, causal=False) == 4 * 64 * 2 * 3 * 100 * 100


def test_prefill_exec_flops_counts_visited_and_kept(bench):
    mask = np.array([[[[0, 2], [1, 0]]]], np.uint8)   # 3 visited tiles, 2 kept
    flops, visited, kept = bench.prefill_exec_flops(mask, 128)
    assert (visited, kept) == (3, 2)
    assert flops == 2 * 128 * 64 * 64 * (3 + 2)


def _mask_two_groups():
    # B=1, Hkv=2, G=2, L=130: tiles of 64, 64 and 2 keys. Group 0 keeps
    # tiles 0 (head 0) and 2 (head 1); group 1 keeps tile 0 only.
    m = np.ones((1, 4, 3), np.uint8)
    m[0, 0, 0] = 0
    m[0, 1, 2] = 0
    m[0, 2, 0] = 0
    return m


def test_decode_bytes(bench):
    dense, actual = bench.decode_bytes(16, 8, 131072, 128)
    assert dense == actual == 2 * 16 * 8 * 131072 * 128 * 2 == 8589934592
    dense, actual = bench.decode_bytes(1, 2, 130, 4, _mask_two_groups(), G=2)
    assert dense == 2 * 1 * 2 * 130 * 4 * 2
    # all of K, plus the V rows of the tiles some head of the group keeps
    assert actual == dense / 2 + (64 + 2 + 64) * 4 * 2


def test_q4_bytes(bench):
    # per key: d/2 bytes of K codes + 4 of K parameters; per V tile and
    # channel: 32 bytes of codes + 4 of parameters
    assert bench.q4_bytes(16, 8, 131072, 128) == 16 * 8 * 131072 * (64 + 4 + 36 * 128 / 64)
    assert bench.q4_bytes(16, 8, 131072, 128) == 2348810240
    got = bench.q4_bytes(1, 2, 130, 4, _mask_two_groups(), G=2)
    assert got == 1 * 2 * 130 * (2 + 4) + 3 * 36 * 4


def test_q2_bytes(bench):
    # per key: d/4 bytes of K codes + 4 of K parameters; per V tile and
    # channel: 16 bytes of codes + 4 of parameters
    assert bench.q2_bytes(16, 8, 131072, 128) == 16 * 8 * 131072 * (32 + 4 + 20 * 128 / 64)
    assert bench.q2_bytes(16, 8, 131072, 128) == 1275068416
    got = bench.q2_bytes(1, 2, 130, 4, _mask_two_groups(), G=2)
    assert got == 1 * 2 * 130 * (1 + 4) + 3 * 20 * 4


def test_measured_traffic_follows_the_sources(bench, monkeypatch):
    for leg, entry in bench.MEASURED_TRAFFIC.items():
        want = entry["bytes"] if bench._source_sha1(entry["sources"]) == entry["sha1"] else None
        assert bench.measured_traffic(leg) == want
    stale = dict(bench.MEASURED_TRAFFIC["decode"], sha1="0" * 40)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, "decode", stale)
    assert bench.measured_traffic("decode") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_runs_on_tiny_inputs(bench):
    # the host leg of bench.py (the oracle timed on a sample), at toy sizes
    import synth
    rng = np.random.default_rng(0)

    def bits(*shape):
        return synth.f32_to_bf16_bits(rng.normal(size=shape).astype(np.float32))
    pq, pk, pv = bits(1, 1, 256, 64), bits(1, 1, 256, 64), bits(1, 1, 256, 64)
    dq, dk, dv = bits(2, 4, 64), bits(2, 2, 300, 64), bits(2, 2, 300, 64)
    pre, dec, dq4, dq2, dqh = bench.cpu_baseline(pq, pk, pv, dq, dk, dv, nblocks=4, nkv=3,
                                                 nkv_q=2, pname="tiny", hybrid_bits=(4, 2))
    for r in (pre, dec, dq4, dq2, dqh):
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
        assert r["host_cores"] == os.cpu_count() and r["cores"] <= r["host_cores"]
    assert pre["unit"] == "TFLOP/s" and dq2["unit"] == "GB/s"
    assert "2-bit" in dq2["sample"] and "4-bit" in dq4["sample"] and "hybrid" in dqh["sample"]
    # without a hybrid width list the hybrid leg is not run
    assert bench.cpu_baseline(pq, pk, pv, dq, dk, dv, nblocks=2, nkv=1, nkv_q=1,
                              pname="tiny")[4] is None
