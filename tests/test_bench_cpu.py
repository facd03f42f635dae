"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and op counts the roofline divides by, the counter-traffic lookup, and the
workload shapes."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_gemm_bytes_decode():
    # int8 W 4096x4096 + int8 xq 8x4096 + xs [8, 32] + ws [32, 32] + bf16 y 8x4096
    assert bench.gemm_bytes(8, 4096, 4096) == 4096 * 4096 + 8 * 4096 + 4 * 8 * 32 + 4 * 32 * 32 + 2 * 8 * 4096
    assert bench.gemm_bytes(8, 4096, 4096) == 16880640


def test_gemm_bytes_ragged_uses_ceil_sized_scales():
    M, N, K = 333, 5000, 4000
    NB, KB = 40, 32
    assert bench.gemm_bytes(M, N, K) == M * K + 4 * M * KB + N * K + 4 * NB * KB + 2 * M * N


def test_gemm_bytes_per_channel_scales():
    M, N, K = 4096, 4096, 4096
    assert bench.gemm_bytes(M, N, K, (1, K)) == M * K + 4 * M + N * K + 4 * N + 2 * M * N


def test_quant_bytes():
    assert bench.quant_bytes(4096, 4096) == 3 * 4096 * 4096 + 4 * 4096 * 32


def test_counter_traffic_needs_matching_sources(tmp_path, monkeypatch):
    rec = {"decode": {"source_digest": "abc", "bytes_per_launch": 123}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "abc")
    assert bench.counter_traffic("decode") == 123
    assert bench.counter_traffic("prefill") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "changed")
    assert bench.counter_traffic("decode") is None


def test_counter_traffic_missing_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("decode") is None


def test_source_digest_is_stable_and_short():
    a, b = bench.source_digest(), bench.source_digest()
    assert a == b and len(a) == 16


@pytest.mark.parametrize("name,shape", [
    ("tiny", (16, 256, 256)), ("decode", (8, 4096, 4096)), ("prefill", (4096, 4096, 4096)),
    ("gate_up", (2048, 4096, 28672)), ("down", (2048, 14336, 4096)), ("ragged", (333, 4000, 5000)),
])
def test_dense_workload_shapes(name, shape):
    c = wl.CONFIGS[name]
    assert (c["M"], c["K"], c["N"]) == shape


def test_moe_workload_shape():
    c = wl.CONFIGS["moe"]
    assert (c["T"], c["H"], c["I"], c["E"], c["topk"]) == (4096, 4096, 14336, 8, 2)


def test_weight_copies_cover_the_cache():
    # enough rotating copies that the 256 MB last-level cache cannot hold them
    n = bench.n_copies(4096 * 4096)
    assert n * 4096 * 4096 >= 256 * 2**20
    assert bench.n_copies(4096 * 4096, override=3) == 3


class _FakeBuf:
    def __init__(self, a):
        self.a = a

    def cpu(self):
        return self

    def numpy(self):
        return self.a


def test_clock_probe_reads_cycles_over_real_time_per_unit():
    """Two samples per compute unit: cycles / real-time ticks * tick rate =
    clock; units are matched by XCD and HW_ID bits [15:8], the XCD's figure
    is the median over its units."""
    import numpy as np
    p = bench.ClockProbe.__new__(bench.ClockProbe)
    p.rate_khz = 100000   # 100 MHz real-time counter

    def place(xcd, cu):
        return (cu << 40) | (0x3 << 32) | xcd   # wave / SIMD bits (low HW_ID bits) are ignored

    b = np.zeros((2, 5, 3), np.int64)
    # XCD 0: two units at 2000 MHz (20 cycles per tick) with unrelated counter
    # origins; XCD 1: one unit at 2200 MHz; the second sample lists them in
    # another order, and a unit seen only once is ignored
    b[0] = [[1000, 500, place(0, 1)], [9_000_000, 500, place(0, 2)], [7000, 501, place(1, 1)],
            [1010, 502, place(0, 1)], [5, 5, place(1, 9)]]
    b[1] = [[7000 + 22 * 1000, 1501, place(1, 1)], [1000 + 20 * 1000, 1500, place(0, 1)],
            [9_000_000 + 20 * 2000, 2500, place(0, 2)], [0, 0, place(0, 7)], [0, 0, place(0, 1)]]
    p.buf = _FakeBuf(b)
    r = p.read()
    assert r["xcds"] == 2 and r["cus"] == 3
    assert r["min"] == 2000.0 and r["max"] == 2200.0 and r["mhz"] == 2100.0
    p.rate_khz = 0
    assert p.read() is None


def test_roofline_scales_the_int8_peak_to_the_observed_clock():
    class W:
        dominant, dominant_ops, dominant_bytes = "k", 2 * 4096 ** 3, 67_600_000
    r = bench.roofline(W, 100e-6, {"mhz": 1800.0, "min": 1790.0, "max": 1810.0, "xcds": 8})
    assert r["bound"] == "mfma"
    assert abs(r["achieved"] - 1374.4) < 0.1 and r["peak"] == 5000.0
    assert r["peak_at_clock"] == 3750.0 and abs(r["frac_at_clock"] - 1374.4 / 3750.0) < 1e-4
