"""Host-side arithmetic of bench.py's roofline ceilings and counted-traffic
fields (no GPU).

Expected values are worked out by hand from the workload shapes: bytes = A
(M*K) + B (N*K) + fp32 scales (M*K/128 and ceil(N/128)*K/128 words) + bf16 D
(2*M*N); ceiling = min(5000 TFLOP/s, 2*M*N*K / bytes * 8 TB/s).
"""
import math

import bench


def test_min_bytes_dense():
    # 64 x 2112 x 7168: 458752 + 15138816 + 14336 + 3808 + 270336 bytes
    want = 64 * 7168 + 2112 * 7168 + 4 * 64 * 56 + 4 * 17 * 56 + 2 * 64 * 2112
    assert bench.min_bytes(64, 2112, 7168) == want == 15886048


def test_min_bytes_grouped():
    # 16 groups of B [4096, 7168] dominate: 16 * 29.36 MB = 469.8 MB
    got = bench.min_bytes(0, 4096, 7168, groups=16)
    assert got == 16 * 4096 * 7168 + 4 * 16 * 32 * 56


def test_ceilings():
    # HBM-bound: 2*64*2112*7168 flops over 15.89 MB at 8 TB/s -> 975.8 TFLOP/s (19.5% of peak)
    c = bench.ceiling_tflops(2.0 * 64 * 2112 * 7168, bench.min_bytes(64, 2112, 7168))
    assert math.isclose(c, 2.0 * 64 * 2112 * 7168 / 15886048 * 8e12 / 1e12, rel_tol=1e-12)
    assert 975 < c < 976.5
    # MFMA-bound: the 4096 x 7168 x 16384 shape is capped at the FP8 peak
    assert bench.ceiling_tflops(2.0 * 4096 * 7168 * 16384, bench.min_bytes(4096, 7168, 16384)) == 5000.0


def _raw_row(name):
    """Raw (FETCH_SIZE KiB, WRITE_SIZE KiB) of one row of the committed counter file."""
    for line in open(bench.TRAFFIC_ROWS_FILE):
        if line.startswith(name + " ="):
            fetch, write = line.split("=", 1)[1].split()
            return float(fetch), float(write)
    raise KeyError(name)


def test_counted_traffic_rows():
    t = bench.counted_traffic()
    if not t:   # kernel sources changed since the counters were taken
        return
    # FETCH_SIZE reads 0.5x of the true bytes, WRITE_SIZE 1.0x, both in KiB per call
    fetch, write = _raw_row("64x2112x7168")
    assert math.isclose(t["64x2112x7168"], (fetch / 0.5 + write) * 1024, rel_tol=1e-12)
    # 64 x 2112 x 7168 moves about 26.9 MB per call (15.9 MB algorithmic plus the split-K partials)
    assert 20e6 < t["64x2112x7168"] < 35e6
    rows = {"%dx%dx%d" % (m, n, k) for m in (64, 128)
            for (n, k) in ((2112, 7168), (24576, 1536), (7168, 16384), (4096, 7168), (7168, 2048))}
    assert rows <= set(t)
    # bytes over 10 us, in GB/s
    assert bench.counted_gbs(t, "64x2112x7168", 10.0) == round(t["64x2112x7168"] / 10e-6 / 1e9, 1)
    assert bench.counted_gbs(t, "no such row", 10.0) is None


def test_counted_traffic_ignored_after_a_kernel_change(monkeypatch):
    monkeypatch.setattr(bench, "gemm_source_sha256", lambda: "0" * 64)
    assert bench.counted_traffic() == {}
