"""Byte accounting used by the peak-memory checks, pinned to the pages' table."""

import os

from flash_attention_head_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mlx3660_peak_memory.tsv")
MiB = 1 << 20


def _rows():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        yield [int(x) for x in line.split()]


def test_input_bytes_and_fused_peak_match_the_microbenchmark_table():
    rows = list(_rows())
    assert len(rows) == 3
    for qL, kL, inputs_mib, peak_mib in rows:
        b = W.io_bytes(1, 16, 8, qL, kL, 256, 2)
        assert b["inputs"] == inputs_mib * MiB
        # a fused kernel that allocates nothing beyond its output peaks at inputs + output
        assert b["inputs"] + b["out"] == peak_mib * MiB


def test_flop_count_of_named_workloads():
    # 4 * B * Hq * D * visible pairs; full causal square: L (L + 1) / 2 pairs per head
    wl = W.WORKLOADS["causal_h64_16k"]
    L = 16384
    assert W.flops(wl) == 4.0 * 64 * 256 * (L * (L + 1) // 2)
    wl = W.WORKLOADS["sliding_32k"]
    pairs = sum(min(p + 1, 1024) for p in range(32768))
    assert W.flops(wl) == 4.0 * 32 * 256 * pairs
    wl = W.WORKLOADS["chunked_prefill_32k"]
    pairs = sum(31744 + i + 1 for i in range(1024))
    assert W.flops(wl) == 4.0 * 16 * 256 * pairs
