"""q/k head dim 192 with v head dim 256 (sdpa_forward_dv) against the fp64 oracle.

The review discussion of ml-explore/mlx PR #3293 names models whose heads
are Q=192/K=192/V=256 and notes that its fused path, gated on equal query
and value head dims, leaves them out.  Here the scores take the 192-long
dot products and each output row is the weighted sum of 256-long value
rows.  Small shapes compare every row; the full-size workload compares
sampled rows in the configuration the benchmark times; zero queries give
the mean of the visible value rows at any size.
"""

import numpy as np
import pytest
import torch

import flash_attention_head_amd as fa
import oracle
from flash_attention_head_amd import workloads as W
from gpu_util import ORACLE_THREADS, TOL, check_close, ensure_library, f64, note, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def oracle_dv(q, k, v, rows=None, *, scale, causal, window, q_offset, dtype):
    return oracle.sdpa_dv_f64(W.bits(q), W.bits(k), W.bits(v), scale=scale, causal=causal, window=window,
                              q_offset=q_offset, dtype=dtype, rows=rows, threads=ORACLE_THREADS)


# (B, Hq, Hkv, qL, kL, dtype, causal, window, q_offset)
CASES = [
    (2, 4, 2, 333, 333, BF16, True, 0, 0),        # ragged tiles and row blocks
    (1, 4, 2, 100, 1000, FP16, True, 77, 900),    # window over a prefix
    (1, 2, 2, 257, 190, FP16, False, 0, 0),       # no mask, qL > kL
    (1, 8, 1, 65, 700, BF16, True, 33, 635),      # G = 8
    (1, 2, 1, 300, 9000, BF16, True, 0, 8700),    # key split + combine
    (1, 4, 2, 4, 2500, FP16, True, 0, 2496),      # verify block
    (2, 2, 1, 1, 700, BF16, False, 0, 0),         # unmasked decode
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}q{c[3]}k{c[4]}c{int(c[6])}w{c[7]}"
                                             for c in CASES])
def test_value_dim_256_matches_the_oracle(case):
    B, Hq, Hkv, qL, kL, dtype, causal, window, q_offset = case
    q, k, v = W.random_qkv(7000 + qL + kL, B, Hq, Hkv, qL, kL, 192, dtype, Dv=256)
    note(f"dk192 dv256 {case}")
    got = run_gpu(q, k, v, causal=causal, window=window, q_offset=q_offset)
    assert tuple(got.shape) == (B, Hq, qL, 256)
    scale = float(np.float32(1.0 / np.sqrt(192)))
    ref = oracle_dv(q, k, v, scale=scale, causal=causal, window=window, q_offset=q_offset, dtype=dtype)
    check_close(f64(got), ref, dtype, f"dk192 dv256 {case}")


def test_value_columns_match_the_equal_dim_calls():
    # the output's leading 192 columns use the same weights as a D = 192
    # call over those value columns; they agree within rounding of the two
    # kernels' accumulation (not bitwise: the P V products differ in blocking)
    q, k, v = W.random_qkv(7100, 1, 4, 2, 200, 1500, 192, BF16, Dv=256)
    note("dk192 dv256 vs D192 on the leading columns")
    wide = f64(run_gpu(q, k, v, causal=True, q_offset=1300))
    lead = f64(run_gpu(q, k, v[..., :192].contiguous(), causal=True, q_offset=1300))
    assert np.abs(wide[..., :192] - lead).max() <= 2 * TOL[BF16]


@pytest.mark.timeout(600)
def test_full_size_workload_on_sampled_rows():
    wl = W.WORKLOADS["causal_dk192_dv256_16k"]
    q, k, v = W.draw(wl)
    note(f"{wl.name} full size")
    got = run_gpu(q, k, v, causal=wl.causal, window=wl.window, q_offset=wl.q_offset)
    assert torch.isfinite(got.float()).all()
    rows = sample_rows(wl, 96, seed=wl.seed)
    ref = oracle_dv(q, k, v, rows, scale=wl.scale, causal=wl.causal, window=wl.window, q_offset=wl.q_offset,
                    dtype=wl.dtype)
    check_close(f64(got.reshape(-1, wl.dv)[torch.from_numpy(rows)]), ref, wl.dtype,
                f"{wl.name} ({rows.size} rows)")


@pytest.mark.timeout(600)
def test_zero_queries_average_visible_values_at_full_size():
    wl = W.WORKLOADS["causal_dk192_dv256_16k"]
    _, k, v = W.draw(wl)
    q = torch.zeros((wl.B, wl.Hq, wl.qL, wl.D), dtype=W.TORCH_DTYPES[wl.dtype])
    note(f"{wl.name} zero queries")
    got = run_gpu(q, k, v, causal=wl.causal, window=wl.window, q_offset=wl.q_offset)
    G = wl.Hq // wl.Hkv
    p = wl.q_offset + np.arange(wl.qL)
    hi = np.minimum(p, wl.kL - 1)
    n = (hi + 1).astype(np.float64)[:, None]
    worst = 0.0
    for hk in sorted({0, wl.Hkv // 2, wl.Hkv - 1}):
        csum = np.zeros((wl.kL + 1, wl.dv))
        np.cumsum(v[0, hk].to(torch.float64).numpy(), axis=0, out=csum[1:])
        mean = csum[hi + 1] / n
        for g in range(G):
            worst = max(worst, float(np.abs(f64(got[0, hk * G + g]) - mean).max()))
    print(f"[parity] {wl.name} zero-query mean: max err {worst:.3e}", flush=True)
    assert worst <= TOL[wl.dtype]


def test_unsupported_pairs_are_rejected_before_any_launch():
    q, k, v = W.random_qkv(7200, 1, 2, 1, 8, 64, 256, FP16, Dv=192)
    with pytest.raises(fa.SdpaError) as e:
        fa.sdpa(q.cuda(), k.cuda(), v.cuda(), causal=True)
    assert e.value.status == fa.SDPA_UNSUPPORTED
