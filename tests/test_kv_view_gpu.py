"""Attention over keys and values held in a KV cache (sdpa_forward_kv_view).

The verify probe of lablup/mlxcel issue #2160 ("Gemma 4 MTP never engages on
CUDA (GB10), verify probe fails") runs over caches: capacity-padded buffers
whose live keys are a prefix ("strided, sliced keys", Current Behavior, 31B)
and sliding-window layers kept as a ring with a cursor (Current Behavior,
12B and 31B; Proposed Solution step 2).  A cache of `cap` rows per head
holds kv_len live keys, logical key j in row (ring_start + j) % cap.

Checked here: parity with the fp64 oracle run on the live keys in logical
order; that a ring view gives the same bytes as the same keys stored from
row 0 (the kernel accumulates in logical order); that rows outside the live
keys are never read (they hold NaN); and that each row of a verify block
over a ring equals, byte for byte, the single-row call over its own trimmed
prefix of the same cache.
"""

import numpy as np
import pytest
import torch

import flash_attention_head_amd as fa
from flash_attention_head_amd import workloads as W
from gpu_util import check_close, ensure_library, f64, note, oracle_full

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def to_cache(x, cap, ring_start):
    """Logical [B, H, n, D] rows into a cache of cap rows, key j at row
    (ring_start + j) % cap; rows holding no live key are NaN."""
    B, H, n, D = x.shape
    cache = torch.full((B, H, cap, D), float("nan"), dtype=x.dtype)
    idx = (ring_start + torch.arange(n)) % cap
    cache[:, :, idx] = x
    return cache


def run_view(q, kc, vc, kv_len, ring_start, **kw):
    out = fa.sdpa_kv_cache(q.cuda(), kc.cuda(), vc.cuda(), kv_len, ring_start=ring_start, **kw)
    torch.cuda.synchronize()
    return out.cpu()


# (B, Hq, Hkv, qL, kL, cap, ring_start, D, dtype, causal, window, q_offset)
CASES = [
    (1, 4, 2, 100, 1000, 1500, 0, 256, BF16, True, 0, 900),       # padded cache, prefix-filled
    (1, 4, 2, 4, 2500, 4000, 700, 256, FP16, True, 0, 2496),      # live run at an offset, no wrap
    (1, 4, 2, 4, 1000, 1000, 963, 256, BF16, True, 0, 996),       # full ring, wrap at an odd row of a tile
    (1, 4, 2, 4, 1000, 1000, 872, 256, FP16, True, 0, 996),       # full ring, wrap at a tile edge
    (1, 4, 2, 3, 2048, 2048, 1001, 256, BF16, True, 1024, 2045),  # sliding ring, window
    (1, 4, 2, 4, 1000, 1500, 1200, 256, FP16, True, 0, 996),      # wrapped, NaN rows in the middle
    (1, 4, 2, 300, 1000, 1000, 517, 256, FP16, True, 0, 700),     # prefill over a wrapped ring
    (1, 4, 2, 200, 9000, 9000, 4321, 256, BF16, True, 500, 8800),  # key split over a wrapped ring
    (2, 2, 1, 2, 700, 800, 750, 256, FP16, False, 0, 0),          # unmasked decode, wrapped
    (1, 4, 1, 4, 700, 700, 333, 512, BF16, True, 0, 696),         # head_dim 512, wrapped
    (1, 2, 1, 100, 600, 640, 601, 512, FP16, True, 0, 500),       # head_dim 512 prefill, wrapped
    (1, 2, 1, 4, 600, 640, 17, 512, BF16, True, 0, 596),          # head_dim 512, offset, no wrap
    (1, 4, 2, 4, 1000, 1000, 963, 128, BF16, True, 0, 996),       # head_dim 128, wrapped ring
    (1, 4, 2, 200, 3000, 3000, 1501, 128, FP16, True, 0, 2800),   # head_dim 128 prefill, wrapped
    (1, 4, 2, 4, 1000, 1000, 963, 192, FP16, True, 0, 996),       # head_dim 192, wrapped ring
    (1, 4, 2, 200, 3000, 3200, 2901, 192, BF16, True, 0, 2800),   # head_dim 192 prefill, wrapped
    (1, 4, 2, 4, 1000, 1000, 963, 64, BF16, True, 0, 996),        # head_dim 64, wrapped ring
    (1, 4, 2, 4, 1000, 1000, 963, 80, FP16, True, 0, 996),        # head_dim 80, wrapped ring
    (1, 4, 2, 200, 3000, 3000, 1501, 80, BF16, True, 0, 2800),    # head_dim 80 prefill, wrapped
]


@pytest.mark.parametrize("case", CASES, ids=[f"q{c[3]}k{c[4]}cap{c[5]}r{c[6]}D{c[7]}" for c in CASES])
def test_cache_views_match_the_oracle(case):
    B, Hq, Hkv, qL, kL, cap, rs, D, dtype, causal, window, q_offset = case
    q, k, v = W.random_qkv(3000 + kL + rs, B, Hq, Hkv, qL, kL, D, dtype)
    note(f"kv view {case}")
    got = f64(run_view(q, to_cache(k, cap, rs), to_cache(v, cap, rs), kL, rs, causal=causal,
                       window=window, q_offset=q_offset))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ref = oracle_full(q, k, v, scale=scale, causal=causal, window=window, q_offset=q_offset,
                      dtype=dtype)
    check_close(got, ref, dtype, f"kv view {case}")


@pytest.mark.parametrize("qL,kL,cap,rs,D", [(4, 3000, 3000, 1234, 256), (4, 3000, 3500, 3301, 256),
                                            (130, 5000, 5000, 2047, 256), (4, 1500, 1500, 1499, 512),
                                            (70, 1500, 1600, 900, 512), (4, 1000, 1000, 962, 128),
                                            (70, 1000, 1000, 961, 128), (4, 1000, 1000, 962, 192)])
def test_ring_view_equals_the_same_keys_from_row_zero(qL, kL, cap, rs, D):
    q, k, v = W.random_qkv(4000 + rs, 1, 8, 2, qL, kL, D, BF16)
    note(f"ring vs row-0 cache q{qL} k{kL} cap{cap} r{rs} D{D}")
    ring = run_view(q, to_cache(k, cap, rs), to_cache(v, cap, rs), kL, rs, causal=True)
    flat = run_view(q, to_cache(k, cap, 0), to_cache(v, cap, 0), kL, 0, causal=True)
    assert torch.equal(ring.view(torch.int16), flat.view(torch.int16))


def _check_verify_rows(q, kc, vc, kL, rs, *, window, what):
    """Each row of a qL-row verify block over the cache equals the single-row
    call over its own trimmed prefix of the same cache, byte for byte."""
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    qL = q.shape[2]
    note(f"{what}: block of {qL} rows")
    block = fa.sdpa_kv_cache(qd, kd, vd, kL, ring_start=rs, causal=True, window=window,
                             q_offset=kL - qL)
    torch.cuda.synchronize()
    for r in range(qL):
        n = kL - qL + r + 1
        note(f"{what}: row {r} over {n} keys")
        one = fa.sdpa_kv_cache(qd[:, :, r:r + 1].contiguous(), kd, vd, n, ring_start=rs, causal=True,
                               window=window, q_offset=n - 1)
        torch.cuda.synchronize()
        a = block[:, :, r:r + 1].contiguous().view(torch.int16)
        b = one.view(torch.int16)
        assert torch.equal(a, b), f"{what}: row {r} differs in {(a != b).sum().item()} elements"


@pytest.mark.timeout(600)
def test_verify_rows_over_a_wrapped_128k_ring_match_single_row_calls():
    wl = W.WORKLOADS["decode_q4_128k"]
    q, k, v = W.draw(wl)
    rs = 54321
    _check_verify_rows(q, to_cache(k, wl.kL, rs), to_cache(v, wl.kL, rs), wl.kL, rs, window=0,
                       what="128k ring")


@pytest.mark.timeout(600)
def test_verify_rows_over_a_sliding_window_ring_match_single_row_calls():
    # the 12B sliding layers: 16 query / 8 KV heads at head_dim 256, window 1024,
    # kept as a ring of 1024 rows whose cursor has wrapped
    q, k, v = W.random_qkv(71, 1, 16, 8, 4, 1024, 256, BF16)
    _check_verify_rows(q, to_cache(k, 1024, 777), to_cache(v, 1024, 777), 1024, 777, window=1024,
                       what="sliding ring 1024")


@pytest.mark.timeout(600)
def test_verify_rows_across_a_chunk_size_step_of_the_key_count():
    # 8 KV heads: were the chunk sized from the live key count it would step
    # from 2048 to 4096 keys between 126976 and 126977 keys, inside this
    # block's rows; sized from the capacity it does not move
    q, k, v = W.random_qkv(72, 1, 16, 8, 4, 126978, 256, FP16)
    cap = 131072
    _check_verify_rows(q, to_cache(k, cap, 0), to_cache(v, cap, 0), 126978, 0, window=0,
                       what="capacity 128k, 126978 keys")
