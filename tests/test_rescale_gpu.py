"""The online softmax's mid-row rescale, forced by inputs whose scores climb.

The kernels keep a per-row reference maximum that moves only when a tile's
maximum beats it by more than 2^8 in base-2 units (the weights then stay at
most 256); when it moves, the output accumulator and the running sum are
scaled by alpha = 2^(old - new), 0 < alpha < 1.  N(0, 1) inputs at scale
1/sqrt(D) almost never trigger that after the first tile, so these tests use
``workloads.ramp_qkv``: each row's scores grow along the keys by up to ~60
natural units, so the reference moves many times per row, and the tiles just
below a move carry weights near 256 (the top of the fp16 range the P operand
is rounded into).  Rows of shrinking scores (their maximum among the first
keys) and rows of both kinds share each workgroup, so the skip taken when no
row of a wave moved runs beside the rescale.

Every entry point is covered (prefill, key split + combine, decode / verify
chunks, a wrapped KV-cache ring, the additive mask array, a value head dim
other than q's) at head dims 64 to 512 in fp16 and bf16, each output row
compared with the fp64 oracle at the stated tolerance.  Each case also
checks, on the host from the scores themselves, that most rows do reach a
tile whose maximum beats their first tile's by more than 8 ln 2.
"""

import math

import numpy as np
import pytest
import torch

import flash_attention_head_amd as fa
import oracle
from flash_attention_head_amd import workloads as W
from gpu_util import ORACLE_THREADS, check_close, ensure_library, f64, note, oracle_dense_rows, oracle_full

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def rows_that_rescale(q, k, *, scale, causal, window, q_offset, tile):
    """Fraction of rows whose visible scores reach a tile whose maximum exceeds
    the maximum of the row's first visible tile by more than 8 ln 2 (natural
    units): such a row moves its reference maximum with 0 < alpha < 1."""
    B, Hq, qL, D = q.shape
    G = Hq // k.shape[1]
    kf = k.to(torch.float64).repeat_interleave(G, dim=1)
    s = (q.to(torch.float64) @ kf.transpose(-1, -2)) * float(np.float32(scale))  # [B, Hq, qL, kL]
    kL = k.shape[2]
    p = q_offset + torch.arange(qL).view(qL, 1)
    j = torch.arange(kL).view(1, kL)
    vis = torch.ones((qL, kL), dtype=torch.bool)
    if causal:
        vis &= j <= p
    if window:
        vis &= (p - j) < window
    s = s.masked_fill(~vis, -math.inf)
    first = j // tile == (torch.argmax(vis.int(), dim=1, keepdim=True) // tile)
    m0 = s.masked_fill(~first, -math.inf).amax(-1)
    return float(((s.amax(-1) - m0) > 8 * math.log(2)).double().mean())


# (B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset)
PREFILL = [
    (1, 4, 2, 333, 1000, 256, FP16, True, 0, 667),
    (1, 4, 2, 333, 1000, 256, BF16, False, 0, 0),
    (2, 8, 2, 200, 700, 512, BF16, True, 0, 500),
    (1, 4, 1, 150, 900, 512, FP16, False, 0, 0),
    (1, 8, 2, 333, 1500, 128, FP16, True, 0, 1167),
    (1, 4, 2, 300, 1200, 128, BF16, False, 0, 0),
    (1, 4, 2, 300, 1200, 64, FP16, True, 0, 900),
    (1, 4, 2, 300, 1200, 64, BF16, False, 0, 0),
    (1, 4, 2, 300, 1200, 80, BF16, True, 0, 900),
    (1, 4, 2, 300, 1200, 192, FP16, True, 0, 900),
    (1, 4, 2, 100, 2000, 256, BF16, True, 600, 1900),     # window: the ramp within 600 keys
    (1, 2, 1, 300, 9000, 256, FP16, True, 0, 8700),      # key split + combine
    (1, 2, 1, 130, 8300, 512, BF16, True, 0, 8170),      # head dim 512 key split
    (1, 4, 2, 4, 5000, 256, FP16, True, 0, 4996),        # verify block: decode chunks
    (1, 4, 2, 1, 5000, 256, BF16, True, 0, 4999),        # decode
    (1, 8, 2, 4, 3000, 512, FP16, True, 0, 2996),        # head dim 512 verify
    (1, 4, 2, 3, 4000, 128, BF16, True, 0, 3997),        # head dim 128 verify
]


@pytest.mark.parametrize("case", PREFILL, ids=[f"q{c[3]}k{c[4]}D{c[5]}{'bf16' if c[6] else 'f16'}c{int(c[7])}w{c[8]}"
                                               for c in PREFILL])
def test_rescaled_rows_match_the_oracle(case):
    B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset = case
    q, k, v = W.ramp_qkv(9000 + qL + kL + D, B, Hq, Hkv, qL, kL, D, dtype)
    scale = float(np.float32(1 / math.sqrt(D)))
    frac = rows_that_rescale(q, k, scale=scale, causal=causal, window=window, q_offset=q_offset,
                             tile=32 if D == 512 else 64)
    note(f"rescale {case} ({frac:.0%} of rows move their reference mid-row)")
    assert frac > 0.4, frac
    out = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, window=window, q_offset=q_offset)
    torch.cuda.synchronize()
    ref = oracle_full(q, k, v, scale=scale, causal=causal, window=window, q_offset=q_offset, dtype=dtype)
    check_close(f64(out.cpu()), ref, dtype, f"rescale {case}")


@pytest.mark.parametrize("qL,D,dtype", [(4, 256, BF16), (300, 256, FP16), (4, 512, FP16), (200, 128, BF16)])
def test_rescaled_rows_over_a_wrapped_cache_ring(qL, D, dtype):
    kL, cap, ring_start = 3000, 3500, 2100  # wraps after 1400 keys
    q, k, v = W.ramp_qkv(9100 + qL + D, 1, 4, 2, qL, kL, D, dtype)
    idx = (ring_start + torch.arange(kL)) % cap
    kc = torch.zeros((1, 2, cap, D), dtype=k.dtype)
    vc = torch.zeros((1, 2, cap, D), dtype=v.dtype)
    kc[:, :, idx], vc[:, :, idx] = k, v
    scale = float(np.float32(1 / math.sqrt(D)))
    note(f"rescale ring qL {qL} D {D}")
    out = fa.sdpa_kv_cache(q.cuda(), kc.cuda(), vc.cuda(), kL, ring_start=ring_start, scale=scale, causal=True)
    torch.cuda.synchronize()
    ref = oracle_full(q, k, v, scale=scale, causal=True, window=0, q_offset=kL - qL, dtype=dtype)
    check_close(f64(out.cpu()), ref, dtype, f"rescale ring qL {qL} D {D}")


@pytest.mark.parametrize("qL,kL,D,dtype", [(300, 1000, 256, FP16), (4, 3000, 256, BF16), (150, 600, 512, BF16),
                                           (200, 900, 64, FP16)])
def test_rescaled_rows_with_an_additive_mask(qL, kL, D, dtype):
    q, k, v = W.ramp_qkv(9200 + qL + D, 1, 4, 2, qL, kL, D, dtype)
    g = torch.Generator().manual_seed(9201 + D)
    bias = (torch.randn((1, 4, qL, kL), generator=g) * 2.0).to(W.TORCH_DTYPES[dtype])
    scale = float(np.float32(1 / math.sqrt(D)))
    note(f"rescale bias qL {qL} kL {kL} D {D}")
    out = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True, bias=bias.cuda())
    torch.cuda.synchronize()
    ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=scale, causal=True,
                               q_offset=kL - qL, dtype=dtype, threads=ORACLE_THREADS)
    check_close(f64(out.cpu()), ref, dtype, f"rescale bias qL {qL} kL {kL} D {D}")


@pytest.mark.parametrize("qL,kL,dtype", [(300, 1200, BF16), (4, 3000, FP16)])
def test_rescaled_rows_with_a_wider_value_head(qL, kL, dtype):
    q, k, v = W.ramp_qkv(9300 + qL, 1, 4, 2, qL, kL, 192, dtype, Dv=256)
    scale = float(np.float32(1 / math.sqrt(192)))
    note(f"rescale dv qL {qL} kL {kL}")
    out = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True)
    torch.cuda.synchronize()
    rows = np.arange(4 * qL, dtype=np.int64)
    ref = oracle_dense_rows(q, k, v, rows, scale=scale, causal=True, window=0, q_offset=kL - qL, dtype=dtype)
    check_close(f64(out.cpu().reshape(-1, 256)), ref, dtype, f"rescale dv qL {qL} kL {kL}")
