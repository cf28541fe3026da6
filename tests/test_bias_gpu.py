"""Attention with an additive mask array (sdpa_forward_bias) against the oracle.

The array mask of lablup/mlxcel issue #672 (Root cause: a windowed/causal
additive mask handed to SDPA; cuDNN takes such an array as a bias), added to
the scaled scores before softmax.  The oracle is oracle.sdpa_bias_f64, the
same plain definition with the bias term.
"""

import numpy as np
import pytest
import torch

import flash_attention_head_amd as fa
import oracle
from flash_attention_head_amd import workloads as W
from gpu_util import ORACLE_THREADS, check_close, ensure_library, f64, note

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def make_bias(seed, shape, dtype, ninf_frac=0.1, sigma=2.0):
    """N(0, sigma) bias rounded to dtype, some entries -inf (never key 0)."""
    g = torch.Generator().manual_seed(seed)
    b = torch.randn(shape, generator=g) * sigma
    if ninf_frac > 0:
        drop = torch.rand(shape, generator=g) < ninf_frac
        drop[..., 0] = False
        b[drop] = float("-inf")
    return b.to(W.TORCH_DTYPES[dtype])


def run_bias(q, k, v, bias, **kw):
    out = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), bias=bias.cuda(), **kw)
    torch.cuda.synchronize()
    return out.cpu()


# (B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset, bias batch, bias heads)
CASES = [
    (2, 4, 2, 333, 333, 256, FP16, True, 0, 0, True, True),      # ragged tiles, full bias
    (1, 4, 2, 100, 1000, 256, BF16, True, 77, 900, False, True),  # window over a prefix, per-head bias
    (1, 2, 2, 257, 190, 256, FP16, False, 0, 0, False, False),   # no causal mask, one shared bias
    (1, 8, 1, 65, 700, 256, BF16, True, 0, 635, True, False),    # G = 8, batch-only bias
    (1, 2, 1, 300, 9000, 256, FP16, True, 0, 8700, False, True),  # key split + combine
    (1, 4, 2, 4, 2500, 256, BF16, True, 0, 2496, False, True),    # verify block (split path)
    (2, 4, 1, 150, 150, 512, BF16, True, 0, 0, True, True),      # head_dim 512
    (1, 2, 1, 130, 4100, 512, FP16, True, 0, 3970, False, False),  # head_dim 512 with key split
    (2, 4, 2, 200, 333, 128, FP16, True, 0, 133, True, True),    # head_dim 128
    (1, 4, 2, 4, 3000, 128, BF16, False, 0, 0, False, True),     # head_dim 128 decode, unmasked
    (2, 4, 2, 200, 333, 192, BF16, True, 0, 133, True, True),    # head_dim 192
    (1, 4, 2, 4, 3000, 192, FP16, True, 0, 2996, False, True),   # head_dim 192 verify block
    (2, 4, 2, 200, 333, 64, FP16, True, 0, 133, True, True),     # head_dim 64
    (2, 4, 2, 200, 333, 80, BF16, True, 0, 133, True, True),     # head_dim 80
    (1, 2, 1, 130, 4100, 80, FP16, True, 0, 3970, False, False),  # head_dim 80 with key split
]


@pytest.mark.parametrize("case", CASES, ids=[f"q{c[3]}k{c[4]}D{c[5]}c{int(c[7])}w{c[8]}b{int(c[10])}{int(c[11])}"
                                             for c in CASES])
def test_bias_matches_the_oracle(case):
    B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset, bb, bh = case
    q, k, v = W.random_qkv(5000 + qL + kL + D, B, Hq, Hkv, qL, kL, D, dtype)
    bias = make_bias(6000 + kL, (B if bb else 1, Hq if bh else 1, qL, kL), dtype)
    note(f"bias {case}")
    got = f64(run_bias(q, k, v, bias, causal=causal, window=window, q_offset=q_offset))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=scale, causal=causal,
                               window=window, q_offset=q_offset, dtype=dtype, threads=ORACLE_THREADS)
    check_close(got, ref, dtype, f"bias {case}")


@pytest.mark.parametrize("B,Hq,Hkv,qL,kL,bb,bh", [(2, 12, 3, 3, 3, False, True), (1, 2, 1, 5, 333, False, False),
                                                  (2, 4, 2, 333, 333, True, True)])
def test_the_last_bias_element_counts_when_kl_is_odd(B, Hq, Hkv, qL, kL, bb, bh):
    # the last row of the bias starts at an odd element (or kL is odd with an
    # even start): the 4-byte word holding its last key reaches 2 bytes past
    # the bias.  That key is visible (causal, the diagonal of the last row)
    # and its bias is large, so reading it as zero would move the row far
    # outside the tolerance
    q, k, v = W.random_qkv(5200 + kL, B, Hq, Hkv, qL, kL, 256, FP16)
    bias = make_bias(5300 + kL, (B if bb else 1, Hq if bh else 1, qL, kL), FP16, ninf_frac=0.0)
    bias[..., -1, -1] = 6.0
    note(f"last bias element, B{B} Hq{Hq} qL{qL} kL{kL}")
    got = run_bias(q, k, v, bias, causal=True, q_offset=kL - qL)
    scale = float(np.float32(1.0 / 16))
    ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=scale, causal=True,
                               q_offset=kL - qL, dtype=FP16, threads=ORACLE_THREADS)
    check_close(f64(got), ref, FP16, f"last bias element, B{B} Hq{Hq} qL{qL} kL{kL}")


def test_rows_with_no_finite_biased_score_are_zero():
    q, k, v = W.random_qkv(5101, 1, 4, 2, 70, 300, 256, BF16)
    bias = make_bias(5102, (1, 4, 70, 300), BF16, ninf_frac=0.0)
    bias[0, 1, 5, :] = float("-inf")    # every key of row 5 of head 1
    bias[0, 3, 69, 200:] = float("-inf")  # the keys row 69 (position 299) sees from 200 on; 0..199 stay
    note("all -inf rows")
    got = run_bias(q, k, v, bias, causal=True, q_offset=230)
    assert torch.isfinite(got.float()).all()
    assert torch.count_nonzero(got[0, 1, 5]) == 0
    scale = float(np.float32(1.0 / 16))
    ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=scale, causal=True,
                               q_offset=230, dtype=BF16, threads=ORACLE_THREADS)
    check_close(f64(got), ref, BF16, "all -inf rows")


@pytest.mark.parametrize("D,qL,kL", [(256, 300, 2000), (512, 100, 700), (128, 4, 5000)])
def test_zero_bias_gives_the_unbiased_bytes(D, qL, kL):
    # s + 0 == s exactly, so the bias instance must reproduce sdpa_forward bit for bit
    q, k, v = W.random_qkv(5200 + D, 1, 4, 2, qL, kL, D, FP16)
    note(f"zero bias D{D}")
    zero = torch.zeros((1, 1, qL, kL), dtype=torch.float16)
    a = run_bias(q, k, v, zero, causal=True)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    b = fa.sdpa(qd, kd, vd, causal=True).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_verify_rows_with_bias_match_single_row_calls():
    # each verify row equals the single-row call over its trimmed prefix, with
    # its own bias row trimmed likewise (a strided view of the same tensor)
    q, k, v = W.random_qkv(5300, 1, 16, 8, 4, 20000, 256, BF16)
    bias = make_bias(5301, (1, 16, 4, 20000), BF16).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    note("verify rows with bias")
    block = fa.sdpa(qd, kd, vd, bias=bias, causal=True, q_offset=20000 - 4)
    torch.cuda.synchronize()
    for r in range(4):
        n = 20000 - 4 + r + 1
        one = fa.sdpa(qd[:, :, r:r + 1].contiguous(), kd[:, :, :n].contiguous(), vd[:, :, :n].contiguous(),
                      bias=bias[:, :, r:r + 1, :n], causal=True, q_offset=n - 1)
        torch.cuda.synchronize()
        assert torch.equal(block[:, :, r:r + 1].contiguous().view(torch.int16), one.view(torch.int16)), r


@pytest.mark.timeout(600)
def test_full_size_bias_workload_on_sampled_rows():
    wl = W.WORKLOADS["chunked_prefill_32k_bias"]
    q, k, v = W.draw(wl)
    bias = W.draw_bias(wl)
    note(f"{wl.name} full size")
    got = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), bias=bias.cuda(), causal=wl.causal, q_offset=wl.q_offset)
    torch.cuda.synchronize()
    got = got.cpu()
    assert torch.isfinite(got.float()).all()
    rng = np.random.default_rng(wl.seed)
    nrows = wl.B * wl.Hq * wl.qL
    rows = np.unique(np.concatenate([np.arange(16), np.arange(nrows - 16, nrows), rng.integers(0, nrows, 64)]))
    ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=wl.scale, causal=wl.causal,
                               q_offset=wl.q_offset, dtype=wl.dtype, rows=rows, threads=ORACLE_THREADS)
    check_close(f64(got.reshape(-1, wl.D)[torch.from_numpy(rows)]), ref, wl.dtype, f"{wl.name} ({rows.size} rows)")


@pytest.mark.parametrize("qL,kL,dtype", [(128, 4097, FP16), (33, 1025, BF16)])
def test_contiguous_odd_bias_ending_on_a_page_boundary(qL, kL, dtype):
    # a [1, 16, qL, kL] bias whose last byte ends a 4 KiB page: the layout the
    # library used to refuse; it must read nothing past the bias and count the
    # last element (set large on the diagonal key of the last row)
    B, Hq, Hkv, D = 1, 16, 8, 256
    q, k, v = W.random_qkv(5400 + kL, B, Hq, Hkv, qL, kL, D, dtype)
    bias = make_bias(5401 + kL, (B, Hq, qL, kL), dtype, ninf_frac=0.0)
    bias[..., -1, -1] = 6.0
    n = bias.numel()
    pool = torch.empty(n + 8192, dtype=bias.dtype, device="cuda")
    end = (pool.data_ptr() + 2 * n + 4095) // 4096 * 4096   # first page boundary at or past n elements
    off = (end - pool.data_ptr()) // 2 - n
    view = pool[off:off + n].view(B, Hq, qL, kL)
    assert (view.data_ptr() + 2 * n) % 4096 == 0
    view.copy_(bias.cuda())
    note(f"bias ending on a page boundary, qL {qL} kL {kL}")
    out = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), bias=view, causal=True)
    torch.cuda.synchronize()
    scale = float(np.float32(1.0 / 16))
    ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=scale, causal=True,
                               q_offset=kL - qL, dtype=dtype, threads=ORACLE_THREADS)
    check_close(f64(out.cpu()), ref, dtype, f"bias ending on a page boundary, qL {qL} kL {kL}")
