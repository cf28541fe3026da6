"""GPU output of the HIP library against the fp64 oracle, element by element.

Small shapes run every row through the oracle; they span several K/V tiles,
several row blocks and ragged tails of both.  The named full-size workloads
run in the launch configuration the benchmark times and are compared on
sampled rows (the oracle computes them one by one), plus closed forms that
hold at any size.
"""

import numpy as np
import pytest
import torch

from flash_attention_head_amd import workloads as W
import flash_attention_head_amd as fa
from gpu_util import (TOL, check_close, ensure_library, f64, launch_rows, note, oracle_dense_rows, oracle_full,
                      oracle_rows, run_gpu, sample_rows)

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


# (B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset)
SMALL = [
    (2, 4, 2, 333, 333, 256, FP16, True, 0, 0),        # ragged tiles and row blocks
    (1, 4, 2, 100, 1000, 256, BF16, True, 0, 900),     # bottom-right chunk over a prefix
    (1, 4, 2, 100, 1000, 256, BF16, True, 77, 900),    # sliding window over a prefix
    (1, 2, 2, 257, 190, 256, FP16, False, 0, 0),       # no mask, qL > kL
    (1, 8, 1, 65, 700, 256, BF16, True, 33, 635),      # G = 8
    (1, 2, 1, 5, 5, 256, FP16, True, 0, 0),            # smallest prefill, one partial tile
    (1, 2, 1, 300, 9000, 256, FP16, True, 0, 8700),    # key split + combine, ragged last split
    (1, 4, 2, 200, 9000, 256, BF16, True, 500, 8800),  # key split with a window
    (1, 4, 1, 150, 150, 512, BF16, True, 0, 0),        # head_dim 512
    (2, 2, 2, 70, 200, 512, FP16, False, 0, 0),
    (1, 4, 2, 96, 400, 512, BF16, True, 40, 304),
    (1, 2, 1, 130, 8300, 512, FP16, True, 0, 8170),    # head_dim 512 with key split
    (1, 4, 2, 1, 2500, 256, BF16, True, 0, 2499),      # decode, three 1024-key chunks
    (1, 4, 2, 4, 2500, 256, FP16, True, 0, 2496),      # verify block
    (1, 4, 2, 3, 2500, 256, BF16, True, 100, 2497),    # verify block with a window
    (1, 8, 2, 4, 1500, 512, BF16, True, 0, 1496),      # verify block at head_dim 512
    (2, 2, 1, 2, 700, 256, FP16, False, 0, 0),         # unmasked decode
    (2, 4, 2, 333, 333, 128, FP16, True, 0, 0),        # head_dim 128: ragged tiles and row blocks
    (1, 4, 2, 100, 1000, 128, BF16, True, 77, 900),    # head_dim 128, window over a prefix
    (1, 2, 1, 300, 9000, 128, FP16, True, 0, 8700),    # head_dim 128 with key split
    (1, 4, 2, 4, 2500, 128, BF16, True, 0, 2496),      # head_dim 128 verify block
    (1, 2, 2, 65, 190, 128, BF16, False, 0, 0),        # head_dim 128, no mask
    (2, 4, 2, 333, 333, 192, BF16, True, 0, 0),        # head_dim 192: ragged tiles and row blocks
    (1, 4, 2, 100, 1000, 192, FP16, True, 77, 900),    # head_dim 192, window over a prefix
    (1, 2, 1, 300, 9000, 192, BF16, True, 0, 8700),    # head_dim 192 with key split
    (1, 4, 2, 4, 2500, 192, FP16, True, 0, 2496),      # head_dim 192 verify block
    (1, 2, 2, 65, 190, 192, FP16, False, 0, 0),        # head_dim 192, no mask
    (2, 4, 2, 333, 333, 64, FP16, True, 0, 0),         # head_dim 64: ragged tiles and row blocks
    (1, 4, 2, 100, 1000, 64, BF16, True, 77, 900),     # head_dim 64, window over a prefix
    (1, 2, 1, 300, 9000, 64, FP16, True, 0, 8700),     # head_dim 64 with key split
    (1, 4, 2, 4, 2500, 64, BF16, True, 0, 2496),       # head_dim 64 verify block
    (2, 4, 2, 333, 333, 80, BF16, True, 0, 0),         # head_dim 80: ragged tiles and row blocks
    (1, 4, 2, 100, 1000, 80, FP16, True, 77, 900),     # head_dim 80, window over a prefix
    (1, 2, 1, 300, 9000, 80, BF16, True, 0, 8700),     # head_dim 80 with key split
    (1, 4, 2, 4, 2500, 80, FP16, True, 0, 2496),       # head_dim 80 verify block
    (1, 2, 2, 65, 190, 80, FP16, False, 0, 0),         # head_dim 80, no mask
]


@pytest.mark.parametrize("D", [256, 192])
@pytest.mark.parametrize("ntile", list(range(1, 14)))
def test_every_tile_count_of_the_step_loop(D, ntile):
    # head dims 192 and 256 run their 64-key tiles in steps of six (K buffer
    # t mod 2, V buffer t mod 3): 1..13 tiles end the loop after every step
    # position and start every V buffer phase; the last tile is ragged
    kL = 64 * ntile - 13 if ntile > 1 else 40
    q, k, v = W.random_qkv(3000 + 20 * ntile + D, 1, 4, 2, 70, kL, D, BF16 if ntile % 2 else FP16)
    dtype = BF16 if ntile % 2 else FP16
    scale = float(np.float32(1.0 / np.sqrt(D)))
    for causal, window in [(False, 0), (True, 100)]:
        if causal and kL < 70:
            continue  # a causal block needs as many keys as rows
        qo = kL - 70 if causal else 0
        note(f"step loop D{D} tiles {ntile} kL {kL} causal {causal}")
        got = f64(run_gpu(q, k, v, causal=causal, window=window, q_offset=qo))
        ref = oracle_full(q, k, v, scale=scale, causal=causal, window=window, q_offset=qo, dtype=dtype)
        check_close(got, ref, dtype, f"step loop D{D} tiles {ntile} causal {causal}")


# Sliding-window prefill at head dim 256 runs a persistent kernel when the row
# blocks outnumber the workgroups that fill the chip once: S = ceil(256 / (B *
# Hkv)) workgroups per KV head, workgroup w running row blocks w, w + S, ...
# (128 packed rows each) in one pipeline.  These shapes all take it, with
# ragged last blocks, several blocks per workgroup and a query offset.
PERSISTENT = [
    (2, 64, 32, 1000, 1000, 256, BF16, True, 200, 0),     # 4 blocks per workgroup, ragged last block
    (1, 32, 16, 4096, 4096, 256, FP16, True, 1024, 0),    # the sliding layer's heads at L 4096
    (1, 64, 32, 1500, 4000, 256, FP16, True, 333, 2500),  # a chunk over a prefix, 3 blocks per workgroup
    (1, 64, 64, 700, 700, 256, BF16, True, 64, 0),        # window of one tile
    (1, 64, 32, 2100, 2100, 256, BF16, True, 700, 0),     # 32 heads, 8 workgroups each, ragged last block
    (2, 16, 8, 2500, 2600, 256, FP16, True, 900, 100),    # two batches of 8 heads, a query offset
]


def _persistent(B, Hq, Hkv, qL, window, D):
    S = -(-256 // (B * Hkv))
    return window > 0 and D == 256 and S < -(-(Hq // Hkv) * qL // 128)


@pytest.mark.parametrize("case", PERSISTENT, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}q{c[3]}k{c[4]}w{c[8]}" for c in PERSISTENT])
def test_persistent_sliding_window_every_row(case):
    B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset = case
    assert _persistent(B, Hq, Hkv, qL, window, D)
    q, k, v = W.random_qkv(1200 + qL + kL, B, Hq, Hkv, qL, kL, D, dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    note(f"persistent {case}")
    got = f64(run_gpu(q, k, v, causal=causal, window=window, q_offset=q_offset))
    ref = oracle_full(q, k, v, scale=scale, causal=causal, window=window, q_offset=q_offset, dtype=dtype)
    check_close(got, ref, dtype, f"persistent {case}")


# More than 8 KV heads (a multiple of 8) without a key split: the workgroup
# index maps so that each of the 8 XCDs runs whole heads one at a time.
XCD_HEADS = [
    (2, 16, 8, 300, 300, 256, BF16, True, 0, 0),        # 16 heads, 3 ragged row blocks each
    (1, 48, 24, 200, 700, 128, FP16, True, 0, 500),     # 24 heads, head dim 128, a chunk over a prefix
    (1, 16, 16, 150, 150, 512, BF16, False, 0, 0),      # head dim 512, unmasked
    (3, 8, 8, 260, 260, 64, FP16, True, 40, 0),          # 24 heads, head dim 64, window
]


@pytest.mark.parametrize("case", XCD_HEADS, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}q{c[3]}D{c[5]}" for c in XCD_HEADS])
def test_heads_run_whole_per_xcd_every_row(case):
    B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset = case
    assert B * Hkv > 8 and (B * Hkv) % 8 == 0 and fa.sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D) == 0
    q, k, v = W.random_qkv(1400 + qL + D, B, Hq, Hkv, qL, kL, D, dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    note(f"xcd heads {case}")
    got = f64(run_gpu(q, k, v, causal=causal, window=window, q_offset=q_offset))
    ref = oracle_full(q, k, v, scale=scale, causal=causal, window=window, q_offset=q_offset, dtype=dtype)
    check_close(got, ref, dtype, f"xcd heads {case}")


def test_persistent_unit_window_returns_the_diagonal_value_rows_exactly():
    q, k, v = W.random_qkv(1299, 1, 64, 64, 600, 600, 256, BF16)
    assert _persistent(1, 64, 64, 600, 1, 256)
    note("persistent window 1")
    got = run_gpu(q, k, v, causal=True, window=1, q_offset=0)
    assert torch.equal(got.view(torch.int16), v.view(torch.int16))


# Two query heads per KV head and window 1: a row block is 64 positions.
# With the query offset a multiple of 64 it sees exactly one 64-key tile, so
# the last steps of a block cannot load the next block's first two tiles and
# the block end loads them; with offset 1 each block sees two tiles and the
# last two steps load them.  Window 1 returns each position's own value row.
@pytest.mark.parametrize("q_offset", [0, 64, 1])
def test_persistent_one_tile_blocks_return_the_diagonal_value_rows_exactly(q_offset):
    qL = 1200
    kL = qL + q_offset
    q, k, v = W.random_qkv(1301 + q_offset, 1, 64, 32, qL, kL, 256, FP16)
    assert _persistent(1, 64, 32, qL, 1, 256)
    note(f"persistent window 1, G 2, q_offset {q_offset}")
    got = run_gpu(q, k, v, causal=True, window=1, q_offset=q_offset)
    want = v[:, :, q_offset:q_offset + qL].repeat_interleave(2, dim=1)
    assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}q{c[3]}k{c[4]}D{c[5]}"
                                             f"{'bf16' if c[6] else 'f16'}c{int(c[7])}w{c[8]}"
                                             for c in SMALL])
def test_small_shapes_every_row(case):
    B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset = case
    q, k, v = W.random_qkv(1000 + qL + kL, B, Hq, Hkv, qL, kL, D, dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    note(f"small {case}")
    got = f64(run_gpu(q, k, v, causal=causal, window=window, q_offset=q_offset))
    ref = oracle_full(q, k, v, scale=scale, causal=causal, window=window, q_offset=q_offset,
                      dtype=dtype)
    check_close(got, ref, dtype, f"small {case}")


def test_tiny_causal_workload_every_row():
    wl = W.WORKLOADS["tiny_causal"]
    q, k, v = W.draw(wl)
    note(wl.name)
    got = f64(run_gpu(q, k, v, causal=wl.causal, window=wl.window, q_offset=wl.q_offset))
    ref = oracle_full(q, k, v, scale=wl.scale, causal=wl.causal, window=wl.window,
                      q_offset=wl.q_offset, dtype=wl.dtype)
    check_close(got, ref, wl.dtype, wl.name)


FULL = [("chunked_prefill_32k", 160), ("causal_h64_16k", 160), ("sliding_32k", 200),
        ("global_d512_32k", 64), ("causal_d64_16k", 96), ("causal_d80_16k", 96), ("causal_d128_16k", 96),
        ("causal_d192_16k", 96), ("causal_dk192_dv256_16k", 64), ("decode_q4_128k", 32),
        ("decode_q1_128k", 16)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_random", FULL, ids=[f[0] for f in FULL])
def test_full_size_workloads_on_sampled_rows(name, n_random):
    # edge and random rows against the C oracle; for the prefill calls also one
    # row of every launched workgroup and of every key split it runs, against
    # the dense (matmul + softmax + matmul) oracle
    wl = W.WORKLOADS[name]
    q, k, v = W.draw(wl)
    note(f"{name} full size")
    got = run_gpu(q, k, v, causal=wl.causal, window=wl.window, q_offset=wl.q_offset)
    assert torch.isfinite(got.float()).all()
    flat = got.reshape(-1, wl.dv)
    rows = sample_rows(wl, n_random, seed=wl.seed)
    ref = oracle_rows(q, k, v, rows, scale=wl.scale, causal=wl.causal, window=wl.window,
                      q_offset=wl.q_offset, dtype=wl.dtype) if wl.dv == wl.D else \
        oracle_dense_rows(q, k, v, rows, scale=wl.scale, causal=wl.causal, window=wl.window,
                          q_offset=wl.q_offset, dtype=wl.dtype)
    check_close(f64(flat[torch.from_numpy(rows)]), ref, wl.dtype, f"{name} ({rows.size} rows)")
    if wl.qL > 4:
        wrows, geo = launch_rows(wl, seed=wl.seed + 1)
        assert geo["covered"] == geo["workgroups"] or wl.window, geo
        ref = oracle_dense_rows(q, k, v, wrows, scale=wl.scale, causal=wl.causal, window=wl.window,
                                q_offset=wl.q_offset, dtype=wl.dtype)
        check_close(f64(flat[torch.from_numpy(wrows)]), ref, wl.dtype,
                    f"{name}: {wrows.size} rows covering {geo['covered']} of {geo['workgroups']} "
                    f"(workgroup, split) pairs")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["decode_q4_128k", "decode_q1_128k"])
def test_benchmarked_decode_call_every_row(name):
    # the call the benchmark times: sdpa_forward_kv_view over a full cache of
    # kL = 131072 rows per head, whose plan is 32 chunks of 4096 keys merged by
    # the many-split combine (two chunks per wave); every row against the oracle
    wl = W.WORKLOADS[name]
    q, k, v = W.draw(wl)
    need = fa.sdpa_workspace_bytes_kv_view(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.kL, wl.D)
    assert need == wl.B * wl.Hq * wl.qL * 32 * (wl.D + 2) * 4, need  # 32 splits of 4096 keys
    note(f"{name} through sdpa_forward_kv_view, capacity {wl.kL}")
    out = fa.sdpa_kv_cache(q.cuda(), k.cuda(), v.cuda(), wl.kL, scale=wl.scale, causal=wl.causal,
                           window=wl.window, q_offset=wl.q_offset)
    torch.cuda.synchronize()
    got = f64(out.cpu())
    ref = oracle_full(q, k, v, scale=wl.scale, causal=wl.causal, window=wl.window, q_offset=wl.q_offset,
                      dtype=wl.dtype)
    check_close(got, ref, wl.dtype, f"{name} kv view (all {got.size // wl.D} rows)")


# the fused-vs-unfused validation grid of ml-explore/mlx PR #3660 (Validation):
# 16 query / 8 KV heads at head dim 256, fp16 and bf16, qL in {1024, 2048}, kL
# in {64K, 128K}; the page names no mask, so each shape runs both unmasked and
# causal bottom-right aligned (a prefill chunk over the prefix)
GRID = [(qL, kL, dt) for dt in (FP16, BF16) for qL in (1024, 2048) for kL in (65536, 131072)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", [FP16, BF16], ids=["f16", "bf16"])
def test_validation_grid_of_the_pages(dtype):
    q_all, k_all, v_all = W.random_qkv(3660 + dtype, 1, 16, 8, 2048, 131072, 256, dtype)
    scale = float(np.float32(1 / 16))
    for qL, kL, _ in [g for g in GRID if g[2] == dtype]:
        q = q_all[:, :, :qL].contiguous()
        k = k_all[:, :, :kL].contiguous()
        v = v_all[:, :, :kL].contiguous()
        rows = sample_rows(W.WORKLOADS["chunked_prefill_32k"].with_(qL=qL, kL=kL), 96, seed=qL + kL)
        for causal in (False, True):
            qo = kL - qL if causal else 0
            note(f"validation grid qL {qL} kL {kL} dtype {dtype} causal {causal}")
            got = run_gpu(q, k, v, causal=causal, q_offset=qo)
            ref = oracle_dense_rows(q, k, v, rows, scale=scale, causal=causal, window=0, q_offset=qo,
                                    dtype=dtype)
            check_close(f64(got.reshape(-1, 256)[torch.from_numpy(rows)]), ref, dtype,
                        f"grid qL {qL} kL {kL} causal {causal} ({rows.size} rows)")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["chunked_prefill_32k", "sliding_32k", "causal_h64_16k",
                                  "global_d512_32k", "decode_q4_128k"])
def test_zero_queries_average_visible_values_at_full_size(name):
    # with Q = 0 every visible key has weight 1/n: each row is the mean of its
    # visible value rows, computed here with fp64 prefix sums.  Checks every
    # row's mask boundaries and the head mapping at full size.
    wl = W.WORKLOADS[name]
    _, k, v = W.draw(wl)
    q = torch.zeros((wl.B, wl.Hq, wl.qL, wl.D), dtype=W.TORCH_DTYPES[wl.dtype])
    note(f"{name} zero queries")
    got = run_gpu(q, k, v, causal=wl.causal, window=wl.window, q_offset=wl.q_offset)
    G = wl.Hq // wl.Hkv
    p = wl.q_offset + np.arange(wl.qL)
    hi = np.minimum(p, wl.kL - 1) if wl.causal else np.full(wl.qL, wl.kL - 1)
    lo = np.maximum(p - wl.window + 1, 0) if wl.window else np.zeros(wl.qL, dtype=np.int64)
    n = (hi - lo + 1).astype(np.float64)[:, None]
    worst = 0.0
    for hk in sorted({0, wl.Hkv // 2, wl.Hkv - 1}):
        csum = np.zeros((wl.kL + 1, wl.D))
        np.cumsum(v[0, hk].to(torch.float64).numpy(), axis=0, out=csum[1:])
        mean = (csum[hi + 1] - csum[lo]) / n
        for g in range(G):
            o = f64(got[0, hk * G + g])
            worst = max(worst, float(np.abs(o - mean).max()))
    print(f"[parity] {name} zero-query mean: max err {worst:.3e}", flush=True)
    assert worst <= TOL[wl.dtype]


@pytest.mark.parametrize("D,dtype", [(256, FP16), (256, BF16), (512, BF16), (192, FP16), (80, BF16),
                                     (64, FP16)])
def test_first_causal_row_and_unit_window_are_exact(D, dtype):
    # causal row 0 at q_offset 0 sees key 0 only; a window of 1 sees key p only:
    # exp2(0) = 1, every other weight is 0, so the output is the value row bitwise
    q, k, v = W.random_qkv(77, 1, 4, 2, 300, 300, D, dtype)
    note(f"exact rows D{D} dtype{dtype}")
    a = run_gpu(q, k, v, causal=True, q_offset=0)
    expect0 = v[:, :, 0].repeat_interleave(2, dim=1)
    assert torch.equal(a[:, :, 0].view(torch.int16), expect0.contiguous().view(torch.int16))
    b = run_gpu(q, k, v, causal=True, window=1, q_offset=0)
    assert torch.equal(b.view(torch.int16), v.repeat_interleave(2, dim=1).view(torch.int16))


@pytest.mark.parametrize("D,qL,kL", [(256, 300, 300), (512, 200, 260), (256, 4, 3000)])
def test_gqa_equals_explicitly_repeated_kv_heads(D, qL, kL):
    G = 4
    q, k, v = W.random_qkv(78, 1, 8, 2, qL, kL, D, BF16)
    note(f"gqa D{D} qL{qL} kL{kL}")
    a = run_gpu(q, k, v, causal=True, q_offset=kL - qL)
    b = run_gpu(q, k.repeat_interleave(G, dim=1).contiguous(),
                v.repeat_interleave(G, dim=1).contiguous(), causal=True, q_offset=kL - qL)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_runs_are_bitwise_deterministic():
    wl = W.WORKLOADS["tiny_causal"].with_(qL=700, kL=5000, q_offset=4300, Hq=8, Hkv=2)
    q, k, v = W.random_qkv(79, 1, 8, 2, 700, 5000, 256, FP16)
    note("determinism")
    a = run_gpu(q, k, v, causal=True, q_offset=wl.q_offset)
    b = run_gpu(q, k, v, causal=True, q_offset=wl.q_offset)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("L", [16384, 32768])
def test_unmasked_h8_long_sequences_are_finite(L):
    # the shape of the M3 Ultra test script in mlx PR #3293: B=1, H=8, D=256,
    # normal inputs, scale 1/sqrt(D), no mask; output shape and finiteness
    q, k, v = W.random_qkv(80 + L, 1, 8, 8, L, L, 256, BF16)
    note(f"unmasked H8 L{L}")
    out = run_gpu(q, k, v, causal=False)
    assert out.shape == (1, 8, L, 256)
    assert torch.isfinite(out.float()).all()
    rows = np.array([0, 1, L - 1, 3 * L + 5, 8 * L - 1], dtype=np.int64)
    ref = oracle_rows(q, k, v, rows, scale=1 / 16, causal=False, window=0, q_offset=0, dtype=BF16)
    check_close(f64(out.reshape(-1, 256)[torch.from_numpy(rows)]), ref, BF16, f"unmasked L{L}")
