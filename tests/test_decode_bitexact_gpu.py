"""Verify rows are bit-identical to single-row decode calls over trimmed keys.

A qL-row verify block at the end of a kL-key cache must give, for row r, the
same bytes as a qL=1 call whose keys are a contiguous copy of the first
kL - qL + r + 1 keys, with the query at the last of them: each verify row as
classic decode issues it (lablup/mlxcel issue #2160, Proposed Solution step
2, and the gemma4_12b_sliding_verify_rows_match_decode_byte_for_byte unit
test of its Acceptance Criteria: head_dim 256, 16 query / 8 KV heads,
width 4, windowed).  No oracle is needed: both sides run on the GPU.
"""

import pytest
import torch

import flash_attention_head_amd as fa
from flash_attention_head_amd import workloads as W
from gpu_util import ensure_library, note

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _check_rows(q, k, v, *, window, what):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qL, kL = q.shape[2], k.shape[2]
    note(f"{what}: block of {qL} rows")
    block = fa.sdpa(qd, kd, vd, causal=True, window=window, q_offset=kL - qL)
    torch.cuda.synchronize()
    for r in range(qL):
        n = kL - qL + r + 1
        note(f"{what}: row {r} over {n} keys")
        ks = kd[:, :, :n].contiguous()
        vs = vd[:, :, :n].contiguous()
        one = fa.sdpa(qd[:, :, r:r + 1].contiguous(), ks, vs, causal=True, window=window,
                      q_offset=n - 1)
        torch.cuda.synchronize()
        a = block[:, :, r:r + 1].contiguous().view(torch.int16)
        b = one.view(torch.int16)
        assert torch.equal(a, b), f"{what}: row {r} differs in {(a != b).sum().item()} elements"
        del ks, vs, one


@pytest.mark.timeout(600)
def test_verify_block_of_four_at_128k_keys():
    wl = W.WORKLOADS["decode_q4_128k"]
    q, k, v = W.draw(wl)
    _check_rows(q, k, v, window=0, what="decode_q4_128k")


@pytest.mark.timeout(600)
def test_windowed_verify_block_of_four_at_128k_keys():
    wl = W.WORKLOADS["decode_q4_128k"]
    q, k, v = W.draw(wl)
    _check_rows(q, k, v, window=1024, what="decode_q4_128k window 1024")


@pytest.mark.timeout(600)
def test_verify_block_at_head_dim_512_global_geometry():
    # Gemma-4 31B global layers: 32 query heads over 4 KV heads at head_dim 512
    q, k, v = W.random_qkv(51, 1, 32, 4, 4, 65536, 512, BF16)
    _check_rows(q, k, v, window=0, what="D512 32/4")


@pytest.mark.timeout(600)
def test_verify_block_at_head_dim_128():
    q, k, v = W.random_qkv(54, 1, 32, 8, 4, 20000, 128, BF16)
    _check_rows(q, k, v, window=0, what="D128 32/8")


@pytest.mark.timeout(600)
def test_verify_block_at_head_dim_192():
    q, k, v = W.random_qkv(55, 1, 32, 8, 4, 20000, 192, BF16)
    _check_rows(q, k, v, window=0, what="D192 32/8")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("D", [64, 80])
def test_verify_block_at_small_head_dims(D):
    q, k, v = W.random_qkv(57 + D, 1, 32, 8, 4, 20000, D, FP16)
    _check_rows(q, k, v, window=0, what=f"D{D} 32/8")


@pytest.mark.timeout(600)
def test_verify_block_with_value_head_dim_256():
    # q/k head dim 192, v head dim 256 (sdpa_forward_dv)
    q, k, v = W.random_qkv(56, 1, 16, 16, 4, 20000, 192, FP16, Dv=256)
    _check_rows(q, k, v, window=0, what="D192 Dv256")
    _check_rows(q, k, v, window=700, what="D192 Dv256 window 700")


@pytest.mark.parametrize("qL", [2, 3])
def test_verify_blocks_of_two_and_three(qL):
    q, k, v = W.random_qkv(52 + qL, 1, 16, 8, qL, 20000, 256, BF16)
    _check_rows(q, k, v, window=0, what=f"qL{qL}")


@pytest.mark.parametrize("kL", [1024, 1025, 1026, 1027, 2050, 3071, 4, 4097, 4099])
def test_rows_straddling_a_chunk_boundary(kL):
    # the block's rows end on both sides of a multiple of the 1024-key chunk;
    # at 4097 and 4099 keys the block has 5 chunks and the first rows' own
    # calls 4, which the merge takes with its few-split kernel
    q, k, v = W.random_qkv(60 + kL, 1, 4, 2, 4, kL, 256, FP16)
    _check_rows(q, k, v, window=0, what=f"kL{kL}")
    _check_rows(q, k, v, window=3, what=f"kL{kL} window 3")


def test_bitexact_with_fp16_and_group_of_eight():
    q, k, v = W.random_qkv(70, 2, 16, 2, 4, 5000, 256, FP16)
    _check_rows(q, k, v, window=700, what="fp16 G8 B2")


@pytest.mark.timeout(600)
def test_rows_whose_prefixes_straddle_a_power_of_two_of_chunks():
    # 8 KV heads and 126978 keys: the rows' prefixes hold 126975..126978 keys,
    # on both sides of 124 * 1024 = 126976, where a chunk sized from the key
    # count to fill 256 workgroups would step from 2048 to 4096 keys
    q, k, v = W.random_qkv(73, 1, 16, 8, 4, 126978, 256, BF16)
    _check_rows(q, k, v, window=0, what="126978 keys")


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_verify_block_spanning_two_row_waves_at_group_of_sixteen(dtype):
    # G = 16 at head dim 256: a 4-row verify block is 64 packed rows, held by
    # two waves, while each single-row call's 16 rows sit in one wave
    q, k, v = W.random_qkv(74, 1, 32, 2, 4, 9000, 256, dtype)
    _check_rows(q, k, v, window=0, what=f"G16 dtype {dtype}")
    _check_rows(q, k, v, window=2000, what=f"G16 window dtype {dtype}")
