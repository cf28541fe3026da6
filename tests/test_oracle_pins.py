"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties the oracle to something it does not share code with: a library
routine (torch's float64 attention, numpy/torch dtype widening, scipy's
softmax), a closed form, or an invariant the definition of attention implies.
``test_oracle_mutants.py`` checks that these pins catch planted mistakes.
"""

import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from flash_attention_head_amd import workloads as W

FP16, BF16 = oracle.FP16, oracle.BF16


def _np_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    t = torch.from_numpy(np.asarray(a, dtype=np.float32)).to(W.TORCH_DTYPES[dtype])
    return W.bits(t)


def _widened(bits: np.ndarray, dtype: int) -> np.ndarray:
    t = torch.from_numpy(bits.view(np.int16)).view(W.TORCH_DTYPES[dtype])
    return t.to(torch.float64).numpy()


def _mask(qL, kL, causal, window, q_offset):
    p = q_offset + np.arange(qL)[:, None]
    j = np.arange(kL)[None, :]
    m = np.ones((qL, kL), dtype=bool)
    if causal:
        m &= j <= p
    if window > 0:
        m &= (p - j) < window
    return m


# ---------------------------------------------------------------- widening --
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_widening_matches_library_for_every_bit_pattern(oracle_lib, dtype):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(allbits, dtype)
    ref = _widened(allbits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------- library routine, brute --
def _torch_ref(q, k, v, scale, causal, window, q_offset, dtype):
    qd = torch.from_numpy(_widened(q, dtype))
    kd = torch.from_numpy(_widened(k, dtype))
    vd = torch.from_numpy(_widened(v, dtype))
    mask = torch.from_numpy(_mask(q.shape[2], k.shape[2], causal, window, q_offset))
    return F.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=float(np.float32(scale)),
                                          enable_gqa=True).numpy()


def _cases():
    heads = [(1, 1), (2, 1), (4, 2)]
    out = []
    seed = 100
    for (Hq, Hkv), qL, kL in itertools.product(heads, [1, 3, 9], [1, 4, 9]):
        for causal, window in [(False, 0), (True, 0), (True, 1), (True, 3)]:
            if causal and qL > kL:
                continue
            offs = [0, kL - qL] if causal else [0]
            for q_offset in sorted(set(offs)):
                seed += 1
                out.append((seed, Hq, Hkv, qL, kL, causal, window, q_offset))
    return out


@pytest.mark.parametrize("case", _cases())
def test_matches_torch_float64_sdpa_bruteforce(oracle_lib, case):
    seed, Hq, Hkv, qL, kL, causal, window, q_offset = case
    for B, D, dtype in [(1, 8, FP16), (2, 5, BF16)]:
        q, k, v = (W.bits(t) for t in W.random_qkv(seed, B, Hq, Hkv, qL, kL, D, dtype))
        scale = 0.37
        got = oracle.sdpa_f64(q, k, v, scale=scale, causal=causal, window=window,
                              q_offset=q_offset, dtype=dtype, threads=2)
        ref = _torch_ref(q, k, v, scale, causal, window, q_offset, dtype)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------ closed forms --
def test_two_keys_closed_form(oracle_lib):
    # one query q=1, keys 0 and 1, values 0 and 4: o = 4 e^s / (1 + e^s)
    q = _np_bits(np.array([1.0]).reshape(1, 1, 1, 1), FP16)
    k = _np_bits(np.array([0.0, 1.0]).reshape(1, 1, 2, 1), FP16)
    v = _np_bits(np.array([0.0, 4.0]).reshape(1, 1, 2, 1), FP16)
    s = float(np.float32(math.log(3.0)))  # weights 1/4 and 3/4 up to fp32 rounding of ln 3
    o = oracle.sdpa_f64(q, k, v, scale=s, dtype=FP16)[0, 0, 0, 0]
    assert abs(o - 4.0 / (1.0 + math.exp(-s))) < 1e-15
    assert abs(o - 3.0) < 1e-6


def test_huge_scores_select_the_largest_key(oracle_lib):
    # scores 0, 5000, 10000, 2500: every weight but the largest underflows to 0,
    # so the output is that key's value row exactly (no overflow on the way)
    dtype = BF16
    q = _np_bits(np.array([100.0]).reshape(1, 1, 1, 1), dtype)
    k = _np_bits(np.array([0.0, 50.0, 100.0, 25.0]).reshape(1, 1, 4, 1), dtype)
    v = _np_bits(np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 4, 1), dtype)
    o = oracle.sdpa_f64(q, k, v, scale=1.0, dtype=dtype)
    assert o[0, 0, 0, 0] == 3.0


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_one_hot_values_give_softmax_weights(oracle_lib, dtype):
    # K = V = identity: output d equals the softmax weight of key d
    D = 7
    rng = np.random.default_rng(7)
    qv = rng.normal(size=D)
    q = _np_bits(qv.reshape(1, 1, 1, D), dtype)
    eye = _np_bits(np.eye(D).reshape(1, 1, D, D), dtype)
    scale = 0.9
    o = oracle.sdpa_f64(q, eye, eye, scale=scale, dtype=dtype)[0, 0, 0]
    ref = scipy.special.softmax(float(np.float32(scale)) * _widened(q, dtype).ravel())
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal,window,q_offset,qL,kL", [
    (False, 0, 0, 37, 300),
    (True, 0, 0, 300, 300),
    (True, 0, 263, 37, 300),
    (True, 50, 0, 300, 300),
    (True, 50, 120, 37, 300),
    (True, 1, 5, 37, 300),
])
def test_zero_queries_average_the_visible_values(oracle_lib, causal, window, q_offset, qL, kL):
    # all scores equal => the output is the plain mean of the visible value rows
    D, dtype = 16, BF16
    _, _, v = W.random_qkv(11, 2, 4, 2, qL, kL, D, dtype)
    q = torch.zeros((2, 4, qL, D), dtype=torch.bfloat16)
    o = oracle.sdpa_f64(W.bits(q), W.bits(v), W.bits(v), scale=0.0625, causal=causal,
                        window=window, q_offset=q_offset, dtype=dtype)
    vd = v.to(torch.float64).numpy()
    csum = np.concatenate([np.zeros((2, 2, 1, D)), np.cumsum(vd, axis=2)], axis=2)
    for i in range(qL):
        p = q_offset + i
        hi = min(p, kL - 1) if causal else kL - 1
        lo = max(p - window + 1, 0) if window > 0 else 0
        mean = (csum[:, :, hi + 1] - csum[:, :, lo]) / (hi - lo + 1)  # [B, Hkv, D]
        np.testing.assert_allclose(o[:, :, i], np.repeat(mean, 2, axis=1), rtol=0, atol=1e-13)


# ------------------------------------------------- special cases from NS --
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_first_causal_query_returns_first_value_row(oracle_lib, dtype):
    q, k, v = (W.bits(t) for t in W.random_qkv(3, 1, 4, 2, 20, 20, 32, dtype))
    o = oracle.sdpa_f64(q, k, v, scale=0.2, causal=True, q_offset=0, dtype=dtype)
    v0 = _widened(v, dtype)[:, :, 0]
    assert np.array_equal(o[:, :, 0], np.repeat(v0, 2, axis=1))


@pytest.mark.parametrize("q_offset", [0, 13])
def test_window_of_one_returns_the_diagonal_value_row(oracle_lib, q_offset):
    dtype = BF16
    q, k, v = (W.bits(t) for t in W.random_qkv(4, 1, 2, 2, 19, 32, 16, dtype))
    o = oracle.sdpa_f64(q, k, v, scale=0.25, causal=True, window=1, q_offset=q_offset,
                        dtype=dtype)
    vd = _widened(v, dtype)
    for i in range(19):
        assert np.array_equal(o[:, :, i], vd[:, :, q_offset + i])


def test_equal_value_rows_give_that_row(oracle_lib):
    dtype = FP16
    q, k, _ = W.random_qkv(5, 1, 2, 1, 11, 40, 24, dtype)
    row = torch.randn((1, 1, 1, 24), generator=torch.Generator().manual_seed(9)).to(torch.float16)
    v = row.expand(1, 1, 40, 24).contiguous()
    for causal, window in [(False, 0), (True, 0), (True, 7)]:
        o = oracle.sdpa_f64(W.bits(q), W.bits(k), W.bits(v), scale=0.3, causal=causal,
                            window=window, q_offset=29, dtype=dtype)
        r = row.to(torch.float64).numpy()[0, 0, 0]
        assert np.max(np.abs(o - r)) <= 1e-15 * max(1.0, np.max(np.abs(r))) * 4


def test_single_key_returns_it_exactly(oracle_lib):
    q, k, v = (W.bits(t) for t in W.random_qkv(6, 2, 2, 1, 5, 1, 9, FP16))
    o = oracle.sdpa_f64(q, k, v, scale=1.0, dtype=FP16)
    assert np.array_equal(o, np.repeat(np.repeat(_widened(v, FP16), 2, axis=1), 5, axis=2))


# -------------------------------------------------------------- invariants --
@pytest.mark.parametrize("G", [2, 4])
def test_gqa_equals_repeated_kv_heads(oracle_lib, G):
    Hkv, dtype = 2, BF16
    q, k, v = W.random_qkv(12, 2, Hkv * G, Hkv, 13, 21, 16, dtype)
    kw = dict(scale=0.125, causal=True, window=6, q_offset=8, dtype=dtype)
    a = oracle.sdpa_f64(W.bits(q), W.bits(k), W.bits(v), **kw)
    kr = k.repeat_interleave(G, dim=1)
    vr = v.repeat_interleave(G, dim=1)
    b = oracle.sdpa_f64(W.bits(q), W.bits(kr), W.bits(vr), **kw)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("window", [0, 5])
def test_rows_equal_calls_over_their_trimmed_key_prefix(oracle_lib, window):
    # a masked row equals an unmasked single-row call over exactly its visible keys
    dtype = FP16
    q, k, v = W.random_qkv(13, 1, 2, 1, 8, 30, 16, dtype)
    q_offset = 22
    o = oracle.sdpa_f64(W.bits(q), W.bits(k), W.bits(v), scale=0.25, causal=True, window=window,
                        q_offset=q_offset, dtype=dtype)
    for i in range(8):
        p = q_offset + i
        lo = max(p - window + 1, 0) if window else 0
        ks = k[:, :, lo:p + 1].contiguous()
        vs = v[:, :, lo:p + 1].contiguous()
        r = oracle.sdpa_f64(W.bits(q[:, :, i:i + 1]), W.bits(ks), W.bits(vs), scale=0.25,
                            dtype=dtype)
        assert np.array_equal(o[:, :, i:i + 1], r)


def test_key_permutation_changes_only_rounding(oracle_lib):
    dtype = BF16
    q, k, v = W.random_qkv(14, 1, 2, 2, 6, 50, 16, dtype)
    perm = torch.randperm(50, generator=torch.Generator().manual_seed(1))
    a = oracle.sdpa_f64(W.bits(q), W.bits(k), W.bits(v), scale=0.25, dtype=dtype)
    b = oracle.sdpa_f64(W.bits(q), W.bits(k[:, :, perm]), W.bits(v[:, :, perm]), scale=0.25,
                        dtype=dtype)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    assert not np.array_equal(W.bits(k), W.bits(k[:, :, perm]))


def test_scale_multiplies_scores(oracle_lib):
    # doubling q (exact) and halving scale (exact) leaves every score unchanged
    dtype = FP16
    q, k, v = W.random_qkv(15, 1, 2, 1, 7, 20, 8, dtype)
    a = oracle.sdpa_f64(W.bits(q), W.bits(k), W.bits(v), scale=0.5, causal=True, q_offset=13,
                        dtype=dtype)
    b = oracle.sdpa_f64(W.bits(q * 2), W.bits(k), W.bits(v), scale=0.25, causal=True,
                        q_offset=13, dtype=dtype)
    assert np.array_equal(a, b)


def test_selected_rows_equal_full_call(oracle_lib):
    dtype = BF16
    q, k, v = (W.bits(t) for t in W.random_qkv(16, 2, 4, 2, 9, 33, 16, dtype))
    kw = dict(scale=0.3, causal=True, window=10, q_offset=24, dtype=dtype)
    full = oracle.sdpa_f64(q, k, v, **kw).reshape(-1, 16)
    rows = np.array([0, 5, 17, 35, 71, 70, 36], dtype=np.int64)
    part = oracle.sdpa_rows_f64(q, k, v, rows, **kw)
    assert np.array_equal(part, full[rows])


def test_thread_count_does_not_change_results(oracle_lib):
    q, k, v = (W.bits(t) for t in W.random_qkv(17, 1, 4, 2, 33, 70, 16, FP16))
    kw = dict(scale=0.3, causal=True, window=0, q_offset=37, dtype=FP16)
    a = oracle.sdpa_f64(q, k, v, threads=1, **kw)
    b = oracle.sdpa_f64(q, k, v, threads=7, **kw)
    assert np.array_equal(a, b)


# ------------------------------------------- additive mask array ("bias") --
def _bias_bits(rng, shape, dtype, ninf_frac=0.0):
    """Random N(0, 2) bias rounded to dtype, with a fraction of -inf entries (never
    a whole row), as bit patterns."""
    b = rng.normal(0.0, 2.0, size=shape).astype(np.float32)
    if ninf_frac > 0:
        drop = rng.random(shape) < ninf_frac
        drop[..., 0] = False  # every row keeps at least key 0
        b[drop] = -np.inf
    return _np_bits(b, dtype)


def _torch_ref_bias(q, k, v, bias, scale, causal, window, q_offset, dtype):
    qd = torch.from_numpy(_widened(q, dtype))
    kd = torch.from_numpy(_widened(k, dtype))
    vd = torch.from_numpy(_widened(v, dtype))
    add = torch.from_numpy(_widened(bias, dtype))
    mask = torch.from_numpy(_mask(q.shape[2], k.shape[2], causal, window, q_offset))
    add = torch.where(mask, add, torch.tensor(float("-inf"), dtype=torch.float64))
    return F.scaled_dot_product_attention(qd, kd, vd, attn_mask=add, scale=float(np.float32(scale)),
                                          enable_gqa=True).numpy()


@pytest.mark.parametrize("bshape", ["11", "B1", "1H", "BH"])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_bias_matches_torch_float64_sdpa_with_a_float_mask(oracle_lib, bshape, causal, window):
    rng = np.random.default_rng(7)
    for (Hq, Hkv), qL, kL, dtype, D in [((2, 1), 3, 9, FP16, 8), ((4, 2), 9, 9, BF16, 5), ((1, 1), 1, 4, BF16, 8)]:
        B = 2
        q_offset = kL - qL if causal else 0
        q, k, v = (W.bits(t) for t in W.random_qkv(300 + qL + kL, B, Hq, Hkv, qL, kL, D, dtype))
        shape = (B if bshape[0] == "B" else 1, Hq if bshape[1] == "H" else 1, qL, kL)
        bias = _bias_bits(rng, shape, dtype, ninf_frac=0.2 if not causal else 0.0)
        got = oracle.sdpa_bias_f64(q, k, v, bias, scale=0.37, causal=causal, window=window,
                                   q_offset=q_offset, dtype=dtype, threads=2)
        ref = _torch_ref_bias(q, k, v, bias, 0.37, causal, window, q_offset, dtype)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_zero_bias_is_the_unbiased_call_bitwise(oracle_lib):
    q, k, v = (W.bits(t) for t in W.random_qkv(401, 2, 4, 2, 5, 11, 8, BF16))
    zero = np.zeros((1, 1, 5, 11), dtype=np.uint16)
    a = oracle.sdpa_bias_f64(q, k, v, zero, scale=0.5, causal=True, q_offset=6, dtype=BF16, threads=2)
    b = oracle.sdpa_f64(q, k, v, scale=0.5, causal=True, q_offset=6, dtype=BF16, threads=2)
    assert np.array_equal(a, b)


def test_minus_inf_bias_drops_exactly_those_keys(oracle_lib):
    # a row whose bias is 0 on a key subset and -inf elsewhere equals the
    # unbiased single-row call over that subset of keys
    rng = np.random.default_rng(11)
    qL, kL, D = 4, 13, 8
    q, k, v = (W.bits(t) for t in W.random_qkv(402, 1, 2, 1, qL, kL, D, FP16))
    keep = rng.random((1, 2, qL, kL)) < 0.5
    keep[..., 3] = True
    bias = np.where(keep, np.uint16(0), _np_bits(np.array([-np.inf], dtype=np.float32), FP16)[0])
    got = oracle.sdpa_bias_f64(q, k, v, bias.astype(np.uint16), scale=0.3, dtype=FP16, threads=2)
    for h in range(2):
        for i in range(qL):
            idx = np.nonzero(keep[0, h, i])[0]
            one = oracle.sdpa_f64(q[:, h:h + 1, i:i + 1], k[:, :, idx], v[:, :, idx], scale=0.3, dtype=FP16,
                                  threads=1)
            assert np.array_equal(got[0, h, i], one[0, 0, 0]), (h, i)


def test_a_constant_bias_per_row_changes_only_rounding(oracle_lib):
    q, k, v = (W.bits(t) for t in W.random_qkv(403, 1, 2, 2, 6, 10, 8, BF16))
    row_const = np.repeat(np.linspace(-3.0, 5.0, 6, dtype=np.float32)[:, None], 10, axis=1)
    bias = _np_bits(row_const[None, None], BF16)
    a = oracle.sdpa_bias_f64(q, k, v, bias, scale=0.4, causal=True, q_offset=4, dtype=BF16, threads=2)
    b = oracle.sdpa_f64(q, k, v, scale=0.4, causal=True, q_offset=4, dtype=BF16, threads=2)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_head_broadcast_bias_equals_an_explicit_repeat(oracle_lib):
    rng = np.random.default_rng(12)
    q, k, v = (W.bits(t) for t in W.random_qkv(404, 2, 4, 2, 3, 7, 8, FP16))
    b1 = _bias_bits(rng, (2, 1, 3, 7), FP16)
    a = oracle.sdpa_bias_f64(q, k, v, b1, scale=0.3, dtype=FP16, threads=2)
    b = oracle.sdpa_bias_f64(q, k, v, np.repeat(b1, 4, axis=1), scale=0.3, dtype=FP16, threads=2)
    assert np.array_equal(a, b)


def test_a_row_with_no_finite_biased_score_is_a_zero_row(oracle_lib):
    q, k, v = (W.bits(t) for t in W.random_qkv(405, 1, 1, 1, 2, 5, 8, BF16))
    f = np.zeros((1, 1, 2, 5), dtype=np.float32)
    f[0, 0, 1, :] = -np.inf
    got = oracle.sdpa_bias_f64(q, k, v, _np_bits(f, BF16), scale=0.3, dtype=BF16, threads=1)
    assert np.array_equal(got[0, 0, 1], np.zeros(8)) and np.isfinite(got).all()
    assert np.abs(got[0, 0, 0]).sum() > 0


def test_bias_row_selection_equals_the_full_call(oracle_lib):
    rng = np.random.default_rng(13)
    q, k, v = (W.bits(t) for t in W.random_qkv(406, 2, 4, 2, 5, 9, 8, BF16))
    bias = _bias_bits(rng, (2, 4, 5, 9), BF16)
    full = oracle.sdpa_bias_f64(q, k, v, bias, scale=0.3, causal=True, q_offset=4, dtype=BF16, threads=2)
    rows = np.array([0, 7, 19, 33, 39], dtype=np.int64)
    sel = oracle.sdpa_bias_f64(q, k, v, bias, scale=0.3, causal=True, q_offset=4, dtype=BF16, rows=rows,
                               threads=2)
    assert np.array_equal(sel, full.reshape(-1, 8)[rows])


# ------------------------------------------------------- value head dim Dv --
# v rows longer than the q/k rows (the Q=192/K=192/V=256 heads named in the
# review discussion of ml-explore/mlx PR #3293): scores from D-long dot
# products, output rows the weighted sums of Dv-long value rows.
def _torch_ref_dv(q, k, v, scale, causal, window, q_offset, dtype):
    qd, kd, vd = (torch.from_numpy(_widened(x, dtype)) for x in (q, k, v))
    mask = torch.from_numpy(_mask(q.shape[2], k.shape[2], causal, window, q_offset))
    return F.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=float(np.float32(scale)),
                                          enable_gqa=True).numpy()


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_value_dim_matches_torch_float64_sdpa(oracle_lib, causal, window):
    for (Hq, Hkv), qL, kL, D, Dv, dtype in [((2, 1), 3, 9, 6, 8, FP16), ((4, 2), 9, 9, 5, 11, BF16),
                                             ((1, 1), 1, 4, 8, 3, FP16)]:
        B = 2
        q_offset = kL - qL if causal else 0
        q, k, _ = (W.bits(t) for t in W.random_qkv(500 + Dv, B, Hq, Hkv, qL, kL, D, dtype))
        v = W.bits(W.random_qkv(600 + Dv, B, Hkv, Hkv, 1, kL, Dv, dtype)[2])
        got = oracle.sdpa_dv_f64(q, k, v, scale=0.37, causal=causal, window=window, q_offset=q_offset,
                                 dtype=dtype, threads=2)
        assert got.shape == (B, Hq, qL, Dv)
        ref = _torch_ref_dv(q, k, v, 0.37, causal, window, q_offset, dtype)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_value_columns_equal_equal_dim_calls_bitwise(oracle_lib):
    # output column c depends on value column c alone, through the same
    # weights: the leading D and the trailing D columns of a Dv-wide result are
    # the equal-dim calls over those value columns, bit for bit
    D, Dv = 6, 10
    q, k, _ = (W.bits(t) for t in W.random_qkv(610, 2, 4, 2, 5, 12, D, BF16))
    v = W.bits(W.random_qkv(611, 2, 2, 2, 1, 12, Dv, BF16)[2])
    got = oracle.sdpa_dv_f64(q, k, v, scale=0.45, causal=True, window=4, q_offset=7, dtype=BF16, threads=2)
    lead = oracle.sdpa_f64(q, k, np.ascontiguousarray(v[..., :D]), scale=0.45, causal=True, window=4,
                           q_offset=7, dtype=BF16, threads=2)
    trail = oracle.sdpa_f64(q, k, np.ascontiguousarray(v[..., Dv - D:]), scale=0.45, causal=True, window=4,
                            q_offset=7, dtype=BF16, threads=2)
    assert np.array_equal(got[..., :D], lead)
    assert np.array_equal(got[..., Dv - D:], trail)


def test_value_dim_equal_to_d_is_the_plain_call_bitwise(oracle_lib):
    q, k, v = (W.bits(t) for t in W.random_qkv(612, 1, 4, 1, 6, 9, 8, FP16))
    a = oracle.sdpa_dv_f64(q, k, v, scale=0.3, causal=True, q_offset=3, dtype=FP16, threads=2)
    b = oracle.sdpa_f64(q, k, v, scale=0.3, causal=True, q_offset=3, dtype=FP16, threads=2)
    assert np.array_equal(a, b)


def test_value_dim_row_selection_equals_the_full_call(oracle_lib):
    q, k, _ = (W.bits(t) for t in W.random_qkv(613, 2, 4, 2, 5, 9, 6, BF16))
    v = W.bits(W.random_qkv(614, 2, 2, 2, 1, 9, 9, BF16)[2])
    full = oracle.sdpa_dv_f64(q, k, v, scale=0.3, causal=True, q_offset=4, dtype=BF16, threads=2)
    rows = np.array([0, 7, 19, 33, 39], dtype=np.int64)
    sel = oracle.sdpa_dv_f64(q, k, v, scale=0.3, causal=True, q_offset=4, dtype=BF16, rows=rows, threads=2)
    assert np.array_equal(sel, full.reshape(-1, 9)[rows])


# ------------------------------------------------------------ 4-bit K / V --
# Affine 4-bit rows (the reading of the 4-bit-at-rest prefix KV cache of
# ml-explore/mlx PR #3660, End-to-end section, in the affine group-64 form
# that lablup/mlxcel issue #2160 names): element d of a row is
# scale[d // 64] * code_d + bias[d // 64]; the codes are packed eight to a
# 32-bit word, element 8w + n in bits 4n .. 4n + 3 of word w.  The expected
# values below are worked out by hand from that definition.

def _u16(values, dtype):
    return _np_bits(np.asarray(values, dtype=np.float32), dtype)


def test_dequant4_golden_words(oracle_lib):
    # one group of 64: scale 0.5, bias -1, so code c gives c / 2 - 1
    words = np.array([[0x76543210, 0xFEDCBA98, 0x00000000, 0xFFFFFFFF,
                       0x0000000F, 0xF0000000, 0x12345678, 0x89ABCDEF]], dtype=np.uint32)
    got = oracle.dequant4_f64(words, _u16([0.5], BF16), _u16([-1.0], BF16), D=64, dtype=BF16)
    expect = ([-1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 2.5]
              + [3.0, 3.5, 4.0, 4.5, 5.0, 5.5, 6.0, 6.5]
              + [-1.0] * 8
              + [6.5] * 8
              + [6.5] + [-1.0] * 7
              + [-1.0] * 7 + [6.5]
              + [3.0, 2.5, 2.0, 1.5, 1.0, 0.5, 0.0, -0.5]
              + [6.5, 6.0, 5.5, 5.0, 4.5, 4.0, 3.5, 3.0])
    assert got.tolist() == [expect]


def test_dequant4_two_groups_and_two_rows(oracle_lib):
    # D = 128: row 0 has groups (scale 1, bias 0) and (scale 2, bias 3);
    # row 1 has (scale 0.25, bias -2) and (scale 4, bias 0.5)
    words = np.full((2, 16), 0x76543210, dtype=np.uint32)
    scales = _u16([[1.0, 2.0], [0.25, 4.0]], FP16)
    biases = _u16([[0.0, 3.0], [-2.0, 0.5]], FP16)
    got = oracle.dequant4_f64(words, scales, biases, D=128, dtype=FP16)
    r0 = [0, 1, 2, 3, 4, 5, 6, 7] * 8 + [3, 5, 7, 9, 11, 13, 15, 17] * 8
    r1 = [-2.0, -1.75, -1.5, -1.25, -1.0, -0.75, -0.5, -0.25] * 8 + [0.5, 4.5, 8.5, 12.5, 16.5, 20.5, 24.5, 28.5] * 8
    assert got.tolist() == [r0, r1]


def _codes_as_values(words: np.ndarray, D: int) -> np.ndarray:
    """The 4-bit codes of packed rows as integers [..., D] (the packing order only)."""
    shifts = 4 * np.arange(8, dtype=np.uint32)
    c = (words[..., :, None] >> shifts) & 0xF
    return c.reshape(words.shape[:-1] + (D,)).astype(np.float64)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_q4kv_with_unit_groups_is_the_plain_call_on_the_codes_bitwise(oracle_lib, dtype):
    # scale 1 and bias 0: every value is its code, exactly representable, so
    # the quantized call must be the plain (pinned) call on those values, bit
    # for bit
    B, Hq, Hkv, qL, kL, D = 2, 4, 2, 5, 9, 128
    q = W.bits(W.random_qkv(710, B, Hq, Hkv, qL, kL, D, dtype)[0])
    kq, _, _, vq, _, _ = W.random_q4kv(711, B, Hkv, kL, D, dtype)
    ones, zeros = _u16(np.ones((B, Hkv, kL, D // 64)), dtype), _u16(np.zeros((B, Hkv, kL, D // 64)), dtype)
    k = _u16(_codes_as_values(W.words(kq), D), dtype)
    v = _u16(_codes_as_values(W.words(vq), D), dtype)
    for causal, window in [(False, 0), (True, 0), (True, 3)]:
        qo = kL - qL if causal else 0
        got = oracle.sdpa_q4kv_f64(q, W.words(kq), ones, zeros, W.words(vq), ones, zeros, scale=0.05,
                                   causal=causal, window=window, q_offset=qo, dtype=dtype, threads=2)
        ref = oracle.sdpa_f64(q, k, v, scale=0.05, causal=causal, window=window, q_offset=qo, dtype=dtype,
                              threads=2)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 4)])
def test_q4kv_matches_a_dense_softmax_over_the_dequantized_rows(oracle_lib, causal, window):
    # random groups: against a dense numpy formulation over the dequantized
    # values (scores, mask, softmax, weighted sum), GQA and batches included
    for (B, Hq, Hkv, qL, kL, D, dtype) in [(2, 4, 2, 6, 11, 64, BF16), (1, 6, 3, 3, 8, 128, FP16)]:
        q = W.bits(W.random_qkv(720 + D, B, Hq, Hkv, qL, kL, D, dtype)[0])
        kq, ks, kb, vq, vs, vb = W.random_q4kv(721 + D, B, Hkv, kL, D, dtype)
        qo = kL - qL if causal else 0
        got = oracle.sdpa_q4kv_f64(q, W.words(kq), W.bits(ks), W.bits(kb), W.words(vq), W.bits(vs), W.bits(vb),
                                   scale=0.11, causal=causal, window=window, q_offset=qo, dtype=dtype,
                                   threads=2)
        kd = oracle.dequant4_f64(W.words(kq), W.bits(ks), W.bits(kb), D=D, dtype=dtype)
        vd = oracle.dequant4_f64(W.words(vq), W.bits(vs), W.bits(vb), D=D, dtype=dtype)
        G = Hq // Hkv
        kd, vd = np.repeat(kd, G, axis=1), np.repeat(vd, G, axis=1)
        s = float(np.float32(0.11)) * np.einsum("bhid,bhjd->bhij", _widened(q, dtype), kd)
        s = np.where(_mask(qL, kL, causal, window, qo)[None, None], s, -np.inf)
        w = np.exp(s - s.max(axis=-1, keepdims=True))
        ref = np.einsum("bhij,bhjd->bhid", w / w.sum(axis=-1, keepdims=True), vd)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_q4kv_row_selection_equals_the_full_call(oracle_lib):
    q = W.bits(W.random_qkv(730, 1, 4, 2, 5, 40, 64, BF16)[0])
    kv = [W.words(t) if t.dtype == torch.int32 else W.bits(t) for t in W.random_q4kv(731, 1, 2, 40, 64, BF16)]
    full = oracle.sdpa_q4kv_f64(q, *kv, scale=0.2, causal=True, q_offset=35, dtype=BF16, threads=2)
    rows = np.array([0, 7, 19], dtype=np.int64)
    sel = oracle.sdpa_q4kv_f64(q, *kv, scale=0.2, causal=True, q_offset=35, dtype=BF16, rows=rows, threads=2)
    assert np.array_equal(sel, full.reshape(-1, 64)[rows])
