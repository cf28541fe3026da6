"""Seeded random small shapes against the fp64 oracle, every output row.

Each case draws its batch, head counts (Hq a multiple of Hkv), query and key
lengths, head dim, dtype, mask (causal or not, window, bottom-right or other
valid q_offset) and entry point from one seed, so that combinations the
hand-picked cases do not name (ragged row blocks with several query heads
per KV head, windows wider than the keys, a q_offset short of the end, qL
above kL without a mask, 4-bit K/V) are exercised too.  A second set of
seeds draws the same kinds of shapes for the additive-mask entry (a bias
broadcast or not over batch and heads, with -inf entries, half of them
views of wider rows) and for q/k head
dim 192 with v head dim 256, and a third set lays the keys and values into
a KV cache of random capacity from a random ring start (16-bit at every
head dim, and 4-bit).  The seeds are fixed: the cases are the same on every
run.
"""

import numpy as np
import pytest
import torch

import flash_attention_head_amd as fa
import oracle
from flash_attention_head_amd import workloads as W
from gpu_util import ORACLE_THREADS, check_close, ensure_library, f64, note, oracle_full
from test_bias_gpu import make_bias

pytestmark = pytest.mark.gpu

HEAD_DIMS = [64, 80, 128, 192, 256, 256, 512]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _case(seed):
    r = np.random.default_rng(seed)
    D = int(r.choice(HEAD_DIMS))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 8]))
    B = int(r.integers(1, 3))
    kL = int(r.integers(1, 1500 if D < 512 else 700))
    decode = r.random() < 0.35
    qL = int(r.integers(1, 5)) if decode else int(r.integers(1, 400))
    causal = bool(r.random() < 0.75)
    if causal and qL > kL:
        qL = kL
    window = int(r.integers(1, kL + 60)) if causal and r.random() < 0.4 else 0
    q_offset = 0
    if causal:
        q_offset = kL - qL if r.random() < 0.7 else int(r.integers(0, kL - qL + 1))
    dtype = W.BF16 if r.random() < 0.5 else W.FP16
    q4 = D == 256 and r.random() < 0.5
    return dict(B=B, Hq=Hkv * G, Hkv=Hkv, qL=qL, kL=kL, D=D, causal=causal, window=window,
                q_offset=q_offset, dtype=dtype, q4=q4)


SEEDS = list(range(700, 760)) + list(range(900, 1000))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_against_the_oracle(seed):
    c = _case(seed)
    note(f"random case {seed}: {c}")
    scale = float(np.float32(1.0 / np.sqrt(c["D"])))
    if c["q4"]:
        q = W.random_qkv(seed, c["B"], c["Hq"], c["Hkv"], c["qL"], 1, 256, c["dtype"])[0]
        kv = W.random_q4kv(seed + 1, c["B"], c["Hkv"], c["kL"], 256, c["dtype"])
        got = fa.sdpa_q4kv(q.cuda(), *(t.cuda() for t in kv), causal=c["causal"], window=c["window"],
                           q_offset=c["q_offset"])
        torch.cuda.synchronize()
        # the exact 4-bit oracle: every element dequantized in double
        ref = oracle.sdpa_q4kv_f64(W.bits(q), W.words(kv[0]), W.bits(kv[1]), W.bits(kv[2]), W.words(kv[3]),
                                   W.bits(kv[4]), W.bits(kv[5]), scale=scale, causal=c["causal"],
                                   window=c["window"], q_offset=c["q_offset"], dtype=c["dtype"],
                                   threads=ORACLE_THREADS)
    else:
        q, k, v = W.random_qkv(seed, c["B"], c["Hq"], c["Hkv"], c["qL"], c["kL"], c["D"], c["dtype"])
        got = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), causal=c["causal"], window=c["window"],
                      q_offset=c["q_offset"])
        torch.cuda.synchronize()
        ref = oracle_full(q, k, v, scale=scale, causal=c["causal"], window=c["window"],
                          q_offset=c["q_offset"], dtype=c["dtype"])
    check_close(f64(got.cpu()), ref, c["dtype"], f"random case {seed}")


BIAS_DV_SEEDS = list(range(760, 800)) + list(range(1000, 1040))


def _case_bias_dv(seed):
    c = _case(seed)
    r = np.random.default_rng(seed + 100000)
    c["q4"] = False
    c["entry"] = "dv" if r.random() < 0.3 else "bias"
    if c["entry"] == "dv":
        c["D"] = 192
    c["bias_b"], c["bias_h"] = bool(r.random() < 0.5), bool(r.random() < 0.5)
    # half the biases are views of wider rows (row stride kL + pad, keys still contiguous)
    c["bias_pad"] = int(r.integers(1, 6)) if r.random() < 0.5 else 0
    return c


@pytest.mark.parametrize("seed", BIAS_DV_SEEDS)
def test_random_shape_with_a_bias_or_value_dim_256_against_the_oracle(seed):
    c = _case_bias_dv(seed)
    note(f"random case {seed}: {c}")
    B, Hq, Hkv, qL, kL, D = c["B"], c["Hq"], c["Hkv"], c["qL"], c["kL"], c["D"]
    mask = dict(causal=c["causal"], window=c["window"], q_offset=c["q_offset"])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    if c["entry"] == "bias":
        q, k, v = W.random_qkv(seed, B, Hq, Hkv, qL, kL, D, c["dtype"])
        wide = make_bias(seed + 1, (B if c["bias_b"] else 1, Hq if c["bias_h"] else 1, qL, kL + c["bias_pad"]),
                         c["dtype"])
        bias = wide[..., :kL]
        # sliced on the device, so that the kernel sees the row stride kL + pad
        gbias = wide.cuda()[..., :kL]
        assert c["bias_pad"] == 0 or gbias.stride(2) == kL + c["bias_pad"]
        got = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), bias=gbias, **mask)
        torch.cuda.synchronize()
        ref = oracle.sdpa_bias_f64(W.bits(q), W.bits(k), W.bits(v), W.bits(bias), scale=scale, dtype=c["dtype"],
                                   threads=ORACLE_THREADS, **mask)
    else:
        q, k, v = W.random_qkv(seed, B, Hq, Hkv, qL, kL, 192, c["dtype"], Dv=256)
        got = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), **mask)
        torch.cuda.synchronize()
        assert tuple(got.shape) == (B, Hq, qL, 256)
        ref = oracle.sdpa_dv_f64(W.bits(q), W.bits(k), W.bits(v), scale=scale, dtype=c["dtype"],
                                 threads=ORACLE_THREADS, **mask)
    check_close(f64(got.cpu()), ref, c["dtype"], f"random case {seed}")


CACHE_SEEDS = list(range(800, 840)) + list(range(1040, 1080))


def _lay(t, cap, start):
    """A [B, H, kL, ...] tensor laid into a cache of `cap` rows from row `start`, wrapping."""
    kL = t.shape[2]
    c = torch.zeros(t.shape[:2] + (cap,) + t.shape[3:], dtype=t.dtype)
    c[:, :, (start + torch.arange(kL)) % cap] = t
    return c


@pytest.mark.parametrize("seed", CACHE_SEEDS)
def test_random_shape_over_a_kv_cache_against_the_oracle(seed):
    c = _case(seed)
    r = np.random.default_rng(seed + 200000)
    cap = c["kL"] + int(r.integers(0, 3000))
    start = int(r.integers(0, cap))
    c.update(cap=cap, ring_start=start)
    note(f"random case {seed}: {c}")
    B, Hq, Hkv, qL, kL, D = c["B"], c["Hq"], c["Hkv"], c["qL"], c["kL"], c["D"]
    mask = dict(causal=c["causal"], window=c["window"], q_offset=c["q_offset"])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    if c["q4"]:
        q = W.random_qkv(seed, B, Hq, Hkv, qL, 1, 256, c["dtype"])[0]
        kv = W.random_q4kv(seed + 1, B, Hkv, kL, 256, c["dtype"])
        got = fa.sdpa_q4kv(q.cuda(), *(_lay(t, cap, start).cuda() for t in kv), kv_len=kL, ring_start=start,
                           **mask)
        torch.cuda.synchronize()
        # the exact 4-bit oracle over the live keys in logical order
        ref = oracle.sdpa_q4kv_f64(W.bits(q), W.words(kv[0]), W.bits(kv[1]), W.bits(kv[2]), W.words(kv[3]),
                                   W.bits(kv[4]), W.bits(kv[5]), scale=scale, dtype=c["dtype"],
                                   threads=ORACLE_THREADS, **mask)
    else:
        q, k, v = W.random_qkv(seed, B, Hq, Hkv, qL, kL, D, c["dtype"])
        got = fa.sdpa_kv_cache(q.cuda(), _lay(k, cap, start).cuda(), _lay(v, cap, start).cuda(), kL,
                               ring_start=start, **mask)
        torch.cuda.synchronize()
        ref = oracle_full(q, k, v, scale=scale, dtype=c["dtype"], **mask)
    check_close(f64(got.cpu()), ref, c["dtype"], f"random case {seed}")
