"""Seeded synthetic inputs and the named workloads they are drawn for.

This module is shared by the tests, the benchmark and the smoke check; it
holds no attention arithmetic (neither the kernels' nor the oracle's), only
shapes, seeds, the random draw and byte/FLOP accounting for reports.

Input recipe: one CPU ``torch.Generator`` per workload, seeded with the
workload's seed; Q, K and V are drawn in that order as float32 standard
normals and cast to the workload's dtype with round-to-nearest-even.  The same
host tensors feed the oracle (as uint16 bit patterns) and the GPU (copied to
the device).  i.i.d. N(0, 1) inputs with scale 1/sqrt(D) are the pages' own
synthetic workload (the M3 Ultra test script in ml-explore/mlx PR #3293, "fix:
add head_dim=256 to fused SDPA full attention kernel").
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

FP16 = 0
BF16 = 1
TORCH_DTYPES = {FP16: torch.float16, BF16: torch.bfloat16}
DTYPE_NAMES = {FP16: "f16", BF16: "bf16"}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    qL: int
    kL: int
    D: int
    dtype: int
    causal: bool
    window: int
    q_offset: int
    seed: int
    what: str
    Dv: int = 0  # head dim of v and the output; 0: D

    @property
    def dv(self) -> int:
        return self.Dv or self.D

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _wl(name, B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset, seed, what, Dv=0):
    return Workload(name, B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset, seed, what, Dv)


# The five workloads the library is measured and checked on.  Shapes follow the
# pages: n_q=16 / n_kv=8 at head_dim 256 over a 32768-key prefix (mlx PR #3660,
# Microbenchmarks); H=64 at L=16384 (mlx PR #3293, Benchmark, H=64 table);
# Gemma-4 31B sliding 32/16/256 window 1024 and global 32/4/512 layers, and a
# 4-row verify block over a long KV cache (mlxcel issue #2160, Current Behavior).
WORKLOADS = {
    "tiny_causal": _wl("tiny_causal", 1, 2, 1, 128, 128, 256, FP16, True, 0, 0, 1,
                       "tiny causal self-attention, B1 Hq2 Hkv1 D256 L128 fp16"),
    "chunked_prefill_32k": _wl("chunked_prefill_32k", 1, 16, 8, 1024, 32768, 256, FP16, True, 0,
                               32768 - 1024, 2,
                               "chunked prefill over a 32K KV prefix, B1 Hq16 Hkv8 D256 qL1024 kL32768 fp16 causal"),
    "causal_h64_16k": _wl("causal_h64_16k", 1, 64, 64, 16384, 16384, 256, BF16, True, 0, 0, 3,
                          "large-head causal self-attention, B1 Hq64 Hkv64 D256 L16384 bf16"),
    "sliding_32k": _wl("sliding_32k", 1, 32, 16, 32768, 32768, 256, BF16, True, 1024, 0, 41,
                       "Gemma-4-31B-like sliding layer, B1 Hq32 Hkv16 D256 L32768 bf16 window 1024"),
    "global_d512_32k": _wl("global_d512_32k", 1, 32, 4, 32768, 32768, 512, BF16, True, 0, 0, 42,
                           "Gemma-4-31B-like global layer, B1 Hq32 Hkv4 D512 L32768 bf16 causal"),
    "causal_d128_16k": _wl("causal_d128_16k", 1, 32, 8, 16384, 16384, 128, BF16, True, 0, 0, 6,
                           "head_dim 128 causal self-attention, B1 Hq32 Hkv8 D128 L16384 bf16"),
    "causal_d64_16k": _wl("causal_d64_16k", 1, 32, 8, 16384, 16384, 64, BF16, True, 0, 0, 10,
                          "head_dim 64 causal self-attention, B1 Hq32 Hkv8 D64 L16384 bf16"),
    "causal_d80_16k": _wl("causal_d80_16k", 1, 32, 8, 16384, 16384, 80, BF16, True, 0, 0, 11,
                          "head_dim 80 causal self-attention, B1 Hq32 Hkv8 D80 L16384 bf16"),
    "causal_d192_16k": _wl("causal_d192_16k", 1, 32, 8, 16384, 16384, 192, BF16, True, 0, 0, 8,
                           "head_dim 192 causal self-attention, B1 Hq32 Hkv8 D192 L16384 bf16"),
    "causal_dk192_dv256_16k": _wl("causal_dk192_dv256_16k", 1, 32, 8, 16384, 16384, 192, BF16, True, 0, 0, 9,
                                  "q/k head dim 192 with v head dim 256, causal, B1 Hq32 Hkv8 L16384 bf16",
                                  Dv=256),
    "chunked_prefill_32k_bias": _wl("chunked_prefill_32k_bias", 1, 16, 8, 1024, 32768, 256, FP16, True, 0,
                                    32768 - 1024, 2,
                                    "chunked_prefill_32k plus one additive mask array [1, 1, 1024, 32768] "
                                    "shared by every head, N(0, 1) fp16 (seed 7)"),
    "decode_q4_128k": _wl("decode_q4_128k", 1, 16, 8, 4, 131072, 256, BF16, True, 0, 131072 - 4, 5,
                          "verify block, B1 Hq16 Hkv8 D256 qL4 kL131072 bf16 causal bottom-right"),
    "decode_q1_128k": _wl("decode_q1_128k", 1, 16, 8, 1, 131072, 256, BF16, True, 0, 131072 - 1, 5,
                          "decode, B1 Hq16 Hkv8 D256 qL1 kL131072 bf16 (row 3 of the qL=4 draw)"),
    "decode_q4kv_128k": _wl("decode_q4kv_128k", 1, 16, 8, 4, 131072, 256, BF16, True, 0, 131072 - 4, 5,
                            "the verify block of decode_q4_128k over 4-bit K/V (random code words, "
                            "per-64 scales/biases, seed 12)"),
}

# workloads whose K and V are 4-bit rows: name -> seed of random_q4kv
Q4KV = {"decode_q4kv_128k": 12}


# workloads that also pass an additive mask array: name -> (bias batch dim, bias head dim, seed)
BIAS = {"chunked_prefill_32k_bias": (1, 1, 7)}


def draw_bias(wl: Workload) -> "torch.Tensor | None":
    """The seeded additive mask array of a workload in BIAS (None for the others)."""
    if wl.name not in BIAS:
        return None
    bb, bh, seed = BIAS[wl.name]
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn((bb, bh, wl.qL, wl.kL), generator=g, dtype=torch.float32).to(TORCH_DTYPES[wl.dtype])


def draw_q4kv(wl: Workload):
    """Q (the draw of the 16-bit workload of the same shape) and the seeded 4-bit
    K/V rows (kq, ks, kb, vq, vs, vb) of a workload in Q4KV."""
    q = draw(WORKLOADS["decode_q4_128k"] if wl.name == "decode_q4kv_128k" else wl)[0]
    return (q,) + random_q4kv(Q4KV[wl.name], wl.B, wl.Hkv, wl.kL, wl.D, wl.dtype)


def q4kv_bytes(wl: Workload) -> int:
    """Bytes of Q, the 4-bit K and V rows (codes, scales, biases) and O, each once."""
    q = wl.B * wl.Hq * wl.qL * wl.D * 2
    rows = 2 * wl.B * wl.Hkv * wl.kL
    return 2 * q + rows * (wl.D // 2 + 2 * (wl.D // 64) * 2)


def draw(wl: Workload, device: str = "cpu"):
    """Seeded Q, K, V for a workload, as torch tensors of its dtype on the CPU.

    ``decode_q1_128k`` shares the qL=4 draw (seed 5) and takes its last query row.
    """
    if wl.name == "decode_q1_128k":
        q4, k, v = draw(WORKLOADS["decode_q4_128k"])
        return q4[:, :, 3:4].contiguous(), k, v
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed)
    dt = TORCH_DTYPES[wl.dtype]
    q = torch.randn((wl.B, wl.Hq, wl.qL, wl.D), generator=g, dtype=torch.float32).to(dt)
    k = torch.randn((wl.B, wl.Hkv, wl.kL, wl.D), generator=g, dtype=torch.float32).to(dt)
    v = torch.randn((wl.B, wl.Hkv, wl.kL, wl.dv), generator=g, dtype=torch.float32).to(dt)
    return q, k, v


def random_qkv(seed: int, B: int, Hq: int, Hkv: int, qL: int, kL: int, D: int, dtype: int,
               std: float = 1.0, Dv: int = 0):
    """Seeded Q, K, V of an arbitrary shape, same recipe as ``draw`` (v's head
    dim is Dv when given, else D)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = TORCH_DTYPES[dtype]
    q = (torch.randn((B, Hq, qL, D), generator=g, dtype=torch.float32) * std).to(dt)
    k = (torch.randn((B, Hkv, kL, D), generator=g, dtype=torch.float32) * std).to(dt)
    v = (torch.randn((B, Hkv, kL, Dv or D), generator=g, dtype=torch.float32) * std).to(dt)
    return q, k, v


def ramp_qkv(seed: int, B: int, Hq: int, Hkv: int, qL: int, kL: int, D: int, dtype: int,
             rise: float = 40.0, Dv: int = 0):
    """Seeded Q, K, V whose scores climb along the keys (same draw order as ``draw``).

    Per (batch, KV head) a direction u of N(0, 1) entries.  Query row i of each
    head is c_i u + N(0, 1), with c_i ~ U(-0.5, 1.5) drawn per row; key j is
    (rise * j / kL) * u / sqrt(D) + N(0, 1); values are N(0, 1).  With scale
    1/sqrt(D) the scores of row i then grow by about c_i * rise over the keys,
    so that the rows with c_i > 0 see later keys overtake every earlier maximum
    again and again, by far more than the same-magnitude noise of N(0, 1)
    inputs ever does; rows with c_i < 0 have their maximum among the first keys.
    Holds none of the attention arithmetic (it only shapes the inputs).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = TORCH_DTYPES[dtype]
    u = torch.randn((B, Hkv, 1, D), generator=g, dtype=torch.float32)
    uq = u.repeat_interleave(Hq // Hkv, dim=1)
    c = torch.rand((B, Hq, qL, 1), generator=g, dtype=torch.float32) * 2.0 - 0.5
    q = (c * uq + torch.randn((B, Hq, qL, D), generator=g, dtype=torch.float32)).to(dt)
    r = (rise * torch.arange(kL, dtype=torch.float32) / kL).view(1, 1, kL, 1)
    k = (r * u / math.sqrt(D) + torch.randn((B, Hkv, kL, D), generator=g, dtype=torch.float32)).to(dt)
    v = torch.randn((B, Hkv, kL, Dv or D), generator=g, dtype=torch.float32).to(dt)
    return q, k, v


def random_q4kv(seed: int, B: int, Hkv: int, kL: int, D: int, dtype: int):
    """Seeded 4-bit K and V rows: (kq, ks, kb, vq, vs, vb).

    kq, vq [B, Hkv, kL, D / 8] int32: code words of uniformly random bits (eight
    4-bit codes each).  ks, vs, kb, vb [B, Hkv, kL, D / 64] in the dtype: a
    scale drawn from U(0.3, 0.5) and a bias of -7.5 * scale + N(0, 0.1) per
    group of 64 elements, so that a group spans about [-3, 3], the range of
    N(0, 1) values quantized 64 at a time.  Holds none of the attention or
    dequantization arithmetic.
    """
    if D % 64:
        raise ValueError("4-bit rows need D to be a multiple of 64")
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = TORCH_DTYPES[dtype]
    out = []
    for _ in range(2):
        words = torch.randint(-(1 << 31), 1 << 31, (B, Hkv, kL, D // 8), generator=g, dtype=torch.int64)
        sc = torch.rand((B, Hkv, kL, D // 64), generator=g, dtype=torch.float32) * 0.2 + 0.3
        bi = -7.5 * sc + 0.1 * torch.randn((B, Hkv, kL, D // 64), generator=g, dtype=torch.float32)
        out += [words.to(torch.int32), sc.to(dt), bi.to(dt)]
    return tuple(out)


def shaped_q4kv(seed: int, B: int, Hq: int, Hkv: int, qL: int, kL: int, dtype: int, kind: str):
    """Seeded Q and 4-bit K/V rows (q, kq, ks, kb, vq, vs, vb) of a chosen shape of values.

    kind "narrow": value groups with scale U(0.09, 0.11) and bias U(2.0, 2.3), so
    that every value and every output lies in [2, 4), where a bf16 spacing is
    2^-6; key groups with scale U(0.05, 0.15) and bias -7.5 scale + N(0, 0.1).
    kind "ramp": query row i is c_i + N(0, 1) in every element, c_i ~ U(-0.5, 1.5)
    per row; key groups have scale U(0.05, 0.1) and a bias that grows from 0 to 4
    along the keys (plus N(0, 0.05)), so that the scores of rows with c_i > 0
    climb by tens of natural units over the keys; values as in ``random_q4kv``.
    Code words are uniformly random bits.  Holds none of the attention or
    dequantization arithmetic.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = TORCH_DTYPES[dtype]
    if kind == "ramp":
        c = torch.rand((B, Hq, qL, 1), generator=g, dtype=torch.float32) * 2.0 - 0.5
        q = (c + torch.randn((B, Hq, qL, 256), generator=g, dtype=torch.float32)).to(dt)
    else:
        q = torch.randn((B, Hq, qL, 256), generator=g, dtype=torch.float32).to(dt)
    out = [q]
    for which in ("k", "v"):
        words = torch.randint(-(1 << 31), 1 << 31, (B, Hkv, kL, 32), generator=g, dtype=torch.int64)
        u = torch.rand((B, Hkv, kL, 4), generator=g, dtype=torch.float32)
        n = torch.randn((B, Hkv, kL, 4), generator=g, dtype=torch.float32)
        if which == "k" and kind == "ramp":
            sc = u * 0.05 + 0.05
            bi = 4.0 * (torch.arange(kL, dtype=torch.float32) / kL).view(1, 1, kL, 1) + 0.05 * n
        elif which == "k":
            sc = u * 0.1 + 0.05
            bi = -7.5 * sc + 0.1 * n
        elif kind == "narrow":
            sc = u * 0.02 + 0.09
            bi = 2.0 + 0.3 * torch.rand((B, Hkv, kL, 4), generator=g, dtype=torch.float32)
        else:
            sc = u * 0.2 + 0.3
            bi = -7.5 * sc + 0.1 * n
        out += [words.to(torch.int32), sc.to(dt), bi.to(dt)]
    return tuple(out)


def words(t: torch.Tensor) -> np.ndarray:
    """uint32 views of a CPU int32 tensor of 4-bit code words."""
    return t.contiguous().numpy().view(np.uint32)


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU fp16/bf16 tensor (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def visible_keys(qL: int, kL: int, causal: bool, window: int, q_offset: int) -> np.ndarray:
    """Number of keys each query row may see (for FLOP accounting), int64 [qL]."""
    p = q_offset + np.arange(qL, dtype=np.int64)
    hi = np.minimum(p, kL - 1) if causal else np.full(qL, kL - 1, dtype=np.int64)
    lo = np.maximum(p - window + 1, 0) if window > 0 else np.zeros(qL, dtype=np.int64)
    return np.maximum(hi - lo + 1, 0)


def flops(wl: Workload) -> float:
    """Algorithmic FLOP: 2 * B * Hq * (D + Dv) * (visible query-key pairs per head),
    i.e. 4 * B * Hq * D * pairs when Dv = D."""
    pairs = int(visible_keys(wl.qL, wl.kL, wl.causal, wl.window, wl.q_offset).sum())
    return 2.0 * wl.B * wl.Hq * (wl.D + wl.dv) * pairs


def io_bytes(B, Hq, Hkv, qL, kL, D, elem_bytes=2, Dv=0) -> dict:
    """Bytes of the inputs and the output, each read or written once (v and
    the output have head dim Dv when given, else D)."""
    Dv = Dv or D
    q = B * Hq * qL * D * elem_bytes
    kv = B * Hkv * kL * (D + Dv) * elem_bytes
    out = B * Hq * qL * Dv * elem_bytes
    return {"q": q, "kv": kv, "out": out, "inputs": q + kv, "total": q + kv + out}
