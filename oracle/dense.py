"""The unfused matmul + softmax + matmul formulation of attention, in numpy fp64.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it, and it imports nothing from the HIP library's package.

It computes the same function as ``sdpa_oracle.c``, written the way the pages
time the non-fused path: a matrix product of the query rows with the keys, a
softmax over each row of that score matrix, and a matrix product of the
weights with the values (ml-explore/mlx PR #3293, Benchmark, the "unfused"
columns; ml-explore/mlx PR #3660, Microbenchmarks and Validation, where the
fused output agrees with it).  The two matrix products are library routines
(numpy's fp64 matmul); nothing else is blocked, fused or reordered.  The
rows asked for are grouped by (batch, query head) and taken a bounded number
at a time, so that the score matrix of one group stays small; that grouping
changes no arithmetic of any row.

The C oracle walks one row at a time; this one exists because the product
form runs the full-size workloads' sampled rows (thousands of rows over up to
131072 keys) in seconds.  Readings are the C oracle's: exact fp16/bf16
widening, scale widened from the fp32 the caller passes, key j visible from
position p = q_offset + i iff j <= p (causal) and p - j < window (window > 0),
query head hq reading KV head hq // (Hq // Hkv), masked keys excluded.

Pins (``tests/test_oracle_dense_pins.py``): torch's float64 scaled_dot_product_attention
on brute-force shapes, zero queries giving the mean of the visible values,
the first causal row and a unit window returning value rows exactly, and
agreement with the C oracle.
"""

from __future__ import annotations

import numpy as np

FP16 = 0
BF16 = 1

# score-matrix elements held at once for one group of rows (about 64 MB)
_MAX_SCORES = 1 << 23


def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp16/bf16 -> float64 of a uint16 bit-pattern array."""
    bits = np.ascontiguousarray(bits).view(np.uint16)
    if dtype == BF16:
        with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def sdpa_dense_rows_f64(q, k, v, rows, *, scale: float, causal: bool = False, window: int = 0,
                        q_offset: int = 0, dtype: int = FP16) -> np.ndarray:
    """Selected output rows, [len(rows), Dv] float64.

    q [B, Hq, qL, D], k [B, Hkv, kL, D], v [B, Hkv, kL, Dv]: uint16 bit patterns of
    fp16 (dtype=FP16) or bf16 (dtype=BF16) values.  rows: flat indices
    (b * Hq + hq) * qL + i.  scale is rounded to fp32 first, as the GPU library
    receives it.
    """
    q = np.ascontiguousarray(q).view(np.uint16)
    k = np.ascontiguousarray(k).view(np.uint16)
    v = np.ascontiguousarray(v).view(np.uint16)
    B, Hq, qL, D = q.shape
    Bk, Hkv, kL, Dk = k.shape
    if Bk != B or Dk != D or v.shape[:3] != k.shape[:3] or Hq % Hkv:
        raise ValueError("shape mismatch between q, k, v")
    Dv = v.shape[3]
    s32 = float(np.float32(scale))
    rows = np.asarray(rows, dtype=np.int64).ravel()
    out = np.zeros((rows.size, Dv), dtype=np.float64)
    G = Hq // Hkv
    bh = rows // qL
    order = np.argsort(bh, kind="stable")
    keys = np.arange(kL, dtype=np.int64)
    start = 0
    while start < order.size:
        group = bh[order[start]]
        end = start
        while end < order.size and bh[order[end]] == group:
            end += 1
        b, hq = divmod(int(group), Hq)
        hk = hq // G
        kd = widen(k[b, hk], dtype)   # [kL, D]
        vd = widen(v[b, hk], dtype)   # [kL, Dv]
        step = max(1, _MAX_SCORES // kL)
        for c0 in range(start, end, step):
            sel = order[c0:min(end, c0 + step)]
            i = rows[sel] % qL
            qd = widen(q[b, hq, i], dtype)          # [n, D]
            s = (qd @ kd.T) * s32                   # scores [n, kL]
            p = (q_offset + i)[:, None]
            vis = np.ones(s.shape, dtype=bool)
            if causal:
                vis &= keys[None, :] <= p
            if window > 0:
                vis &= (p - keys[None, :]) < window
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
            l = e.sum(axis=1, keepdims=True)
            o = e @ vd
            out[sel] = np.where(l > 0, o / np.where(l > 0, l, 1.0), 0.0)
        start = end
    return out
