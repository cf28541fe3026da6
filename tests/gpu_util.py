"""Helpers of the GPU tests: run the HIP library, compare against the oracle."""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import flash_attention_head_amd as fa
import oracle
from flash_attention_head_amd import workloads as W

# the stated bar: max abs error against the fp64 oracle, by dtype
TOL = {W.FP16: 5e-3, W.BF16: 1.5e-2}
ORACLE_THREADS = min(16, oracle.default_threads())


def ensure_library():
    if not os.path.exists(fa.library_path()):
        from flash_attention_head_amd import build

        build.build()
    fa.load_library()


def note(msg: str):
    """Name the case on stdout before a GPU step, so a fault can be attributed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, *, causal, window=0, q_offset=None, scale=None):
    """Copy CPU inputs to the GPU, run the library, return the CPU output."""
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = fa.sdpa(qd, kd, vd, scale=scale, causal=causal, window=window, q_offset=q_offset)
    torch.cuda.synchronize()
    return out.cpu()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def rounded(ref: np.ndarray, dtype: int) -> np.ndarray:
    return torch.from_numpy(ref).to(W.TORCH_DTYPES[dtype]).to(torch.float64).numpy()


def check_close(got: np.ndarray, ref: np.ndarray, dtype: int, what: str):
    """Max abs error against the unrounded oracle within the dtype's tolerance."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    worst = float(err.max()) if err.size else 0.0
    # diagnostics: error left after rounding the oracle to the output dtype
    err_r = float(np.abs(got - rounded(ref, dtype)).max()) if err.size else 0.0
    print(f"[parity] {what}: max|gpu-oracle| = {worst:.3e} (vs rounded oracle {err_r:.3e}), "
          f"tol {TOL[dtype]:.1e}", flush=True)
    assert worst <= TOL[dtype], f"{what}: max abs err {worst} > {TOL[dtype]}"
    return worst


def oracle_full(q, k, v, *, scale, causal, window, q_offset, dtype):
    return oracle.sdpa_f64(W.bits(q), W.bits(k), W.bits(v), scale=scale, causal=causal,
                           window=window, q_offset=q_offset, dtype=dtype, threads=ORACLE_THREADS)


def oracle_rows(q, k, v, rows, *, scale, causal, window, q_offset, dtype):
    return oracle.sdpa_rows_f64(W.bits(q), W.bits(k), W.bits(v), rows, scale=scale,
                                causal=causal, window=window, q_offset=q_offset, dtype=dtype,
                                threads=ORACLE_THREADS)


def sample_rows(wl: W.Workload, n_random: int, seed: int, edge: int = 8) -> np.ndarray:
    """Flat row indices: heads {0, mid, last} at the first/last `edge` rows, plus random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in {0, wl.B - 1}:
        for hq in {0, wl.Hq // 2, wl.Hq - 1}:
            base = (b * wl.Hq + hq) * wl.qL
            for i in list(range(min(edge, wl.qL))) + list(range(max(0, wl.qL - edge), wl.qL)):
                rows.add(base + i)
    total = wl.B * wl.Hq * wl.qL
    rows.update(int(x) for x in rng.integers(0, total, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)


def launch_rows(wl: W.Workload, seed: int) -> tuple[np.ndarray, dict]:
    """Rows that give every launched workgroup of the prefill kernel, and every
    key split it runs, at least one checked output row.

    The launch geometry follows the library's documented plan: a workgroup
    holds 128 packed rows (64 at head dim 512) of one (batch, KV head), packed
    row r being query position r // G of query head hkv * G + r % G; key splits,
    when used, are equal runs of a multiple of 1024 keys, their count read back
    from the workspace size (B * Hq * qL * nsplit * (Dv + 2) * 4 bytes).  For
    each (workgroup, split) with at least one visible key a seeded random packed
    row that sees a key of that split is taken.
    """
    rng = np.random.default_rng(seed)
    BM = 64 if wl.D == 512 else 128
    G = wl.Hq // wl.Hkv
    ws = fa.sdpa_workspace_bytes_dv(wl.B, wl.Hq, wl.Hkv, wl.qL, wl.kL, wl.D, wl.dv)
    per = wl.B * wl.Hq * wl.qL * (wl.dv + 2) * 4
    nsplit = max(1, ws // per)
    assert ws in (0, nsplit * per), (ws, per)
    split_len = -(-(-(-wl.kL // nsplit)) // 1024) * 1024 if nsplit > 1 else wl.kL
    assert -(-wl.kL // split_len) == nsplit
    npacked = G * wl.qL
    mblocks = -(-npacked // BM)
    r = np.arange(npacked, dtype=np.int64)
    pos = wl.q_offset + r // G
    hi = np.minimum(pos, wl.kL - 1) if wl.causal else np.full(npacked, wl.kL - 1)
    lo = np.maximum(pos - wl.window + 1, 0) if wl.window else np.zeros(npacked, dtype=np.int64)
    rows, pairs = [], 0
    for s in range(nsplit):
        s0, s1 = s * split_len, min(wl.kL, (s + 1) * split_len) - 1
        sees = (lo <= s1) & (hi >= s0)
        for mb in range(mblocks):
            cand = np.nonzero(sees[mb * BM:(mb + 1) * BM])[0]
            if cand.size == 0:
                continue
            pairs += 1
            pr = mb * BM + int(rng.choice(cand))
            for b in range(wl.B):
                for hkv in range(wl.Hkv):
                    hq = hkv * G + pr % G
                    rows.append((b * wl.Hq + hq) * wl.qL + pr // G)
    geo = {"block_rows": BM, "mblocks": mblocks, "nsplit": nsplit, "split_len": split_len,
           "workgroups": wl.B * wl.Hkv * mblocks * nsplit, "covered": pairs * wl.B * wl.Hkv}
    return np.unique(np.array(rows, dtype=np.int64)), geo


def oracle_dense_rows(q, k, v, rows, *, scale, causal, window, q_offset, dtype):
    return oracle.sdpa_dense_rows_f64(W.bits(q), W.bits(k), W.bits(v), rows, scale=scale, causal=causal,
                                      window=window, q_offset=q_offset, dtype=dtype)
