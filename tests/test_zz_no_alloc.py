"""sdpa_forward_noalloc against sdpa_forward, through the C ABI.

The entry point for callers that cannot allocate runs sdpa_forward's kernels
with the key-split partials in the library's own per-GPU scratch array, so
its output must be sdpa_forward's byte for byte (and so within the oracle's
tolerance).  Two calls in a row, the second smaller, check that a call does
not depend on what the previous one left in the shared array; a call with no
key split needs no scratch at all.
"""

import ctypes

import numpy as np
import pytest
import torch

import flash_attention_head_amd as fa
from flash_attention_head_amd import workloads as W
from gpu_util import check_close, ensure_library, f64, note, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu

FP16, BF16 = W.FP16, W.BF16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _both(q, k, v, *, causal, window, q_offset):
    """(sdpa_forward output, sdpa_forward_noalloc output), both through the C ABI."""
    B, Hq, qL, D = q.shape
    Hkv, kL = k.shape[1], k.shape[2]
    dtype = fa.SDPA_FP16 if q.dtype == torch.float16 else fa.SDPA_BF16
    scale = float(np.float32(1 / np.sqrt(D)))
    stream = torch.cuda.current_stream().cuda_stream
    need = fa.sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    a = torch.empty_like(q)
    rc = fa.sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), B, Hq, Hkv, qL, kL, D, scale,
                         int(causal), window, q_offset, dtype, ws.data_ptr() if need else None, need, stream)
    assert rc == fa.SDPA_OK, fa.sdpa_last_error()
    b = torch.full_like(q, float("nan"))
    rc = fa.sdpa_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), b.data_ptr(), B, Hq, Hkv, qL, kL, D,
                                 scale, int(causal), window, q_offset, dtype, stream)
    assert rc == fa.SDPA_OK, fa.sdpa_last_error()
    torch.cuda.synchronize()
    return a.cpu(), b.cpu(), need


# (B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset): each pair runs
# the larger call first, then a smaller one over the same scratch
PAIRS = [
    ((1, 16, 8, 1024, 32768, 256, FP16, True, 0, 31744),     # chunked prefill: 2 key splits, 32 MiB
     (1, 4, 2, 4, 2500, 256, BF16, True, 0, 2496)),         # verify block: 3 chunks
    ((1, 8, 2, 4, 60000, 512, BF16, True, 1000, 59996),      # head dim 512 verify, windowed
     (1, 2, 1, 300, 9000, 512, FP16, True, 0, 8700)),       # head dim 512 prefill with 2 splits
    ((2, 4, 2, 1, 20000, 128, FP16, False, 0, 0),            # unmasked decode, two batches
     (1, 4, 2, 333, 333, 128, BF16, True, 0, 0)),           # no key split: no scratch used
]


@pytest.mark.parametrize("first,second", PAIRS, ids=["prefill-then-verify", "d512", "d128"])
def test_noalloc_calls_equal_sdpa_forward_bytes(first, second):
    for n, case in enumerate((first, second)):
        B, Hq, Hkv, qL, kL, D, dtype, causal, window, q_offset = case
        q, k, v = W.random_qkv(7700 + qL + kL + D, B, Hq, Hkv, qL, kL, D, dtype)
        note(f"noalloc call {n + 1}: {case}")
        a, b, need = _both(q.cuda(), k.cuda(), v.cuda(), causal=causal, window=window, q_offset=q_offset)
        assert need <= fa.NOALLOC_SCRATCH_BYTES
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), case
        wl = W.WORKLOADS["tiny_causal"].with_(B=B, Hq=Hq, Hkv=Hkv, qL=qL, kL=kL, D=D, dtype=dtype)
        rows = sample_rows(wl, 32, seed=n)
        ref = oracle_rows(q, k, v, rows, scale=float(np.float32(1 / np.sqrt(D))), causal=causal, window=window,
                          q_offset=q_offset if causal else 0, dtype=dtype)
        check_close(f64(b.reshape(-1, D)[torch.from_numpy(rows)]), ref, dtype, f"noalloc {case}")
