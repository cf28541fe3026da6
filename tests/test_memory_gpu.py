"""Device memory: the library allocates nothing, and peak memory is O(L).

The page layout followed is the mlx PR #3660 Microbenchmarks table (inputs,
fused peak; "fused transient ~16 MB regardless of kL"): with caller-owned
buffers the peak is exactly inputs + output + workspace, and the workspace
grows with the number of key chunks, never with qL * kL.
"""

import pytest
import torch

import flash_attention_head_amd as fa
from flash_attention_head_amd import workloads as W
from gpu_util import ensure_library, note

pytestmark = pytest.mark.gpu

MiB = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _alloc(B, Hq, Hkv, qL, kL, D, dtype=torch.float16):
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    q = torch.randn((B, Hq, qL, D), device="cuda", dtype=dtype, generator=g)
    k = torch.randn((B, Hkv, kL, D), device="cuda", dtype=dtype, generator=g)
    v = torch.randn((B, Hkv, kL, D), device="cuda", dtype=dtype, generator=g)
    return q, k, v


def _peak_of_call(q, k, v, **kw):
    """Peak torch-allocated bytes of one sdpa call, inputs included."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    out = fa.sdpa(q, k, v, **kw)
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated(), out


@pytest.mark.timeout(300)
def test_peak_is_inputs_plus_output_plus_workspace_and_linear_in_kL():
    rows = []
    for qL, kL in [(1024, 8192), (1024, 16384), (1024, 32768), (1024, 65536), (1024, 131072),
                   (2048, 65536), (2048, 131072)]:
        note(f"peak memory qL{qL} kL{kL}")
        q, k, v = _alloc(1, 16, 8, qL, kL, 256)
        inputs = sum(t.numel() * t.element_size() for t in (q, k, v))
        ws = fa.sdpa_workspace_bytes(1, 16, 8, qL, kL, 256)
        peak, out = _peak_of_call(q, k, v, causal=True)
        outb = out.numel() * out.element_size()
        rows.append((qL, kL, inputs / MiB, peak / MiB, (peak - inputs) / MiB, ws / MiB))
        # torch's caching allocator rounds blocks up; allow that slack only
        assert peak - inputs - outb - ws <= 4 * MiB, rows[-1]
        # transient (output + workspace) never grows like qL * kL
        assert ws <= 16 * qL * 32 * 258 * 4
        del q, k, v, out
    print("\nqL\tkL\tinputs MiB\tpeak MiB\tpeak-inputs MiB\tworkspace MiB")
    for r in rows:
        print("%d\t%d\t%.0f\t%.0f\t%.1f\t%.1f" % r, flush=True)


@pytest.mark.timeout(300)
def test_peak_of_the_64_head_causal_layer_is_linear_in_L():
    # the 64-query/64-KV-head layer at head dim 256 (the shape of the large-head
    # causal workload) over L = 2K .. 16K: every call fills the chip without a
    # key split, so the peak is inputs + output, 4 x L x 64 x 256 x 2 bytes
    for L in (2048, 4096, 8192, 16384):
        note(f"peak memory 64 heads L{L}")
        q, k, v = _alloc(1, 64, 64, L, L, 256, torch.bfloat16)
        inputs = sum(t.numel() * t.element_size() for t in (q, k, v))
        assert fa.sdpa_workspace_bytes(1, 64, 64, L, L, 256) == 0
        peak, out = _peak_of_call(q, k, v, causal=True)
        outb = out.numel() * out.element_size()
        print(f"64 heads L {L}: inputs {inputs / MiB:.0f} MiB, peak {peak / MiB:.0f} MiB", flush=True)
        assert 0 <= peak - inputs - outb <= 4 * MiB, (L, peak, inputs, outb)
        assert peak <= 4 * L * 64 * 256 * 2 + 4 * MiB
        del q, k, v, out


def test_library_allocates_no_device_memory():
    q, k, v = _alloc(1, 16, 8, 4, 131072, 256, torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(fa.sdpa_workspace_bytes(1, 16, 8, 4, 131072, 256), dtype=torch.uint8,
                     device="cuda")
    note("no-alloc check (warm-up)")
    fa.sdpa(q, k, v, causal=True, out=out, workspace=ws)  # first call loads the code objects
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        fa.sdpa(q, k, v, causal=True, out=out, workspace=ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0
