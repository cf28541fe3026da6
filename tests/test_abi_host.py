"""The C ABI library on the host: it loads without a GPU, exports what the
header declares, and rejects bad arguments with a status code and a message
before it touches the GPU (CPU only; no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import flash_attention_head_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa_mi355x.h")
SIZE_MAX = ctypes.c_size_t(-1).value


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        from flash_attention_head_amd import build

        build.build()
    return fa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(sdpa_\w+)\s*\(", text, flags=re.M))


def test_header_declares_the_binding_names():
    assert _declared_functions() == set(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert fa.sdpa_version() >= 100
    assert fa.sdpa_last_error() == ""


def test_only_the_c_abi_is_exported(lib):
    out = os.popen(f"nm -D --defined-only {fa.library_path()}").read()
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert syms == set(fa.EXPORTED_SYMBOLS), syms


# a valid argument set; individual tests break one argument at a time
GOOD = dict(q=0x1000, k=0x100000, v=0x200000, out=0x300000, B=1, Hq=4, Hkv=2, qL=8, kL=64, D=256,
            scale=0.0625, causal=1, window=0, q_offset=56, dtype=fa.SDPA_BF16, workspace=0x400000,
            workspace_bytes=1 << 30, stream=None)
ORDER = ["q", "k", "v", "out", "B", "Hq", "Hkv", "qL", "kL", "D", "scale", "causal", "window",
         "q_offset", "dtype", "workspace", "workspace_bytes", "stream"]


def _call(**kw):
    args = dict(GOOD, **kw)
    return fa.sdpa_forward(*[args[n] for n in ORDER])


BAD = [
    (dict(q=None), fa.SDPA_INVALID_ARG, "non-null"),
    (dict(out=None), fa.SDPA_INVALID_ARG, "non-null"),
    (dict(B=0), fa.SDPA_INVALID_ARG, ">= 1"),
    (dict(kL=-3), fa.SDPA_INVALID_ARG, ">= 1"),
    (dict(Hq=3), fa.SDPA_INVALID_ARG, "multiple"),
    (dict(D=96), fa.SDPA_UNSUPPORTED, "head_dim"),
    (dict(D=160), fa.SDPA_UNSUPPORTED, "head_dim"),
    (dict(dtype=2), fa.SDPA_UNSUPPORTED, "dtype"),
    (dict(scale=float("nan")), fa.SDPA_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), fa.SDPA_INVALID_ARG, "scale"),
    (dict(scale=-1.0), fa.SDPA_INVALID_ARG, "scale"),
    (dict(scale=0.0), fa.SDPA_INVALID_ARG, "scale"),
    (dict(causal=2), fa.SDPA_INVALID_ARG, "causal"),
    (dict(window=-1), fa.SDPA_INVALID_ARG, "window"),
    (dict(causal=0, window=16), fa.SDPA_INVALID_ARG, "requires causal"),
    (dict(q_offset=57), fa.SDPA_INVALID_ARG, "q_offset"),
    (dict(q_offset=-1), fa.SDPA_INVALID_ARG, "q_offset"),
    (dict(qL=65, q_offset=0), fa.SDPA_INVALID_ARG, "q_offset"),
    (dict(out=0x1000 + 64), fa.SDPA_INVALID_ARG, "overlap"),
    (dict(out=0x100000 + 4096), fa.SDPA_INVALID_ARG, "overlap"),
    (dict(qL=2, q_offset=62, workspace=None), fa.SDPA_WORKSPACE_TOO_SMALL, "workspace"),
    (dict(qL=2, q_offset=62, workspace_bytes=16), fa.SDPA_WORKSPACE_TOO_SMALL, "workspace"),
]


@pytest.mark.parametrize("kw,status,words", BAD, ids=[str(b[0]) for b in BAD])
def test_bad_arguments_return_status_and_message(lib, kw, status, words):
    assert _call(**kw) == status
    assert words in fa.sdpa_last_error()


def test_message_is_per_thread(lib):
    import threading

    assert _call(B=0) == fa.SDPA_INVALID_ARG
    seen = []
    t = threading.Thread(target=lambda: seen.append(fa.sdpa_last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert ">= 1" in fa.sdpa_last_error()


def test_workspace_is_zero_without_a_split(lib):
    # self-attention with enough row blocks to fill the chip: no split
    assert fa.sdpa_workspace_bytes(1, 64, 64, 16384, 16384, 256) == 0
    assert fa.sdpa_workspace_bytes(1, 32, 16, 32768, 32768, 256) == 0
    assert fa.sdpa_workspace_bytes(1, 32, 4, 32768, 32768, 512) == 0
    assert fa.sdpa_workspace_bytes(1, 2, 1, 128, 128, 256) == 0


def decode_chunks(ws, B, Hq, qL, D):
    """Key chunks of a decode/verify call, read off its workspace size."""
    per = B * Hq * qL * (D + 2) * 4  # one fp32 (m, l, O[D]) partial per row and chunk
    assert ws % per == 0
    return ws // per


def test_decode_chunks_depend_on_the_shape_not_on_qL(lib):
    # verify rows must see exactly the chunks a single-row call sees
    for (B, Hq, Hkv, kL, D) in [(1, 16, 8, 131072, 256), (1, 32, 4, 32768, 512), (2, 8, 2, 5000, 256),
                                (1, 16, 8, 1000, 256), (4, 64, 8, 65536, 256)]:
        n = {qL: decode_chunks(fa.sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D), B, Hq, qL, D)
             for qL in (1, 2, 3, 4)}
        assert len(set(n.values())) == 1, n
        nv = {qL: decode_chunks(fa.sdpa_workspace_bytes_kv_view(B, Hq, Hkv, qL, kL, 2 * kL, D), B, Hq, qL, D)
              for qL in (1, 2, 3, 4)}
        assert len(set(nv.values())) == 1, nv


def test_plain_decode_chunks_are_1024_keys_whatever_kL(lib):
    # a verify block over kL keys and the single-row calls over each row's
    # trimmed prefix (kL - 3 .. kL keys) must share chunk boundaries: with no
    # cache capacity given the chunk cannot depend on kL at all
    for (B, Hq, Hkv) in [(1, 16, 8), (1, 32, 4), (4, 64, 8)]:
        for kL in (1, 1023, 1024, 1025, 126976, 126977, 131072, 1 << 20):
            n = decode_chunks(fa.sdpa_workspace_bytes(B, Hq, Hkv, 4, kL, 256), B, Hq, 4, 256)
            assert n == -(-kL // 1024), (B, Hkv, kL, n)


def kv_view_chunk(B, Hq, Hkv, kL, cap, D=256):
    n = decode_chunks(fa.sdpa_workspace_bytes_kv_view(B, Hq, Hkv, 4, kL, cap, D), B, Hq, 4, D)
    return next(c for c in (1024 << k for k in range(21)) if -(-kL // c) == n)


def test_cache_decode_chunk_depends_on_the_capacity_not_on_kL(lib):
    # every call over one cache (any live key count) gets the same chunk size
    for (B, Hq, Hkv, cap) in [(1, 16, 8, 131072), (1, 16, 8, 200000), (1, 32, 4, 65536), (2, 8, 2, 1 << 20)]:
        sizes = {kv_view_chunk(B, Hq, Hkv, kL, cap) for kL in (cap, cap - 1, cap - 3, cap // 2 + 5)}
        assert len(sizes) == 1, (B, Hkv, cap, sizes)


def test_cache_decode_chunk_is_the_largest_that_fills_the_chip(lib):
    # chunk = 1024 * 2^k at absolute key positions: the largest for which the
    # (b, kv head) x chunk workgroups of a full cache still make one full
    # round of 256
    for (B, Hq, Hkv, cap) in [(1, 16, 8, 131072), (1, 16, 8, 4096), (1, 8, 8, 1 << 20), (2, 32, 16, 65536)]:
        chunk = kv_view_chunk(B, Hq, Hkv, cap, cap)
        heads, n = B * Hkv, -(-cap // chunk)
        assert chunk == 1024 or heads * n >= 256
        assert heads * -(-cap // (2 * chunk)) < 256
    # the verify workload: 8 KV heads x 32 chunks of 4096 keys = 256 workgroups
    assert kv_view_chunk(1, 16, 8, 131072, 131072) == 4096


def test_kv_view_rejects_bad_views(lib):
    for (kL, cap, ring) in [(10, 9, 0), (10, 10, 10), (10, 10, -1), (10, 20, 20)]:
        rc = lib.sdpa_forward_kv_view(1, 1, 1, 1, 1, 2, 1, 1, kL, cap, ring, 256, ctypes.c_float(0.0625), 1, 0,
                                      kL - 1, 0, None, 0, None)
        assert rc == fa.SDPA_INVALID_ARG, (kL, cap, ring, rc)
        assert "kv_capacity" in fa.sdpa_last_error() or "ring_start" in fa.sdpa_last_error()
    assert fa.sdpa_workspace_bytes_kv_view(1, 2, 1, 1, 10, 9, 256) == ctypes.c_size_t(-1).value


def test_workspace_is_linear_in_key_chunks_not_quadratic(lib):
    for qL in (1, 2, 4):
        prev = None
        for kL in (1000, 1024, 1025, 4096, 65536, 131072, 1 << 20):
            ws = fa.sdpa_workspace_bytes(1, 16, 8, qL, kL, 256)
            assert ws <= 16 * qL * (-(-kL // 1024)) * (256 + 2) * 4
            if prev is not None:
                assert ws >= prev
            prev = ws
    # a chunked prefill over a long prefix splits its keys: bounded by rows * splits * D
    ws = fa.sdpa_workspace_bytes(1, 16, 8, 1024, 32768, 256)
    assert 0 < ws <= 16 * 1024 * 32 * (256 + 2) * 4


def test_workspace_of_rejected_shapes_is_size_max(lib):
    assert fa.sdpa_workspace_bytes(1, 4, 2, 8, 64, 160) == SIZE_MAX
    assert fa.sdpa_workspace_bytes(1, 3, 2, 8, 64, 256) == SIZE_MAX
    assert fa.sdpa_workspace_bytes(0, 4, 2, 8, 64, 256) == SIZE_MAX


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    import importlib

    monkeypatch.setenv("SDPA_MI355X_LIB", str(tmp_path / "missing.so"))
    mod = importlib.reload(fa)
    try:
        with pytest.raises(RuntimeError, match="no fallback"):
            mod.sdpa_version()
    finally:
        monkeypatch.delenv("SDPA_MI355X_LIB")
        importlib.reload(fa)


def test_bias_entry_point_rejects_bad_bias_arguments(lib):
    f = ctypes.c_float(0.0625)
    base = dict(q=0x1000, k=0x100000, v=0x200000, bias=0x400000, sb=0, sh=0, sq=64, out=0x300000)

    def call(**kw):
        a = dict(base, **kw)
        return lib.sdpa_forward_bias(a["q"], a["k"], a["v"], a["bias"], a["sb"], a["sh"], a["sq"], a["out"],
                                     1, 4, 2, 8, 64, 256, f, 1, 0, 56, 0, None, 0, None)

    assert call(bias=None) == fa.SDPA_INVALID_ARG and "bias" in fa.sdpa_last_error()
    assert call(sq=-1) == fa.SDPA_INVALID_ARG and "stride" in fa.sdpa_last_error()
    assert call(sh=1 << 31) == fa.SDPA_UNSUPPORTED and "2^30" in fa.sdpa_last_error()
    assert call(bias=0x300000 - 64) == fa.SDPA_INVALID_ARG and "overlap" in fa.sdpa_last_error()
    # kL odd and a bias (4 rows of 63 keys, 504 bytes) that ends on a 4 KiB page
    # boundary: the kernels read nothing past the bias, so the layout passes every
    # bias check.  The call stops at the next check instead (a verify block needs
    # a workspace and none is given), before anything could be launched.
    rc = lib.sdpa_forward_bias(0x1000, 0x100000, 0x200000, 0x400000 - 504, 0, 0, 63, 0x300000,
                               1, 4, 2, 4, 63, 256, f, 1, 0, 59, 0, None, 0, None)
    assert rc == fa.SDPA_WORKSPACE_TOO_SMALL, (rc, fa.sdpa_last_error())


# sdpa_forward_dv: q/k head dim D, v and out head dim Dv
DV_ORDER = ["q", "k", "v", "out", "B", "Hq", "Hkv", "qL", "kL", "D", "Dv", "scale", "causal", "window",
            "q_offset", "dtype", "workspace", "workspace_bytes", "stream"]


def _call_dv(**kw):
    args = {**GOOD, "D": 192, "Dv": 256, **kw}
    return fa.sdpa_forward_dv(*[args[n] for n in DV_ORDER])


@pytest.mark.parametrize("D,Dv", [(256, 192), (128, 256), (192, 512), (256, 512), (96, 96), (192, 128), (64, 80)])
def test_value_dim_pairs_outside_the_supported_set_are_rejected(lib, D, Dv):
    assert _call_dv(D=D, Dv=Dv) == fa.SDPA_UNSUPPORTED
    assert "head" in fa.sdpa_last_error()
    assert fa.sdpa_workspace_bytes_dv(1, 4, 2, 2, 5000, D, Dv) == SIZE_MAX


def test_value_dim_entry_checks_the_other_arguments_like_sdpa_forward(lib):
    assert _call_dv(B=0) == fa.SDPA_INVALID_ARG and ">= 1" in fa.sdpa_last_error()
    assert _call_dv(q_offset=57) == fa.SDPA_INVALID_ARG and "q_offset" in fa.sdpa_last_error()
    # out is [B, Hq, qL, 256]: 16 KiB here, so from 8 KiB below k it reaches into k
    assert _call_dv(out=0x100000 - 8192) == fa.SDPA_INVALID_ARG and "overlap" in fa.sdpa_last_error()
    # v is [B, Hkv, kL, 256] (64 KiB): out just past its 48 KiB of a D = 192 view still overlaps
    assert _call_dv(out=0x200000 + 49152) == fa.SDPA_INVALID_ARG and "overlap" in fa.sdpa_last_error()
    assert _call_dv(qL=2, q_offset=62, workspace_bytes=16) == fa.SDPA_WORKSPACE_TOO_SMALL


def test_value_dim_workspace_counts_value_columns(lib):
    # decode: one (m, l, O[Dv]) fp32 partial per row and 1024-key chunk
    ws = fa.sdpa_workspace_bytes_dv(1, 16, 8, 4, 5000, 192, 256)
    assert ws == 16 * 4 * 5 * (256 + 2) * 4
    assert fa.sdpa_workspace_bytes_dv(1, 16, 8, 4, 5000, 192, 192) == fa.sdpa_workspace_bytes(1, 16, 8, 4, 5000, 192)
    assert fa.sdpa_workspace_bytes_dv(1, 64, 64, 16384, 16384, 192, 256) == 0


# sdpa_forward_q4kv: decode / verify over 4-bit K and V
Q4_BASE = dict(q=0x1000, kq=0x100000, ks=0x180000, kb=0x190000, vq=0x200000, vs=0x280000, vb=0x290000,
               out=0x300000, B=1, Hq=4, Hkv=2, qL=4, kL=64, cap=64, ring=0, D=256, scale=0.0625, causal=1, window=0,
               q_offset=60, dtype=fa.SDPA_BF16, workspace=0x400000, workspace_bytes=1 << 30, stream=None)
Q4_ORDER = ["q", "kq", "ks", "kb", "vq", "vs", "vb", "out", "B", "Hq", "Hkv", "qL", "kL", "cap", "ring", "D",
            "scale", "causal", "window", "q_offset", "dtype", "workspace", "workspace_bytes", "stream"]


def _call_q4(**kw):
    args = dict(Q4_BASE, **kw)
    return fa.sdpa_forward_q4kv(*[args[n] for n in Q4_ORDER])


def test_q4kv_entry_point_rejects_what_it_does_not_take(lib):
    assert _call_q4(D=128) == fa.SDPA_UNSUPPORTED and "256" in fa.sdpa_last_error()
    for name in ("ks", "kb", "vs", "vb"):
        assert _call_q4(**{name: None}) == fa.SDPA_INVALID_ARG and "non-null" in fa.sdpa_last_error()
    assert _call_q4(kq=None) == fa.SDPA_INVALID_ARG
    assert _call_q4(Hq=3) == fa.SDPA_INVALID_ARG and "multiple" in fa.sdpa_last_error()
    assert _call_q4(q_offset=61) == fa.SDPA_INVALID_ARG and "q_offset" in fa.sdpa_last_error()
    assert _call_q4(workspace_bytes=16) == fa.SDPA_WORKSPACE_TOO_SMALL
    assert _call_q4(cap=63) == fa.SDPA_INVALID_ARG and "kv_capacity" in fa.sdpa_last_error()
    assert _call_q4(ring=64) == fa.SDPA_INVALID_ARG and "ring_start" in fa.sdpa_last_error()
    # a head's code words are addressed by 32-bit byte offsets: 2^25 rows at most
    assert _call_q4(cap=(1 << 25) + 1) == fa.SDPA_UNSUPPORTED and "33554432" in fa.sdpa_last_error()
    # out is [1, 4, 4, 256] fp16/bf16 = 8 KiB: starting 4 KiB before kq it reaches into kq, and
    # starting inside the scales of K it overlaps them
    assert _call_q4(out=0x100000 - 4096) == fa.SDPA_INVALID_ARG and "overlap" in fa.sdpa_last_error()
    assert _call_q4(out=0x180000 + 256) == fa.SDPA_INVALID_ARG and "overlap" in fa.sdpa_last_error()


# sdpa_forward_noalloc: sdpa_forward without workspace arguments
NOALLOC_ORDER = [n for n in ORDER if n not in ("workspace", "workspace_bytes")]


def _call_noalloc(**kw):
    args = dict(GOOD, **kw)
    return fa.sdpa_forward_noalloc(*[args[n] for n in NOALLOC_ORDER])


def test_noalloc_entry_point_checks_arguments_before_any_hip_call(lib):
    # the same checks and codes as sdpa_forward, all before the scratch array
    # is looked up (no call here reaches the GPU)
    assert _call_noalloc(q=None) == fa.SDPA_INVALID_ARG and "non-null" in fa.sdpa_last_error()
    assert _call_noalloc(D=96) == fa.SDPA_UNSUPPORTED
    assert _call_noalloc(Hq=3) == fa.SDPA_INVALID_ARG
    assert _call_noalloc(q_offset=57) == fa.SDPA_INVALID_ARG and "q_offset" in fa.sdpa_last_error()
    assert _call_noalloc(dtype=7) == fa.SDPA_UNSUPPORTED
    assert _call_noalloc(window=5, causal=0) == fa.SDPA_INVALID_ARG
    assert _call_noalloc(out=0x1000) == fa.SDPA_INVALID_ARG and "overlap" in fa.sdpa_last_error()


def test_noalloc_entry_point_rejects_calls_beyond_its_scratch(lib):
    # a verify block of 4 rows over 2^21 keys at 64 query heads needs
    # 64 * 4 * 2048 * 258 * 4 bytes of partials, past the 64 MiB array
    B, Hq, Hkv, qL, kL, D = 1, 64, 8, 4, 1 << 21, 256
    need = fa.sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    rc = fa.sdpa_forward_noalloc(0x1000, 0x10000000, 0x40000000, 0x100000, B, Hq, Hkv, qL, kL, D, 0.0625, 1, 0,
                                 kL - qL, fa.SDPA_BF16, None)
    assert rc == fa.SDPA_WORKSPACE_TOO_SMALL
    assert str(need) in fa.sdpa_last_error() and str(fa.NOALLOC_SCRATCH_BYTES) in fa.sdpa_last_error()


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define SDPA_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == fa.NOALLOC_SCRATCH_BYTES
