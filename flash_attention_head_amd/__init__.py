"""Fused scaled-dot-product attention for AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libsdpa_mi355x.so``
(``include/sdpa_mi355x.h``).  Every step of the computation runs in the HIP
kernels of that library; this package only marshals arguments.  PyTorch is
used for device memory and streams.  There is no fallback: if the library is
missing or cannot be loaded, every call raises.

Raw entry points (same names and arguments as the C functions, pointers as
integers): ``sdpa_forward``, ``sdpa_workspace_bytes``, ``sdpa_forward_kv_view``,
``sdpa_workspace_bytes_kv_view``, ``sdpa_forward_bias``, ``sdpa_forward_dv``,
``sdpa_workspace_bytes_dv``, ``sdpa_forward_q4kv``, ``sdpa_forward_noalloc``, ``sdpa_last_error``,
``sdpa_version``.
Convenience wrappers on torch tensors: ``sdpa`` (contiguous K/V, optionally an
additive mask array, optionally a value head dim other than q's),
``sdpa_kv_cache`` (K/V in a cache, possibly a wrapped ring) and ``sdpa_q4kv``
(decode / verify over 4-bit K/V).
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "SDPA_OK", "SDPA_INVALID_ARG", "SDPA_UNSUPPORTED", "SDPA_WORKSPACE_TOO_SMALL",
    "SDPA_HIP_ERROR", "SDPA_FP16", "SDPA_BF16", "SdpaError", "library_path", "load_library",
    "sdpa_forward", "sdpa_workspace_bytes", "sdpa_forward_kv_view", "sdpa_workspace_bytes_kv_view",
    "sdpa_forward_bias", "sdpa_forward_dv", "sdpa_workspace_bytes_dv", "sdpa_forward_q4kv",
    "sdpa_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "sdpa_last_error", "sdpa_version", "sdpa",
    "sdpa_kv_cache", "sdpa_q4kv", "EXPORTED_SYMBOLS",
]

SDPA_OK = 0
SDPA_INVALID_ARG = 1
SDPA_UNSUPPORTED = 2
SDPA_WORKSPACE_TOO_SMALL = 3
SDPA_HIP_ERROR = 4
SDPA_FP16 = 0
SDPA_BF16 = 1

EXPORTED_SYMBOLS = ("sdpa_forward", "sdpa_workspace_bytes", "sdpa_forward_kv_view",
                    "sdpa_workspace_bytes_kv_view", "sdpa_forward_bias", "sdpa_forward_dv",
                    "sdpa_workspace_bytes_dv", "sdpa_forward_q4kv", "sdpa_forward_noalloc", "sdpa_last_error",
                    "sdpa_version")

# SDPA_NOALLOC_SCRATCH_BYTES of the header: the largest workspace sdpa_forward_noalloc serves
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

# (q/k head dim, v head dim) pairs the library takes
HEAD_DIMS = ((64, 64), (80, 80), (128, 128), (192, 192), (256, 256), (512, 512), (192, 256))

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


class SdpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sdpa status {status}: {message}")
        self.status = status
        self.message = message


def library_path() -> str:
    return os.environ.get("SDPA_MI355X_LIB", os.path.join(_PKG, "libsdpa_mi355x.so"))


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m flash_attention_head_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sdpa_forward.argtypes = [vp, vp, vp, vp] + [ci] * 6 + [ctypes.c_float] + [ci] * 4 + [vp, sz, vp]
    lib.sdpa_forward.restype = ci
    lib.sdpa_workspace_bytes.argtypes = [ci] * 6
    lib.sdpa_workspace_bytes.restype = sz
    lib.sdpa_forward_kv_view.argtypes = [vp, vp, vp, vp] + [ci] * 8 + [ctypes.c_float] + [ci] * 4 + [vp, sz, vp]
    lib.sdpa_forward_kv_view.restype = ci
    lib.sdpa_workspace_bytes_kv_view.argtypes = [ci] * 7
    lib.sdpa_workspace_bytes_kv_view.restype = sz
    ll = ctypes.c_longlong
    lib.sdpa_forward_bias.argtypes = [vp, vp, vp, vp, ll, ll, ll, vp] + [ci] * 6 + [ctypes.c_float] + [ci] * 4 + [vp, sz, vp]
    lib.sdpa_forward_bias.restype = ci
    lib.sdpa_forward_dv.argtypes = [vp, vp, vp, vp] + [ci] * 7 + [ctypes.c_float] + [ci] * 4 + [vp, sz, vp]
    lib.sdpa_forward_dv.restype = ci
    lib.sdpa_workspace_bytes_dv.argtypes = [ci] * 7
    lib.sdpa_workspace_bytes_dv.restype = sz
    lib.sdpa_forward_q4kv.argtypes = [vp] * 8 + [ci] * 8 + [ctypes.c_float] + [ci] * 4 + [vp, sz, vp]
    lib.sdpa_forward_q4kv.restype = ci
    lib.sdpa_forward_noalloc.argtypes = [vp, vp, vp, vp] + [ci] * 6 + [ctypes.c_float] + [ci] * 4 + [vp]
    lib.sdpa_forward_noalloc.restype = ci
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_version.argtypes = []
    lib.sdpa_version.restype = ci
    _lib = lib
    return lib


# ----------------------------------------------------------- raw C entry points
def sdpa_forward(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype,
                 workspace, workspace_bytes, stream) -> int:
    """``int sdpa_forward(...)`` of the C ABI; pointer arguments are integers."""
    return load_library().sdpa_forward(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window,
                                       q_offset, dtype, workspace, workspace_bytes, stream)


def sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D) -> int:
    """``size_t sdpa_workspace_bytes(...)``; (size_t)-1 for rejected shapes."""
    return load_library().sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D)


def sdpa_forward_kv_view(q, k, v, out, B, Hq, Hkv, qL, kL, kv_capacity, ring_start, D, scale, causal,
                         window, q_offset, dtype, workspace, workspace_bytes, stream) -> int:
    """``int sdpa_forward_kv_view(...)`` of the C ABI; pointer arguments are integers."""
    return load_library().sdpa_forward_kv_view(q, k, v, out, B, Hq, Hkv, qL, kL, kv_capacity,
                                               ring_start, D, scale, causal, window, q_offset,
                                               dtype, workspace, workspace_bytes, stream)


def sdpa_workspace_bytes_kv_view(B, Hq, Hkv, qL, kL, kv_capacity, D) -> int:
    """``size_t sdpa_workspace_bytes_kv_view(...)``; (size_t)-1 for rejected arguments."""
    return load_library().sdpa_workspace_bytes_kv_view(B, Hq, Hkv, qL, kL, kv_capacity, D)


def sdpa_forward_bias(q, k, v, bias, bias_stride_b, bias_stride_h, bias_stride_q, out, B, Hq, Hkv, qL, kL,
                      D, scale, causal, window, q_offset, dtype, workspace, workspace_bytes, stream) -> int:
    """``int sdpa_forward_bias(...)`` of the C ABI; pointer arguments are integers."""
    return load_library().sdpa_forward_bias(q, k, v, bias, bias_stride_b, bias_stride_h, bias_stride_q, out,
                                            B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype,
                                            workspace, workspace_bytes, stream)


def sdpa_forward_dv(q, k, v, out, B, Hq, Hkv, qL, kL, D, Dv, scale, causal, window, q_offset, dtype,
                    workspace, workspace_bytes, stream) -> int:
    """``int sdpa_forward_dv(...)`` of the C ABI; pointer arguments are integers."""
    return load_library().sdpa_forward_dv(q, k, v, out, B, Hq, Hkv, qL, kL, D, Dv, scale, causal, window,
                                          q_offset, dtype, workspace, workspace_bytes, stream)


def sdpa_workspace_bytes_dv(B, Hq, Hkv, qL, kL, D, Dv) -> int:
    """``size_t sdpa_workspace_bytes_dv(...)``; (size_t)-1 for rejected shapes."""
    return load_library().sdpa_workspace_bytes_dv(B, Hq, Hkv, qL, kL, D, Dv)


def sdpa_forward_q4kv(q, kq, ks, kb, vq, vs, vb, out, B, Hq, Hkv, qL, kL, kv_capacity, ring_start, D, scale,
                      causal, window, q_offset, dtype, workspace, workspace_bytes, stream) -> int:
    """``int sdpa_forward_q4kv(...)`` of the C ABI; pointer arguments are integers."""
    return load_library().sdpa_forward_q4kv(q, kq, ks, kb, vq, vs, vb, out, B, Hq, Hkv, qL, kL, kv_capacity,
                                            ring_start, D, scale, causal, window, q_offset, dtype, workspace,
                                            workspace_bytes, stream)


def sdpa_forward_noalloc(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype,
                         stream) -> int:
    """``int sdpa_forward_noalloc(...)`` of the C ABI (sdpa_forward without a workspace
    argument: the library's own per-GPU scratch array); pointer arguments are integers."""
    return load_library().sdpa_forward_noalloc(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window,
                                               q_offset, dtype, stream)


def sdpa_last_error() -> str:
    return load_library().sdpa_last_error().decode()


def sdpa_version() -> int:
    return load_library().sdpa_version()


# --------------------------------------------------------- torch tensor wrappers
def _check_tensors(q, k, v, value_dim=False):
    """Sizes and dtype code; with value_dim, v's last size may differ from q's
    (it is then returned as an eighth value)."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, L, D]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, Hq, qL, D = q.shape
    Bk, Hkv, L, Dk = k.shape
    same = tuple(v.shape) == tuple(k.shape) or (value_dim and tuple(v.shape[:3]) == tuple(k.shape[:3]))
    if not same or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    sizes = (B, Hq, Hkv, qL, L, D, (SDPA_FP16 if q.dtype == torch.float16 else SDPA_BF16))
    return sizes + (v.shape[3],) if value_dim else sizes


def _prepare(q, need, D, out, workspace, stream, Dv=None):
    import torch

    Dv = D if Dv is None else Dv
    oshape = tuple(q.shape[:3]) + (Dv,)
    if out is None:
        out = torch.empty(oshape, dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != oshape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {oshape} tensor of q's dtype")
    if need == ctypes.c_size_t(-1).value:
        raise SdpaError(SDPA_UNSUPPORTED if (D, Dv) not in HEAD_DIMS else SDPA_INVALID_ARG,
                        sdpa_last_error())
    ws_ptr, ws_bytes = 0, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return out, ws_ptr, ws_bytes, stream


def sdpa(q, k, v, *, scale: float | None = None, causal: bool = False, window: int = 0,
         q_offset: int | None = None, bias=None, out=None, workspace=None, stream=None):
    """softmax(scale * q k^T + mask) v on device tensors.

    q: [B, Hq, qL, D], k: [B, Hkv, kL, D], v: [B, Hkv, kL, Dv], contiguous fp16 or
    bf16 tensors on one GPU; D = Dv in {64, 80, 128, 192, 256, 512}, or D = 192 with
    Dv = 256 (sdpa_forward_dv, no bias); Hq a multiple of Hkv.  The result is
    [B, Hq, qL, Dv].  scale defaults to 1/sqrt(D) (as fp32).  With causal, query row i sits at key position q_offset + i;
    q_offset defaults to kL - qL (queries aligned to the end of the keys).
    window > 0 limits each row to its last `window` keys (requires causal).
    bias: an optional additive mask array of q's dtype, a tensor that broadcasts to
    [B, Hq, qL, kL] with contiguous keys (size-1 or stride-0 dimensions broadcast).
    Runs on `stream` (default: torch's current stream) without synchronising.
    """
    B, Hq, Hkv, qL, kL, D, dtype, Dv = _check_tensors(q, k, v, value_dim=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q_offset is None:
        q_offset = kL - qL if causal else 0
    if Dv != D:
        if bias is not None:
            raise ValueError("a bias is not supported with a value head dim other than q's")
        need = sdpa_workspace_bytes_dv(B, Hq, Hkv, qL, kL, D, Dv)
        out, ws_ptr, ws_bytes, stream = _prepare(q, need, D, out, workspace, stream, Dv)
        rc = sdpa_forward_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, qL, kL,
                             D, Dv, float(scale), int(bool(causal)), int(window), int(q_offset), dtype, ws_ptr,
                             ws_bytes, stream.cuda_stream)
        if rc != SDPA_OK:
            raise SdpaError(rc, sdpa_last_error())
        return out
    need = sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D)
    out, ws_ptr, ws_bytes, stream = _prepare(q, need, D, out, workspace, stream)
    if bias is None:
        rc = sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, qL, kL,
                          D, float(scale), int(bool(causal)), int(window), int(q_offset), dtype, ws_ptr,
                          ws_bytes, stream.cuda_stream)
    else:
        if bias.dtype != q.dtype or not bias.is_cuda or bias.dim() != 4:
            raise ValueError("bias must be a 4-D GPU tensor of q's dtype")
        bshape = tuple(bias.shape)
        if bshape[2:] != (qL, kL) or bshape[0] not in (1, B) or bshape[1] not in (1, Hq):
            raise ValueError(f"bias {bshape} does not broadcast to {(B, Hq, qL, kL)}")
        if kL > 1 and bias.stride(3) != 1:
            raise ValueError("bias keys must be contiguous")
        sb, sh, sq = (0 if bshape[i] == 1 else bias.stride(i) for i in range(3))
        rc = sdpa_forward_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(), sb, sh, sq,
                               out.data_ptr(), B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)),
                               int(window), int(q_offset), dtype, ws_ptr, ws_bytes, stream.cuda_stream)
    if rc != SDPA_OK:
        raise SdpaError(rc, sdpa_last_error())
    return out


def sdpa_kv_cache(q, k_cache, v_cache, kv_len: int, *, ring_start: int = 0,
                  scale: float | None = None, causal: bool = False, window: int = 0,
                  q_offset: int | None = None, out=None, workspace=None, stream=None):
    """``sdpa`` over keys and values held in a KV cache.

    k_cache and v_cache: [B, Hkv, capacity, D]; kv_len live keys, logical key j
    in row (ring_start + j) % capacity of its head (a wrapped ring when
    ring_start + kv_len > capacity).  Positions and masks refer to logical key
    indices; q_offset defaults to kv_len - qL.  Decode and verify calls
    (qL <= 4) over one cache use key chunks fixed by (B, Hkv, capacity), so a
    verify row and the single-row call over its trimmed prefix agree byte for
    byte.
    """
    B, Hq, Hkv, qL, cap, D, dtype = _check_tensors(q, k_cache, v_cache)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q_offset is None:
        q_offset = kv_len - qL if causal else 0
    need = sdpa_workspace_bytes_kv_view(B, Hq, Hkv, qL, int(kv_len), cap, D)
    out, ws_ptr, ws_bytes, stream = _prepare(q, need, D, out, workspace, stream)
    rc = sdpa_forward_kv_view(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B,
                              Hq, Hkv, qL, int(kv_len), cap, int(ring_start), D, float(scale),
                              int(bool(causal)), int(window), int(q_offset), dtype, ws_ptr, ws_bytes,
                              stream.cuda_stream)
    if rc != SDPA_OK:
        raise SdpaError(rc, sdpa_last_error())
    return out


def sdpa_q4kv(q, kq, ks, kb, vq, vs, vb, *, kv_len: int | None = None, ring_start: int = 0,
              scale: float | None = None, causal: bool = False, window: int = 0, q_offset: int | None = None,
              out=None, workspace=None, stream=None):
    """``sdpa_kv_cache`` over a 4-bit KV cache (``sdpa_forward_q4kv``): decode / verify
    steps and chunked prefill over a 4-bit prefix.

    q: [B, Hq, qL, 256] fp16 or bf16.  kq, vq: [B, Hkv, capacity, 32] int32 code words
    (element 8 w + n of a row in bits 4 n .. 4 n + 3 of word w).  ks, kb, vs, vb:
    [B, Hkv, capacity, 4] of q's dtype, the scale and bias of each 64-element group;
    element d of a row is scale[d // 64] * code_d + bias[d // 64].  kv_len live keys
    (default: the capacity), logical key j in row (ring_start + j) % capacity.  Decode
    and verify calls over one cache use key chunks fixed by (B, Hkv, capacity), so a
    verify row and the single-row call over its trimmed key count agree byte for byte.
    """
    import torch

    if q.dim() != 4 or kq.dim() != 4 or vq.dim() != 4:
        raise ValueError("q and the code words must be 4-D")
    B, Hq, qL, D = q.shape
    Bk, Hkv, cap, W = kq.shape
    if q.dtype not in (torch.float16, torch.bfloat16) or kq.dtype != torch.int32 or vq.dtype != torch.int32:
        raise ValueError("q must be fp16/bf16 and the code words int32")
    if Bk != B or W * 8 != D or tuple(vq.shape) != tuple(kq.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kq {tuple(kq.shape)}, vq {tuple(vq.shape)}")
    for t in (ks, kb, vs, vb):
        if tuple(t.shape) != (B, Hkv, cap, D // 64) or t.dtype != q.dtype:
            raise ValueError("scales and biases must be [B, Hkv, capacity, D / 64] tensors of q's dtype")
    ts = (q, kq, ks, kb, vq, vs, vb)
    if not all(t.is_cuda and t.is_contiguous() for t in ts):
        raise ValueError("all inputs must be contiguous GPU tensors")
    dtype = SDPA_FP16 if q.dtype == torch.float16 else SDPA_BF16
    kL = cap if kv_len is None else int(kv_len)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q_offset is None:
        q_offset = kL - qL if causal else 0
    need = sdpa_workspace_bytes_kv_view(B, Hq, Hkv, qL, kL, cap, D)
    out, ws_ptr, ws_bytes, stream = _prepare(q, need, D, out, workspace, stream)
    rc = sdpa_forward_q4kv(*(t.data_ptr() for t in ts), out.data_ptr(), B, Hq, Hkv, qL, kL, cap, int(ring_start), D,
                           float(scale), int(bool(causal)), int(window), int(q_offset), dtype, ws_ptr, ws_bytes,
                           stream.cuda_stream)
    if rc != SDPA_OK:
        raise SdpaError(rc, sdpa_last_error())
    return out
