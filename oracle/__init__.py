"""fp64 CPU oracle for scaled-dot-product attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
in ``flash_attention_head_amd`` never imports it, and it imports nothing from
there: the two share no code.

The arithmetic lives in ``sdpa_oracle.c`` (plain C, double precision, one
row at a time, ascending key order); this module only builds and loads that
library and marshals numpy arrays of fp16/bf16 bit patterns into it.
What it computes, and the readings taken where the pages leave a step open,
are stated in the header of ``sdpa_oracle.c``.

``dense.py`` holds the same function written as the unfused matrix product,
softmax and matrix product in numpy (``sdpa_dense_rows_f64``), for row checks
at full size.

Every function here has a pin in ``tests/test_oracle_pins.py`` or
``tests/test_oracle_dense_pins.py``; none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .dense import sdpa_dense_rows_f64  # noqa: F401  (numpy, no C library)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdpa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_sdpa.so")
# A test may point the whole suite at another build of the oracle (a planted
# mistake, built from a modified copy of the source) through this variable.
_LIB_OVERRIDE = os.environ.get("SDPA_ORACLE_LIB")

FP16 = 0
BF16 = 1

_lib = None


def build(out_path: str = _LIB, src_path: str = _SRC, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc (no fast-math: the C order of operations holds)."""
    cmd = [
        "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared",
        "-pthread", *extra_flags, src_path, "-o", out_path + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def load(path: str = _LIB):
    """Load a built oracle library (building the default one if it is absent)."""
    global _lib
    if path == _LIB and _LIB_OVERRIDE:
        path = _LIB_OVERRIDE
        if _lib is not None:
            return _lib
        lib = load(path)
        _lib = lib
        return lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if path != _LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    ci = ctypes.c_int
    lib.oracle_sdpa_f64.argtypes = [u16p, u16p, u16p, f64p] + [ci] * 6 + [ctypes.c_float] + [ci] * 5
    lib.oracle_sdpa_f64.restype = ci
    lib.oracle_sdpa_rows_f64.argtypes = (
        [u16p, u16p, u16p, f64p] + [ci] * 6 + [ctypes.c_float] + [ci] * 4 + [i64p, ctypes.c_int64, ci]
    )
    lib.oracle_sdpa_rows_f64.restype = ci
    i64 = ctypes.c_int64
    lib.oracle_sdpa_bias_f64.argtypes = (
        [u16p, u16p, u16p, u16p, i64, i64, i64, f64p] + [ci] * 6 + [ctypes.c_float] + [ci] * 4 + [i64p, i64, ci]
    )
    lib.oracle_sdpa_bias_f64.restype = ci
    lib.oracle_sdpa_dv_f64.argtypes = (
        [u16p, u16p, u16p, f64p] + [ci] * 7 + [ctypes.c_float] + [ci] * 4 + [i64p, i64, ci]
    )
    lib.oracle_sdpa_dv_f64.restype = ci
    lib.oracle_widen.argtypes = [u16p, f64p, ctypes.c_int64, ci]
    lib.oracle_widen.restype = None
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.oracle_sdpa_q4kv_f64.argtypes = (
        [u16p, u32p, u16p, u16p, u32p, u16p, u16p, f64p] + [ci] * 6 + [ctypes.c_float] + [ci] * 4 + [i64p, i64, ci]
    )
    lib.oracle_sdpa_q4kv_f64.restype = ci
    lib.oracle_dequant4.argtypes = [u32p, u16p, u16p, f64p, i64, ci, ci]
    lib.oracle_dequant4.restype = None
    if path == _LIB:
        _lib = lib
    return lib


def _bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype not in (np.uint16, np.int16):
        raise TypeError("oracle inputs are fp16/bf16 bit patterns as uint16 arrays")
    return a.view(np.uint16)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, Hq, qL, D = q.shape
    Bk, Hkv, kL, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k, v")
    return B, Hq, Hkv, qL, kL, D


def sdpa_f64(q, k, v, *, scale: float, causal: bool = False, window: int = 0, q_offset: int = 0,
             dtype: int = FP16, threads: int | None = None, lib=None) -> np.ndarray:
    """All output rows, [B, Hq, qL, D] float64.

    q, k, v: uint16 bit patterns of fp16 (dtype=FP16) or bf16 (dtype=BF16) values;
    scale: converted to fp32 first, as the GPU library receives it.
    """
    lib = lib or load()
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, Hq, Hkv, qL, kL, D = _check_shapes(q, k, v)
    out = np.empty((B, Hq, qL, D), dtype=np.float64)
    rc = lib.oracle_sdpa_f64(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        _ptr(out, ctypes.c_double), B, Hq, Hkv, qL, kL, D, float(np.float32(scale)),
        int(bool(causal)), int(window), int(q_offset), int(dtype), int(threads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_sdpa_f64 failed ({rc})")
    return out


def sdpa_rows_f64(q, k, v, rows, *, scale: float, causal: bool = False, window: int = 0,
                  q_offset: int = 0, dtype: int = FP16, threads: int | None = None,
                  lib=None) -> np.ndarray:
    """Selected rows, [len(rows), D] float64; rows are flat indices (b*Hq + hq)*qL + i."""
    lib = lib or load()
    q, k, v = _bits(q), _bits(k), _bits(v)
    B, Hq, Hkv, qL, kL, D = _check_shapes(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, D), dtype=np.float64)
    rc = lib.oracle_sdpa_rows_f64(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        _ptr(out, ctypes.c_double), B, Hq, Hkv, qL, kL, D, float(np.float32(scale)),
        int(bool(causal)), int(window), int(q_offset), int(dtype), _ptr(rows, ctypes.c_int64),
        int(rows.size), int(threads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_sdpa_rows_f64 failed ({rc})")
    return out


def widen(bits, dtype: int, lib=None) -> np.ndarray:
    """Exact fp16/bf16 -> float64 widening of a uint16 bit-pattern array."""
    lib = lib or load()
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_widen(_ptr(b, ctypes.c_uint16), _ptr(out, ctypes.c_double), b.size, int(dtype))
    return out


def sdpa_bias_f64(q, k, v, bias, *, scale: float, causal: bool = False, window: int = 0,
                  q_offset: int = 0, dtype: int = FP16, rows=None, threads: int | None = None,
                  lib=None) -> np.ndarray:
    """Output rows with an additive mask array added to the scaled scores.

    bias: uint16 bit patterns (the input dtype), shape [Bb, Hb, qL, kL] with Bb in
    {1, B} and Hb in {1, Hq} (1 broadcasts).  rows=None: every row, [B, Hq, qL, D];
    else the flat rows (b*Hq + hq)*qL + i, [len(rows), D].
    """
    lib = lib or load()
    q, k, v, bias = _bits(q), _bits(k), _bits(v), _bits(bias)
    B, Hq, Hkv, qL, kL, D = _check_shapes(q, k, v)
    if bias.ndim != 4 or bias.shape[2:] != (qL, kL) or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, Hq):
        raise ValueError(f"bias shape {bias.shape} does not broadcast to {(B, Hq, qL, kL)}")
    sq = kL
    sh = 0 if bias.shape[1] == 1 else qL * kL
    sb = 0 if bias.shape[0] == 1 else bias.shape[1] * qL * kL
    if rows is None:
        out = np.empty((B, Hq, qL, D), dtype=np.float64)
        rptr, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, D), dtype=np.float64)
        rptr, nrows = _ptr(rows, ctypes.c_int64), rows.size
    rc = lib.oracle_sdpa_bias_f64(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        _ptr(bias, ctypes.c_uint16), sb, sh, sq, _ptr(out, ctypes.c_double), B, Hq, Hkv, qL, kL, D,
        float(np.float32(scale)), int(bool(causal)), int(window), int(q_offset), int(dtype), rptr, nrows,
        int(threads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_sdpa_bias_f64 failed ({rc})")
    return out


def sdpa_dv_f64(q, k, v, *, scale: float, causal: bool = False, window: int = 0, q_offset: int = 0,
                dtype: int = FP16, rows=None, threads: int | None = None, lib=None) -> np.ndarray:
    """Output rows when v's head dim Dv may differ from q's and k's D.

    q [B, Hq, qL, D], k [B, Hkv, kL, D], v [B, Hkv, kL, Dv] (uint16 bit patterns).
    rows=None: every row, [B, Hq, qL, Dv]; else the flat rows (b*Hq + hq)*qL + i,
    [len(rows), Dv].
    """
    lib = lib or load()
    q, k, v = _bits(q), _bits(k), _bits(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, Hq, qL, D = q.shape
    Bk, Hkv, kL, Dk = k.shape
    if v.shape[:3] != k.shape[:3] or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k, v")
    Dv = v.shape[3]
    if rows is None:
        out = np.empty((B, Hq, qL, Dv), dtype=np.float64)
        rptr, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, Dv), dtype=np.float64)
        rptr, nrows = _ptr(rows, ctypes.c_int64), rows.size
    rc = lib.oracle_sdpa_dv_f64(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        _ptr(out, ctypes.c_double), B, Hq, Hkv, qL, kL, D, Dv, float(np.float32(scale)),
        int(bool(causal)), int(window), int(q_offset), int(dtype), rptr, nrows,
        int(threads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_sdpa_dv_f64 failed ({rc})")
    return out


def _words(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype not in (np.uint32, np.int32):
        raise TypeError("4-bit codes are packed in 32-bit words (uint32 arrays)")
    return a.view(np.uint32)


def dequant4_f64(codes, scales, biases, *, D: int, dtype: int = FP16, lib=None) -> np.ndarray:
    """The values of 4-bit rows: codes [..., D / 8] words, scales and biases [..., D / 64]
    (uint16 bit patterns of the dtype); returns [..., D] float64."""
    lib = lib or load()
    codes, scales, biases = _words(codes), _bits(scales), _bits(biases)
    if D % 64 or codes.shape[-1] != D // 8 or scales.shape[-1] != D // 64 or biases.shape != scales.shape:
        raise ValueError("4-bit rows: codes [..., D/8], scales and biases [..., D/64], D a multiple of 64")
    n = codes.size // (D // 8)
    if scales.size != n * (D // 64):
        raise ValueError("codes and scales describe different row counts")
    out = np.empty(codes.shape[:-1] + (D,), dtype=np.float64)
    lib.oracle_dequant4(_ptr(codes, ctypes.c_uint32), _ptr(scales, ctypes.c_uint16), _ptr(biases, ctypes.c_uint16),
                        _ptr(out, ctypes.c_double), n, D, int(dtype))
    return out


def sdpa_q4kv_f64(q, kq, ks, kb, vq, vs, vb, *, scale: float, causal: bool = False, window: int = 0,
                  q_offset: int = 0, dtype: int = FP16, rows=None, threads: int | None = None,
                  lib=None) -> np.ndarray:
    """Output rows with 4-bit K and V.

    q [B, Hq, qL, D] (uint16 bit patterns); kq, vq [B, Hkv, kL, D / 8] uint32 code words;
    ks, kb, vs, vb [B, Hkv, kL, D / 64] scales and biases (uint16 bit patterns of the dtype).
    rows=None: every row, [B, Hq, qL, D]; else the flat rows (b*Hq + hq)*qL + i, [len(rows), D].
    """
    lib = lib or load()
    q = _bits(q)
    kq, vq = _words(kq), _words(vq)
    ks, kb, vs, vb = _bits(ks), _bits(kb), _bits(vs), _bits(vb)
    if q.ndim != 4 or kq.ndim != 4:
        raise ValueError("q and the code words must be [B, H, L, ...]")
    B, Hq, qL, D = q.shape
    Bk, Hkv, kL, W = kq.shape
    if Bk != B or W * 8 != D or D % 64 or vq.shape != kq.shape:
        raise ValueError("shape mismatch between q and the 4-bit K/V")
    for a in (ks, kb, vs, vb):
        if a.shape != (B, Hkv, kL, D // 64):
            raise ValueError("scales and biases must be [B, Hkv, kL, D / 64]")
    if rows is None:
        out = np.empty((B, Hq, qL, D), dtype=np.float64)
        rptr, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, D), dtype=np.float64)
        rptr, nrows = _ptr(rows, ctypes.c_int64), rows.size
    rc = lib.oracle_sdpa_q4kv_f64(
        _ptr(q, ctypes.c_uint16), _ptr(kq, ctypes.c_uint32), _ptr(ks, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
        _ptr(vq, ctypes.c_uint32), _ptr(vs, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
        _ptr(out, ctypes.c_double), B, Hq, Hkv, qL, kL, D, float(np.float32(scale)),
        int(bool(causal)), int(window), int(q_offset), int(dtype), rptr, nrows,
        int(threads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_sdpa_q4kv_f64 failed ({rc})")
    return out
