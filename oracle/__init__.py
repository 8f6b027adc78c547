"""CPU fp64 oracle for GQA flash-decode attention (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the CPU
baseline leg of the benchmark may import this module; the product path never
does.  It shares no code with the HIP library.

Every function takes the raw bf16 bit patterns (numpy uint16) that the GPU
path receives (or, for the *_fp8 functions, OCP FP8 E4M3 bytes as numpy uint8
plus one fp32 scale per K / V tensor), int32 lengths / page tables, and a
float32 scale, and returns float64 outputs of shape [B, Hq, D].  See oracle.c
for the definition and the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-shared", "-fPIC", "-Wall", "-Wextra"]

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c with gcc (always recompiles).  Each process writes its own temporary
    file and renames it into place, so concurrent builds (parallel test workers) do not collide."""
    tmp = f"{out}.{os.getpid()}.tmp"
    subprocess.check_call(["gcc", *CFLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load the built oracle, building it first if nothing is built."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p):
        build(out=p)
    lib = ctypes.CDLL(p)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    ci, cf = ctypes.c_int, ctypes.c_float
    lib.oracle_decode.argtypes = [u16p, u16p, u16p, i32p, ci, ci, ci, ci, ci, cf, f64p]
    lib.oracle_decode_split.argtypes = [u16p, u16p, u16p, i32p, ci, ci, ci, ci, ci, cf, ci, f64p]
    lib.oracle_paged_decode.argtypes = [u16p, u16p, u16p, i32p, i32p, ci, ci, ci, ci, ci, ci, ci,
                                        cf, f64p]
    lib.oracle_paged_decode_split.argtypes = [u16p, u16p, u16p, i32p, i32p, ci, ci, ci, ci, ci,
                                              ci, ci, cf, ci, f64p]
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_decode_fp8.argtypes = [u16p, u8p, u8p, i32p, ci, ci, ci, ci, ci, cf, cf, cf, ci, f64p]
    lib.oracle_paged_decode_fp8.argtypes = [u16p, u8p, u8p, i32p, i32p, ci, ci, ci, ci, ci, ci, ci,
                                            cf, cf, cf, ci, f64p]
    lib.oracle_decode_mq.argtypes = [u16p, u16p, u16p, i32p, ci, ci, ci, ci, ci, ci, cf, ci, f64p]
    lib.oracle_paged_decode_mq.argtypes = [u16p, u16p, u16p, i32p, i32p, ci, ci, ci, ci, ci, ci,
                                           ci, ci, cf, ci, f64p]
    for fn in (lib.oracle_decode, lib.oracle_decode_split, lib.oracle_paged_decode,
               lib.oracle_paged_decode_split, lib.oracle_max_threads, lib.oracle_decode_fp8,
               lib.oracle_paged_decode_fp8, lib.oracle_decode_mq, lib.oracle_paged_decode_mq):
        fn.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ci]
    lib.oracle_set_threads.restype = None
    if path is None:
        _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs must be passed as uint16 bit patterns")
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def decode(q, k, v, seq_lens, scale, *, chunk: int = 0, lib=None) -> np.ndarray:
    """Contiguous cache: q [B,Hq,D], k/v [B,Hkv,S_max,D] (uint16 bf16 bits)."""
    lib = lib or load()
    q, k, v, seq_lens = _u16(q), _u16(k), _u16(v), _i32(seq_lens)
    B, Hq, D = q.shape
    Bk, Hkv, S_max, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or seq_lens.shape != (B,):
        raise ValueError("shape mismatch")
    out = np.empty((B, Hq, D), dtype=np.float64)
    args = [_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
            _ptr(seq_lens, ctypes.c_int32), B, Hq, Hkv, D, S_max, ctypes.c_float(scale)]
    if chunk > 0:
        rc = lib.oracle_decode_split(*args, chunk, _ptr(out, ctypes.c_double))
    else:
        rc = lib.oracle_decode(*args, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return out


def paged_decode(q, k_pool, v_pool, seq_lens, page_table, scale, *, chunk: int = 0,
                 lib=None) -> np.ndarray:
    """Paged cache: k/v pools [P,Hkv,page_size,D], page_table [B,max_pages] int32."""
    lib = lib or load()
    q, k_pool, v_pool = _u16(q), _u16(k_pool), _u16(v_pool)
    seq_lens, page_table = _i32(seq_lens), _i32(page_table)
    B, Hq, D = q.shape
    P, Hkv, ps, Dk = k_pool.shape
    if v_pool.shape != k_pool.shape or Dk != D or seq_lens.shape != (B,) or \
            page_table.ndim != 2 or page_table.shape[0] != B:
        raise ValueError("shape mismatch")
    max_pages = page_table.shape[1]
    out = np.empty((B, Hq, D), dtype=np.float64)
    args = [_ptr(q, ctypes.c_uint16), _ptr(k_pool, ctypes.c_uint16),
            _ptr(v_pool, ctypes.c_uint16), _ptr(seq_lens, ctypes.c_int32),
            _ptr(page_table, ctypes.c_int32), B, Hq, Hkv, D, ps, P, max_pages,
            ctypes.c_float(scale)]
    if chunk > 0:
        rc = lib.oracle_paged_decode_split(*args, chunk, _ptr(out, ctypes.c_double))
    else:
        rc = lib.oracle_paged_decode(*args, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_paged_decode failed with code {rc}")
    return out


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("fp8 inputs must be passed as uint8 E4M3 bytes")
    return a


def decode_fp8(q, k, v, seq_lens, scale, k_scale, v_scale, *, chunk: int = 0,
               lib=None) -> np.ndarray:
    """Contiguous E4M3 cache: k/v [B,Hkv,S_max,D] uint8, one fp32 scale per tensor."""
    lib = lib or load()
    q, k, v, seq_lens = _u16(q), _u8(k), _u8(v), _i32(seq_lens)
    B, Hq, D = q.shape
    Bk, Hkv, S_max, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or seq_lens.shape != (B,):
        raise ValueError("shape mismatch")
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_decode_fp8(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint8),
                               _ptr(v, ctypes.c_uint8), _ptr(seq_lens, ctypes.c_int32), B, Hq,
                               Hkv, D, S_max, ctypes.c_float(scale), ctypes.c_float(k_scale),
                               ctypes.c_float(v_scale), int(chunk), _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_decode_fp8 failed with code {rc}")
    return out


def paged_decode_fp8(q, k_pool, v_pool, seq_lens, page_table, scale, k_scale, v_scale, *,
                     chunk: int = 0, lib=None) -> np.ndarray:
    """Paged E4M3 cache: k/v pools [P,Hkv,page_size,D] uint8, page_table [B,max_pages]."""
    lib = lib or load()
    q, k_pool, v_pool = _u16(q), _u8(k_pool), _u8(v_pool)
    seq_lens, page_table = _i32(seq_lens), _i32(page_table)
    B, Hq, D = q.shape
    P, Hkv, ps, Dk = k_pool.shape
    if v_pool.shape != k_pool.shape or Dk != D or seq_lens.shape != (B,) or \
            page_table.ndim != 2 or page_table.shape[0] != B:
        raise ValueError("shape mismatch")
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_paged_decode_fp8(_ptr(q, ctypes.c_uint16), _ptr(k_pool, ctypes.c_uint8),
                                     _ptr(v_pool, ctypes.c_uint8), _ptr(seq_lens, ctypes.c_int32),
                                     _ptr(page_table, ctypes.c_int32), B, Hq, Hkv, D, ps, P,
                                     page_table.shape[1], ctypes.c_float(scale),
                                     ctypes.c_float(k_scale), ctypes.c_float(v_scale), int(chunk),
                                     _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_paged_decode_fp8 failed with code {rc}")
    return out


def decode_mq(q, k, v, seq_lens, scale, *, chunk: int = 0, lib=None) -> np.ndarray:
    """Multi-query decode, contiguous bf16 cache: q [B,M,Hq,D]; query i of sequence b attends
    to keys 0 .. len-M+i.  Returns [B,M,Hq,D]."""
    lib = lib or load()
    q, k, v, seq_lens = _u16(q), _u16(k), _u16(v), _i32(seq_lens)
    B, M, Hq, D = q.shape
    Bk, Hkv, S_max, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or seq_lens.shape != (B,):
        raise ValueError("shape mismatch")
    out = np.empty((B, M, Hq, D), dtype=np.float64)
    rc = lib.oracle_decode_mq(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                              _ptr(v, ctypes.c_uint16), _ptr(seq_lens, ctypes.c_int32), B, M, Hq,
                              Hkv, D, S_max, ctypes.c_float(scale), int(chunk),
                              _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_decode_mq failed with code {rc}")
    return out


def paged_decode_mq(q, k_pool, v_pool, seq_lens, page_table, scale, *, chunk: int = 0,
                    lib=None) -> np.ndarray:
    """Multi-query decode over a paged bf16 cache: q [B,M,Hq,D]."""
    lib = lib or load()
    q, k_pool, v_pool = _u16(q), _u16(k_pool), _u16(v_pool)
    seq_lens, page_table = _i32(seq_lens), _i32(page_table)
    B, M, Hq, D = q.shape
    P, Hkv, ps, Dk = k_pool.shape
    if v_pool.shape != k_pool.shape or Dk != D or seq_lens.shape != (B,) or \
            page_table.ndim != 2 or page_table.shape[0] != B:
        raise ValueError("shape mismatch")
    out = np.empty((B, M, Hq, D), dtype=np.float64)
    rc = lib.oracle_paged_decode_mq(_ptr(q, ctypes.c_uint16), _ptr(k_pool, ctypes.c_uint16),
                                    _ptr(v_pool, ctypes.c_uint16), _ptr(seq_lens, ctypes.c_int32),
                                    _ptr(page_table, ctypes.c_int32), B, M, Hq, Hkv, D, ps, P,
                                    page_table.shape[1], ctypes.c_float(scale), int(chunk),
                                    _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_paged_decode_mq failed with code {rc}")
    return out


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())


def set_threads(n: int, lib=None) -> None:
    (lib or load()).oracle_set_threads(int(n))
