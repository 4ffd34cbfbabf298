"""ctypes loader for the plain C float64 attention oracle (test only).

``build()`` compiles ``oracle/c/paged_attn_oracle.c`` with gcc and OpenMP
into ``oracle/c/libpkv_oracle.so``. ``attention()`` calls it on host arrays.
The oracle is described in the C source's header.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "c", "paged_attn_oracle.c")
LIB = os.path.join(_HERE, "c", "libpkv_oracle.so")
_DT = {"f32": 0, "bf16": 1}
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc -O2 -fopenmp); returns the library path."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        lib.pkv_oracle_attention.restype = ctypes.c_int
        lib.pkv_oracle_attention.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int]
        lib.pkv_oracle_attention_q8.restype = ctypes.c_int
        lib.pkv_oracle_attention_q8.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int]
        lib.pkv_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().pkv_oracle_max_threads()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def attention(q, q_dtype: str, k_pool, v_pool, kv_dtype: str, tables, lens,
              scale: float, block_size: int, rows=None, threads: int = 0):
    """Run the C oracle.

    q: [B, nq, Hq, D]; pools: [NB, Hkv, bs, D] (float32 arrays, or uint16/int16
    bit patterns for bf16); tables: [B, max_blocks] int32; lens: [B] int32.
    ``rows``: optional int64 flat row ids (b * nq + i) * Hq + h. Returns
    (out [n_rows, D] or [B, nq, Hq, D], lse) as float64.
    """
    lib = _load()

    def prep(a, dt):
        if dt == "f32":
            return np.ascontiguousarray(a, dtype=np.float32)
        return np.ascontiguousarray(np.asarray(a).view(np.uint16))

    qa, ka, va = prep(q, q_dtype), prep(k_pool, kv_dtype), prep(v_pool, kv_dtype)
    B, nq, Hq, D = qa.shape
    NB, Hkv, bs, Dk = ka.shape
    if Dk != D or bs != block_size:
        raise ValueError("pool shape does not match")
    tb = np.ascontiguousarray(tables, dtype=np.int32)
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    if rows is None:
        n = B * nq * Hq
        rw = None
    else:
        rw = np.ascontiguousarray(rows, dtype=np.int64)
        n = rw.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    rc = lib.pkv_oracle_attention(
        _ptr(qa), _DT[q_dtype], _ptr(ka), _ptr(va), _DT[kv_dtype], _ptr(tb),
        tb.shape[1], _ptr(ln), B, nq, Hq, Hkv, D, bs, NB, float(scale),
        None if rw is None else _ptr(rw), n, _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"C oracle rejected its input (code {rc})")
    if rows is None:
        return out.reshape(B, nq, Hq, D), lse.reshape(B, nq, Hq)
    return out, lse


def attention_q8(q, q_dtype: str, k_codes, v_codes, k_scales, v_scales, tables, lens,
                 scale: float, block_size: int, rows=None, threads: int = 0):
    """The C walk over a pool of per-row int8 codes: element = code * scale.

    k_codes, v_codes: int8 [NB, Hkv, bs, D]; k_scales, v_scales: float32
    [NB, Hkv, bs]. Other arguments and the result as in ``attention``."""
    lib = _load()
    qa = (np.ascontiguousarray(q, dtype=np.float32) if q_dtype == "f32"
          else np.ascontiguousarray(np.asarray(q).view(np.uint16)))
    kc = np.ascontiguousarray(k_codes, dtype=np.int8)
    vc = np.ascontiguousarray(v_codes, dtype=np.int8)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    B, nq, Hq, D = qa.shape
    NB, Hkv, bs, Dk = kc.shape
    if Dk != D or bs != block_size or ks.shape != (NB, Hkv, bs) or vs.shape != ks.shape \
            or vc.shape != kc.shape:
        raise ValueError("pool shape does not match")
    tb = np.ascontiguousarray(tables, dtype=np.int32)
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    if rows is None:
        n = B * nq * Hq
        rw = None
    else:
        rw = np.ascontiguousarray(rows, dtype=np.int64)
        n = rw.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    rc = lib.pkv_oracle_attention_q8(
        _ptr(qa), _DT[q_dtype], _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), _ptr(tb),
        tb.shape[1], _ptr(ln), B, nq, Hq, Hkv, D, bs, NB, float(scale),
        None if rw is None else _ptr(rw), n, _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"C oracle rejected its input (code {rc})")
    if rows is None:
        return out.reshape(B, nq, Hq, D), lse.reshape(B, nq, Hq)
    return out, lse
