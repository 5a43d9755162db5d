"""fp64 CPU oracle for small-q GQA decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it shares no code with them: the C source here has its own binary16 decoder,
its own round-to-nearest-even encoder and its own attention loop.

The computation follows FlashRT pull request #185 ("feat(structures): ggml host
adapter -- llama.cpp distribution for pi0.5 on Thor (SM110)"): the commit that
introduces the decomposed decode attention defines the operation
(``softmax(scale * Q K^T + mask) V`` over one f16 KV head shared by all query
heads, at most 16 query tokens), and the GQA-collapse commit fixes the t-major
row order ``r = t*n_head + h`` and the ``[hd, n_head, n_tok]`` destination.

Every function here has a pin in ``tests/test_oracle.py`` that does not go
through this package's own arithmetic (exhaustive checks against numpy's
binary16 conversions, brute force, closed forms, invariants and an independent
library attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "decode_attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

Q_F32 = 0             # f32 query values, used exactly
Q_F16 = 1             # f16 query bits (the pre-rounded handoff), used exactly
Q_F32_ROUND_F16 = 2   # f32 query values rounded to f16 (RNE) first

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f32_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16_rne.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16_rne_rows.restype = None
        lib.oracle_f32_to_f16_rne_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int64]
        lib.oracle_qkv_post_f64.restype = None
        lib.oracle_qkv_post_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_decode_attn_f64.restype = ctypes.c_int
        lib.oracle_decode_attn_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.oracle_decode_attn_gqa_f64.restype = ctypes.c_int
        lib.oracle_decode_attn_gqa_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int]
        _lib = lib
    return _lib


def f16_to_f64(bits) -> np.ndarray:
    """Widen binary16 bit patterns (uint16 array) to float64, element by element."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    flat_in, flat_out = b.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_f16_to_f64(int(flat_in[i]))
    return out


def f32_to_f16_rne(x) -> np.ndarray:
    """Round float32 values to binary16 bits, nearest-even, element by element."""
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in, flat_out = a.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_f32_to_f16_rne(float(flat_in[i]))
    return out


def f16_copy(src) -> np.ndarray:
    """The batched f32 -> f16 row copy: every float32 rounded to binary16 bits
    (nearest even) on its own; returns uint16 of the same shape."""
    lib = _load()
    a = np.ascontiguousarray(src, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib.oracle_f32_to_f16_rne_rows(a.ctypes.data, out.ctypes.data, int(a.size))
    return out


def qkv_post(qkv, pos, n_head: int, n_kv_head: int, n_tok: int, hd: int, base: float,
             q_scale: float):
    """RoPE (NeoX form) and the query scale applied to one instance's fused QKV
    projection output, in fp64.

    qkv : [n_tok, (n_head + 2*n_kv_head) * hd] float32;  pos : [n_tok] int
    returns q [n_tok, n_head, hd], k [n_kv_head, n_tok, hd], v [n_kv_head, n_tok, hd]
    """
    lib = _load()
    a = np.ascontiguousarray(qkv, dtype=np.float32)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    if a.size != n_tok * (n_head + 2 * n_kv_head) * hd or p.size != n_tok or hd % 2:
        raise ValueError("oracle: qkv_post sizes do not match")
    q = np.empty((n_tok, n_head, hd), dtype=np.float64)
    k = np.empty((n_kv_head, n_tok, hd), dtype=np.float64)
    v = np.empty((n_kv_head, n_tok, hd), dtype=np.float64)
    lib.oracle_qkv_post_f64(a.ctypes.data, p.ctypes.data, int(n_head), int(n_kv_head),
                            int(n_tok), int(hd), float(base), float(q_scale), q.ctypes.data,
                            k.ctypes.data, v.ctypes.data)
    return q, k, v


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def decode_attn(q, k, v, mask, n_head: int, n_tok: int, n_kv: int, hd: int,
                scale: float, q_kind: int = Q_F32, threads: int = 0,
                return_threads: bool = False, n_kv_head: int = 1):
    """One instance of decode attention in fp64.

    q    : [n_tok, n_head, hd] float32 (Q_F32, Q_F32_ROUND_F16) or uint16 f16 bits (Q_F16)
    k, v : [n_kv, hd] uint16 f16 bits; with n_kv_head > 1, [n_kv_head, n_kv, hd]
           (query head h uses KV head h // (n_head // n_kv_head))
    mask : [n_tok, n_kv] uint16 f16 bits, or None (all zero); shared by all heads
    returns [n_tok, n_head, hd] float64  (== ggml's [hd, n_head, n_tok])
    """
    lib = _load()
    qdt = np.uint16 if q_kind == Q_F16 else np.float32
    qa = np.ascontiguousarray(q, dtype=qdt)
    ka = np.ascontiguousarray(k, dtype=np.uint16)
    va = np.ascontiguousarray(v, dtype=np.uint16)
    kv_size = n_kv_head * n_kv * hd
    if qa.size != n_tok * n_head * hd or ka.size != kv_size or va.size != kv_size:
        raise ValueError("oracle: tensor sizes do not match the shape arguments")
    ma = None
    if mask is not None:
        ma = np.ascontiguousarray(mask, dtype=np.uint16)
        if ma.size != n_tok * n_kv:
            raise ValueError("oracle: mask size does not match [n_tok, n_kv]")
    out = np.empty((n_tok, n_head, hd), dtype=np.float64)
    used = lib.oracle_decode_attn_gqa_f64(
        qa.ctypes.data, int(q_kind), ka.ctypes.data, va.ctypes.data,
        None if ma is None else ma.ctypes.data, out.ctypes.data,
        int(n_head), int(n_kv_head), int(n_tok), int(n_kv), int(hd), float(scale),
        int(threads))
    if used < 0:
        raise RuntimeError("oracle_decode_attn_f64 failed")
    return (out, used) if return_threads else out
