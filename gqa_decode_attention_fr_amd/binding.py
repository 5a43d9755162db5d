"""Thin ctypes binding over libfrattn.so (include/fr_decode_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Functions carry the C entry points' names, take
torch CUDA tensors (or raw device addresses as ints) and the current torch
stream by default, and raise FrError on a non-zero status.  There is no
fallback: if the library is missing this module raises when first used.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfrattn.so")

FR_OK = 0
FR_ERR_INVALID = -1
FR_ERR_UNSUPPORTED = -2
FR_ERR_CAPTURE = -3
FR_ERR_HIP = -4
FR_ERR_WORKSPACE = -5

FR_Q_F32 = 0
FR_Q_F16 = 1

FR_Q_ROUND_F16 = 0x1
FR_VARIANT_FUSED = 0x2
FR_VARIANT_DECOMPOSED = 0x4
FR_PLAN_UNMASKED = 0x8

# shape limits (fr_decode_attn.h)
FR_MAX_TOKENS = 64
FR_MAX_TOKENS_UNMASKED = 16384
FR_MAX_HEADS = 1024
FR_MAX_COPIES = 4096
FR_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol the header declares (checked by the ABI tests).
EXPORTED = ("fr_decode_attn", "fr_decode_attn_q16", "fr_decode_attn_batched",
            "fr_decode_attn_ex", "fr_decode_attn_gqa", "fr_decode_attn_gqa_noalloc",
            "fr_decode_attn_workspace_size",
            "fr_decode_attn_reserve", "fr_decode_attn_workspace_query",
            "fr_decode_attn_workspace_release",
            "fr_decode_attn_plan", "fr_decode_attn_profile_events", "fr_f16_copy_batch",
            "fr_qkv_post",
            "fr_status_str",
            "fr_abi_version")

PLAN_FIELDS = ("variant", "n_split", "chunk", "waves", "tiles", "n_rowblk", "grid", "launches")


class F16Copy(ctypes.Structure):
    """struct fr_f16_copy: n float32 at src -> binary16 bits at dst."""
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("n", ctypes.c_int64)]


class FrError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m gqa_decode_attention_fr_amd.build`")
    try:  # load torch's HIP runtime first so that torch and the library share one
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, u32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_uint, ctypes.c_size_t)
    single = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
    lib.fr_decode_attn.argtypes = single
    lib.fr_decode_attn_q16.argtypes = single
    batched = [vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, i32, i32, i32, f32]
    lib.fr_decode_attn_batched.argtypes = batched + [vp]
    lib.fr_decode_attn_ex.argtypes = batched + [u32, vp, sz, vp]
    lib.fr_decode_attn_gqa.argtypes = (batched[:5] + [vp] + batched[5:12] + [i32, i64] +
                                       batched[12:] + [u32, vp, sz, vp])
    lib.fr_decode_attn_gqa_noalloc.argtypes = (batched[:5] + [vp] + batched[5:12] + [i32, i64] +
                                               batched[12:] + [u32, vp])
    for fn in ("fr_decode_attn", "fr_decode_attn_q16", "fr_decode_attn_batched",
               "fr_decode_attn_ex", "fr_decode_attn_gqa", "fr_decode_attn_gqa_noalloc",
               "fr_decode_attn_reserve",
               "fr_decode_attn_plan",
               "fr_abi_version"):
        getattr(lib, fn).restype = i32
    lib.fr_decode_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, u32,
                                                  ctypes.POINTER(i32)]
    lib.fr_decode_attn_workspace_size.restype = sz
    lib.fr_decode_attn_reserve.argtypes = [i32, i32, i32, i32, i32, u32]
    lib.fr_decode_attn_workspace_query.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(sz),
                                                   ctypes.POINTER(i32)]
    lib.fr_decode_attn_workspace_query.restype = i32
    lib.fr_decode_attn_workspace_release.argtypes = []
    lib.fr_decode_attn_workspace_release.restype = i32
    lib.fr_decode_attn_plan.argtypes = [i32, i32, i32, i32, i32, u32, ctypes.POINTER(i32), i32]
    lib.fr_qkv_post.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32,
                                i32, i32, i32, f32, f32, vp]
    lib.fr_qkv_post.restype = i32
    lib.fr_f16_copy_batch.argtypes = [ctypes.POINTER(F16Copy), i32, vp]
    lib.fr_f16_copy_batch.restype = i32
    lib.fr_decode_attn_profile_events.argtypes = [vp, vp]
    lib.fr_decode_attn_profile_events.restype = i32
    lib.fr_status_str.argtypes = [i32]
    lib.fr_status_str.restype = ctypes.c_char_p
    lib.fr_abi_version.argtypes = []
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().fr_status_str(int(status)).decode()


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(st: int, what: str) -> None:
    if st != FR_OK:
        raise FrError(st, what)


def fr_decode_attn(q, k, v, mask, out, n_head, n_tok, n_kv, hd, scale, stream=None) -> None:
    """f32 q [n_tok, n_head, hd]; f16 k, v [n_kv, hd]; f16 mask [n_tok, n_kv] or None;
    fp32 out [n_tok, n_head, hd]."""
    _check(load().fr_decode_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(out), n_head,
                                 n_tok, n_kv, hd, scale, _stream(stream)), "fr_decode_attn")


def fr_decode_attn_q16(q16, k, v, mask, out, n_head, n_tok, n_kv, hd, scale,
                       stream=None) -> None:
    """Pre-rounded f16 q [n_tok, n_head, hd]; otherwise as fr_decode_attn."""
    _check(load().fr_decode_attn_q16(_ptr(q16), _ptr(k), _ptr(v), _ptr(mask), _ptr(out),
                                     n_head, n_tok, n_kv, hd, scale, _stream(stream)),
           "fr_decode_attn_q16")


def fr_decode_attn_batched(q, q_format, k, v, mask, out, n_inst, q_stride, kv_stride,
                           mask_stride, out_stride, n_head, n_tok, n_kv, hd, scale,
                           stream=None) -> None:
    _check(load().fr_decode_attn_batched(_ptr(q), q_format, _ptr(k), _ptr(v), _ptr(mask),
                                         _ptr(out), n_inst, q_stride, kv_stride, mask_stride,
                                         out_stride, n_head, n_tok, n_kv, hd, scale,
                                         _stream(stream)), "fr_decode_attn_batched")


def fr_decode_attn_ex(q, q_format, k, v, mask, out, n_inst, q_stride, kv_stride, mask_stride,
                      out_stride, n_head, n_tok, n_kv, hd, scale, flags=0, workspace=None,
                      workspace_bytes=0, stream=None) -> None:
    _check(load().fr_decode_attn_ex(_ptr(q), q_format, _ptr(k), _ptr(v), _ptr(mask), _ptr(out),
                                    n_inst, q_stride, kv_stride, mask_stride, out_stride, n_head,
                                    n_tok, n_kv, hd, scale, flags, _ptr(workspace),
                                    workspace_bytes, _stream(stream)), "fr_decode_attn_ex")


def fr_decode_attn_gqa(q, q_format, k, v, mask, out, n_inst, q_stride, kv_stride, mask_stride,
                       out_stride, n_head, n_kv_head, kv_head_stride, n_tok, n_kv, hd, scale,
                       flags=0, workspace=None, workspace_bytes=0, stream=None,
                       kv_len=None) -> None:
    """As fr_decode_attn_ex with n_kv_head KV heads per instance ([n_kv_head, n_kv, hd]
    blocks kv_head_stride elements apart); query head h reads KV head
    h // (n_head // n_kv_head).  kv_len: None or a device int32 tensor of n_inst
    valid key counts."""
    _check(load().fr_decode_attn_gqa(_ptr(q), q_format, _ptr(k), _ptr(v), _ptr(mask),
                                     _ptr(kv_len), _ptr(out), n_inst, q_stride, kv_stride, mask_stride,
                                     out_stride, n_head, n_kv_head, kv_head_stride, n_tok, n_kv,
                                     hd, scale, flags, _ptr(workspace), workspace_bytes,
                                     _stream(stream)), "fr_decode_attn_gqa")


def fr_decode_attn_gqa_noalloc(q, q_format, k, v, mask, out, n_inst, q_stride, kv_stride,
                               mask_stride, out_stride, n_head, n_kv_head, kv_head_stride, n_tok,
                               n_kv, hd, scale, flags=0, stream=None, kv_len=None) -> None:
    """fr_decode_attn_gqa without a workspace: partials in the library's fixed
    device array (FR_NOALLOC_SCRATCH_BYTES); no allocation of any kind."""
    _check(load().fr_decode_attn_gqa_noalloc(_ptr(q), q_format, _ptr(k), _ptr(v), _ptr(mask),
                                             _ptr(kv_len), _ptr(out), n_inst, q_stride,
                                             kv_stride, mask_stride, out_stride, n_head,
                                             n_kv_head, kv_head_stride, n_tok, n_kv, hd, scale,
                                             flags, _stream(stream)),
           "fr_decode_attn_gqa_noalloc")


def fr_decode_attn_workspace_size(n_inst, n_head, n_tok, n_kv, hd, flags=0) -> int:
    st = ctypes.c_int(0)
    n = load().fr_decode_attn_workspace_size(n_inst, n_head, n_tok, n_kv, hd, flags,
                                             ctypes.byref(st))
    _check(st.value, "fr_decode_attn_workspace_size")
    return int(n)


def fr_decode_attn_reserve(n_inst, n_head, n_tok, n_kv, hd, flags=0) -> None:
    _check(load().fr_decode_attn_reserve(n_inst, n_head, n_tok, n_kv, hd, flags),
           "fr_decode_attn_reserve")


def fr_decode_attn_workspace_query() -> tuple[int, int, int]:
    """(address, bytes, retired buffers) of the current device's library workspace."""
    p, n, r = ctypes.c_void_p(), ctypes.c_size_t(), ctypes.c_int()
    _check(load().fr_decode_attn_workspace_query(ctypes.byref(p), ctypes.byref(n),
                                                 ctypes.byref(r)),
           "fr_decode_attn_workspace_query")
    return int(p.value or 0), int(n.value), int(r.value)


def fr_decode_attn_workspace_release() -> None:
    _check(load().fr_decode_attn_workspace_release(), "fr_decode_attn_workspace_release")


def fr_decode_attn_plan(n_inst, n_head, n_tok, n_kv, hd, flags=0) -> dict:
    info = (ctypes.c_int * len(PLAN_FIELDS))()
    _check(load().fr_decode_attn_plan(n_inst, n_head, n_tok, n_kv, hd, flags, info,
                                      len(PLAN_FIELDS)), "fr_decode_attn_plan")
    return dict(zip(PLAN_FIELDS, list(info)))


def fr_qkv_post(qkv, pos, q16, k_cache, v_cache, n_inst, qkv_stride, pos_stride, q16_stride,
                cache_stride, cache_head_stride, n_head, n_kv_head, n_tok, hd, capacity,
                rope_base, q_scale, stream=None) -> None:
    """RoPE + query scale + f16 rows: q16 for the window, K/V into the caches."""
    _check(load().fr_qkv_post(_ptr(qkv), _ptr(pos), _ptr(q16), _ptr(k_cache), _ptr(v_cache),
                              n_inst, qkv_stride, pos_stride, q16_stride, cache_stride,
                              cache_head_stride, n_head, n_kv_head, n_tok, hd, capacity,
                              rope_base, q_scale, _stream(stream)), "fr_qkv_post")


def fr_f16_copy_batch(copies, stream=None) -> None:
    """copies: sequence of (src, dst, n) with src float32 and dst float16/uint16
    device tensors or raw pointers; one batched f32 -> f16 conversion call."""
    arr = (F16Copy * max(1, len(copies)))()
    for i, (src, dst, n) in enumerate(copies):
        arr[i] = F16Copy(_ptr(src), _ptr(dst), int(n))
    _check(load().fr_f16_copy_batch(arr, len(copies), _stream(stream)), "fr_f16_copy_batch")


def fr_decode_attn_profile_events(start, stop) -> None:
    """start/stop: raw hipEvent_t handles (ints) or None, None to turn timing off."""
    _check(load().fr_decode_attn_profile_events(start, stop), "fr_decode_attn_profile_events")


def fr_status_str(status: int) -> str:
    return status_str(status)


def fr_abi_version() -> int:
    return int(load().fr_abi_version())
