"""Helpers for the GPU tests: move seeded numpy inputs to the device, call the
C ABI through the binding, compare with the oracle at the stated tolerance."""
from __future__ import annotations

import sys

import numpy as np

# Acceptance bar for floating point: max-abs error and relative L2 error of
# the fp32 output against the fp64 oracle.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def say(msg: str) -> None:
    """Name the GPU case before it runs (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, torch):
    """numpy -> torch CUDA tensor with the same bytes (uint16 f16 bits become float16)."""
    if x is None:
        return None
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.float16)).cuda()
    return torch.from_numpy(a).cuda()


def errors(got: np.ndarray, want: np.ndarray) -> tuple[float, float]:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    max_abs = float(np.max(np.abs(got - want))) if got.size else 0.0
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want) / denom) if denom > 0 else float(np.linalg.norm(got))
    return max_abs, rel


def assert_close(got, want, what: str = "") -> None:
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = errors(got, want)
    assert max_abs <= MAX_ABS and rel <= REL_L2, \
        f"{what}: max_abs={max_abs:.3e} (<= {MAX_ABS}) rel_l2={rel:.3e} (<= {REL_L2})"


def oracle_instances(oracle, case, n_head, n_tok, n_kv, hd, scale, q_kind) -> np.ndarray:
    outs = []
    n_inst = case["k"].shape[0]
    for i in range(n_inst):
        m = None if case["mask"] is None else case["mask"][i]
        outs.append(oracle.decode_attn(case["q"][i], case["k"][i], case["v"][i], m, n_head, n_tok,
                                       n_kv, hd, scale, q_kind=q_kind))
    return np.stack(outs)


def run_gpu(case, n_head, n_tok, n_kv, hd, scale, flags=0, q_f16=False, torch=None,
            entry="ex") -> np.ndarray:
    """Runs the HIP path on every instance of `case` in one call; returns
    [n_inst, n_tok, n_head, hd] float32."""
    import gqa_decode_attention_fr_amd as F
    n_inst = case["k"].shape[0]
    q = dev(case["q"], torch)
    k = dev(case["k"], torch)
    v = dev(case["v"], torch)
    mask = dev(case["mask"], torch)
    M = n_head * n_tok
    out = torch.full((n_inst, n_tok, n_head, hd), float("nan"), dtype=torch.float32,
                     device="cuda")
    fmt = F.FR_Q_F16 if q_f16 else F.FR_Q_F32
    if entry == "single":
        assert n_inst == 1 and flags == 0
        fn = F.fr_decode_attn_q16 if q_f16 else F.fr_decode_attn
        fn(q, k, v, mask, out, n_head, n_tok, n_kv, hd, scale)
    else:
        F.fr_decode_attn_ex(q, fmt, k, v, mask, out, n_inst, M * hd, n_kv * hd,
                            0 if mask is None else n_tok * n_kv, M * hd, n_head, n_tok, n_kv,
                            hd, scale, flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _padded_kv(x, pad_rows, fill):
    """[n_inst, n_kvh, n_kv, hd] -> the same with pad_rows extra rows per KV
    head holding `fill` (f16 bits), which the kernels must never read."""
    if pad_rows == 0:
        return x
    n_inst, n_kvh, n_kv, hd = x.shape
    out = np.full((n_inst, n_kvh, n_kv + pad_rows, hd), fill, dtype=np.uint16)
    out[:, :, :n_kv] = x
    return out


def run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=0, q_f16=False, pad_rows=0,
            kv_len=None, kv_override=None):
    """fr_decode_attn_gqa on every instance of `c` (k, v as [n_inst, n_kvh, n_kv, hd])
    in one call; returns [n_inst, n_tok, n_head, hd] float32."""
    import torch
    import gqa_decode_attention_fr_amd as F
    n_inst = c["q"].shape[0]
    kf = _padded_kv(c["k"] if kv_override is None else kv_override[0], pad_rows, 0x7BFF)
    vf = _padded_kv(c["v"] if kv_override is None else kv_override[1], pad_rows, 0x7BFF)
    q, k, v, mask = dev(c["q"], torch), dev(kf, torch), dev(vf, torch), dev(c["mask"], torch)
    M = n_head * n_tok
    kvh_stride = (n_kv + pad_rows) * hd
    out = torch.full((n_inst, n_tok, n_head, hd), float("nan"), dtype=torch.float32,
                     device="cuda")
    F.fr_decode_attn_gqa(q, F.FR_Q_F16 if q_f16 else F.FR_Q_F32, k, v, mask, out, n_inst,
                         M * hd, n_kvh * kvh_stride, 0 if mask is None else n_tok * n_kv,
                         M * hd, n_head, n_kvh, kvh_stride, n_tok, n_kv, hd, scale, flags,
                         kv_len=None if kv_len is None else
                         torch.tensor(kv_len, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_gqa(oracle, c, n_head, n_kvh, n_tok, n_kv, hd, scale, q_kind):
    outs = []
    for i in range(c["q"].shape[0]):
        m = None if c["mask"] is None else c["mask"][i]
        outs.append(oracle.decode_attn(c["q"][i], c["k"][i], c["v"][i], m, n_head, n_tok, n_kv,
                                       hd, scale, q_kind=q_kind, n_kv_head=n_kvh))
    return np.stack(outs)
