"""Seeded synthetic inputs for small-q GQA decode attention.

This module holds no attention arithmetic.  It only draws inputs, so that the
HIP path and the fp64 oracle can be fed the same bytes; neither side imports
the other.

The workload shapes stand in for the pi0.5 action-decode attention that
FlashRT pull request #185 ("feat(structures): ggml host adapter -- llama.cpp
distribution for pi0.5 on Thor (SM110)") routes through its decomposed decode
attention: at most 16 query tokens, every query head sharing one f16 KV head
padded to the flash-attention KQ stride with zeroed pad rows (the prefill QKV
window commit of the same pull request pads and zeroes that way), and an f16
0/-inf additive mask.  The real workload (trained weights, camera frames) is
not available, so values are drawn from normal distributions.

Draw order per instance, from ``numpy.random.default_rng(seed)`` (PCG64):
  1. Q  = standard_normal((n_tok, n_head, hd)) * sigma_q, float64 -> float32
         (f16 workloads then round float32 -> float16, nearest-even)
  2. K  = standard_normal((n_valid, hd)) * sigma_kv, float64 -> float16
         (several KV heads: standard_normal((n_kv_head, n_valid, hd)))
  3. V  = same as K
  4. extras: the outlier rows of K (chosen without replacement, scaled in f16)
Then the n_kv - n_valid pad rows are appended as zeros and the mask is built.
All instances of one workload are drawn in sequence from the same generator.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F16_ZERO = np.uint16(0x0000)
F16_NEG_INF = np.uint16(0xFC00)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_head: int
    n_tok: int
    n_kv: int            # padded key count (the KV row stride of the mask)
    n_valid: int         # keys that are not padding
    hd: int
    n_inst: int = 1      # independent instances per call batch
    q_dtype: str = "f32"  # "f32" or "f16" (pre-rounded handoff)
    sigma_q: float = 1.0
    sigma_kv: float = 1.0
    mask_kind: str = "zero"   # "zero" | "pad" | "causal_tail" | "none" (no mask passed)
    k_outlier_frac: float = 0.0
    k_outlier_scale: float = 1.0
    seed: int = 0
    n_kv_head: int = 1   # KV heads; query head h reads KV head h // (n_head // n_kv_head)
    dynamic_len: bool = False  # valid keys passed as device counts instead of a mask

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.hd)

    @property
    def M(self) -> int:
        return self.n_head * self.n_tok

    def algorithmic_bytes(self) -> int:
        """Bytes one call must move at minimum, summed over instances:
        K and V over keys visible to at least one query, Q, the full mask,
        and the fp32 output."""
        qb = 4 if self.q_dtype == "f32" else 2
        mask_bytes = 0 if self.mask_kind == "none" else self.n_tok * self.n_kv * 2
        per = (2 * self.n_kv_head * self.n_valid * self.hd * 2 + self.M * self.hd * qb
               + mask_bytes + self.M * self.hd * 4)
        return per * self.n_inst

    def flops(self) -> int:
        """Two contractions over the valid keys, summed over instances."""
        return 4 * self.M * self.n_valid * self.hd * self.n_inst


# The five workloads the library is measured and checked on.
TINY = Workload("tiny_h8_hd256_t1_kv64", n_head=8, n_tok=1, n_kv=64, n_valid=64, hd=256)
PI05_ACTION_STEP = Workload("pi05_action_step_h8_hd256_t10_kv1024_x18", n_head=8, n_tok=10,
                            n_kv=1024, n_valid=968, hd=256, n_inst=18, sigma_kv=0.5,
                            mask_kind="pad")
H16_HD128_Q16 = Workload("h16_hd128_t16_kv4096_q16", n_head=16, n_tok=16, n_kv=4096,
                         n_valid=4096, hd=128, q_dtype="f16")
CAUSAL_TAIL = Workload("causal_tail_h8_hd256_t16_kv2048", n_head=8, n_tok=16, n_kv=2048,
                       n_valid=2048, hd=256, mask_kind="causal_tail",
                       k_outlier_frac=0.05, k_outlier_scale=8.0)
LONG_CONTEXT = Workload("long_context_h32_hd128_t16_kv32768", n_head=32, n_tok=16,
                        n_kv=32768, n_valid=32000, hd=128, mask_kind="pad")

WORKLOADS = [TINY, PI05_ACTION_STEP, H16_HD128_Q16, CAUSAL_TAIL, LONG_CONTEXT]

# Beyond the pages' one KV head: grouped-query decode with 8 KV heads of 4
# query heads each, 4 query tokens (a short speculative-verify window), 4096
# keys, 8 independent sequences per call.
GQA_KV8 = Workload("gqa_h32_kv8_hd128_t4_kv4096_x8", n_head=32, n_tok=4, n_kv=4096,
                   n_valid=4096, hd=128, n_inst=8, n_kv_head=8)
# A speculative-verify step past the pages' 16 tokens: 64 draft tokens checked
# at once against 8192 keys, the last 64 of them the draft tokens themselves
# (causal among them), 32 query heads on 8 KV heads.
SPEC_VERIFY_T64 = Workload("spec_verify_h32_kv8_hd128_t64_kv8192", n_head=32, n_tok=64,
                           n_kv=8192, n_valid=8192, hd=128, n_kv_head=8,
                           mask_kind="causal_tail")
# The prefix-LM prefill attention of the pages: every one of the 968 prefix
# tokens attends over the same 968 keys (row-uniform, pad-only mask), so no
# mask is passed and the padded tail of the 1024-key buffer is excluded by a
# device-side valid count.
PREFILL_PI05 = Workload("prefill_pi05_h8_hd256_t968_kv1024", n_head=8, n_tok=968, n_kv=1024,
                        n_valid=968, hd=256, sigma_kv=0.5, mask_kind="none", dynamic_len=True)
# Plain one-token grouped-query decode (32 query heads on 8 KV heads, 8
# sequences of 4096 keys): each unit has 4 query rows, a quarter of a tile.
GQA_DECODE_T1 = Workload("gqa_decode_h32_kv8_hd128_t1_kv4096_x8", n_head=32, n_tok=1,
                         n_kv=4096, n_valid=4096, hd=128, n_inst=8, n_kv_head=8)
# Head size 80: a vision-encoder attention (16 heads, each its own KV head,
# over 256 patch tokens) for 2 camera views, unmasked.
VISION_HD80 = Workload("vision_mha_h16_hd80_t256_x2", n_head=16, n_tok=256, n_kv=256,
                       n_valid=256, hd=80, n_inst=2, n_kv_head=16, mask_kind="none")
EXTRA_WORKLOADS = [GQA_KV8, GQA_DECODE_T1, SPEC_VERIFY_T64, PREFILL_PI05, VISION_HD80]

BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}


def f16_bits(x: np.ndarray) -> np.ndarray:
    """float array -> binary16 bit patterns (numpy's nearest-even cast)."""
    return np.asarray(x).astype(np.float16).view(np.uint16)


def build_mask(w: Workload) -> np.ndarray:
    """[n_tok, n_kv] f16 bits for the workload's mask kind."""
    m = np.full((w.n_tok, w.n_kv), F16_ZERO, dtype=np.uint16)
    if w.mask_kind in ("zero", "none"):   # "none": an all-zero mask that is not passed
        pass
    elif w.mask_kind == "pad":
        m[:, w.n_valid:] = F16_NEG_INF
    elif w.mask_kind == "causal_tail":
        # the last n_tok keys are the query tokens themselves: token t sees
        # every earlier key and query keys 0..t
        base = w.n_kv - w.n_tok
        for t in range(w.n_tok):
            m[t, base + t + 1:] = F16_NEG_INF
    else:
        raise ValueError(f"unknown mask kind {w.mask_kind!r}")
    return m


def generate(w: Workload, seed: int | None = None) -> dict:
    """Draw every instance of a workload.

    Returns a dict with
      q    [n_inst, n_tok, n_head, hd] float32, or uint16 f16 bits if q_dtype == "f16"
      k, v [n_inst, n_kv, hd] uint16 f16 bits (pad rows zero); with several KV
           heads [n_inst, n_kv_head, n_kv, hd]
      mask [n_inst, n_tok, n_kv] uint16 f16 bits
      outlier_rows [n_inst, n_outliers] int64 (empty when there are none)
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    n_out = int(round(w.k_outlier_frac * w.n_valid))
    if n_out and w.n_kv_head != 1:
        raise ValueError("outlier rows are defined for one KV head only")
    qs, ks, vs, outs = [], [], [], []
    for _ in range(w.n_inst):
        q = (rng.standard_normal((w.n_tok, w.n_head, w.hd)) * w.sigma_q).astype(np.float32)
        if w.q_dtype == "f16":
            q = f16_bits(q)
        heads = () if w.n_kv_head == 1 else (w.n_kv_head,)
        k = np.zeros(heads + (w.n_kv, w.hd), dtype=np.uint16)
        v = np.zeros(heads + (w.n_kv, w.hd), dtype=np.uint16)
        k[..., :w.n_valid, :] = f16_bits(
            rng.standard_normal(heads + (w.n_valid, w.hd)) * w.sigma_kv)
        v[..., :w.n_valid, :] = f16_bits(
            rng.standard_normal(heads + (w.n_valid, w.hd)) * w.sigma_kv)
        rows = np.zeros((0,), dtype=np.int64)
        if n_out:
            rows = np.sort(rng.choice(w.n_valid, size=n_out, replace=False))
            kf = k[rows].view(np.float16).astype(np.float32) * np.float32(w.k_outlier_scale)
            k[rows] = f16_bits(kf)  # x8 is exact in f16 at these magnitudes
        qs.append(q)
        ks.append(k)
        vs.append(v)
        outs.append(rows)
    mask = np.broadcast_to(build_mask(w), (w.n_inst, w.n_tok, w.n_kv)).copy()
    return {"q": np.stack(qs), "k": np.stack(ks), "v": np.stack(vs), "mask": mask,
            "outlier_rows": np.stack(outs)}


def random_case(seed: int, n_head: int, n_tok: int, n_kv: int, hd: int,
                q_dtype: str = "f32", mask_kind: str = "random", sigma: float = 1.0,
                neg_inf_frac: float = 0.2, n_inst: int = 1, n_kv_head: int = 1) -> dict:
    """Small random cases for parity sweeps (ragged shapes, random masks).

    mask_kind: "none" (no mask), "zero", "random" (each entry -inf with
    probability neg_inf_frac, else a finite value in [-2, 2] rounded to f16),
    or "full_row" (random, with token 0's row entirely -inf).
    k and v are [n_inst, n_kv, hd], or [n_inst, n_kv_head, n_kv, hd] when
    n_kv_head > 1.
    """
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((n_inst, n_tok, n_head, hd)) * sigma).astype(np.float32)
    if q_dtype == "f16":
        q = f16_bits(q)
    kv_shape = (n_inst, n_kv, hd) if n_kv_head == 1 else (n_inst, n_kv_head, n_kv, hd)
    k = f16_bits(rng.standard_normal(kv_shape) * sigma)
    v = f16_bits(rng.standard_normal(kv_shape) * sigma)
    mask = None
    if mask_kind == "zero":
        mask = np.zeros((n_inst, n_tok, n_kv), dtype=np.uint16)
    elif mask_kind in ("random", "full_row"):
        vals = f16_bits(rng.uniform(-2.0, 2.0, size=(n_inst, n_tok, n_kv)))
        neg = rng.random((n_inst, n_tok, n_kv)) < neg_inf_frac
        mask = np.where(neg, F16_NEG_INF, vals).astype(np.uint16)
        if mask_kind == "full_row":
            mask[:, 0, :] = F16_NEG_INF
    elif mask_kind != "none":
        raise ValueError(f"unknown mask kind {mask_kind!r}")
    return {"q": q, "k": k, "v": v, "mask": mask}
