"""Brute-force decode attention in pure Python (tiny inputs only).

TEST INFRASTRUCTURE ONLY: it exists to pin the C oracle.  It uses neither
numpy arithmetic nor the C oracle's helpers: binary16 values are decoded with
the standard library's ``struct`` half-precision format, sums use
``math.fsum`` (correctly rounded), and the softmax is the textbook
``exp(s_j) / sum_i exp(s_i)`` with no max subtraction, which is only safe for
the small logits used in the tests.

Same operation as the oracle: FlashRT pull request #185 ("feat(structures):
ggml host adapter -- llama.cpp distribution for pi0.5 on Thor (SM110)"), the
decomposed decode attention commit, with t-major rows from the GQA-collapse
commit.
"""
from __future__ import annotations

import math
import struct


def half_bits_to_float(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]


def float_to_half_bits(x: float) -> int:
    """Python's own binary16 packing (round to nearest even)."""
    return struct.unpack("<H", struct.pack("<e", x))[0]


def decode_attn(q, k, v, mask, n_head, n_tok, n_kv, hd, scale, q_is_f16=False, n_kv_head=1):
    """q: flat list (len n_tok*n_head*hd) of floats, or of f16 bits if q_is_f16;
    k, v: flat lists of f16 bits (n_kv_head*n_kv*hd; query head h reads KV head
    h // (n_head // n_kv_head)); mask: flat list of f16 bits (n_tok*n_kv) or
    None.  Returns a flat list in [n_tok][n_head][hd] order."""
    qf = [half_bits_to_float(x) for x in q] if q_is_f16 else [float(x) for x in q]
    kf = [half_bits_to_float(x) for x in k]
    vf = [half_bits_to_float(x) for x in v]
    out = []
    for t in range(n_tok):
        for h in range(n_head):
            r = t * n_head + h
            qr = qf[r * hd:(r + 1) * hd]
            kv0 = (h // (n_head // n_kv_head)) * n_kv * hd   # this head's K/V rows
            weights = []
            for j in range(n_kv):
                mj = 0.0 if mask is None else half_bits_to_float(mask[t * n_kv + j])
                if mj == -math.inf:
                    weights.append(0.0)
                    continue
                dot = math.fsum(qr[e] * kf[kv0 + j * hd + e] for e in range(hd))
                weights.append(math.exp(scale * dot + mj))
            total = math.fsum(weights)
            for d in range(hd):
                if total == 0.0:
                    out.append(0.0)
                else:
                    out.append(math.fsum(weights[j] * vf[kv0 + j * hd + d]
                                         for j in range(n_kv)) / total)
    return out
