"""Pins for the fp64 oracle: checks that do not go through the oracle's own
arithmetic (exhaustive binary16 conversions against numpy and the standard
library, pure-Python brute force, hand-worked cases, closed forms, invariants,
and an independent library attention).  CPU only."""
import json
import math
import os
import struct

import numpy as np
import pytest

from oracle import brute
from gqa_decode_attention_fr_amd.workloads import f16_bits, random_case

HERE = os.path.dirname(os.path.abspath(__file__))
NEG_INF = 0xFC00


def _f16(x):
    return f16_bits(np.asarray(x, dtype=np.float64))


# --------------------------------------------------------------------------- conversions

def test_f16_decode_exhaustive(oracle_mod):
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle_mod.f16_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0
    # and agree with the standard library's own half-precision decoder
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x7C00, 0xFC00, 0xC000):
        assert got[b] == struct.unpack("<e", struct.pack("<H", b))[0]


def _rne_test_values():
    rng = np.random.default_rng(123)
    vals = [0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.996, 65520.0, 65536.0, 1e10,
            2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
            1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11)]
    f16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.arange(1, 0x7C01, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (f16 + nxt) / 2.0  # exact ties (representable in f32)
    vals = np.concatenate([np.array(vals), f16, -f16, mids, -mids,
                           np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(0)),
                           rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000)])
    return vals.astype(np.float32)


def test_f32_to_f16_rne_matches_numpy_and_stdlib(oracle_mod):
    x = _rne_test_values()
    got = oracle_mod.f32_to_f16_rne(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    # the standard library's packer (rounds to nearest even; raises on overflow)
    for xv, g in zip(x[:4000:7], got[:4000:7]):
        if abs(float(xv)) < 65520.0:
            assert g == struct.unpack("<H", struct.pack("<e", float(xv)))[0]
    nan = oracle_mod.f32_to_f16_rne(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_f16_row_copy_matches_numpy_and_the_element_rounding(oracle_mod):
    """The batched copy rounds each element on its own: numpy's nearest-even
    cast (an independent implementation) and the element-wise oracle agree."""
    x = _rne_test_values()
    got = oracle_mod.f16_copy(x)
    with np.errstate(over="ignore"):
        assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    assert np.array_equal(got[:5000], oracle_mod.f32_to_f16_rne(x[:5000]))
    assert oracle_mod.f16_copy(np.zeros(0, dtype=np.float32)).size == 0


# --------------------------------------------------------------------------- brute force

def _oracle_case(oracle_mod, c, n_head, n_tok, n_kv, hd, scale, q_kind):
    m = None if c["mask"] is None else c["mask"][0]
    return oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], m, n_head, n_tok, n_kv,
                                  hd, scale, q_kind=q_kind)


@pytest.mark.parametrize("seed", range(24))
def test_oracle_matches_brute_force(oracle_mod, seed):
    rng = np.random.default_rng(1000 + seed)
    n_head, n_tok = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    n_kv, hd = int(rng.integers(1, 7)), int(rng.integers(1, 9))
    q_kind = [oracle_mod.Q_F32, oracle_mod.Q_F16, oracle_mod.Q_F32_ROUND_F16][seed % 3]
    mask_kind = ["random", "none", "full_row", "zero"][seed % 4]
    c = random_case(seed, n_head, n_tok, n_kv, hd,
                    q_dtype="f16" if q_kind == oracle_mod.Q_F16 else "f32",
                    mask_kind=mask_kind, sigma=0.7, neg_inf_frac=0.3)
    if c["mask"] is not None and n_kv > 1 and n_tok > 1:
        # one token row sees exactly one key
        c["mask"][0, n_tok - 1, :] = NEG_INF
        c["mask"][0, n_tok - 1, n_kv // 2] = 0
    scale = float(np.float32(1.0 / math.sqrt(hd)))
    got = _oracle_case(oracle_mod, c, n_head, n_tok, n_kv, hd, scale, q_kind).reshape(-1)
    q = c["q"][0].reshape(-1).tolist()
    if q_kind == oracle_mod.Q_F32_ROUND_F16:
        q = [brute.half_bits_to_float(brute.float_to_half_bits(x)) for x in q]
    want = brute.decode_attn(q, c["k"][0].reshape(-1).tolist(), c["v"][0].reshape(-1).tolist(),
                             None if c["mask"] is None else c["mask"][0].reshape(-1).tolist(),
                             n_head, n_tok, n_kv, hd, scale,
                             q_is_f16=(q_kind == oracle_mod.Q_F16))
    want = np.array(want)
    tol = 1e-12 * max(1.0, float(np.max(np.abs(want))))
    assert np.max(np.abs(got - want)) <= tol


@pytest.mark.parametrize("seed", range(12))
def test_gqa_oracle_matches_brute_force(oracle_mod, seed):
    """Several KV heads: query head h reads KV head h // (n_head // n_kv_head)."""
    rng = np.random.default_rng(3000 + seed)
    n_kv_head, group = int(rng.integers(2, 4)), int(rng.integers(1, 3))
    n_head, n_tok = n_kv_head * group, int(rng.integers(1, 4))
    n_kv, hd = int(rng.integers(1, 6)), int(rng.integers(1, 7))
    q_kind = [oracle_mod.Q_F32, oracle_mod.Q_F16][seed % 2]
    c = random_case(seed, n_head, n_tok, n_kv, hd,
                    q_dtype="f16" if q_kind == oracle_mod.Q_F16 else "f32",
                    mask_kind=["random", "none", "full_row"][seed % 3], sigma=0.7,
                    neg_inf_frac=0.3, n_kv_head=n_kv_head)
    scale = float(np.float32(1.0 / math.sqrt(hd)))
    m = None if c["mask"] is None else c["mask"][0]
    got = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], m, n_head, n_tok, n_kv, hd,
                                 scale, q_kind=q_kind, n_kv_head=n_kv_head).reshape(-1)
    want = np.array(brute.decode_attn(c["q"][0].reshape(-1).tolist(),
                                      c["k"][0].reshape(-1).tolist(),
                                      c["v"][0].reshape(-1).tolist(),
                                      None if m is None else m.reshape(-1).tolist(),
                                      n_head, n_tok, n_kv, hd, scale,
                                      q_is_f16=(q_kind == oracle_mod.Q_F16),
                                      n_kv_head=n_kv_head))
    tol = 1e-12 * max(1.0, float(np.max(np.abs(want))))
    assert np.max(np.abs(got - want)) <= tol


def test_gqa_single_key_selects_each_groups_value_row(oracle_mod):
    """With one key, head h's output is row 0 of KV head h // G exactly: pins
    the head-to-group mapping (a transposed or off-by-one mapping picks the
    wrong row)."""
    n_head, n_kvh, n_tok, hd = 12, 4, 3, 8
    c = random_case(41, n_head, n_tok, 1, hd, mask_kind="none", n_kv_head=n_kvh)
    out = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], None, n_head, n_tok, 1, hd,
                                 0.3, n_kv_head=n_kvh)
    vals = c["v"][0][:, 0, :].view(np.float16).astype(np.float64)     # [n_kvh, hd]
    for h in range(n_head):
        assert np.array_equal(out[:, h, :], np.broadcast_to(vals[h // (n_head // n_kvh)],
                                                             (n_tok, hd)))


def test_gqa_identical_keys_give_each_groups_mean(oracle_mod):
    """Identical keys inside each KV head: every head of a group outputs the
    mean of that group's value rows (the softmax is uniform)."""
    n_head, n_kvh, n_tok, n_kv, hd = 6, 3, 2, 7, 4
    c = random_case(43, n_head, n_tok, n_kv, hd, mask_kind="none", n_kv_head=n_kvh)
    k = c["k"][0].copy()
    k[:, :, :] = k[:, :1, :]
    out = oracle_mod.decode_attn(c["q"][0], k, c["v"][0], None, n_head, n_tok, n_kv, hd, 0.5,
                                 n_kv_head=n_kvh)
    v = c["v"][0].view(np.float16).astype(np.float64)
    for h in range(n_head):
        want = np.array([math.fsum(v[h // 2, :, d]) / n_kv for d in range(hd)])
        np.testing.assert_allclose(out[:, h, :], np.broadcast_to(want, (n_tok, hd)),
                                   rtol=1e-14, atol=1e-15)


def test_hand_worked_cases(oracle_mod):
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        mask = None
        if c["mask"] is not None:
            mask = _f16([-np.inf if m == "-inf" else m for m in c["mask"]])
        out = oracle_mod.decode_attn(np.array(c["q"], dtype=np.float32), _f16(c["k"]),
                                     _f16(c["v"]), mask, c["n_head"], c["n_tok"], c["n_kv"],
                                     c["hd"], c["scale"])
        np.testing.assert_allclose(out.reshape(-1), c["expected"], rtol=1e-15, atol=0,
                                   err_msg=c["name"])


# --------------------------------------------------------------------------- closed forms

def test_single_key_returns_v_row(oracle_mod):
    c = random_case(5, 3, 4, 1, 16, mask_kind="none")
    out = _oracle_case(oracle_mod, c, 3, 4, 1, 16, 0.25, oracle_mod.Q_F32)
    v0 = c["v"][0, 0].view(np.float16).astype(np.float64)
    assert np.array_equal(out, np.broadcast_to(v0, out.shape))


def test_single_unmasked_key_returns_that_row(oracle_mod):
    c = random_case(6, 2, 3, 9, 8, mask_kind="zero")
    mask = np.full((3, 9), NEG_INF, dtype=np.uint16)
    for t in range(3):
        mask[t, 2 * t + 1] = 0
    out = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], mask, 2, 3, 9, 8, 0.5)
    vf = c["v"][0].view(np.float16).astype(np.float64)
    for t in range(3):
        assert np.array_equal(out[t], np.broadcast_to(vf[2 * t + 1], (2, 8)))


def test_two_keys_sigmoid_closed_form(oracle_mod):
    # q = a*e0, K_j = b_j*e0: logits are exactly scale*a*b_j (all values exact in f16/f32)
    hd = 4
    a, b0, b1, scale = 1.5, 0.75, -1.25, 0.5
    q = np.zeros((1, 1, hd), dtype=np.float32)
    q[0, 0, 0] = a
    k = np.zeros((2, hd))
    k[0, 0], k[1, 0] = b0, b1
    v = np.array([[1.0, -2.0, 0.5, 3.0], [4.0, 0.25, -1.0, 2.0]])
    out = oracle_mod.decode_attn(q, _f16(k), _f16(v), None, 1, 1, 2, hd, scale)
    s0, s1 = scale * a * b0, scale * a * b1
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(out[0, 0], w0 * v[0] + w1 * v[1], rtol=1e-15, atol=1e-15)


def test_zero_scale_gives_mean_of_v(oracle_mod):
    c = random_case(7, 4, 2, 37, 32, mask_kind="zero")
    out = _oracle_case(oracle_mod, c, 4, 2, 37, 32, 0.0, oracle_mod.Q_F32)
    mean = c["v"][0].view(np.float16).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=1e-13, atol=1e-15)


def test_identical_keys_give_mean_of_visible_values(oracle_mod):
    rng = np.random.default_rng(8)
    n_kv, hd = 50, 16
    krow = _f16(rng.standard_normal(hd))
    k = np.broadcast_to(krow, (n_kv, hd)).copy()
    c = random_case(8, 3, 2, n_kv, hd)
    mask = np.zeros((2, n_kv), dtype=np.uint16)
    mask[0, ::3] = NEG_INF
    mask[1, 40:] = NEG_INF
    out = oracle_mod.decode_attn(c["q"][0], k, c["v"][0], mask, 3, 2, n_kv, hd, 0.3)
    vf = c["v"][0].view(np.float16).astype(np.float64)
    for t in range(2):
        vis = mask[t] == 0
        np.testing.assert_allclose(out[t], np.broadcast_to(vf[vis].mean(axis=0), (3, hd)),
                                   rtol=1e-13, atol=1e-15)


def test_rows_normalise_to_one(oracle_mod):
    c = random_case(9, 5, 3, 200, 64, mask_kind="random", sigma=2.0)
    ones = np.full_like(c["v"][0], 0x3C00)
    out = oracle_mod.decode_attn(c["q"][0], c["k"][0], ones, c["mask"][0], 5, 3, 200, 64, 0.125)
    assert np.max(np.abs(out - 1.0)) <= 1e-14


def test_fully_masked_row_is_zero(oracle_mod):
    c = random_case(10, 2, 3, 20, 8, mask_kind="full_row")
    out = _oracle_case(oracle_mod, c, 2, 3, 20, 8, 0.5, oracle_mod.Q_F32)
    assert np.array_equal(out[0], np.zeros((2, 8)))
    assert np.all(np.abs(out[1:]) > 0)


# --------------------------------------------------------------------------- invariants

def test_masked_keys_contribute_exactly_zero(oracle_mod):
    c = random_case(11, 4, 3, 40, 32, mask_kind="random")
    mask = c["mask"][0].copy()
    dead = [3, 17, 29, 39]
    mask[:, dead] = NEG_INF
    k2, v2 = c["k"][0].copy(), c["v"][0].copy()
    k2[dead] = _f16(np.full((len(dead), 32), 60000.0))
    v2[dead] = _f16(np.full((len(dead), 32), -60000.0))
    a = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], mask, 4, 3, 40, 32, 0.2)
    b = oracle_mod.decode_attn(c["q"][0], k2, v2, mask, 4, 3, 40, 32, 0.2)
    assert np.array_equal(a, b)


def test_collapsed_gqa_equals_per_head_batched(oracle_mod):
    """The GQA-collapse commit of FlashRT pull request #185 says one contraction
    over all n_head*n_tok t-major rows is numerically identical to the per-head
    batched form; in fp64 with the same per-row summation order it is bitwise."""
    n_head, n_tok, n_kv, hd = 6, 5, 70, 24
    c = random_case(12, n_head, n_tok, n_kv, hd, mask_kind="random")
    full = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], c["mask"][0],
                                  n_head, n_tok, n_kv, hd, 0.2)
    for h in range(n_head):
        qh = np.ascontiguousarray(c["q"][0][:, h:h + 1, :])
        one = oracle_mod.decode_attn(qh, c["k"][0], c["v"][0], c["mask"][0],
                                     1, n_tok, n_kv, hd, 0.2)
        assert np.array_equal(one[:, 0, :], full[:, h, :])


def test_mask_row_shift_invariance(oracle_mod):
    c = random_case(13, 3, 4, 64, 16, mask_kind="zero")
    rng = np.random.default_rng(13)
    base = rng.integers(-3, 3, size=(4, 64)).astype(np.float64)
    base[rng.random((4, 64)) < 0.25] = -np.inf
    shifted = base.copy()
    shifted[2] += 5.0  # exact in f16; -inf stays -inf
    a = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], _f16(base), 3, 4, 64, 16, 0.25)
    b = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], _f16(shifted), 3, 4, 64, 16, 0.25)
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-14)


def test_key_permutation_invariance(oracle_mod):
    c = random_case(14, 3, 2, 90, 16, mask_kind="random")
    perm = np.random.default_rng(14).permutation(90)
    a = _oracle_case(oracle_mod, c, 3, 2, 90, 16, 0.25, oracle_mod.Q_F32)
    b = oracle_mod.decode_attn(c["q"][0], c["k"][0][perm], c["v"][0][perm],
                               c["mask"][0][:, perm], 3, 2, 90, 16, 0.25)
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-14)


def test_linear_in_v(oracle_mod):
    rng = np.random.default_rng(15)
    c = random_case(15, 2, 3, 33, 8, mask_kind="random")
    v1 = rng.integers(-8, 8, size=(33, 8)).astype(np.float64)
    v2 = rng.integers(-8, 8, size=(33, 8)).astype(np.float64)
    args = (c["q"][0], c["k"][0])
    o1 = oracle_mod.decode_attn(*args, _f16(v1), c["mask"][0], 2, 3, 33, 8, 0.4)
    o2 = oracle_mod.decode_attn(*args, _f16(v2), c["mask"][0], 2, 3, 33, 8, 0.4)
    o12 = oracle_mod.decode_attn(*args, _f16(v1 + v2), c["mask"][0], 2, 3, 33, 8, 0.4)
    o2x = oracle_mod.decode_attn(*args, _f16(2 * v1), c["mask"][0], 2, 3, 33, 8, 0.4)
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-13, atol=1e-13)
    assert np.array_equal(o2x, 2 * o1)


def test_thread_count_does_not_change_bits(oracle_mod):
    c = random_case(16, 8, 4, 300, 64, mask_kind="random")
    a = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], c["mask"][0], 8, 4, 300, 64,
                               0.125, threads=1)
    b = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], c["mask"][0], 8, 4, 300, 64,
                               0.125, threads=4)
    assert np.array_equal(a, b)


def test_q16_and_rounded_f32_query_agree(oracle_mod):
    """The pages' f16 Q handoff rounds from the same f32 values the gather
    reads, so f32 input rounded to f16 equals pre-rounded f16 input."""
    c = random_case(17, 4, 4, 50, 32, mask_kind="random")
    q16 = f16_bits(c["q"][0])
    a = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], c["mask"][0], 4, 4, 50, 32, 0.2,
                               q_kind=oracle_mod.Q_F32_ROUND_F16)
    b = oracle_mod.decode_attn(q16, c["k"][0], c["v"][0], c["mask"][0], 4, 4, 50, 32, 0.2,
                               q_kind=oracle_mod.Q_F16)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- library cross-check

def test_gqa_matches_torch_sdpa_float64(oracle_mod):
    torch = pytest.importorskip("torch")
    n_head, n_kvh, n_tok, n_kv, hd = 8, 2, 5, 131, 32
    c = random_case(77, n_head, n_tok, n_kv, hd, mask_kind="random", neg_inf_frac=0.1,
                    n_kv_head=n_kvh)
    scale = 0.2
    out = oracle_mod.decode_attn(c["q"][0], c["k"][0], c["v"][0], c["mask"][0], n_head, n_tok,
                                 n_kv, hd, scale, n_kv_head=n_kvh)
    q = torch.from_numpy(c["q"][0].astype(np.float64)).permute(1, 0, 2)       # [h, t, d]
    k = torch.from_numpy(c["k"][0].view(np.float16).astype(np.float64))      # [kvh, kv, d]
    v = torch.from_numpy(c["v"][0].view(np.float16).astype(np.float64))
    k = k.repeat_interleave(n_head // n_kvh, dim=0)                          # heads of a group
    v = v.repeat_interleave(n_head // n_kvh, dim=0)
    m = torch.from_numpy(c["mask"][0].view(np.float16).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), attn_mask=m, scale=scale)[0]
    ref = ref.permute(1, 0, 2).numpy()
    finite = np.isfinite(ref).all(axis=(1, 2))
    np.testing.assert_allclose(out[finite], ref[finite], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_matches_torch_sdpa_float64(oracle_mod, seed):
    torch = pytest.importorskip("torch")
    n_head, n_tok, n_kv, hd = 8, 6, 257, 64
    c = random_case(200 + seed, n_head, n_tok, n_kv, hd, mask_kind="random", neg_inf_frac=0.1)
    scale = 0.125
    out = _oracle_case(oracle_mod, c, n_head, n_tok, n_kv, hd, scale, oracle_mod.Q_F32)
    q = torch.from_numpy(c["q"][0].astype(np.float64)).permute(1, 0, 2)       # [h, t, d]
    k = torch.from_numpy(c["k"][0].view(np.float16).astype(np.float64))
    v = torch.from_numpy(c["v"][0].view(np.float16).astype(np.float64))
    k = k.unsqueeze(0).expand(n_head, n_kv, hd)
    v = v.unsqueeze(0).expand(n_head, n_kv, hd)
    m = torch.from_numpy(c["mask"][0].view(np.float16).astype(np.float64))   # [t, kv]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), attn_mask=m, scale=scale)[0]
    ref = ref.permute(1, 0, 2).numpy()
    finite = np.isfinite(ref).all(axis=(1, 2))
    np.testing.assert_allclose(out[finite], ref[finite], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- qkv_post (RoPE)

def _qkv_case(seed, n_head, n_kvh, n_tok, hd):
    rng = np.random.default_rng(seed)
    qkv = rng.standard_normal((n_tok, (n_head + 2 * n_kvh) * hd)).astype(np.float32)
    pos = rng.integers(0, 5000, n_tok).astype(np.int32)
    return qkv, pos


def test_rope_matches_complex_rotation(oracle_mod):
    """NeoX RoPE is pair (i, i + hd/2) as one complex number times
    exp(i * p * base^(-2i/hd)): numpy's complex arithmetic, not the oracle's
    cos/sin expansion.  A wrong sign, pairing or frequency fails here."""
    n_head, n_kvh, n_tok, hd, base, s = 3, 1, 4, 16, 10000.0, 0.37
    qkv, pos = _qkv_case(11, n_head, n_kvh, n_tok, hd)
    q, k, v = oracle_mod.qkv_post(qkv, pos, n_head, n_kvh, n_tok, hd, base, s)
    half = hd // 2
    freq = base ** (-2.0 * np.arange(half) / hd)
    x = qkv.astype(np.float64).reshape(n_tok, n_head + 2 * n_kvh, hd)
    rot = np.exp(1j * pos[:, None, None].astype(np.float64) * freq[None, None, :])
    zq = (x[:, :n_head, :half] + 1j * x[:, :n_head, half:]) * rot * s
    zk = (x[:, n_head:n_head + n_kvh, :half] + 1j * x[:, n_head:n_head + n_kvh, half:]) * rot
    np.testing.assert_allclose(q, np.concatenate([zq.real, zq.imag], -1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, np.concatenate([zk.real, zk.imag], -1).transpose(1, 0, 2),
                               rtol=0, atol=1e-12)
    assert np.array_equal(v, x[:, n_head + n_kvh:, :].transpose(1, 0, 2))


def test_rope_position_zero_is_identity(oracle_mod):
    n_head, n_kvh, n_tok, hd = 4, 2, 3, 8
    qkv, _ = _qkv_case(12, n_head, n_kvh, n_tok, hd)
    q, k, v = oracle_mod.qkv_post(qkv, np.zeros(n_tok, np.int32), n_head, n_kvh, n_tok, hd,
                                  10000.0, 0.5)
    x = qkv.astype(np.float64).reshape(n_tok, n_head + 2 * n_kvh, hd)
    assert np.array_equal(q, x[:, :n_head] * 0.5)
    assert np.array_equal(k, x[:, n_head:n_head + n_kvh].transpose(1, 0, 2))


def test_rope_scores_depend_only_on_relative_position(oracle_mod):
    """<rope(q, m), rope(k, n)> is a function of m - n: shifting both
    positions leaves every query-key score unchanged."""
    n_head, n_kvh, n_tok, hd = 2, 1, 5, 32
    qkv, pos = _qkv_case(13, n_head, n_kvh, n_tok, hd)
    q0, k0, _ = oracle_mod.qkv_post(qkv, pos, n_head, n_kvh, n_tok, hd, 10000.0, 1.0)
    q1, k1, _ = oracle_mod.qkv_post(qkv, pos + 777, n_head, n_kvh, n_tok, hd, 10000.0, 1.0)
    s0 = np.einsum("thd,usd->thus", q0, k0.transpose(1, 0, 2))
    s1 = np.einsum("thd,usd->thus", q1, k1.transpose(1, 0, 2))
    np.testing.assert_allclose(s0, s1, rtol=0, atol=1e-9)
    # and each rotated pair keeps its length
    x = qkv.astype(np.float64).reshape(n_tok, n_head + 2 * n_kvh, hd)[:, :n_head]
    h = hd // 2
    np.testing.assert_allclose(q0[..., :h] ** 2 + q0[..., h:] ** 2,
                               x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-12)


def _closed_form(expr: str) -> float:
    """Evaluates a hand-derived closed form: numbers, + - * and cos/sin only."""
    import re
    assert re.fullmatch(r"[0-9.\s+\-*()cosin]*", expr), expr
    return float(eval(expr, {"__builtins__": {}}, {"cos": math.cos, "sin": math.sin}))


def test_rope_hand_derived_cases(oracle_mod):
    """The RoPE frequency schedule and the NeoX pairing against hand-derived
    closed forms (tests/golden/rope_neox_cases.json): exact angles at small
    positions, each output a cos/sin expression written from the definition."""
    with open(os.path.join(HERE, "golden", "rope_neox_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        qkv = np.array(c["qkv"], dtype=np.float32)
        q, k, v = oracle_mod.qkv_post(qkv, np.array(c["pos"], dtype=np.int32), c["n_head"],
                                      c["n_kv_head"], c["n_tok"], c["hd"], c["base"],
                                      c["q_scale"])
        for name, got in (("q", q), ("k", k), ("v", v)):
            want = np.vectorize(_closed_form, otypes=[np.float64])(np.array(c[name], dtype=object))
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15,
                                       err_msg=f"{c['name']} {name}")

