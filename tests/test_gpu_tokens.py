"""GPU parity above the pages' 16 query tokens (up to 64: a speculative-verify
window).  Calls with more than 16 tokens run in 8-wave workgroups, which stage
mask rows for up to 64 tokens; both mask load paths (16-byte direct loads for
aligned rows, register staging otherwise) and both variants are checked
against the fp64 oracle."""
import math

import numpy as np
import pytest

from gqa_decode_attention_fr_amd import workloads as W
from gpu_util import assert_close, errors, oracle_gqa, run_gqa, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
FUSED, DECOMP = 0x2, 0x4
NEG_INF = 0xFC00


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_fr_amd as F
    F.binding.load()
    yield


def causal_tail_mask(n_inst, n_tok, n_kv):
    """The last n_tok keys are the query tokens: token t sees every earlier key
    and query keys 0..t (the verify step of speculative decoding)."""
    m = np.zeros((n_inst, n_tok, n_kv), dtype=np.uint16)
    base = n_kv - n_tok
    for t in range(n_tok):
        m[:, t, base + t + 1:] = NEG_INF
    return m


MANY = [  # n_inst, n_head, n_kv_head, n_tok, n_kv, hd, q dtype, mask kind
    (1, 8, 1, 17, 1000, 256, "f32", "random"),        # 16-byte mask loads
    (1, 8, 1, 32, 2048, 256, "f32", "causal"),
    (2, 4, 1, 64, 4096, 128, "f32", "random"),
    (1, 8, 1, 64, 999, 256, "f32", "random"),         # register-staged mask rows
    (1, 16, 4, 48, 1531, 128, "f16", "random"),
    (3, 2, 1, 33, 333, 64, "f32", "full_row"),
    (1, 32, 8, 64, 8192, 128, "f32", "causal"),       # 256 rows per KV head
    (2, 1, 1, 64, 65, 256, "f32", "none"),
]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", MANY, ids=lambda s: "n{}_h{}_g{}_t{}_kv{}_d{}_{}_{}".format(*s))
def test_many_token_parity(oracle_mod, shape, variant):
    n_inst, n_head, n_kvh, n_tok, n_kv, hd, qd, mk = shape
    say(f"tokens {shape} variant={variant}")
    c = W.random_case(MANY.index(shape) + 900, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind="zero" if mk == "causal" else mk, n_inst=n_inst,
                      n_kv_head=n_kvh)
    if mk == "causal":
        c["mask"] = causal_tail_mask(n_inst, n_tok, n_kv)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant,
                  q_f16=(qd == "f16"))
    want = oracle_gqa(oracle_mod, c, n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] tokens {shape} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, str(shape))
    if mk == "full_row":
        assert np.array_equal(got[:, 0], np.zeros_like(got[:, 0]))


def test_sixty_four_tokens_plan_eight_waves():
    import gqa_decode_attention_fr_amd as F
    assert F.fr_decode_attn_plan(1, 8, 64, 999, 256)["waves"] == 8
    assert F.fr_decode_attn_plan(1, 8, 16, 999, 256)["waves"] == 4


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_spec_verify_workload_full_size(oracle_mod, variant):
    """The measured 64-token verify workload, every element."""
    w = W.SPEC_VERIFY_T64
    say(f"workload {w.name} variant={variant}")
    g = W.generate(w)
    got = run_gqa(g, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant)
    want = oracle_gqa(oracle_mod, g, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd, w.scale,
                      oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] {w.name} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, w.name)


def test_prefill_full_size(oracle_mod):
    """The pages' prefix-LM prefill: 968 query tokens over the same 968 keys of
    a 1024-row buffer, no mask, the padded tail excluded by a device count
    (fused) or by n_kv itself (decomposed); every element against the oracle
    over the valid keys."""
    import gqa_decode_attention_fr_amd as F
    w = W.PREFILL_PI05
    say(f"workload {w.name}")
    g = W.generate(w)
    c = dict(g, mask=None)
    c["k"], c["v"] = g["k"][:, None], g["v"][:, None]
    got = run_gqa(c, w.n_head, 1, w.n_tok, w.n_kv, w.hd, w.scale, kv_len=[w.n_valid])
    cv = dict(c, k=np.ascontiguousarray(c["k"][:, :, :w.n_valid]),
              v=np.ascontiguousarray(c["v"][:, :, :w.n_valid]))
    want = oracle_gqa(oracle_mod, cv, w.n_head, 1, w.n_tok, w.n_valid, w.hd, w.scale,
                      oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] {w.name} fused max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, w.name)
    got_d = run_gqa(cv, w.n_head, 1, w.n_tok, w.n_valid, w.hd, w.scale, flags=DECOMP)
    max_abs, rel = errors(got_d, want)
    print(f"[parity] {w.name} decomposed max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got_d, want, w.name + " decomposed")


def test_gqa_prefill_f16_query(oracle_mod):
    say("gqa prefill f16 Q")
    n_head, n_kvh, n_tok, n_kv, hd, valid = 16, 2, 300, 333, 128, 300
    c = W.random_case(950, n_head, n_tok, n_kv, hd, q_dtype="f16", mask_kind="none",
                      n_kv_head=n_kvh)
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, q_f16=True, kv_len=[valid])
    cv = dict(c, k=np.ascontiguousarray(c["k"][:, :, :valid]),
              v=np.ascontiguousarray(c["v"][:, :, :valid]))
    want = oracle_gqa(oracle_mod, cv, n_head, n_kvh, n_tok, valid, hd, scale, oracle_mod.Q_F16)
    assert_close(got, want, "gqa prefill")


LARGEST = [  # n_inst, n_head, n_kv_head, n_tok, n_kv, hd, q dtype, mask kind
    (1, 1, 1, 16384, 200, 64, "f32", "none"),      # the unmasked token limit
    (1, 2, 2, 16384, 77, 128, "f16", "none"),      # ... with two KV heads, one query head each
    (1, 1024, 1, 2, 300, 128, "f32", "random"),    # the head limit, masked
    (1, 1024, 8, 16, 130, 64, "f32", "random"),    # the head limit, 128 query heads per KV head
]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", LARGEST, ids=lambda s: "n{}_h{}_g{}_t{}_kv{}_d{}_{}_{}".format(*s))
def test_largest_accepted_row_counts(oracle_mod, shape, variant):
    """The largest query-token count (no mask) and head count the library
    accepts, element by element against the oracle."""
    import gqa_decode_attention_fr_amd as F
    n_inst, n_head, n_kvh, n_tok, n_kv, hd, qd, mk = shape
    assert n_tok <= (F.FR_MAX_TOKENS_UNMASKED if mk == "none" else F.FR_MAX_TOKENS)
    assert n_head <= F.FR_MAX_HEADS
    say(f"largest {shape} variant={variant}")
    c = W.random_case(LARGEST.index(shape) + 950, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind=mk, n_inst=n_inst, n_kv_head=n_kvh)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant,
                  q_f16=(qd == "f16"))
    want = oracle_gqa(oracle_mod, c, n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] largest {shape} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, str(shape))
