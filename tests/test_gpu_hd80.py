"""GPU parity at head size 80 (the three-launch decomposition, whose QK^T
contraction runs over 96 dimensions with the last 16 zero), against the fp64
oracle: decode shapes with masks, several KV heads with f16 queries, a
vision-style unmasked attention of 256 tokens, and the query/KV producer."""
import math

import numpy as np
import pytest

from gqa_decode_attention_fr_amd import workloads as W
from gpu_util import assert_close, errors, oracle_gqa, run_gqa, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_fr_amd as F
    F.binding.load()
    yield


HD80 = [  # n_inst, n_head, n_kv_head, n_tok, n_kv, q dtype, mask kind
    (1, 8, 1, 10, 1000, "f32", "random"),
    (2, 16, 2, 4, 577, "f16", "random"),
    (1, 1, 1, 1, 1, "f32", "none"),
    (1, 16, 16, 256, 256, "f32", "none"),     # vision-style: every token sees every key
    (3, 12, 4, 33, 129, "f32", "full_row"),
]


@pytest.mark.parametrize("shape", HD80, ids=lambda s: "n{}_h{}_g{}_t{}_kv{}_{}_{}".format(*s))
def test_hd80_parity(oracle_mod, shape):
    import gqa_decode_attention_fr_amd as F
    n_inst, n_head, n_kvh, n_tok, n_kv, qd, mk = shape
    hd = 80
    say(f"hd80 {shape}")
    assert F.fr_decode_attn_plan(n_inst * n_kvh, n_head // n_kvh, n_tok, n_kv, hd)["variant"] == 2
    c = W.random_case(HD80.index(shape) + 1100, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind=mk, n_inst=n_inst, n_kv_head=n_kvh)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, q_f16=(qd == "f16"))
    want = oracle_gqa(oracle_mod, c, n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] hd80 {shape} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, str(shape))
    if mk == "full_row":
        assert np.array_equal(got[:, 0], np.zeros_like(got[:, 0]))
