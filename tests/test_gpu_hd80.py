"""GPU parity at head size 80, against the fp64 oracle, in both variants: the
fused kernel runs it in the hd-128 layout (query columns past 80 zero, row
granules past 80 repeating in-row ones, output columns past 80 not stored),
the decomposition over a 96-wide QK^T.  Decode shapes with masks, several KV
heads with f16 queries, a vision-style unmasked attention of 256 tokens, a
single key, fully masked rows, and device key counts (fused)."""
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


FUSED, DECOMP = 0x2, 0x4


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", HD80, ids=lambda s: "n{}_h{}_g{}_t{}_kv{}_{}_{}".format(*s))
def test_hd80_parity(oracle_mod, shape, variant):
    n_inst, n_head, n_kvh, n_tok, n_kv, qd, mk = shape
    hd = 80
    say(f"hd80 {shape} variant={variant}")
    c = W.random_case(HD80.index(shape) + 1100, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind=mk, n_inst=n_inst, n_kv_head=n_kvh)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant, q_f16=(qd == "f16"))
    want = oracle_gqa(oracle_mod, c, n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] hd80 {shape} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, str(shape))
    if mk == "full_row":
        assert np.array_equal(got[:, 0], np.zeros_like(got[:, 0]))


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_hd80_device_key_counts(oracle_mod, variant):
    """Head size 80 with device key counts, both variants (the padded tail of
    K/V set to NaN on the GPU side: a load of it would poison the output)."""
    n_inst, n_head, n_kvh, n_tok, n_kv, hd = 3, 16, 2, 5, 700, 80
    lens = [700, 333, 0]
    say("hd80 kv_len")
    c = W.random_case(1190, n_head, n_tok, n_kv, hd, mask_kind="random", n_inst=n_inst,
                      n_kv_head=n_kvh)
    mask = c["mask"].copy()
    kg, vg = c["k"].copy(), c["v"].copy()
    for i, L in enumerate(lens):
        mask[i, :, L:] = 0xFC00
        kg[i, :, L:] = 0x7E00
        vg[i, :, L:] = 0x7E00
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant, kv_len=lens,
                  kv_override=(kg, vg))
    want = oracle_gqa(oracle_mod, dict(c, mask=mask), n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F32)
    assert_close(got, want, "hd80 kv_len")
    assert np.array_equal(got[2], np.zeros_like(got[2]))


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_vision_workload_full_size(oracle_mod, variant):
    w = W.VISION_HD80
    say(f"workload {w.name} variant={variant}")
    g = W.generate(w)
    c = dict(g, mask=None)
    got = run_gqa(c, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant)
    want = oracle_gqa(oracle_mod, c, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd, w.scale,
                      oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] {w.name} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, w.name)
