"""A seeded random sweep of the whole window against the fp64 oracle: head
sizes 64/80/128/256, 1 to 8 KV heads with 1 to 16 query heads each, 1 to 64
masked or up to 299 unmasked query tokens, 1 to 2999 keys, f32 and f16
queries, every mask kind, padded KV-head strides, device key counts (with the
hidden K/V rows set to NaN), and both variants."""
import math

import numpy as np
import pytest

from gqa_decode_attention_fr_amd import workloads as W
from gpu_util import assert_close, oracle_gqa, run_gqa, say
from test_gpu_gqa import _hide_past

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
N_CASES = 150


def _cases():
    rng = np.random.default_rng(20251202)
    out = []
    while len(out) < N_CASES:
        hd = int(rng.choice([64, 80, 128, 256]))
        n_kvh = int(rng.choice([1, 1, 2, 3, 4, 8]))
        grp = int(rng.choice([1, 2, 4, 5, 7, 8, 16]))
        mk = str(rng.choice(["random", "zero", "none", "full_row", "random"]))
        n_tok = int(rng.integers(1, 65)) if mk != "none" else int(rng.integers(1, 300))
        if rng.random() < 0.5:
            n_tok = min(n_tok, 16)
        n_kv = int(rng.integers(1, 3000))
        n_inst = int(rng.integers(1, 4))
        qd = str(rng.choice(["f32", "f16"]))
        variant = int(rng.choice([0x2, 0x4, 0x0]))      # fused, decomposed, planner's choice
        lens = None
        if rng.random() < 0.3:
            lens = [int(x) for x in rng.integers(-3, n_kv + 5, size=n_inst)]
        pad = int(rng.choice([0, 0, 8, 56]))
        if n_inst * n_kvh * grp * n_tok * n_kv > 40_000_000:   # keeps the oracle fast
            continue
        out.append((len(out), n_inst, n_kvh * grp, n_kvh, n_tok, n_kv, hd, qd, mk, variant, pad,
                    lens))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_sweep(oracle_mod, case):
    idx, n_inst, n_head, n_kvh, n_tok, n_kv, hd, qd, mk, variant, pad, lens = case
    say(f"sweep {case}")
    c = W.random_case(20_000 + idx, n_head, n_tok, n_kv, hd, q_dtype=qd, mask_kind=mk,
                      n_inst=n_inst, n_kv_head=n_kvh)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    seen, override = (c, None) if lens is None else _hide_past(c, lens, n_kv)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant,
                  q_f16=(qd == "f16"), pad_rows=pad, kv_len=lens, kv_override=override)
    want = oracle_gqa(oracle_mod, seen, n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    assert_close(got, want, str(case))
