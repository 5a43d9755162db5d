"""GPU parity of the query/KV producer (fr_qkv_post: NeoX RoPE, query scale,
f16 rows) against the fp64 oracle, and of the chain it feeds: its f16 query
rows and KV cache through fr_decode_attn_q16 against the oracle attention.

Rounding criterion.  The kernel rotates in fp32 and rounds to f16; the oracle
value is exact to fp64.  An f16 output must equal the oracle value rounded to
nearest-even, except where the oracle value lies within the fp32 evaluation
error of the midpoint between two f16 neighbours: there either neighbour is a
faithful result.  The bound used, 8 * 2^-24 * (|x_i| + |x_{i+hd/2}|) * |scale|,
covers the rounding of cos/sin to fp32, two products, a sum and the scale."""
import math

import numpy as np
import pytest

from gpu_util import MAX_ABS, REL_L2, assert_close, errors, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
CANARY = 0x5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_fr_amd as F
    F.binding.load()
    yield


def check_rounding(got_bits, exact, bound, what):
    want = exact.astype(np.float16)
    got = got_bits.view(np.float16)
    bad = np.nonzero(got.view(np.uint16) != want.view(np.uint16))
    if bad[0].size == 0:
        return 0
    g = got[bad].astype(np.float64)
    w = want[bad].astype(np.float64)
    e = exact[bad]
    # neighbours in f16, and the exact value within the bound of their midpoint
    step = np.nextafter(want[bad], got[bad]).astype(np.float64)
    assert np.array_equal(step, g), f"{what}: an output is not a neighbour of the nearest f16"
    assert (np.abs(e - (g + w) / 2) <= bound[bad]).all(), f"{what}: rounding decision differs"
    return bad[0].size


def pair_bound(x, scale):
    """Per-element bound for rotated heads x [..., hd] (see the module text)."""
    h = x.shape[-1] // 2
    b = 8 * 2.0 ** -24 * (np.abs(x[..., :h]) + np.abs(x[..., h:])) * abs(scale)
    return np.concatenate([b, b], -1).astype(np.float64)


def run_qkv(qkv, pos, n_head, n_kvh, hd, capacity, base, q_scale, cache_fill=CANARY):
    import gqa_decode_attention_fr_amd as F
    n_inst, n_tok = qkv.shape[0], qkv.shape[1]
    q_d = torch.from_numpy(qkv).cuda()
    p_d = torch.from_numpy(pos).cuda()
    q16 = torch.zeros((n_inst, n_tok, n_head, hd), dtype=torch.int16, device="cuda")
    kc = torch.full((n_inst, n_kvh, capacity, hd), cache_fill, dtype=torch.int16, device="cuda")
    vc = torch.full_like(kc, cache_fill)
    F.fr_qkv_post(q_d, p_d, q16, kc, vc, n_inst, qkv[0].size, n_tok, n_tok * n_head * hd,
                  n_kvh * capacity * hd, capacity * hd, n_head, n_kvh, n_tok, hd, capacity,
                  base, q_scale)
    torch.cuda.synchronize()
    return (q16.cpu().numpy().view(np.uint16), kc.cpu().numpy().view(np.uint16),
            vc.cpu().numpy().view(np.uint16))


CASES = [  # n_inst, n_head, n_kv_head, n_tok, hd, capacity, base, q_scale
    (18, 8, 1, 10, 256, 1024, 10000.0, 0.0625),     # the pi0.5 step, as benchmarked
    (1, 32, 8, 4, 128, 40000, 500000.0, 1.0),
    (3, 16, 2, 1, 64, 64, 10000.0, 0.125),
    (1, 4, 4, 64, 128, 8192, 1000000.0, 0.088),
    (2, 8, 2, 5, 80, 512, 10000.0, 0.11),            # head size 80
]


def _random_cases(n):
    """Seeded random shapes: head sizes 64 to 256, 1 to 32 query and 1 to 8 KV
    heads, 1 to 64 tokens, caches up to 40 000 rows, three RoPE bases."""
    rng = np.random.default_rng(424242)
    out = []
    for _ in range(n):
        hd = int(rng.choice([64, 80, 128, 256]))
        n_tok = int(rng.integers(1, 65))
        cap = int(rng.choice([n_tok + 1 + int(rng.integers(0, 64)), 1024, 8192, 40000]))
        n_kvh = int(rng.integers(1, 9)) if cap <= 8192 else 1
        out.append((int(rng.integers(1, 5)), int(rng.integers(1, 33)), n_kvh, n_tok, hd, cap,
                    float(rng.choice([10000.0, 500000.0, 1000000.0])),
                    float(rng.uniform(0.05, 1.0))))
    return out


ALL_CASES = CASES + _random_cases(40)


@pytest.mark.parametrize("case", ALL_CASES, ids=lambda c: "n{}_h{}_g{}_t{}_d{}_c{}".format(*c[:6]))
def test_qkv_post_rounding_and_rows(oracle_mod, case):
    n_inst, n_head, n_kvh, n_tok, hd, cap, base, qs = case
    say(f"qkv_post {case}")
    rng = np.random.default_rng(ALL_CASES.index(case) + 40)
    qkv = rng.standard_normal((n_inst, n_tok, (n_head + 2 * n_kvh) * hd)).astype(np.float32)
    # distinct positions per instance; instance 0 also takes the largest angle
    pos = np.stack([rng.choice(cap - 1, n_tok, replace=False) for _ in range(n_inst)])
    pos = pos.astype(np.int32)
    pos[0, 0] = cap - 1
    q16, kc, vc = run_qkv(qkv, pos, n_head, n_kvh, hd, cap, base, qs)
    flips = 0
    for i in range(n_inst):
        q, k, v = oracle_mod.qkv_post(qkv[i], pos[i], n_head, n_kvh, n_tok, hd, base, qs)
        x = qkv[i].astype(np.float64).reshape(n_tok, n_head + 2 * n_kvh, hd)
        flips += check_rounding(q16[i], q, pair_bound(x[:, :n_head], qs), f"q inst {i}")
        kx = x[:, n_head:n_head + n_kvh].transpose(1, 0, 2)
        flips += check_rounding(kc[i][:, pos[i]], k, pair_bound(kx, 1.0), f"k inst {i}")
        assert np.array_equal(vc[i][:, pos[i]], oracle_mod.f16_copy(v.astype(np.float32)))
        untouched = np.ones(cap, dtype=bool)
        untouched[pos[i]] = False
        assert (kc[i][:, untouched] == CANARY).all() and (vc[i][:, untouched] == CANARY).all()
    total = q16.size + n_inst * n_kvh * n_tok * hd
    print(f"[parity] qkv_post {case}: {flips} of {total} outputs on the other side of a tie")
    assert flips <= max(10, total // 100)


def test_positions_outside_the_cache_are_not_stored(oracle_mod):
    say("qkv_post out-of-range positions")
    n_head, n_kvh, n_tok, hd, cap = 4, 2, 4, 64, 16
    rng = np.random.default_rng(3)
    qkv = rng.standard_normal((1, n_tok, (n_head + 2 * n_kvh) * hd)).astype(np.float32)
    pos = np.array([[-1, 16, 3, 1 << 30]], dtype=np.int32)
    q16, kc, vc = run_qkv(qkv, pos, n_head, n_kvh, hd, cap, 10000.0, 1.0)
    rows = np.ones(cap, dtype=bool)
    rows[3] = False
    assert (kc[0][:, rows] == CANARY).all() and (vc[0][:, rows] == CANARY).all()
    assert (kc[0][:, 3] != CANARY).any()
    q, _, _ = oracle_mod.qkv_post(qkv[0], pos[0], n_head, n_kvh, n_tok, hd, 10000.0, 1.0)
    x = qkv[0].astype(np.float64).reshape(n_tok, n_head + 2 * n_kvh, hd)
    check_rounding(q16[0], q, pair_bound(x[:, :n_head], 1.0), "q")  # q rows always written


def test_producer_feeds_the_window(oracle_mod):
    """qkv_post for 10 new tokens appended after a 958-token prefix, then the
    window over the cache with its f16 queries (fr_decode_attn_q16), against
    the oracle attention on the oracle's own producer outputs."""
    import gqa_decode_attention_fr_amd as F
    say("qkv_post -> decode window")
    n_head, n_tok, hd, cap, prefix, base, qs = 8, 10, 256, 1024, 958, 10000.0, 1.0
    rng = np.random.default_rng(21)
    qkv = (rng.standard_normal((1, n_tok, (n_head + 2) * hd)) * 0.5).astype(np.float32)
    pos = (prefix + np.arange(n_tok, dtype=np.int32))[None]
    prev_k = (rng.standard_normal((prefix, hd)) * 0.5).astype(np.float16)
    prev_v = (rng.standard_normal((prefix, hd)) * 0.5).astype(np.float16)
    kc = torch.zeros((cap, hd), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:prefix] = torch.from_numpy(prev_k).cuda()
    vc[:prefix] = torch.from_numpy(prev_v).cuda()
    q16 = torch.zeros((n_tok, n_head, hd), dtype=torch.float16, device="cuda")
    F.fr_qkv_post(torch.from_numpy(qkv).cuda(), torch.from_numpy(pos).cuda(), q16, kc, vc, 1,
                  0, 0, 0, 0, 0, n_head, 1, n_tok, hd, cap, base, qs)
    # causal over the new tokens; keys past the last token masked
    mask = np.zeros((n_tok, cap), dtype=np.float16)
    for t in range(n_tok):
        mask[t, prefix + t + 1:] = -np.inf
    m_d = torch.from_numpy(mask).cuda()
    out = torch.empty((n_tok, n_head, hd), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(hd)
    F.fr_decode_attn_q16(q16, kc, vc, m_d, out, n_head, n_tok, cap, hd, scale)
    torch.cuda.synchronize()
    q, k, v = oracle_mod.qkv_post(qkv[0], pos[0], n_head, 1, n_tok, hd, base, qs)
    k_all = np.zeros((cap, hd), dtype=np.float16)
    v_all = np.zeros((cap, hd), dtype=np.float16)
    k_all[:prefix], v_all[:prefix] = prev_k, prev_v
    k_all[prefix:prefix + n_tok] = k[0].astype(np.float16)
    v_all[prefix:prefix + n_tok] = v[0].astype(np.float16)
    want = oracle_mod.decode_attn(q.astype(np.float16).view(np.uint16), k_all.view(np.uint16),
                                  v_all.view(np.uint16), mask.view(np.uint16), n_head, n_tok,
                                  cap, hd, scale, q_kind=oracle_mod.Q_F16)
    got = out.cpu().numpy()
    max_abs, rel = errors(got, want)
    print(f"[parity] producer->window max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, "producer -> window")


def test_graph_replays_follow_device_positions():
    import gqa_decode_attention_fr_amd as F
    say("qkv_post graph replay")
    n_head, n_kvh, n_tok, hd, cap = 8, 2, 3, 128, 64
    rng = np.random.default_rng(8)
    qkv = torch.from_numpy(rng.standard_normal((n_tok, (n_head + 2 * n_kvh) * hd))
                           .astype(np.float32)).cuda()
    pos = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    q16 = torch.zeros((n_tok, n_head, hd), dtype=torch.int16, device="cuda")
    kc = torch.zeros((n_kvh, cap, hd), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)

    def call():
        F.fr_qkv_post(qkv, pos, q16, kc, vc, 1, 0, 0, 0, 0, cap * hd, n_head, n_kvh, n_tok, hd,
                      cap, 10000.0, 0.5)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    for step, new in enumerate(([5, 6, 7], [60, 61, 63], [9, 0, 30])):
        pos.copy_(torch.tensor(new, dtype=torch.int32))
        for t in (q16, kc, vc):
            t.zero_()
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        eager = [t.clone() for t in (q16, kc, vc)]
        for t in (q16, kc, vc):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip((q16, kc, vc), eager):
            assert torch.equal(t, e), f"replay {step} positions {new}"
