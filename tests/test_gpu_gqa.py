"""GPU parity of the several-KV-head entry point (fr_decode_attn_gqa): query
head h attends over KV head h // (n_head // n_kv_head).  Checked against the
fp64 oracle at the acceptance tolerance, and bit for bit against separate
one-KV-head calls on each group's query heads with the same key splits.  Also
its device-side valid key counts, against the oracle with those keys masked,
eagerly and from one captured graph replayed with changing counts."""
import math

import numpy as np
import pytest

from gqa_decode_attention_fr_amd import workloads as W
from gpu_util import assert_close, dev, errors, oracle_gqa, run_gqa, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
FUSED, DECOMP = 0x2, 0x4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_fr_amd as F
    F.binding.load()
    yield


GQA = [  # n_inst, n_head, n_kv_head, n_tok, n_kv, hd, q dtype, mask kind, pad rows per KV head
    (2, 32, 8, 4, 1000, 128, "f32", "random", 0),      # 4 query heads per KV head
    (1, 16, 2, 16, 4096, 128, "f16", "zero", 0),
    (3, 8, 8, 10, 333, 64, "f32", "random", 0),       # one query head per KV head
    (1, 28, 4, 1, 2048, 128, "f32", "none", 0),       # single-token decode, 7 per group
    (2, 12, 3, 16, 777, 256, "f32", "full_row", 0),
    (1, 64, 8, 16, 8192, 128, "f32", "random", 0),    # 128 rows per unit
    (2, 8, 2, 10, 968, 256, "f32", "random", 56),     # padded head stride
    (1, 40, 5, 3, 1531, 64, "f16", "random", 8),
]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", GQA, ids=lambda s: "n{}_h{}_g{}_t{}_kv{}_d{}_{}_{}_p{}".format(*s))
def test_gqa_parity(oracle_mod, shape, variant):
    n_inst, n_head, n_kvh, n_tok, n_kv, hd, qd, mk, pad = shape
    say(f"gqa {shape} variant={variant}")
    c = W.random_case(GQA.index(shape) + 500, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind=mk, n_inst=n_inst, n_kv_head=n_kvh)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant,
                  q_f16=(qd == "f16"), pad_rows=pad)
    want = oracle_gqa(oracle_mod, c, n_head, n_kvh, n_tok, n_kv, hd, scale,
                      oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] gqa {shape} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, str(shape))
    if mk == "full_row":
        assert np.array_equal(got[:, 0], np.zeros_like(got[:, 0]))


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_gqa_equals_one_call_per_group(monkeypatch, variant):
    """Each group of query heads through the one-KV-head entry point, with the
    key splits forced equal: the grouped call must match bit for bit (only
    where rows are read and written differs)."""
    import gqa_decode_attention_fr_amd as F
    n_inst, n_head, n_kvh, n_tok, n_kv, hd = 2, 24, 4, 7, 1500, 128
    G = n_head // n_kvh
    say(f"gqa per-group identity variant={variant}")
    monkeypatch.setenv("FR_FORCE_SPLITS", "6")
    c = W.random_case(601, n_head, n_tok, n_kv, hd, mask_kind="random", n_inst=n_inst,
                      n_kv_head=n_kvh)
    scale = 1.0 / math.sqrt(hd)
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant)
    for i in range(n_inst):
        for kh in range(n_kvh):
            qg = np.ascontiguousarray(c["q"][i][:, kh * G:(kh + 1) * G, :])
            out = torch.full((n_tok, G, hd), float("nan"), dtype=torch.float32, device="cuda")
            F.fr_decode_attn_ex(dev(qg, torch), F.FR_Q_F32, dev(c["k"][i, kh], torch),
                                dev(c["v"][i, kh], torch), dev(c["mask"][i], torch), out, 1,
                                0, 0, 0, 0, G, n_tok, n_kv, hd, scale, variant)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), got[i][:, kh * G:(kh + 1) * G, :]), \
                f"instance {i} KV head {kh}"


def test_gqa_with_one_kv_head_equals_ex():
    """n_kv_head = 1 is the pages' window: the same bits as fr_decode_attn_ex."""
    import gqa_decode_attention_fr_amd as F
    w = W.PI05_ACTION_STEP
    say("gqa one KV head == ex")
    g = W.generate(w)
    c = dict(g)
    c["k"], c["v"] = g["k"][:, None], g["v"][:, None]
    got = run_gqa(c, w.n_head, 1, w.n_tok, w.n_kv, w.hd, w.scale)
    from gpu_util import run_gpu
    ref = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("w", [W.GQA_KV8, W.GQA_DECODE_T1], ids=lambda w: w.name)
@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_gqa_workload_full_size(oracle_mod, variant, w):
    """The measured several-KV-head workloads, every element, both variants."""
    say(f"workload {w.name} variant={variant}")
    g = W.generate(w)
    got = run_gqa(g, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant)
    want = oracle_gqa(oracle_mod, g, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd, w.scale,
                      oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] {w.name} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, w.name)


F16_NAN = 0x7E00
NEG_INF = 0xFC00


def _hide_past(c, kv_len, n_kv):
    """The oracle's view of valid key counts: keys j >= L masked (-inf) for
    every token; and the GPU's inputs with those K/V rows set to NaN, which
    would poison the output if any were read."""
    n_inst, n_tok = c["q"].shape[0], c["q"].shape[1]
    mask = (np.zeros((n_inst, n_tok, n_kv), dtype=np.uint16) if c["mask"] is None
            else c["mask"].copy())
    kg, vg = c["k"].copy(), c["v"].copy()
    for i, L in enumerate(kv_len):
        L = min(max(L, 0), n_kv)
        mask[i, :, L:] = NEG_INF
        kg[i, ..., L:, :] = F16_NAN
        vg[i, ..., L:, :] = F16_NAN
    return dict(c, mask=mask), (kg, vg)


KV_LEN = [  # n_head, n_kv_head, n_tok, n_kv, hd, mask kind, valid counts per instance
    (16, 2, 5, 1000, 128, "random", [1000, 0, 1, 777, 64, 1100, -5]),
    (8, 1, 10, 1024, 256, "none", [968, 968, 500, 1024]),
    (32, 8, 4, 4096, 128, "zero", [4096, 2048, 33, 4000]),
    (12, 3, 16, 333, 64, "random", [333, 320, 65, 0]),
    (8, 2, 3, 64, 256, "zero", [64, 0, 10]),          # one key block: no split
]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", KV_LEN, ids=lambda s: "h{}_g{}_t{}_kv{}_d{}_{}".format(*s[:6]))
def test_device_valid_key_counts(oracle_mod, shape, variant):
    n_head, n_kvh, n_tok, n_kv, hd, mk, lens = shape
    say(f"kv_len {shape} variant={variant}")
    c = W.random_case(KV_LEN.index(shape) + 700, n_head, n_tok, n_kv, hd, mask_kind=mk,
                      n_inst=len(lens), n_kv_head=n_kvh)
    if n_kvh == 1:
        c["k"], c["v"] = c["k"][:, None], c["v"][:, None]
    scale = 1.0 / math.sqrt(hd)
    c_or, kv_nan = _hide_past(c, lens, n_kv)
    gpu_in = dict(c)
    got = run_gqa(gpu_in, n_head, n_kvh, n_tok, n_kv, hd, scale, flags=variant, kv_len=lens,
                  kv_override=kv_nan)
    want = oracle_gqa(oracle_mod, c_or, n_head, n_kvh, n_tok, n_kv, hd, scale, oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] kv_len {shape} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, str(shape))
    for i, L in enumerate(lens):
        if L <= 0:
            assert np.array_equal(got[i], np.zeros_like(got[i])), f"instance {i}"


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_graph_replays_follow_device_key_counts(variant):
    """One graph captured with a device key-count array; between replays the
    host writes new counts, and every replay equals an eager call with them."""
    import gqa_decode_attention_fr_amd as F
    n_inst, n_head, n_kvh, n_tok, n_kv, hd = 3, 16, 4, 4, 2048, 128
    say(f"graph replays with changing kv_len, variant={variant}")
    c = W.random_case(801, n_head, n_tok, n_kv, hd, mask_kind="none", n_inst=n_inst,
                      n_kv_head=n_kvh)
    scale = 1.0 / math.sqrt(hd)
    M = n_head * n_tok
    units, grp = n_inst * n_kvh, n_head // n_kvh
    F.fr_decode_attn_reserve(units, grp, n_tok, n_kv, hd, variant)
    q, k, v = dev(c["q"], torch), dev(c["k"], torch), dev(c["v"], torch)
    lens = torch.full((n_inst,), n_kv, dtype=torch.int32, device="cuda")
    out = torch.zeros((n_inst, n_tok, n_head, hd), dtype=torch.float32, device="cuda")

    def call():
        F.fr_decode_attn_gqa(q, F.FR_Q_F32, k, v, None, out, n_inst, M * hd,
                             n_kvh * n_kv * hd, 0, M * hd, n_head, n_kvh, n_kv * hd, n_tok,
                             n_kv, hd, scale, variant, kv_len=lens)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    for step, new in enumerate(([2048, 2048, 2048], [1, 100, 1999], [0, 64, 65], [513, 0, 2048])):
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        eager = out.clone()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {step} with counts {new}"


def _gqa_selector_case(n_inst, n_head, n_kvh, n_tok, n_kv, hd, seed):
    """Per KV head, K_j = 2048 e_j for j < min(hd, n_kv); query row (t, h)
    is e_{pi}: its logits are 128 at key pi of its own KV head and 0
    elsewhere, so exp(-128) vanishes in fp32 and out[t][h] must be V[h/G][pi]
    bit for bit.  V differs between KV heads, so a row that reads another KV
    head's keys or values fails."""
    rng = np.random.default_rng(seed)
    n_dir = min(hd, n_kv)
    M = n_head * n_tok
    pi = (np.arange(n_inst * M).reshape(n_inst, n_tok, n_head) * 29 + 5) % n_dir
    k = np.zeros((n_inst, n_kvh, n_kv, hd), dtype=np.float64)
    k[:, :, np.arange(n_dir), np.arange(n_dir)] = 2048.0
    q = np.zeros((n_inst, n_tok, n_head, hd), dtype=np.float32)
    for i in range(n_inst):
        for t in range(n_tok):
            q[i, t, np.arange(n_head), pi[i, t]] = 1.0
    v = W.f16_bits(rng.standard_normal((n_inst, n_kvh, n_kv, hd)))
    case = {"q": q, "k": W.f16_bits(k), "v": v,
            "mask": np.zeros((n_inst, n_tok, n_kv), dtype=np.uint16)}
    return case, pi


SELECT = [  # n_inst, n_head, n_kv_head, n_tok, n_kv, hd
    (2, 8, 4, 3, 200, 128),
    (1, 32, 8, 16, 1024, 128),
    (3, 12, 3, 5, 100, 64),
    (1, 16, 2, 10, 968, 256),
    (1, 8, 2, 4, 90, 80),       # head size 80
]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", SELECT, ids=lambda s: "n{}_h{}_g{}_t{}_kv{}_d{}".format(*s))
def test_gqa_selector_bit_exact(shape, variant):
    n_inst, n_head, n_kvh, n_tok, n_kv, hd = shape
    say(f"gqa selector {shape} variant={variant}")
    c, pi = _gqa_selector_case(n_inst, n_head, n_kvh, n_tok, n_kv, hd, SELECT.index(shape))
    got = run_gqa(c, n_head, n_kvh, n_tok, n_kv, hd, 1.0 / 16, flags=variant)
    vf = c["v"].view(np.float16).astype(np.float32)
    G = n_head // n_kvh
    want = np.empty_like(got)
    for i in range(n_inst):
        for t in range(n_tok):
            for h in range(n_head):
                want[i, t, h] = vf[i, h // G, pi[i, t, h]]
    assert np.array_equal(got, want)


def test_gqa_writes_only_its_output_and_repeats_bitwise():
    """Guard bands before, between and after the instances' outputs stay
    untouched, and a second call gives the same bits."""
    import gqa_decode_attention_fr_amd as F
    n_inst, n_head, n_kvh, n_tok, n_kv, hd = 3, 16, 4, 6, 1500, 128
    say("gqa guard bands and determinism")
    c = W.random_case(1201, n_head, n_tok, n_kv, hd, mask_kind="random", n_inst=n_inst,
                      n_kv_head=n_kvh)
    M = n_head * n_tok
    guard = 4096
    stride = M * hd + guard                   # a guard band between instances too
    buf = torch.full((guard + n_inst * stride,), 12345.0, dtype=torch.float32, device="cuda")
    q, k, v, m = (dev(c[x], torch) for x in ("q", "k", "v", "mask"))
    outs = []
    for _ in range(2):
        buf.fill_(12345.0)
        out = buf[guard:]
        F.fr_decode_attn_gqa(q, F.FR_Q_F32, k, v, m, out, n_inst, M * hd, n_kvh * n_kv * hd,
                             n_tok * n_kv, stride, n_head, n_kvh, n_kv * hd, n_tok, n_kv, hd,
                             1.0 / math.sqrt(hd))
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        written = np.zeros(host.size, dtype=bool)
        for i in range(n_inst):
            written[guard + i * stride:guard + i * stride + M * hd] = True
        assert (host[~written] == 12345.0).all()
        assert np.isfinite(host[written]).all() and (host[written] != 12345.0).mean() > 0.99
        outs.append(host[written].copy())
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_kv_blocks_beyond_4_gib(oracle_mod, variant):
    """KV heads and instances placed 4 to 12 GiB into K and V (64-bit base
    offsets from kv_stride and kv_head_stride), against the oracle.  The row
    just before and just after every block holds NaN: a kernel that read it
    would turn its output rows into NaN."""
    import gqa_decode_attention_fr_amd as F
    n_inst, n_head, n_kvh, n_tok, n_kv, hd = 2, 4, 2, 3, 300, 128
    kvh_stride = (1 << 31) + 37 * hd                # elements: 4 GiB + 37 rows
    kv_stride = n_kvh * kvh_stride + 11 * hd
    total = (n_inst - 1) * kv_stride + (n_kvh - 1) * kvh_stride + (n_kv + 1) * hd
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * 2 * total + (4 << 30):
        pytest.skip("needs about 26 GB of free device memory")
    say(f"kv blocks beyond 4 GiB variant={variant}")
    c = W.random_case(900, n_head, n_tok, n_kv, hd, q_dtype="f32", mask_kind="random",
                      n_inst=n_inst, n_kv_head=n_kvh)
    nan_row = torch.full((hd,), float("nan"), dtype=torch.float16, device="cuda")
    bufs = []
    for name in ("k", "v"):
        t = torch.empty(total, dtype=torch.float16, device="cuda")
        for i in range(n_inst):
            for h in range(n_kvh):
                off = i * kv_stride + h * kvh_stride
                t[off:off + n_kv * hd] = dev(c[name][i, h].reshape(-1), torch)
                t[off + n_kv * hd:off + (n_kv + 1) * hd] = nan_row
                if off >= hd:
                    t[off - hd:off] = nan_row
        bufs.append(t)
    k, v = bufs
    q, mask = dev(c["q"], torch), dev(c["mask"], torch)
    M = n_head * n_tok
    out = torch.full((n_inst, n_tok, n_head, hd), float("nan"), dtype=torch.float32,
                     device="cuda")
    scale = 1.0 / math.sqrt(hd)
    F.fr_decode_attn_gqa(q, F.FR_Q_F32, k, v, mask, out, n_inst, M * hd, kv_stride,
                         n_tok * n_kv, M * hd, n_head, n_kvh, kvh_stride, n_tok, n_kv, hd,
                         scale, variant)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del k, v, bufs
    torch.cuda.empty_cache()
    want = oracle_gqa(oracle_mod, c, n_head, n_kvh, n_tok, n_kv, hd, scale, oracle_mod.Q_F32)
    max_abs, rel = errors(got, want)
    print(f"[parity] kv beyond 4 GiB variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, "kv blocks beyond 4 GiB")
