"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on the
five measured workloads at full size, ragged random shapes, and the edge cases
(single key, fully masked rows, no mask, maximum tokens), plus bit-exact layout,
determinism, no out-of-bounds writes, and the f16-Q handoff identity."""
import dataclasses
import math
import os

import numpy as np
import pytest

from gqa_decode_attention_fr_amd import workloads as W
from gpu_util import (MAX_ABS, REL_L2, assert_close, dev, errors, oracle_instances, run_gpu,
                      say)

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


_ORACLE_CACHE = {}


def _oracle_workload(oracle, w, g, q_kind):
    key = (w.name, q_kind)
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = oracle_instances(oracle, g, w.n_head, w.n_tok, w.n_kv, w.hd,
                                              w.scale, q_kind)
    return _ORACLE_CACHE[key]


def _q_kind(oracle, w, flags=0):
    if w.q_dtype == "f16":
        return oracle.Q_F16
    return oracle.Q_F32_ROUND_F16 if flags & 0x1 else oracle.Q_F32


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("w", W.WORKLOADS, ids=lambda w: w.name)
def test_workload_parity_full_size(oracle_mod, w, variant):
    say(f"workload {w.name} variant={variant}")
    g = W.generate(w)
    got = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant,
                  q_f16=(w.q_dtype == "f16"), torch=torch)
    want = _oracle_workload(oracle_mod, w, g, _q_kind(oracle_mod, w))
    max_abs, rel = errors(got, want)
    print(f"[parity] {w.name} variant={variant} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert_close(got, want, w.name)


@pytest.mark.parametrize("w", [W.TINY, W.H16_HD128_Q16], ids=lambda w: w.name)
def test_single_entry_points(oracle_mod, w):
    say(f"single entry {w.name}")
    g = W.generate(w)
    got = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, q_f16=(w.q_dtype == "f16"),
                  torch=torch, entry="single")
    want = _oracle_workload(oracle_mod, w, g, _q_kind(oracle_mod, w))
    assert_close(got, want, w.name)


RANDOM = [  # n_head, n_tok, n_kv, hd, q dtype, mask kind
    (1, 1, 1, 64, "f32", "none"),
    (1, 1, 1, 256, "f32", "zero"),
    (3, 5, 77, 128, "f32", "random"),
    (7, 16, 1000, 256, "f32", "random"),
    (2, 3, 129, 64, "f16", "random"),
    (16, 16, 300, 128, "f32", "full_row"),
    (5, 9, 4097, 64, "f32", "random"),
    (12, 11, 640, 256, "f16", "none"),
    (33, 7, 2500, 128, "f32", "random"),
    (64, 16, 8192, 128, "f32", "zero"),      # M = 1024: several row blocks
    (1, 16, 65, 256, "f32", "random"),
    (40, 16, 1531, 64, "f32", "random"),
]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", RANDOM, ids=lambda s: "h{}_t{}_kv{}_d{}_{}_{}".format(*s))
def test_random_shapes(oracle_mod, shape, variant):
    n_head, n_tok, n_kv, hd, qd, mk = shape
    say(f"random {shape} variant={variant}")
    c = W.random_case(RANDOM.index(shape) + 100, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind=mk)
    scale = 1.0 / math.sqrt(hd)
    got = run_gpu(c, n_head, n_tok, n_kv, hd, scale, flags=variant, q_f16=(qd == "f16"),
                  torch=torch)
    want = oracle_instances(oracle_mod, c, n_head, n_tok, n_kv, hd, scale,
                            oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    assert_close(got, want, str(shape))
    if mk == "full_row":  # token 0 sees no key: its rows are exactly zero
        assert np.array_equal(got[0, 0], np.zeros((n_head, hd), dtype=np.float32))


FORCED_WAVES = [  # n_head, n_tok, n_kv, hd, q dtype, mask kind, waves (the other count than planned)
    (8, 10, 1000, 256, "f32", "random", 8),
    (20, 16, 700, 256, "f32", "random", 4),    # M = 320: 20 tiles, planned as 8 waves
    (20, 16, 700, 256, "f16", "none", 4),
    (16, 16, 4096, 128, "f16", "zero", 8),
    (64, 16, 2048, 128, "f32", "random", 4),
    (9, 5, 333, 64, "f16", "random", 8),
    (3, 16, 129, 128, "f32", "full_row", 8),
]


@pytest.mark.parametrize("shape", FORCED_WAVES, ids=lambda s: "h{}_t{}_kv{}_d{}_{}_{}_w{}".format(*s))
def test_forced_wave_counts(oracle_mod, shape, monkeypatch):
    """Both instantiated workgroup shapes (4 and 8 waves) against the oracle,
    on shapes whose plan would pick the other one."""
    import gqa_decode_attention_fr_amd as F
    n_head, n_tok, n_kv, hd, qd, mk, waves = shape
    say(f"forced waves {shape}")
    monkeypatch.setenv("FR_FORCE_WAVES", str(waves))
    assert F.fr_decode_attn_plan(1, n_head, n_tok, n_kv, hd)["waves"] == waves
    c = W.random_case(FORCED_WAVES.index(shape) + 300, n_head, n_tok, n_kv, hd, q_dtype=qd,
                      mask_kind=mk)
    scale = 1.0 / math.sqrt(hd)
    got = run_gpu(c, n_head, n_tok, n_kv, hd, scale, q_f16=(qd == "f16"), torch=torch)
    want = oracle_instances(oracle_mod, c, n_head, n_tok, n_kv, hd, scale,
                            oracle_mod.Q_F16 if qd == "f16" else oracle_mod.Q_F32)
    assert_close(got, want, str(shape))


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_round_f16_flag_matches_oracle(oracle_mod, variant):
    w = W.CAUSAL_TAIL
    say(f"round-f16 flag variant={variant}")
    g = W.generate(w)
    got = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant | 0x1, torch=torch)
    want = oracle_instances(oracle_mod, g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale,
                            oracle_mod.Q_F32_ROUND_F16)
    # the pages' f16 rounding of Q is part of this mode, so both sides round
    assert_close(got, want, "round_f16")


def _selector_case(n_head, n_tok, n_kv, hd, seed=0):
    """K_j = 2048 e_j for j < hd (zero beyond), Q_r = e_{pi(r)}, scale 1/16:
    row r's logits are 128 at key pi(r) and 0 elsewhere, so exp(-128) vanishes
    in fp32 and out[r] must equal V[pi(r)] bit for bit."""
    rng = np.random.default_rng(seed)
    M = n_head * n_tok
    n_dir = min(hd, n_kv)
    pi = (np.arange(M) * 37 + 11) % n_dir
    k = np.zeros((n_kv, hd), dtype=np.float64)
    k[np.arange(n_dir), np.arange(n_dir)] = 2048.0
    q = np.zeros((n_tok, n_head, hd), dtype=np.float32)
    q.reshape(M, hd)[np.arange(M), pi] = 1.0
    v = W.f16_bits(rng.standard_normal((n_kv, hd)))
    case = {"q": q[None], "k": W.f16_bits(k)[None], "v": v[None],
            "mask": np.zeros((1, n_tok, n_kv), dtype=np.uint16)}
    return case, pi


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
@pytest.mark.parametrize("shape", [(8, 1, 64, 256), (8, 10, 1024, 256), (16, 16, 4096, 128),
                                   (8, 16, 2048, 256), (32, 16, 32768, 128), (3, 7, 100, 64)])
def test_selector_layout_bit_exact(shape, variant):
    n_head, n_tok, n_kv, hd = shape
    say(f"selector {shape} variant={variant}")
    case, pi = _selector_case(n_head, n_tok, n_kv, hd)
    got = run_gpu(case, n_head, n_tok, n_kv, hd, 1.0 / 16, flags=variant, torch=torch)
    vf = case["v"][0].view(np.float16).astype(np.float32)
    want = vf[pi].reshape(n_tok, n_head, hd)
    assert np.array_equal(got[0], want)


def test_q16_handoff_is_bit_identical_to_rounded_f32():
    """FlashRT PR #185, qkv_post handoff commit: f16 Q rounded from the same
    f32 values gives bit-identical results to the gather path."""
    w = W.PI05_ACTION_STEP
    say("q16 handoff identity")
    g = W.generate(w)
    q16 = {**g, "q": g["q"].astype(np.float16).view(np.uint16)}
    for variant in (FUSED, DECOMP):
        a = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant | 0x1,
                    torch=torch)
        b = run_gpu(q16, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant, q_f16=True,
                    torch=torch)
        assert np.array_equal(a, b)


def test_run_to_run_deterministic():
    say("determinism")
    for w in (W.PI05_ACTION_STEP, W.LONG_CONTEXT):
        g = W.generate(w)
        a = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch)
        b = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch)
        assert np.array_equal(a, b)


def test_hi_lo_query_is_more_accurate_than_rounded(oracle_mod):
    """The f32 entry keeps q at ~22 bits; rounding q to f16 (the pages' gather)
    measurably moves the causal-tail workload with its x8 key outliers."""
    w = W.CAUSAL_TAIL
    say("hi/lo accuracy")
    g = W.generate(w)
    want = _oracle_workload(oracle_mod, w, g, oracle_mod.Q_F32)
    hilo = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch)
    rounded = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=0x1, torch=torch)
    assert errors(hilo, want)[0] < errors(rounded, want)[0]


@pytest.mark.parametrize("variant", [FUSED, DECOMP], ids=["fused", "decomposed"])
def test_no_writes_outside_out(variant):
    """The call writes its output rows and nothing else: guard bands around
    out keep their canary, and q, k, v and the mask are bitwise unchanged."""
    import gqa_decode_attention_fr_amd as F
    say(f"canary guard bands and untouched inputs, variant={variant}")
    w = W.PI05_ACTION_STEP
    g = W.generate(w)
    M = w.M
    n = w.n_inst * M * w.hd
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
    out = buf[guard:guard + n]
    ins = {x: dev(g[x], torch) for x in ("q", "k", "v", "mask")}
    F.fr_decode_attn_ex(ins["q"], F.FR_Q_F32, ins["k"], ins["v"], ins["mask"], out, w.n_inst,
                        M * w.hd, w.n_kv * w.hd, w.n_tok * w.n_kv, M * w.hd, w.n_head, w.n_tok,
                        w.n_kv, w.hd, w.scale, variant)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 12345.0) and np.all(b[-guard:] == 12345.0)
    assert np.all(np.isfinite(b[guard:guard + n]))
    for x, t in ins.items():
        after = t.cpu().numpy()
        assert np.array_equal(after.view(np.uint8), np.ascontiguousarray(g[x]).view(np.uint8)), x


def test_masked_keys_do_not_matter():
    """Keys hidden from every token may hold any finite values."""
    w = W.PI05_ACTION_STEP
    say("masked garbage invariance")
    g = W.generate(w)
    g2 = {**g, "k": g["k"].copy(), "v": g["v"].copy()}
    g2["k"][:, w.n_valid:] = W.f16_bits(np.full((w.n_kv - w.n_valid, w.hd), 3.0e4))
    g2["v"][:, w.n_valid:] = W.f16_bits(np.full((w.n_kv - w.n_valid, w.hd), -6.0e4))
    for variant in (FUSED, DECOMP):
        a = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant, torch=torch)
        b = run_gpu(g2, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, flags=variant, torch=torch)
        assert np.array_equal(a, b)


def test_null_mask_equals_zero_mask():
    say("null mask")
    c = W.random_case(3, 8, 4, 500, 128, mask_kind="zero")
    a = run_gpu(c, 8, 4, 500, 128, 0.1, torch=torch)
    b = run_gpu({**c, "mask": None}, 8, 4, 500, 128, 0.1, torch=torch)
    assert np.array_equal(a, b)


def test_batched_equals_single_calls(monkeypatch):
    """One batched call over 18 instances gives the same bits as 18 single
    calls with the same split plan."""
    import gqa_decode_attention_fr_amd as F
    w = W.PI05_ACTION_STEP
    say("batched vs single")
    monkeypatch.setenv("FR_FORCE_SPLITS", "8")
    g = W.generate(w)
    batched = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch)
    for i in (0, 7, 17):
        one = {key: g[key][i:i + 1] for key in ("q", "k", "v", "mask")}
        single = run_gpu(one, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch,
                         entry="single")
        assert np.array_equal(single[0], batched[i])
    assert F.fr_decode_attn_plan(1, w.n_head, w.n_tok, w.n_kv, w.hd)["n_split"] == 8


def test_shared_mask_stride_zero(oracle_mod):
    import gqa_decode_attention_fr_amd as F
    w = W.PI05_ACTION_STEP
    say("mask stride 0")
    g = W.generate(w)
    M = w.M
    out = torch.empty((w.n_inst, w.n_tok, w.n_head, w.hd), dtype=torch.float32, device="cuda")
    F.fr_decode_attn_batched(dev(g["q"], torch), F.FR_Q_F32, dev(g["k"], torch),
                             dev(g["v"], torch), dev(g["mask"][0], torch), out, w.n_inst,
                             M * w.hd, w.n_kv * w.hd, 0, M * w.hd, w.n_head, w.n_tok, w.n_kv,
                             w.hd, w.scale)
    torch.cuda.synchronize()
    ref = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, torch=torch)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_caller_workspace(oracle_mod):
    import gqa_decode_attention_fr_amd as F
    w = W.H16_HD128_Q16
    say("caller workspace")
    g = W.generate(w)
    M = w.M
    need = F.fr_decode_attn_workspace_size(1, w.n_head, w.n_tok, w.n_kv, w.hd)
    assert need > 0
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.n_tok, w.n_head, w.hd), dtype=torch.float32, device="cuda")
    args = (dev(g["q"][0], torch), F.FR_Q_F16, dev(g["k"][0], torch), dev(g["v"][0], torch),
            dev(g["mask"][0], torch), out, 1, 0, 0, 0, 0, w.n_head, w.n_tok, w.n_kv, w.hd,
            w.scale, 0)
    with pytest.raises(F.FrError) as e:
        F.fr_decode_attn_ex(*args, workspace=ws, workspace_bytes=need - 1)
    assert e.value.status == F.FR_ERR_WORKSPACE
    F.fr_decode_attn_ex(*args, workspace=ws, workspace_bytes=need)
    torch.cuda.synchronize()
    ref = run_gpu(g, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale, q_f16=True, torch=torch)
    assert np.array_equal(out.cpu().numpy(), ref[0])


def test_graph_capture_replays_match_eager():
    """Capture-safe use (FlashRT-llama.cpp development guide, 'Caches'): with the
    workspace reserved, calls can be captured; every replay equals eager."""
    import gqa_decode_attention_fr_amd as F
    w = W.PI05_ACTION_STEP
    say("graph capture")
    g = W.generate(w)
    M = w.M
    F.fr_decode_attn_reserve(w.n_inst, w.n_head, w.n_tok, w.n_kv, w.hd)
    q, k, v, m = (dev(g[x], torch) for x in ("q", "k", "v", "mask"))
    out = torch.zeros((w.n_inst, w.n_tok, w.n_head, w.hd), dtype=torch.float32, device="cuda")

    def call():
        F.fr_decode_attn_batched(q, F.FR_Q_F32, k, v, m, out, w.n_inst, M * w.hd,
                                 w.n_kv * w.hd, w.n_tok * w.n_kv, M * w.hd, w.n_head, w.n_tok,
                                 w.n_kv, w.hd, w.scale)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    for it in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {it}"
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_capture_refuses_to_grow_workspace():
    import gqa_decode_attention_fr_amd as F
    say("capture without reserve")
    # a shape whose decomposed workspace dwarfs anything reserved so far
    n_head, n_tok, n_kv, hd = 64, 16, 65536, 64
    need = F.fr_decode_attn_workspace_size(1, n_head, n_tok, n_kv, hd, DECOMP)
    assert need > 256 << 20
    q = torch.zeros((n_tok, n_head, hd), dtype=torch.float32, device="cuda")
    k = torch.zeros((n_kv, hd), dtype=torch.float16, device="cuda")
    v = torch.zeros((n_kv, hd), dtype=torch.float16, device="cuda")
    out = torch.zeros((n_tok, n_head, hd), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    status = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            try:
                F.fr_decode_attn_ex(q, F.FR_Q_F32, k, v, None, out, 1, 0, 0, 0, 0, n_head,
                                    n_tok, n_kv, hd, 0.125, DECOMP)
            except F.FrError as e:
                status = e.status
    torch.cuda.synchronize()
    assert status == F.FR_ERR_CAPTURE


def _hip_alloc_range(ptr: int):
    """(base, size) of the live device allocation holding ptr, or None when no
    allocation holds it (hipMemGetAddressRange of the HIP runtime torch loaded)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    st = hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(ptr))
    return (int(base.value or 0), int(size.value)) if st == 0 else None


def test_graph_survives_workspace_growth():
    """A graph captured after a reserve keeps working after a larger eager call
    has grown the library workspace: the outgrown buffer is retired, not freed
    (FlashRT-llama.cpp development guide, 'Caches (all capture-safe)')."""
    import gqa_decode_attention_fr_amd as F
    say("graph across workspace growth")
    torch.cuda.synchronize()
    F.fr_decode_attn_workspace_release()
    assert F.fr_decode_attn_workspace_query() == (0, 0, 0)
    w = W.H16_HD128_Q16
    g = W.generate(w)
    F.fr_decode_attn_reserve(1, w.n_head, w.n_tok, w.n_kv, w.hd)
    p0, n0, r0 = F.fr_decode_attn_workspace_query()
    assert p0 != 0 and n0 >= F.fr_decode_attn_workspace_size(1, w.n_head, w.n_tok, w.n_kv, w.hd)
    assert r0 == 0
    q, k, v, m = (dev(g[x][0], torch) for x in ("q", "k", "v", "mask"))
    out = torch.zeros((w.n_tok, w.n_head, w.hd), dtype=torch.float32, device="cuda")

    def call():
        F.fr_decode_attn_q16(q, k, v, m, out, w.n_head, w.n_tok, w.n_kv, w.hd, w.scale)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # an eager call with a larger workspace grows the library's buffer
    big = dict(n_head=32, n_tok=16, n_kv=32768, hd=128)
    need_big = F.fr_decode_attn_workspace_size(1, *big.values())
    assert need_big > n0
    bq = torch.zeros((big["n_tok"], big["n_head"], big["hd"]), dtype=torch.float32, device="cuda")
    bk = torch.zeros((big["n_kv"], big["hd"]), dtype=torch.float16, device="cuda")
    bo = torch.empty_like(bq)
    F.fr_decode_attn(bq, bk, bk, None, bo, big["n_head"], big["n_tok"], big["n_kv"], big["hd"],
                     0.088)
    torch.cuda.synchronize()
    p1, n1, r1 = F.fr_decode_attn_workspace_query()
    assert p1 != p0 and n1 >= need_big and r1 == 1
    # the retired buffer is still a live allocation of its full size
    rng = _hip_alloc_range(p0)
    assert rng is not None and rng[0] == p0 and rng[1] >= n0
    # fresh allocations in between may take any freed memory
    junk = [torch.full((4 << 20,), float("nan"), device="cuda") for _ in range(8)]
    for it in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {it} after growth"
        call()   # eager work between replays (uses the grown buffer)
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    del junk, graph
