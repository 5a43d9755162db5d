"""fr_decode_attn_gqa_noalloc, the entry point that allocates nothing: its
split partials live in the library's fixed device array.  Checked through the
C ABI against fr_decode_attn_gqa (same plan, same kernels: bit for bit) and
against the fp64 oracle at the acceptance bar, on two calls in a row, the
second smaller; in graph capture with no reserve; and the size limit."""
import numpy as np
import pytest

from gqa_decode_attention_fr_amd import workloads as W
from gpu_util import assert_close, dev, oracle_gqa, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_fr_amd as F
    F.binding.load()
    yield


def _inputs(w, g):
    """Device tensors of a workload with k, v as [n_inst, n_kv_head, n_kv, hd]."""
    k, v = g["k"], g["v"]
    if w.n_kv_head == 1:
        k, v = k[:, None], v[:, None]
    mask = None if w.mask_kind == "none" else g["mask"]
    return dev(g["q"], torch), dev(k, torch), dev(v, torch), dev(mask, torch), k.shape


def _call(F, entry, w, q, k, v, m, kv_len=None):
    M = w.n_head * w.n_tok
    out = torch.full((w.n_inst, w.n_tok, w.n_head, w.hd), float("nan"), dtype=torch.float32,
                     device="cuda")
    fmt = F.FR_Q_F16 if w.q_dtype == "f16" else F.FR_Q_F32
    kvh_stride = w.n_kv * w.hd
    args = (q, fmt, k, v, m, out, w.n_inst, M * w.hd, w.n_kv_head * kvh_stride,
            0 if m is None else w.n_tok * w.n_kv, M * w.hd, w.n_head, w.n_kv_head, kvh_stride,
            w.n_tok, w.n_kv, w.hd, w.scale, 0)
    if entry == "noalloc":
        F.fr_decode_attn_gqa_noalloc(*args, kv_len=kv_len)
    else:
        F.fr_decode_attn_gqa(*args, kv_len=kv_len)
    return out


@pytest.mark.parametrize("pair", [
    (W.PI05_ACTION_STEP, W.CAUSAL_TAIL),        # 18 instances, then one smaller call
    (W.LONG_CONTEXT, W.GQA_KV8),                # the largest partials, then several KV heads
], ids=lambda p: f"{p[0].name}->{p[1].name}")
def test_two_calls_match_the_workspace_entry(oracle_mod, pair):
    import gqa_decode_attention_fr_amd as F
    for w in pair:
        say(f"noalloc {w.name}")
        assert F.fr_decode_attn_workspace_size(w.n_inst * w.n_kv_head,
                                               w.n_head // w.n_kv_head, w.n_tok, w.n_kv,
                                               w.hd) <= F.FR_NOALLOC_SCRATCH_BYTES
        g = W.generate(w)
        q, k, v, m, _ = _inputs(w, g)
        got = _call(F, "noalloc", w, q, k, v, m)
        ref = _call(F, "gqa", w, q, k, v, m)
        torch.cuda.synchronize()
        got, ref = got.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref), f"{w.name}: noalloc differs from the workspace entry"
        q_kind = oracle_mod.Q_F16 if w.q_dtype == "f16" else oracle_mod.Q_F32
        n_check = min(w.n_inst, 2)   # the oracle on the first instances (seconds)
        sub = {x: g[x][:n_check] for x in ("q", "k", "v", "mask")}
        want = oracle_gqa(oracle_mod, sub, w.n_head, w.n_kv_head, w.n_tok, w.n_kv, w.hd,
                          w.scale, q_kind)
        assert_close(got[:n_check], want, w.name)


def test_device_key_counts_and_repeat():
    """Device-side valid counts through the fixed array, twice (the array keeps
    the last call's contents; every partial read is written first)."""
    import gqa_decode_attention_fr_amd as F
    w = W.GQA_DECODE_T1
    say(f"noalloc kv_len {w.name}")
    g = W.generate(w)
    q, k, v, m, _ = _inputs(w, g)
    lens = torch.tensor([4096, 1, 0, 2000, 4095, 64, 65, 3000], dtype=torch.int32,
                        device="cuda")
    a = _call(F, "noalloc", w, q, k, v, m, kv_len=lens)
    b = _call(F, "gqa", w, q, k, v, m, kv_len=lens)
    c = _call(F, "noalloc", w, q, k, v, m, kv_len=lens)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_graph_capture_without_reserve():
    """Captured with no reserve (nothing to allocate), replayed several times with
    eager calls in between: every replay equals the eager result."""
    import gqa_decode_attention_fr_amd as F
    w = W.H16_HD128_Q16
    say(f"noalloc capture {w.name}")
    g = W.generate(w)
    q, k, v, m, _ = _inputs(w, g)
    M = w.n_head * w.n_tok
    out = torch.zeros((w.n_inst, w.n_tok, w.n_head, w.hd), dtype=torch.float32, device="cuda")

    def call():
        F.fr_decode_attn_gqa_noalloc(q, F.FR_Q_F16, k, v, m, out, 1, 0, 0, 0, 0, w.n_head, 1, 0,
                                     w.n_tok, w.n_kv, w.hd, w.scale, 0)

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
    for it in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {it}"
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    del graph


def test_oversized_call_is_declined():
    import gqa_decode_attention_fr_amd as F
    say("noalloc oversized")
    n_head, n_tok, n_kv, hd = 64, 16, 65536, 256
    assert F.fr_decode_attn_workspace_size(1, n_head, n_tok, n_kv, hd,
                                           F.FR_PLAN_UNMASKED) > F.FR_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((n_tok, n_head, hd), dtype=torch.float32, device="cuda")
    kv = torch.zeros((n_kv, hd), dtype=torch.float16, device="cuda")
    out = torch.full((n_tok, n_head, hd), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(F.FrError) as e:
        F.fr_decode_attn_gqa_noalloc(q, F.FR_Q_F32, kv, kv, None, out, 1, 0, 0, 0, 0, n_head, 1,
                                     0, n_tok, n_kv, hd, 0.0625, 0)
    assert e.value.status == F.FR_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing launched
