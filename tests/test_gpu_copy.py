"""GPU parity of the batched f32 -> f16 row copies (fr_f16_copy_batch) against
the oracle's nearest-even rounding, bit for bit: every finite binary16 value,
every tie between neighbours and the values next to them, the overflow and
subnormal boundaries, signed zeros and infinities; ragged lengths, unaligned
pointers (the element path), more copies than one launch carries, empty
copies, guard bands around every destination, and graph replay."""
import numpy as np
import pytest

from gpu_util import say

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


def special_values(seed=0):
    f16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.arange(1, 0x7C01, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((f16 + nxt) / 2.0).astype(np.float32)          # exact ties in f32
    rng = np.random.default_rng(seed)
    vals = np.concatenate([
        f16.astype(np.float32), -f16.astype(np.float32), mids, -mids,
        np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
        np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.996, 65520.0, 1e30, -1e30,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1e-30, -1e-30],
                 dtype=np.float32),
        (rng.standard_normal(50000) * 10.0 ** rng.integers(-8, 5, 50000)).astype(np.float32),
    ])
    return vals


def run_copies(pieces, offsets, guard=64):
    """Copies piece i (float32 numpy) into its own destination region of one
    uint16 buffer, starting `offsets[i]` elements into a source buffer and a
    destination region (offsets that are not multiples of 4 / 8 break 16-byte
    alignment).  Returns (outputs, guard bands intact)."""
    import gqa_decode_attention_fr_amd as F
    src_tot = sum(o + len(p) + 8 for p, o in zip(pieces, offsets))
    dst_tot = sum(guard + o + len(p) + guard for p, o in zip(pieces, offsets))
    src = torch.zeros(src_tot, dtype=torch.float32, device="cuda")
    dst = torch.full((dst_tot,), CANARY, dtype=torch.int16, device="cuda")
    copies, spans = [], []
    s_at = d_at = 0
    for p, o in zip(pieces, offsets):
        src[s_at + o:s_at + o + len(p)] = torch.from_numpy(p).cuda()
        d0 = d_at + guard + o
        copies.append((src.data_ptr() + 4 * (s_at + o), dst.data_ptr() + 2 * d0, len(p)))
        spans.append((d0, len(p)))
        s_at += o + len(p) + 8
        d_at += guard + o + len(p) + guard
    F.fr_f16_copy_batch(copies)
    torch.cuda.synchronize()
    host = dst.cpu().numpy().view(np.uint16)
    outs = [host[d0:d0 + n] for d0, n in spans]
    written = np.zeros(dst_tot, dtype=bool)
    for d0, n in spans:
        written[d0:d0 + n] = True
    guards_ok = bool((host[~written] == CANARY).all())
    return outs, guards_ok


def test_every_rounding_case_bitwise(oracle_mod):
    say("f16 copy: rounding cases")
    vals = special_values()
    cuts = [0, 1, 7, 8, 9, 1000, 65537, len(vals) // 2, len(vals)]
    pieces = [vals[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    offsets = [0, 1, 3, 8, 5, 0, 2, 0]       # several pieces take the element path
    outs, guards_ok = run_copies(pieces, offsets)
    assert guards_ok
    for i, (p, got) in enumerate(zip(pieces, outs)):
        want = oracle_mod.f16_copy(p)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (f"piece {i}: {bad.size} differ, first x={p[bad[0]]!r} "
                               f"got {got[bad[0]]:#06x} want {want[bad[0]]:#06x}")


def test_more_copies_than_one_launch_and_empty_ones(oracle_mod):
    say("f16 copy: 150 copies")
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 3000, 150)]
    lens[3] = lens[70] = 0
    pieces = [(rng.standard_normal(n) * 3).astype(np.float32) for n in lens]
    offsets = [int(x) for x in rng.integers(0, 9, 150)]
    outs, guards_ok = run_copies(pieces, offsets)
    assert guards_ok
    for p, got in zip(pieces, outs):
        assert np.array_equal(got, oracle_mod.f16_copy(p))


def test_pi05_encoder_kv_tail_copies(oracle_mod):
    """The pages' case: per layer, the K and V rows of the 968-token prefix into
    f16 buffers: 18 layers x 2 tensors in one call."""
    import gqa_decode_attention_fr_amd as F
    say("f16 copy: 36 encoder KV tensors")
    rng = np.random.default_rng(7)
    srcs = [torch.from_numpy((rng.standard_normal((968, 256)) * 0.5).astype(np.float32)).cuda()
            for _ in range(36)]
    dsts = [torch.empty((1024, 256), dtype=torch.float16, device="cuda") for _ in range(36)]
    F.fr_f16_copy_batch([(s, d, s.numel()) for s, d in zip(srcs, dsts)])
    torch.cuda.synchronize()
    for s, d in zip(srcs, dsts):
        got = d[:968].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle_mod.f16_copy(s.cpu().numpy()))


def test_graph_replay_equals_eager():
    import gqa_decode_attention_fr_amd as F
    say("f16 copy: graph replay")
    rng = np.random.default_rng(9)
    srcs = [torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
            for n in (4096, 777, 8)]
    dsts = [torch.zeros(s.numel(), dtype=torch.float16, device="cuda") for s in srcs]

    def call():
        F.fr_f16_copy_batch([(s, d, s.numel()) for s, d in zip(srcs, dsts)])

    call()
    torch.cuda.synchronize()
    eager = [d.clone() for d in dsts]
    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            call()
    torch.cuda.current_stream().wait_stream(st)
    for it in range(3):
        for d in dsts:
            d.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for d, e in zip(dsts, eager):
            assert torch.equal(d.view(torch.int16), e.view(torch.int16)), f"replay {it}"


def test_copies_may_share_a_source(oracle_mod):
    """Sources may overlap (only destinations are checked): three copies of
    one source, and one of its second half, all equal the oracle's rounding."""
    import gqa_decode_attention_fr_amd as F
    say("f16 copy: shared source")
    rng = np.random.default_rng(13)
    src = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).cuda()
    dsts = [torch.zeros(5000, dtype=torch.float16, device="cuda") for _ in range(3)]
    half = torch.zeros(2500, dtype=torch.float16, device="cuda")
    F.fr_f16_copy_batch([(src, d, 5000) for d in dsts] +
                        [(src.data_ptr() + 4 * 2500, half, 2500)])
    torch.cuda.synchronize()
    want = oracle_mod.f16_copy(src.cpu().numpy())
    for d in dsts:
        assert np.array_equal(d.cpu().numpy().view(np.uint16), want)
    assert np.array_equal(half.cpu().numpy().view(np.uint16), want[2500:])
