"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, rejects bad arguments before any HIP call, and plans sensibly."""
import ctypes
import os
import re
import subprocess

import pytest

from gqa_decode_attention_fr_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fr_decode_attn.h")

# Fake but 256-byte-aligned device addresses: calls that fail validation never
# touch them, and these tests only make calls that fail validation.
Q, K, V, MASK, OUT = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fr_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    declared = header_functions()
    assert set(declared) == set(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", out, re.M), name


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_is_plain_c(tmp_path, lang):
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "fr_decode_attn.h"\nint main(void){return fr_abi_version();}\n')
    cc = "gcc" if lang == "c" else "g++"
    subprocess.run([cc, "-fsyntax-only", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}",
                    str(src)], check=True)


def test_abi_version_and_status_strings():
    assert B.fr_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert B.fr_status_str(st).startswith("FR_")
    assert "unknown" in B.fr_status_str(7)


def call(**kw):
    a = dict(q=Q, fmt=B.FR_Q_F32, k=K, v=V, mask=MASK, out=OUT, n_inst=1, qs=0, kvs=0, ms=0,
             os_=0, n_head=8, n_tok=10, n_kv=1024, hd=256, scale=0.0625, flags=0, ws=None,
             ws_bytes=0)
    a.update(kw)
    return B.load().fr_decode_attn_ex(a["q"], a["fmt"], a["k"], a["v"], a["mask"], a["out"],
                                      a["n_inst"], a["qs"], a["kvs"], a["ms"], a["os_"],
                                      a["n_head"], a["n_tok"], a["n_kv"], a["hd"], a["scale"],
                                      a["flags"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.FR_ERR_INVALID),
    (dict(k=None), B.FR_ERR_INVALID),
    (dict(v=None), B.FR_ERR_INVALID),
    (dict(out=None), B.FR_ERR_INVALID),
    (dict(n_tok=0), B.FR_ERR_INVALID),
    (dict(n_kv=0), B.FR_ERR_INVALID),
    (dict(n_head=0), B.FR_ERR_INVALID),
    (dict(n_inst=0), B.FR_ERR_INVALID),
    (dict(n_tok=65), B.FR_ERR_UNSUPPORTED),
    (dict(n_tok=64, n_kv=1 << 25), B.FR_ERR_UNSUPPORTED),  # mask offsets past 2^31 bytes
    (dict(n_kv=(1 << 26) + 1), B.FR_ERR_UNSUPPORTED),
    (dict(hd=96), B.FR_ERR_UNSUPPORTED),
    (dict(hd=512), B.FR_ERR_UNSUPPORTED),
    (dict(n_head=1025), B.FR_ERR_UNSUPPORTED),
    (dict(q=Q + 8), B.FR_ERR_INVALID),
    (dict(k=K + 2), B.FR_ERR_INVALID),
    (dict(out=OUT + 4), B.FR_ERR_INVALID),
    (dict(mask=MASK + 1), B.FR_ERR_INVALID),
    (dict(out=Q), B.FR_ERR_INVALID),                       # out aliases q
    (dict(out=K + 0x1000), B.FR_ERR_INVALID),              # out inside k
    (dict(scale=float("nan")), B.FR_ERR_INVALID),
    (dict(scale=float("inf")), B.FR_ERR_INVALID),
    (dict(flags=0x80), B.FR_ERR_INVALID),
    (dict(flags=B.FR_VARIANT_FUSED | B.FR_VARIANT_DECOMPOSED), B.FR_ERR_INVALID),
    (dict(fmt=B.FR_Q_F16, flags=B.FR_Q_ROUND_F16), B.FR_ERR_INVALID),
    (dict(fmt=2), B.FR_ERR_INVALID),
    (dict(n_inst=2, os_=100), B.FR_ERR_INVALID),           # out stride < M*hd
    (dict(n_inst=2, os_=8 * 10 * 256, kvs=5), B.FR_ERR_INVALID),  # kv stride breaks alignment
    (dict(n_inst=2, os_=8 * 10 * 256, ms=-1), B.FR_ERR_INVALID),
    (dict(ws=0x900000, ws_bytes=16), B.FR_ERR_WORKSPACE),  # caller workspace too small
    # a caller workspace the kernels would write over an input or the output
    # (the plan's workspace here is about 1.3 MB: each range below starts in or
    # just before the named tensor)
    (dict(ws=Q, ws_bytes=1 << 24), B.FR_ERR_INVALID),            # from q on
    (dict(ws=0x280000, ws_bytes=1 << 24), B.FR_ERR_INVALID),     # from v on (k ends there)
    (dict(ws=0x3F0000, ws_bytes=1 << 24), B.FR_ERR_INVALID),     # from the mask on
    (dict(ws=0x4FFF00, ws_bytes=1 << 24), B.FR_ERR_INVALID),     # over out
])
def test_rejected_before_any_launch(kw, status):
    assert call(**kw) == status


def gqa_call(**kw):
    a = dict(q=Q, fmt=B.FR_Q_F32, k=K, v=V, mask=MASK, out=OUT, n_inst=1, qs=0, kvs=0, ms=0,
             os_=0, n_head=8, n_kvh=2, kvhs=1024 * 128, n_tok=4, n_kv=1024, hd=128,
             scale=0.088, flags=0, ws=None, ws_bytes=0, kvl=None)
    a.update(kw)
    return B.load().fr_decode_attn_gqa(a["q"], a["fmt"], a["k"], a["v"], a["mask"], a["kvl"],
                                       a["out"],
                                       a["n_inst"], a["qs"], a["kvs"], a["ms"], a["os_"],
                                       a["n_head"], a["n_kvh"], a["kvhs"], a["n_tok"], a["n_kv"],
                                       a["hd"], a["scale"], a["flags"], a["ws"], a["ws_bytes"],
                                       None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_kvh=0), B.FR_ERR_INVALID),
    (dict(n_kvh=3), B.FR_ERR_INVALID),                       # does not divide n_head
    (dict(n_kvh=16), B.FR_ERR_INVALID),
    (dict(kvhs=1024 * 128 - 8), B.FR_ERR_INVALID),           # heads would overlap
    (dict(kvhs=1024 * 128 + 4), B.FR_ERR_INVALID),           # breaks 16-byte alignment
    (dict(n_inst=2, os_=32 * 128, kvs=1024 * 128), B.FR_ERR_INVALID),  # instance < 2 heads
    (dict(out=K + 1024 * 128 * 2), B.FR_ERR_INVALID),        # out inside the second KV head
    (dict(n_tok=65), B.FR_ERR_UNSUPPORTED),
    (dict(q=None), B.FR_ERR_INVALID),
    (dict(kvl=0x600002), B.FR_ERR_INVALID),                  # misaligned key counts
    (dict(kvl=OUT + 64), B.FR_ERR_INVALID),                  # key counts inside out
    (dict(kvl=0x900100, ws=0x900000, ws_bytes=1 << 20), B.FR_ERR_INVALID),  # ... in the workspace
    (dict(ws=K + 0x40000, ws_bytes=1 << 20), B.FR_ERR_INVALID),  # workspace over k
])
def test_gqa_rejected_before_any_launch(kw, status):
    assert gqa_call(**kw) == status


def noalloc_call(**kw):
    a = dict(q=Q, fmt=B.FR_Q_F32, k=K, v=V, mask=MASK, out=OUT, n_inst=1, qs=0, kvs=0, ms=0,
             os_=0, n_head=8, n_kvh=1, kvhs=0, n_tok=10, n_kv=1024, hd=256, scale=0.0625,
             flags=0, kvl=None)
    a.update(kw)
    return B.load().fr_decode_attn_gqa_noalloc(a["q"], a["fmt"], a["k"], a["v"], a["mask"],
                                               a["kvl"], a["out"], a["n_inst"], a["qs"],
                                               a["kvs"], a["ms"], a["os_"], a["n_head"],
                                               a["n_kvh"], a["kvhs"], a["n_tok"], a["n_kv"],
                                               a["hd"], a["scale"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.FR_ERR_INVALID),
    (dict(out=Q), B.FR_ERR_INVALID),
    (dict(n_tok=65), B.FR_ERR_UNSUPPORTED),
    (dict(n_kvh=3), B.FR_ERR_INVALID),
    (dict(flags=0x80), B.FR_ERR_INVALID),
    (dict(kvl=OUT), B.FR_ERR_INVALID),
    # plans whose partials exceed the fixed 32 MiB array: declined before any HIP call
    # (fake addresses 1 GiB apart: these tensors are large)
    (dict(q=1 << 30, k=2 << 30, v=3 << 30, out=4 << 30, mask=None, n_head=32, n_tok=16,
          n_kv=1 << 20, hd=128, flags=B.FR_VARIANT_DECOMPOSED), B.FR_ERR_WORKSPACE),
    (dict(q=1 << 30, k=2 << 30, v=3 << 30, out=4 << 30, mask=None, n_head=64, n_tok=16,
          n_kv=65536, hd=256), B.FR_ERR_WORKSPACE),
])
def test_noalloc_rejected_before_any_launch(kw, status):
    assert noalloc_call(**kw) == status


def test_noalloc_limit_matches_workspace_sizes():
    """The workloads this library measures all fit the fixed array."""
    for shape in [(18, 8, 10, 1024, 256), (1, 16, 16, 4096, 128), (1, 8, 16, 2048, 256),
                  (1, 32, 16, 32768, 128), (64, 4, 4, 4096, 128)]:
        assert B.fr_decode_attn_workspace_size(*shape) <= B.FR_NOALLOC_SCRATCH_BYTES, shape


def test_gqa_with_one_kv_head_validates_like_ex():
    # one KV head ignores the head stride; the rest of the checks are shared
    for kw in (dict(n_tok=65), dict(hd=96), dict(out=Q), dict(scale=float("nan"))):
        a = dict(kw)
        assert gqa_call(n_kvh=1, kvhs=-5, **a) == call(**a)


def test_single_entry_points_validate_too():
    lib = B.load()
    assert lib.fr_decode_attn(None, K, V, MASK, OUT, 8, 1, 64, 256, 0.0625, None) == B.FR_ERR_INVALID
    assert lib.fr_decode_attn_q16(Q, K, V, MASK, OUT, 8, 65, 64, 256, 0.0625, None) == \
        B.FR_ERR_UNSUPPORTED
    assert lib.fr_decode_attn_batched(Q, B.FR_Q_F32, K, V, MASK, OUT, 3, 0, 0, 0, 16, 8, 1, 64,
                                      256, 0.0625, None) == B.FR_ERR_INVALID


SHAPES = [(1, 8, 1, 64, 256), (18, 8, 10, 1024, 256), (1, 16, 16, 4096, 128),
          (1, 8, 16, 2048, 256), (1, 32, 16, 32768, 128), (3, 5, 7, 1000, 64), (1, 1, 1, 1, 64),
          (1, 8, 24, 2000, 256), (2, 4, 64, 4096, 128), (1, 1, 17, 77, 64)]
SHAPES_80 = [(1, 8, 10, 1000, 80), (2, 16, 256, 256, 80)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("flags", [0, B.FR_VARIANT_DECOMPOSED])
def test_plan_covers_keys_and_rows(shape, flags):
    n_inst, n_head, n_tok, n_kv, hd = shape
    p = B.fr_decode_attn_plan(*shape, flags)
    M = n_head * n_tok
    assert p["variant"] == (2 if flags else 1)
    assert p["chunk"] % 64 == 0
    assert p["n_split"] * p["chunk"] >= n_kv > (p["n_split"] - 1) * p["chunk"]  # no empty split
    assert p["waves"] * p["tiles"] * 16 * p["n_rowblk"] >= M
    assert p["grid"] == n_inst * p["n_rowblk"] * p["n_split"]
    tiles_total = -(-M // 16)
    if flags:
        assert p["waves"] == 4 and p["tiles"] == {256: 1, 128: 2, 80: 4, 64: 4}[hd]
    else:
        # 8 waves above 16 tiles, and for more tokens than 4 waves stage mask rows for
        assert p["tiles"] == 1 and p["waves"] == (4 if tiles_total <= 16 and n_tok <= 16 else 8)
        # one workgroup per compute unit at most, unless instances x row blocks exceed it
        assert p["grid"] <= max(256, n_inst * p["n_rowblk"])
    ws = B.fr_decode_attn_workspace_size(*shape, flags)
    if flags == 0:
        rows = n_inst * p["n_split"] * M
        assert ws == (0 if p["n_split"] == 1 else -(-(rows * hd * 4 + rows * 8) // 256) * 256)
        assert B.fr_decode_attn_plan(*shape, B.FR_Q_ROUND_F16) == p   # format-independent
        assert B.fr_decode_attn_workspace_size(*shape, B.FR_Q_ROUND_F16) == ws
        assert p["launches"] == (1 if p["n_split"] == 1 else 2)
    else:
        assert ws >= n_inst * M * n_kv * 6 and p["launches"] >= 3


@pytest.mark.parametrize("shape,want", [
    # (n_inst, n_head, n_tok, n_kv, hd) -> (waves, row blocks, splits, keys per split)
    ((18, 8, 10, 1024, 256), (4, 2, 6, 192)),     # 36 row blocks: 7 splits fit, 3 blocks each
    # 16 tiles: 4-tile row blocks and 2-block splits would leave 128 workgroups,
    # so 2-tile row blocks: 8 x 32 = 256
    ((1, 16, 16, 4096, 128), (4, 8, 32, 128)),
    # 8 tiles, 32 key blocks: 4-tile row blocks give 64 workgroups, 2-tile ones 128
    ((1, 8, 16, 2048, 256), (4, 4, 32, 64)),
    ((1, 32, 16, 32768, 128), (8, 4, 64, 512)),   # 32 tiles: 8 waves, 256 workgroups
    ((1, 8, 1, 64, 256), (4, 1, 1, 64)),
])
def test_plan_shapes(shape, want):
    p = B.fr_decode_attn_plan(*shape, 0)
    assert (p["waves"], p["n_rowblk"], p["n_split"], p["chunk"]) == want


@pytest.mark.parametrize("shape", SHAPES_80)
@pytest.mark.parametrize("flags", [0, B.FR_VARIANT_DECOMPOSED])
def test_plan_covers_keys_and_rows_at_hd80(shape, flags):
    n_inst, n_head, n_tok, n_kv, hd = shape
    p = B.fr_decode_attn_plan(*shape, flags)
    assert p["variant"] == (2 if flags else 1)
    assert p["tiles"] == (4 if flags else 1)
    assert p["n_split"] * p["chunk"] >= n_kv > (p["n_split"] - 1) * p["chunk"]
    assert p["waves"] * p["tiles"] * 16 * p["n_rowblk"] >= n_head * n_tok
    rows = n_inst * p["n_split"] * n_head * n_tok
    if not flags:   # partials of 80 columns
        ws = B.fr_decode_attn_workspace_size(*shape, B.FR_PLAN_UNMASKED)
        plan_u = B.fr_decode_attn_plan(*shape, B.FR_PLAN_UNMASKED)
        rows_u = n_inst * plan_u["n_split"] * n_head * n_tok
        assert ws == (0 if plan_u["n_split"] == 1 else -(-(rows_u * 80 * 4 + rows_u * 8) // 256) * 256)
    assert rows >= 0


def test_unmasked_prefill_plans_four_wave_row_blocks():
    """An unmasked call with many rows (the prefill) plans 4-wave row blocks
    and fewer key splits; masked calls keep their plan; the workspace size
    without the bit covers both."""
    shape = (1, 8, 968, 1024, 256)
    masked = B.fr_decode_attn_plan(*shape, 0)
    unmasked = B.fr_decode_attn_plan(*shape, B.FR_PLAN_UNMASKED)
    assert (masked["waves"], masked["n_split"]) == (8, 4)
    assert (unmasked["waves"], unmasked["n_split"], unmasked["n_rowblk"]) == (4, 2, 121)
    both = B.fr_decode_attn_workspace_size(*shape, 0)
    only = B.fr_decode_attn_workspace_size(*shape, B.FR_PLAN_UNMASKED)
    rows = 8 * 968
    assert only == -(-(2 * rows * 256 * 4 + 2 * rows * 8) // 256) * 256
    assert both == -(-(4 * rows * 256 * 4 + 4 * rows * 8) // 256) * 256 >= only
    # few rows: the bit changes nothing; more than 16 tokens unmasked may stay at 4 waves
    assert B.fr_decode_attn_plan(18, 8, 10, 1024, 256, B.FR_PLAN_UNMASKED) == \
        B.fr_decode_attn_plan(18, 8, 10, 1024, 256, 0)
    assert B.fr_decode_attn_plan(1, 1, 40, 500, 128, B.FR_PLAN_UNMASKED)["waves"] == 4
    assert B.fr_decode_attn_plan(1, 1, 40, 500, 128, 0)["waves"] == 8


def test_head_size_80_plans():
    assert B.fr_decode_attn_plan(1, 8, 10, 1000, 80, 0)["variant"] == 1
    assert B.fr_decode_attn_plan(1, 8, 10, 1000, 80, B.FR_VARIANT_DECOMPOSED)["variant"] == 2
    ws = B.fr_decode_attn_workspace_size(1, 8, 10, 1000, 80, B.FR_VARIANT_DECOMPOSED)
    assert ws >= 80 * 1024 * 6


def test_unmasked_calls_take_long_query_counts():
    # a masked call stops at 64 tokens; an unmasked one (prefill) goes on
    assert call(n_tok=65) == B.FR_ERR_UNSUPPORTED
    assert call(n_tok=16385, mask=None) == B.FR_ERR_UNSUPPORTED
    assert call(n_tok=968, mask=None, out=0x900000, flags=0x80) == B.FR_ERR_INVALID  # sizes ok
    p = B.fr_decode_attn_plan(1, 8, 968, 968, 256, 0)
    assert p["waves"] == 8 and p["n_rowblk"] * 8 * 16 >= 8 * 968


def test_many_tokens_take_eight_waves(monkeypatch):
    monkeypatch.setenv("FR_FORCE_WAVES", "4")
    assert B.fr_decode_attn_plan(1, 8, 16, 1024, 256, 0)["waves"] == 4
    assert B.fr_decode_attn_plan(1, 8, 17, 1024, 256, 0)["waves"] == 8
    assert B.fr_decode_attn_plan(1, 2, 64, 1024, 128, 0)["waves"] == 8


def test_forced_split_count(monkeypatch):
    monkeypatch.setenv("FR_FORCE_SPLITS", "4")
    p = B.fr_decode_attn_plan(18, 8, 10, 1024, 256, 0)
    assert p["n_split"] == 4 and p["chunk"] == 256


def test_sizes_rejected_by_helpers():
    with pytest.raises(B.FrError) as e:
        B.fr_decode_attn_workspace_size(1, 8, 16385, 64, 256)
    assert e.value.status == B.FR_ERR_UNSUPPORTED
    info = (ctypes.c_int * 8)()
    assert B.load().fr_decode_attn_plan(1, 8, 1, 64, 96, 0, info, 8) == B.FR_ERR_UNSUPPORTED


def copy_call(entries, n=None):
    arr = (B.F16Copy * max(1, len(entries)))()
    for i, (s, d, cnt) in enumerate(entries):
        arr[i] = B.F16Copy(s, d, cnt)
    return B.load().fr_f16_copy_batch(arr, len(entries) if n is None else n, None)


@pytest.mark.parametrize("entries,n,status", [
    ([], -1, B.FR_ERR_INVALID),
    ([(Q, K, 16)], 4097, B.FR_ERR_INVALID),                 # above FR_MAX_COPIES
    ([(Q, K, -1)], None, B.FR_ERR_INVALID),
    ([(None, K, 16)], None, B.FR_ERR_INVALID),
    ([(Q, None, 16)], None, B.FR_ERR_INVALID),
    ([(Q + 2, K, 16)], None, B.FR_ERR_INVALID),             # src not 4-byte aligned
    ([(Q, K + 1, 16)], None, B.FR_ERR_INVALID),             # dst not 2-byte aligned
    ([(Q, Q + 8, 16)], None, B.FR_ERR_INVALID),             # dst overlaps its source
    ([(Q, K, 16), (V, K + 16, 16)], None, B.FR_ERR_INVALID),  # two destinations overlap
    ([(Q, K, 16), (V, Q + 60, 16)], None, B.FR_ERR_INVALID),  # dst over another source
    ([], 0, B.FR_OK),                                        # nothing to do, no launch
    ([(None, None, 0), (Q, None, 0)], None, B.FR_OK),        # empty copies are skipped
])
def test_copy_batch_validation(entries, n, status):
    assert copy_call(entries, n) == status


def test_copy_batch_null_array():
    assert B.load().fr_f16_copy_batch(None, 3, None) == B.FR_ERR_INVALID


def qkv_call(**kw):
    a = dict(qkv=Q, pos=MASK, q16=OUT, kc=K, vc=V, n_inst=1, qs=0, ps=0, q16s=0, cs=0,
             chs=0, n_head=8, n_kvh=1, n_tok=10, hd=256, cap=1024, base=10000.0, qscale=0.0625)
    a.update(kw)
    return B.load().fr_qkv_post(a["qkv"], a["pos"], a["q16"], a["kc"], a["vc"], a["n_inst"],
                                a["qs"], a["ps"], a["q16s"], a["cs"], a["chs"], a["n_head"],
                                a["n_kvh"], a["n_tok"], a["hd"], a["cap"], a["base"],
                                a["qscale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), B.FR_ERR_INVALID),
    (dict(pos=None), B.FR_ERR_INVALID),
    (dict(q16=None), B.FR_ERR_INVALID),
    (dict(vc=None), B.FR_ERR_INVALID),                      # K cache without V cache
    (dict(hd=96), B.FR_ERR_UNSUPPORTED),
    (dict(n_tok=16385), B.FR_ERR_UNSUPPORTED),
    (dict(base=0.0), B.FR_ERR_INVALID),
    (dict(base=float("inf")), B.FR_ERR_INVALID),
    (dict(qscale=float("nan")), B.FR_ERR_INVALID),
    (dict(cap=0), B.FR_ERR_INVALID),
    (dict(n_kvh=2, chs=100), B.FR_ERR_INVALID),              # KV heads would overlap
    (dict(n_inst=2, qs=10, q16s=8 * 10 * 256, cs=1 << 20), B.FR_ERR_INVALID),
    (dict(q16=Q + 64), B.FR_ERR_INVALID),                    # q16 overlaps qkv
    (dict(kc=OUT + 4096), B.FR_ERR_INVALID),                 # K cache overlaps q16
])
def test_qkv_post_rejected_before_any_launch(kw, status):
    assert qkv_call(**kw) == status


def test_copy_batch_overlap_check_scales():
    """4096 copies, the only overlap between the first and the last destination
    (far apart in the list): rejected, and quickly (the check sorts the ranges
    instead of comparing every pair)."""
    import time
    n = 4096
    entries = [(0x10000000 + i * 0x1000, 0x40000000 + i * 0x1000, 256) for i in range(n)]
    entries[-1] = (entries[-1][0], entries[0][1] + 64, 256)     # lands inside destination 0
    t = time.perf_counter()
    assert copy_call(entries) == B.FR_ERR_INVALID
    assert time.perf_counter() - t < 0.5


def test_plain_c_consumer_compiles_and_links(tmp_path):
    """tests/c_consumer.c (run on the GPU by test_gpu_c_consumer.py) builds
    against the header and the library with gcc alone."""
    from c_consumer_build import build_consumer
    if not os.path.exists(os.path.join("/opt/rocm", "lib", "libamdhip64.so")):
        pytest.skip("HIP runtime not installed")
    exe = build_consumer(tmp_path / "c_consumer")
    assert os.path.getsize(exe) > 0


def test_binding_constants_match_the_header():
    """Every FR_ constant the binding mirrors has the header's value."""
    text = open(HEADER).read()
    defs = {m.group(1): int(m.group(2), 0)
            for m in re.finditer(r"#define\s+(FR_\w+)\s+(0x[0-9a-fA-F]+|\d+)u?\b", text)}
    enums = {m.group(1): int(m.group(2))
             for m in re.finditer(r"\b(FR_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text)}
    both = {**defs, **enums}
    mirrored = [n for n in dir(B) if n.startswith("FR_") and isinstance(getattr(B, n), int)]
    assert {"FR_MAX_TOKENS", "FR_MAX_TOKENS_UNMASKED", "FR_MAX_HEADS", "FR_PLAN_UNMASKED"} <= set(mirrored)
    for n in mirrored:
        assert n in both, n
        assert getattr(B, n) == both[n], n


def test_plan_invariants_over_random_shapes():
    """Seeded random shapes, masked and unmasked plans of the fused variant:
    every key and row is covered with no empty split, the grid is what the
    plan says, the wave rules hold, and the default workspace size covers
    both plans' partials."""
    import numpy as np
    rng = np.random.default_rng(77)
    for _ in range(600):
        n_inst = int(rng.integers(1, 65))
        n_head = int(rng.integers(1, 129))
        unmasked = bool(rng.random() < 0.5)
        n_tok = int(rng.integers(1, 4097 if unmasked else 65))
        n_kv = int(rng.integers(1, 100_001))
        hd = int(rng.choice([64, 80, 128, 256]))
        if n_inst * n_head * n_tok > (1 << 24):
            continue
        shape = (n_inst, n_head, n_tok, n_kv, hd)
        flags = B.FR_PLAN_UNMASKED if unmasked else 0
        p = B.fr_decode_attn_plan(*shape, flags)
        M = n_head * n_tok
        tiles_total = -(-M // 16)
        assert p["variant"] == 1 and p["tiles"] == 1 and p["waves"] in (4, 8), shape
        assert p["chunk"] % 64 == 0, shape
        assert p["n_split"] * p["chunk"] >= n_kv > (p["n_split"] - 1) * p["chunk"], shape
        assert p["n_rowblk"] * p["waves"] * 16 >= M, shape
        assert p["n_rowblk"] <= tiles_total, shape                      # no empty row block
        assert p["grid"] == n_inst * p["n_rowblk"] * p["n_split"], shape
        assert p["grid"] <= max(256, n_inst * p["n_rowblk"]), shape
        if not unmasked and n_tok > 16:
            assert p["waves"] == 8, shape                              # mask rows for 64 tokens
        if tiles_total <= 16 and n_tok <= 16:
            assert p["waves"] == 4, shape
        need = 0 if p["n_split"] == 1 else n_inst * p["n_split"] * M * (hd * 4 + 8)
        assert B.fr_decode_attn_workspace_size(*shape, flags) >= need, shape
        assert B.fr_decode_attn_workspace_size(*shape, 0) >= need, shape  # covers both plans
