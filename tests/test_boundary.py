"""C-ABI boundary on the CPU: the library loads, exports what the header
declares, and rejects every invalid argument before touching the device.

Calls here pass made-up device addresses; every one of them is invalid for
another reason, so nothing is ever enqueued (validation runs before any HIP
call).  The restated rules are those of mlx-native 0.18.0
src/ops/row_exact_matvec.rs validate().
"""
import ctypes
import glob
import json
import os
import re

import pytest

import quantized_few_row_amd as qfr
from quantized_few_row_amd import Schedule, Strides, Weight

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "page_constants.json")))

# Made-up, well-aligned device addresses (never dereferenced).
WP, XP, YP = 0x7F0000000000, 0x7F1000000000, 0x7F2000000000


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(row_exact_[a-z_]+)\s*\(", text, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = qfr.load_library()
    declared = _declared_functions()
    assert len(declared) == 15, declared
    for name in declared:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_binding_names_mirror_the_abi():
    for name in _declared_functions():
        assert callable(getattr(qfr, name)), name


def test_row_bytes_match_page():
    for name, blk in GOLDEN["blocks"].items():
        if name.startswith("_"):
            continue
        for nb in (1, 3, 16, 56):
            assert qfr.row_exact_row_bytes(Weight[name], blk["values"] * nb) == blk["bytes"] * nb
    assert qfr.row_exact_row_bytes(Weight.F16, 512) == 1024
    assert qfr.row_exact_row_bytes(Weight.F32, 512) == 2048
    assert qfr.row_exact_row_bytes(Weight.BF16, 512) == 1024
    assert qfr.row_exact_row_bytes(7, 512) == 0


def test_weight_order_matches_page():
    # the page's five types in its index() order, then the dense extension
    assert [w.name for w in Weight] == GOLDEN["weight_type_order"]["value"] + ["F32", "BF16"]
    assert qfr.MAX_ROWS == GOLDEN["max_rows"]["value"]


def test_stride_helpers_match_page_examples():
    g = GOLDEN["grouped_token_major_example"]
    s = qfr.grouped_token_major(g["m"], g["groups"], g["n"], g["k"])
    assert s.astuple() == tuple(g["strides"][f] for f in ("x_row_stride", "x_batch_stride", "y_row_stride",
                                                            "y_batch_stride"))
    c = GOLDEN["contiguous_example"]
    s = qfr.contiguous(c["m"], c["n"], c["k"])
    assert s.astuple() == tuple(c["strides"][f] for f in ("x_row_stride", "x_batch_stride", "y_row_stride",
                                                            "y_batch_stride"))


def test_required_bytes_is_strided_extent():
    # contiguous: W rows * row_bytes, x m*k floats, y m*n floats
    w, x, y = qfr.row_exact_required_bytes(Weight.Q8_0, 4096, 4096, 8, 1)
    assert (w, x, y) == (4096 * 4352, 8 * 4096 * 4, 8 * 4096 * 4)
    g = GOLDEN["grouped_token_major_example"]
    s = qfr.grouped_token_major(g["m"], g["groups"], g["n"], g["k"])
    w, x, y = qfr.row_exact_required_bytes(Weight.Q5_0, g["n"], g["k"], g["m"], g["groups"], s)
    # last element + 1: (batch-1)*bs + (m-1)*rs + cols
    assert x == 4 * ((g["groups"] - 1) * g["k"] + (g["m"] - 1) * g["groups"] * g["k"] + g["k"])
    assert y == 4 * ((g["groups"] - 1) * g["n"] + (g["m"] - 1) * g["groups"] * g["n"] + g["n"])
    assert x == 4 * g["m"] * g["groups"] * g["k"] and y == 4 * g["m"] * g["groups"] * g["n"]
    assert w == g["groups"] * g["n"] * (g["k"] // 32) * 22


def _mv(wt=Weight.Q8_0, W=WP, x=XP, y=YP, n=64, k=256, m=4, batch=1, strides=None, schedule=None):
    lib = qfr.load_library()
    sp = ctypes.byref(strides) if strides is not None else None
    if schedule is None:
        rc = lib.row_exact_mv(int(wt), W, x, y, n, k, m, batch, sp, None)
    else:
        rc = lib.row_exact_mv_scheduled(int(wt), W, x, y, n, k, m, batch, sp, ctypes.byref(schedule), None)
    return rc, qfr.row_exact_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(m=0), -1, "m = 0: a call takes 1 to 8 input rows"),
    (dict(m=9), -1, "m = 9: a call takes 1 to 8 input rows"),
    (dict(n=0), -1, "every dimension must be at least 1"),
    (dict(k=0), -1, "every dimension must be at least 1"),
    (dict(batch=0), -1, "every dimension must be at least 1"),
    (dict(wt=7), -1, "weight type 7 is not one of"),
    (dict(wt=-1), -1, "weight type -1 is not one of"),
    (dict(wt=Weight.Q8_0, k=48), -1, "divisible by 32"),
    (dict(wt=Weight.Q4_K, k=512 + 32), -1, "divisible by 256"),
    (dict(wt=Weight.Q6_K, k=128), -1, "divisible by 256"),
    (dict(wt=Weight.Q5_0, k=16), -1, "divisible by 32"),
    (dict(wt=Weight.F16, k=6), -1, "divisible by 4"),
    (dict(wt=Weight.F32, k=10), -1, "divisible by 4"),
    (dict(wt=Weight.BF16, k=2), -1, "divisible by 4"),
    (dict(n=1 << 31), -5, "at most 2^31 - 1 weight rows"),
    (dict(n=0xFFFFFFFF), -5, "at most 2^31 - 1 weight rows"),
    (dict(W=0), -1, "non-NULL"),
    (dict(y=0), -1, "non-NULL"),
    (dict(x=XP + 4), -2, "x must sit on a 16-byte boundary"),
    (dict(strides=Strides(258, 0, 64, 0)), -3, "multiples of 4"),
    (dict(strides=Strides(256, 2, 64, 0), batch=2), -3, "multiples of 4"),
    (dict(wt=Weight.Q4_K, W=WP + 4), -2, "16-byte"),
    (dict(wt=Weight.F16, W=WP + 4, k=64), -2, "8-byte"),
    (dict(wt=Weight.BF16, W=WP + 4, k=64), -2, "8-byte"),
    (dict(wt=Weight.F32, W=WP + 8, k=64), -2, "16-byte"),
    (dict(wt=Weight.Q8_0, W=WP + 1), -2, "2-byte"),
    (dict(wt=Weight.Q6_K, W=WP + 3), -2, "2-byte"),
    (dict(wt=Weight.Q5_0, W=WP + 5), -2, "2-byte"),
    (dict(y=YP + 2), -2, "y must sit on a 4-byte boundary"),
])
def test_invalid_arguments(kw, code, text):
    before = qfr.row_exact_launch_count()
    rc, msg = _mv(**kw)
    assert rc == code, (rc, msg)
    assert msg.startswith("row_exact_mv: ") and text in msg, msg
    assert qfr.row_exact_launch_count() == before


@pytest.mark.parametrize("wt,k", [(Weight.Q8_0, 256), (Weight.Q6_K, 512), (Weight.Q5_0, 256)])
def test_two_byte_aligned_weights_pass_the_alignment_check(wt, k):
    # the page's validate() asks 2-byte alignment of these three types; the
    # call is refused afterwards for an unrelated reason (y overlapping W),
    # which shows the alignment was accepted
    for off in (2, 6, 10, 14):
        rc, msg = _mv(wt=wt, W=WP + off, y=WP + 64, k=k)
        assert rc == -4 and "y overlaps the bytes of W" in msg, (off, msg)


# Output layouts: element (b, j, i) at b*y_batch_stride + j*y_row_stride + i.
@pytest.mark.parametrize("m,n,batch,s", [
    # batch 1: rows need y_row_stride >= n
    (4, 64, 1, Strides(256, 0, 63, 0)),
    (2, 64, 1, Strides(256, 0, 0, 0)),
    # m == 1, batch > 1: batches need y_batch_stride >= n
    (1, 64, 3, Strides(256, 256, 0, 63)),
    # token-major (row stride larger): rows must clear every batch entry
    (2, 64, 3, Strides(256, 256, 191, 64)),
    (2, 64, 3, Strides(256, 256, 192, 63)),
    # batch-major (batch stride larger)
    (3, 64, 2, Strides(256, 1024, 64, 191)),
    (3, 64, 2, Strides(256, 1024, 63, 1000)),
    # equal strides with two entries on both axes never nest
    (2, 64, 2, Strides(256, 256, 512, 512)),
    # interleaved rows and entries: n = 1, elements j*3 + b*2 are
    # {0, 2, 4, 3, 5, 7}, all distinct, but the layout does not nest, and the
    # page's rule refuses it too
    (2, 1, 3, Strides(256, 256, 3, 2)),
])
def test_output_layouts_that_do_not_nest_are_refused(m, n, batch, s):
    rc, msg = _mv(m=m, n=n, batch=batch, strides=s)
    assert rc == -4 and "writes some element twice" in msg, msg


@pytest.mark.parametrize("m,n,batch,s", [
    (1, 64, 1, Strides(256, 0, 0, 0)),           # one row: its stride is irrelevant
    (4, 64, 1, Strides(256, 0, 64, 0)),          # contiguous rows
    (1, 64, 3, Strides(256, 256, 0, 64)),        # one row per entry, entries back to back
    (2, 64, 3, Strides(256, 256, 192, 64)),      # token-major, tight
    (3, 64, 2, Strides(256, 1024, 64, 192)),     # batch-major, tight
    (2, 64, 3, Strides(256, 256, 1 << 20, 64)),  # token-major, loose
])
def test_nested_output_layouts_pass_the_layout_check(m, n, batch, s):
    # refused afterwards only because y overlaps W (a different message)
    rc, msg = _mv(m=m, n=n, batch=batch, strides=s, y=WP + 64)
    assert rc == -4 and "y overlaps the bytes of W" in msg, msg


def test_output_must_not_overlap_inputs():
    rc, msg = _mv(y=WP + 64)
    assert rc == -4 and "y overlaps the bytes of W" in msg
    rc, msg = _mv(y=XP + 1024)
    assert rc == -4 and "y overlaps the bytes of W" in msg


@pytest.mark.parametrize("sched,text", [
    (Schedule(3, 1, 8, 1, 1 << 30), "k_split (3) must be 1, 2, 4 or 8"),
    (Schedule(16, 1, 8, 1, 1 << 30), "k_split (16) must be 1, 2, 4 or 8"),
    (Schedule(4, 1, 8, 1, 1 << 30), "k_split (4) exceeds the 2 whole wave steps of a Q8_0 row of k = 4096"),
    (Schedule(2, 1, 3, 1, 1 << 30), "waves_per_workgroup (3) must be a multiple of k_split (2)"),
    (Schedule(2, 1, 8, 1, 1000), "k_chunk (1000) must be >= k (4096) or a multiple of 2048"),
    (Schedule(1, 3, 8, 1, 1 << 30), "rows_per_wave"),
    (Schedule(1, 1, 0, 1, 1 << 30), "waves_per_workgroup"),
    (Schedule(1, 1, 9, 1, 1 << 30), "waves_per_workgroup"),
    (Schedule(1, 1, 8, 0, 1 << 30), "workgroups_per_batch"),
    (Schedule(1, 1, 8, 4, 1000), "k_chunk"),
    (Schedule(1, 1, 8, 4, 1 << 30, 8), "lanes_per_row (8) must be 0 (derived), 16, 32 or 64"),
    (Schedule(1, 1, 8, 4, 1 << 30, 48), "lanes_per_row (48) must be"),
    (Schedule(1, 1, 8, 4, 1 << 30, 128), "lanes_per_row (128) must be"),
    (Schedule(2, 1, 8, 4, 1 << 30, 32), "lanes_per_row (32): a k_split (2) needs 64 lanes per row"),
])
def test_invalid_schedule(sched, text):
    rc, msg = _mv(k=4096, schedule=sched)
    assert rc == -6 and text in msg, msg


def test_k_split_needs_rows_of_64_lanes():
    # F16 rows of k = 256 are 32 pieces (32 lanes per row): never split
    rc, msg = _mv(wt=Weight.F16, k=256, schedule=Schedule(2, 1, 8, 1, 1 << 30))
    assert rc == -6 and "k_split (2): F16 rows of k = 256 (at most 32 pieces) are not split" in msg, msg


def test_lanes_per_row_limited_by_row_offsets():
    # a lane addresses the rows of its wave's slots by 32-bit offsets: (64 /
    # lanes) * rows_per_wave * row bytes must stay below 2^32.  Q8_0 rows of
    # k = 2^28 are 285,212,672 bytes: 16 lanes x 4 rows (16 row offsets) pass
    # 2^32 bytes and are refused; 64 lanes are always fine.
    big = 1 << 28
    rc, msg = _mv(n=8, k=big, m=1, schedule=Schedule(1, 4, 8, 1, 2048, 16))
    assert rc == -6 and "too long for the 32-bit row offsets" in msg, msg
    rc, msg = _mv(n=8, k=big, m=1, schedule=Schedule(1, 4, 8, 1, 2048, 64))
    assert "lanes_per_row" not in msg, msg


def test_null_schedule():
    lib = qfr.load_library()
    rc = lib.row_exact_mv_scheduled(1, WP, XP, YP, 64, 256, 4, 1, None, None, None)
    assert rc == -6


def test_extent_overflow():
    # x extent (batch-1)*xbs + (m-1)*xrs + k in bytes beyond 2^62
    rc, msg = _mv(n=64, k=256, m=8, batch=0xFFFFFFFF,
                  strides=Strides(0xFFFFFFFC, 0xFFFFFFFC, 64, 0xFFFFFFFF))
    assert rc == -5, msg


def test_dequant_validation():
    lib = qfr.load_library()
    assert lib.row_exact_dequant(1, WP, YP, 0, 64, None) == -1
    assert lib.row_exact_dequant(1, WP, YP, 4, 40, None) == -1
    assert lib.row_exact_dequant(2, WP + 4, YP, 4, 256, None) == -2
    assert lib.row_exact_dequant(1, WP, WP + 8, 4, 64, None) == -4
    assert lib.row_exact_dequant(9, WP, YP, 4, 64, None) == -1
    # 2-byte-aligned Q8_0 / Q6_K / Q5_0 rows pass the alignment check (then
    # refused: out overlaps W), a 1-byte offset does not
    for wt, k in ((1, 64), (3, 256), (4, 64)):
        assert lib.row_exact_dequant(wt, WP + 2, WP + 8, 4, k, None) == -4
        assert lib.row_exact_dequant(wt, WP + 1, YP, 4, k, None) == -2


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(qfr, "_lib", None)
    monkeypatch.setattr(qfr, "_LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(qfr.LibraryMissing):
        qfr.row_exact_row_bytes(1, 32)


def test_stream_read_probe_rejects_bad_arguments():
    lib = qfr.load_library()
    assert lib.row_exact_stream_read_shapes() >= 1
    cases = [
        ((0, 1024, YP, 0), -1),                 # NULL buffer
        ((WP, 1024, 0, 0), -1),                 # NULL sink
        ((WP, 0, YP, 0), -1),                   # empty
        ((WP, 1000, YP, 0), -1),                # not a multiple of 16
        ((WP, 1024, YP, 99), -1),               # unknown shape
        ((WP + 8, 1024, YP, 0), -2),            # misaligned buffer
        ((WP, 1024, YP + 2, 0), -2),            # misaligned sink
    ]
    before = qfr.row_exact_launch_count()
    for args, code in cases:
        assert lib.row_exact_stream_read(*args, None) == code, args
        assert "stream_read" in qfr.row_exact_last_error()
    assert qfr.row_exact_launch_count() == before


def _gather(ids=XP + 0x100000, num_experts=4, W=WP, x=XP, y=YP, n=64, k=256, m=2, batch=3, wt=Weight.Q8_0):
    lib = qfr.load_library()
    st = Strides(k, 0, batch * n, n)  # one token's x for every entry, token-major y
    return lib.row_exact_mv_gather(int(wt), W, num_experts, ids, x, y, n, k, m, batch, ctypes.byref(st), None), \
        qfr.row_exact_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(ids=0), -1, "expert_ids"),
    (dict(num_experts=0), -1, "num_experts"),
    (dict(ids=XP + 0x100002), -2, "expert_ids must sit on a 4-byte boundary"),
    (dict(ids=YP + 8), -4, "expert_ids"),
    (dict(m=0), -1, "m = 0"),
    (dict(wt=9), -1, "weight type 9"),
])
def test_gather_invalid_arguments(kw, code, text):
    before = qfr.row_exact_launch_count()
    rc, msg = _gather(**kw)
    assert rc == code, (rc, msg)
    assert text in msg, msg
    assert qfr.row_exact_launch_count() == before


def test_gather_weight_extent_counts_expert_sets():
    # y placed just past W's 4 sets of 64 Q8_0 rows: no overlap with 4 sets,
    # overlap when W holds 5 sets
    rb = qfr.row_exact_row_bytes(Weight.Q8_0, 256)
    y = WP + 4 * 64 * rb
    rc, msg = _gather(num_experts=5, y=y, ids=XP + 0x100000)
    assert rc == -4 and "y overlaps the bytes of W" in msg


RP, GP, HP = 0x7F3000000000, 0x7F4000000000, 0x7F5000000000


def _norm(r=RP, g=GP, h=HP, eps=1e-5, x=XP, y=YP, W=WP, n=64, k=256, m=4, wt=Weight.Q8_0):
    lib = qfr.load_library()
    rc = lib.row_exact_mv_add_rmsnorm(int(wt), W, x, r, g, eps, h, y, n, k, m, 1, None, None)
    return rc, qfr.row_exact_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(r=0), -1, "r must be"),
    (dict(eps=-1.0), -1, "eps"),
    (dict(eps=float("nan")), -1, "eps"),
    (dict(eps=float("inf")), -1, "eps"),
    (dict(r=RP + 4), -2, "16-byte"),
    (dict(g=GP + 8), -2, "16-byte"),
    (dict(h=HP + 4), -2, "16-byte"),
    (dict(h=XP + 16), -4, "h overlaps"),
    (dict(h=RP), -4, "h overlaps"),
    (dict(h=YP), -4, "overlap"),
    (dict(r=YP), -4, "overlaps"),
    (dict(m=9), -1, "m = 9"),
])
def test_add_rmsnorm_invalid_arguments(kw, code, text):
    before = qfr.row_exact_launch_count()
    rc, msg = _norm(**kw)
    assert rc == code, (rc, msg)
    assert text in msg, msg
    assert qfr.row_exact_launch_count() == before


WK = 0x7F6000000000


def _norm_ws(work=WK, work_bytes=1 << 20, batch=1, strides=None, **kw):
    lib = qfr.load_library()
    a = dict(r=RP, g=GP, h=HP, eps=1e-5, x=XP, y=YP, W=WP, n=64, k=256, m=4, wt=Weight.Q8_0)
    a.update(kw)
    sp = ctypes.byref(strides) if strides is not None else None
    rc = lib.row_exact_mv_add_rmsnorm_ws(int(a["wt"]), a["W"], a["x"], a["r"], a["g"], a["eps"], a["h"], a["y"], a["n"],
                                         a["k"], a["m"], batch, sp, work, work_bytes, None)
    return rc, qfr.row_exact_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(work=0), -1, "work must be"),
    (dict(work=WK + 8), -2, "work must sit on a 16-byte boundary"),
    (dict(work_bytes=4 * 256 * 4), -1, "the call needs"),
    (dict(work=YP), -4, "work overlaps"),
    (dict(work=XP + 16), -4, "work overlaps"),
    (dict(work=HP), -4, "work overlaps"),
    (dict(work=GP), -4, "work overlaps"),
    (dict(m=9), -1, "m = 9"),
    (dict(r=0), -1, "r must be"),
])
def test_add_rmsnorm_ws_invalid_arguments(kw, code, text):
    before = qfr.row_exact_launch_count()
    rc, msg = _norm_ws(**kw)
    assert rc == code, (rc, msg)
    assert text in msg, msg
    assert qfr.row_exact_launch_count() == before


def test_norm_work_bytes_is_the_header_formula():
    # u (batch*m*k floats) rounded up to 256 bytes, then batch*m doubles
    assert qfr.norm_work_bytes(256, 4, 1) == 4096 + 32
    assert qfr.norm_work_bytes(4, 1, 1) == 256 + 8
    assert qfr.norm_work_bytes(4096, 8, 16) == 16 * 8 * 4096 * 4 + 16 * 8 * 8


C2, W2 = 0x7F7000000000, 0x7F8000000000


def _resid(work=WK, work_bytes=1 << 20, batch=1, strides=None, **kw):
    lib = qfr.load_library()
    a = dict(h=RP, x=XP, w=GP, c=C2, w2=W2, eps=1e-5, eps2=1e-5, hout=HP, y=YP, W=WP, n=64, k=256, m=4,
             wt=Weight.Q8_0)
    a.update(kw)
    sp = ctypes.byref(strides) if strides is not None else None
    rc = lib.row_exact_mv_residual_rmsnorm_ws(int(a["wt"]), a["W"], a["h"], a["x"], a["w"], a["c"], a["w2"], a["eps"],
                                              a["eps2"], a["hout"], a["y"], a["n"], a["k"], a["m"], batch, sp, work,
                                              work_bytes, None)
    return rc, qfr.row_exact_last_error()


@pytest.mark.parametrize("kw,code,text", [
    (dict(h=0), -1, "h must be a non-NULL device pointer"),
    (dict(eps=-1.0), -1, "eps and eps2 must be finite and >= 0"),
    (dict(eps2=float("inf")), -1, "eps and eps2 must be finite and >= 0"),
    (dict(eps2=float("nan")), -1, "eps and eps2 must be finite and >= 0"),
    (dict(c=C2 + 4), -2, "h, w, c, w2 and hout must be 16-byte aligned"),
    (dict(hout=HP + 8), -2, "16-byte aligned"),
    (dict(w2=YP), -4, "y overlaps h, w, c or w2"),
    (dict(h=YP + 64), -4, "y overlaps"),
    (dict(hout=XP), -4, "hout overlaps"),
    (dict(hout=RP + 16), -4, "hout overlaps"),          # part of h, not h itself
    (dict(hout=GP), -4, "hout overlaps"),
    (dict(work=0), -1, "work must be"),
    (dict(work=WK + 8), -2, "work must sit on a 16-byte boundary"),
    (dict(work_bytes=4 * 256 * 4), -1, "the call needs"),
    (dict(work=HP), -4, "work overlaps"),
    (dict(work=C2), -4, "work overlaps"),
    (dict(x=0), -1, ""),
    (dict(m=9), -1, "m = 9"),
])
def test_residual_rmsnorm_ws_invalid_arguments(kw, code, text):
    before = qfr.row_exact_launch_count()
    rc, msg = _resid(**kw)
    assert rc == code, (rc, msg)
    assert text in msg, msg
    assert qfr.row_exact_launch_count() == before


def test_residual_rmsnorm_ws_in_place_and_optional_vectors_pass_the_checks():
    # hout == h (in place) and NULL w / c / w2 are valid; with no GPU the call
    # then fails only at the launch, after every argument check (with a GPU
    # these placeholder addresses would be launched on: not run there)
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers: only where no GPU is visible")
    for kw in (dict(hout=RP), dict(w=0, c=0, w2=0, hout=0)):
        rc, msg = _resid(**kw)
        assert rc == -7, (kw, rc, msg)


# Extents that only the work buffer's layout adds: the normalisation's grid
# of batch x m workgroups, the u view's batch stride m x k (32 bits), and the
# work size itself.  Each call is refused before the first of its two
# launches (x broadcast over the batch keeps the operands' own extents small).
_M8_BIG_BATCH = dict(n=1, k=32, m=8, batch=(1 << 28) + 1, strides=Strides(32, 0, 1, 8), work_bytes=1 << 40)
_M8_LONG_ROWS = dict(n=1, k=1 << 29, m=8, batch=2, strides=Strides(1 << 29, 0, 1, 8), work_bytes=1 << 36)


@pytest.mark.parametrize("case,text", [
    (_M8_BIG_BATCH, "normalised rows exceed one launch"),
    (_M8_LONG_ROWS, "exceed the 32-bit batch stride"),
])
def test_two_launch_norm_extents_refused_before_any_launch(case, text):
    before = qfr.row_exact_launch_count()
    rc, msg = _norm_ws(**case)
    assert rc == -5 and text in msg, (rc, msg)
    rc, msg = _resid(w=0, c=0, w2=0, **case)
    assert rc == -5 and text in msg, (rc, msg)
    assert qfr.row_exact_launch_count() == before


def test_work_size_overflow_refused():
    # batch x m x k floats of 2^62 bytes or more: refused, not wrapped to a
    # small size that a small buffer would satisfy
    s = Strides(1 << 30, 0, 1, 8)
    for f in (_norm_ws, _resid):
        # W (2^28 sets of one 1.1 GB row) placed above every other operand
        rc, msg = f(W=1 << 63, n=1, k=1 << 30, m=8, batch=1 << 28, strides=s, work_bytes=(1 << 64) - 1)
        assert rc == -5 and "spans 2^62 bytes" in msg, (rc, msg)
