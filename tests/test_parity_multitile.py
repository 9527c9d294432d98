"""GPU parity with a small persistent grid (DIAGMM_MAX_WORKGROUPS): every workgroup walks
many tiles, so the continuation prefetch, the prefetch of a tile that starts a new strip,
load batches held across tiles, empty tail blocks of short residue classes and both slot
chunks of a row block all run at sizes the oracle checks in full.
"""
import math

import pytest
import torch

import datagen
import oracle
import sliding_window_attention_diagmm_amd as dm
from _util import assert_bits_equal, check_close, in_range_mask

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, d, w, w_upper, dilation, in, out, workgroups)
CASES = [
    (1, 2048, 3, 64, 256, 256, 0, "f16", "f16", 8),
    (1, 2048, 2, 64, 300, 300, 0, "f16", "f16", 8),   # 601 slots: two qk slot chunks
    (1, 2048, 3, 64, 256, 256, 3, "f16", "f16", 8),
    (2, 1100, 2, 64, 128, 40, 2, "bf16", "f32", 5),
    (1, 1500, 2, 32, 200, 200, 0, "f16", "f16", 3),
    (1, 900, 2, 128, 96, 96, 1, "bf16", "bf16", 7),
    # the strip split for pv and pvT: 7 workgroups per strip of 8 row blocks (2 of 44 idle),
    # and 2 per strip of 5 row blocks (ragged last blocks of 8 and 19 rows)
    (1, 1366, 2, 64, 200, 200, 3, "f16", "f16", 44),
    (2, 1100, 1, 64, 96, 30, 4, "bf16", "f32", 16),
]


def _ids(c):
    b, n, h, d, w, wu, dil, i, o, wg = c
    return f"b{b}n{n}h{h}d{d}w{w}u{wu}s{dil}-{i}-{o}-wg{wg}"


def test_grid_cap_shapes_the_plan(monkeypatch):
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", "8")
    for mode in ("qk", "pv", "pvT"):
        pl = dm.diagmm_plan(mode, 1, 2048, 3, 64, 256, 256, 0, torch.float16)
        # qk's units are row ranges of at most 208 rows (30 here), pv/pvT's 64-row tiles
        assert pl["workgroups"] <= 8 and pl["tiles"] >= 3 * pl["workgroups"], (mode, pl)


def test_strip_split_choice(monkeypatch):
    """pv and pvT split the tiles strip by strip where that shortens the busiest
    workgroup's list: at n=4096, h=12, w=256, dilation 3 a strip (one residue class of one
    head) has 21 full row blocks and one of 22 rows, so 7 workgroups per strip take 3 or
    3 + the short one, against 4 full ones for 24 workgroups of the flat split."""
    monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS", raising=False)
    for mode in ("pv", "pvT"):
        pl = dm.diagmm_plan(mode, 1, 4096, 12, 64, 256, 256, 3, torch.float16)
        if pl["workgroups"] == 256:
            assert pl["strip_workgroups"] == 7, pl
        for args in ((1, 4096, 12, 64, 256, 256, 0), (12, 4096, 12, 64, 256, 0, 0),
                     (1, 32768, 12, 64, 4096, 4096, 0)):
            assert dm.diagmm_plan(mode, *args, torch.float16)["strip_workgroups"] == 0
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", "44")
    for mode in ("pv", "pvT"):
        assert dm.diagmm_plan(mode, 1, 1366, 2, 64, 200, 200, 3,
                              torch.float16)["strip_workgroups"] == 7
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", "16")
    for mode in ("pv", "pvT"):
        assert dm.diagmm_plan(mode, 2, 1100, 1, 64, 96, 30, 4,
                              torch.bfloat16)["strip_workgroups"] == 2
    # qk cuts every strip into as many row ranges as the workgroups allow (one each)
    assert dm.diagmm_plan("qk", 2, 1100, 1, 64, 96, 30, 4,
                          torch.bfloat16)["strip_workgroups"] == 2
    monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS")
    for dil, g in ((0, 21), (3, 7)):
        pl = dm.diagmm_plan("qk", 1, 4096, 12, 64, 256, 256, dil, torch.float16)
        if pl["workgroups"] == 256:
            assert pl["strip_workgroups"] == g, pl


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_small_grid_matches_oracle(case, monkeypatch):
    b, n, h, d, w, wu, dil, ind, outd, wg = case
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", str(wg))
    g = datagen.rng(77)
    sc = 1.0 / math.sqrt(d)
    q = datagen.normal(g, (b, n, h, d), ind, sc)
    k = datagen.normal(g, (b, n, h, d), ind, sc)
    v = datagen.normal(g, (b, n, h, d), ind, sc)
    probs = datagen.softmax_rows(g, (b, n, h, w + wu + 1), ind)
    mask = in_range_mask(b, n, h, w, wu, dil)
    pad = -0.75

    s_gpu = dm.diagmm_qk(q.cuda(), k.cuda(), w, wu, dil, pad, out_dtype=DT[outd]).cpu()
    check_close(s_gpu, oracle.qk(q, k, w, wu, dil, pad, out_dtype=torch.float64), DT[ind],
                "qk", mask)
    assert_bits_equal(s_gpu[~mask], oracle.qk(q, k, w, wu, dil, pad,
                                              out_dtype=DT[outd])[~mask], "qk padding")

    pc = probs.cuda()
    o_gpu = dm.diagmm_pv(pc, v.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(o_gpu, oracle.pv(probs, v, w, wu, dil, out_dtype=torch.float64), DT[ind], "pv")
    x_gpu = dm.diagmm_pvT(pc, q.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(x_gpu, oracle.pvT(probs, q, w, wu, dil, out_dtype=torch.float64), DT[ind],
                "pvT")
    if ind != "f32":
        p_gpu = dm.diagmm_banded_softmax(pc, w, wu, dil, 0.5).cpu()
        check_close(p_gpu, oracle.softmax(probs, w, wu, dil, 0.5, out_dtype=torch.float64),
                    DT[ind], "softmax", mask)


def test_qk_takes_the_fewest_slot_chunks_when_tiles_suffice(monkeypatch):
    """The persistent tile kernel (f32 outputs, or DIAGMM_QK=tiles): one chunk at the
    benchmark shape (384 tiles for 256 units); more only when the fewest leave under 1.4
    tiles per unit (a 65-slot band of 512 positions: 4 tiles)."""
    monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS", raising=False)
    monkeypatch.setenv("DIAGMM_QK", "tiles")
    for dil in (0, 3):
        pl = dm.diagmm_plan("qk", 1, 4096, 12, 64, 256, 256, dil, torch.float16)
        if pl["workgroups"] == 256:
            assert pl["slots_per_tile"] == 513, pl
    assert dm.diagmm_plan("qk", 1, 2048, 2, 64, 300, 300, 0, torch.float16)["slots_per_tile"] < 601
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", "8")
    pl = dm.diagmm_plan("qk", 1, 512, 1, 64, 32, 32, 0, torch.float16)
    assert pl["tiles"] >= 8 and pl["slots_per_tile"] < 65, pl


def test_qk_stream_plan_balances_row_ranges(monkeypatch):
    """The streaming qk kernel (16-bit in and out) cuts every strip into the same number of
    row ranges of at most 208 class rows: at n = 4096, h = 12 (one strip per head, three
    per head at dilation 3) that is 252 ranges of at most 196 rows for 256 units, so no
    unit stores more than 196 / 192 of the average; every range covers all K slots."""
    monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS", raising=False)
    monkeypatch.delenv("DIAGMM_QK", raising=False)
    for dil, g in ((0, 21), (3, 7)):
        pl = dm.diagmm_plan("qk", 1, 4096, 12, 64, 256, 256, dil, torch.float16)
        if pl["workgroups"] != 256:
            continue
        assert pl["kernel"] == "qk_stream", pl
        assert pl["strip_workgroups"] == g and pl["tiles"] == 252, pl
        assert pl["rows_per_tile"] == 196 and pl["slots_per_tile"] == 513, pl
    # f32 outputs stay on the tile kernel
    assert dm.diagmm_plan("qk", 1, 4096, 12, 64, 256, 256, 0, torch.float16,
                          torch.float32)["kernel"] == "qk_mfma"
    # the key window streams through a ring, so any width works: K = 8193 at n = 32768
    pl = dm.diagmm_plan("qk", 1, 32768, 12, 64, 4096, 4096, 0, torch.float16)
    assert pl["kernel"] == "qk_stream" and pl["slots_per_tile"] == 8193, pl


def test_tile_order(monkeypatch):
    """pvT deals each XCD's tiles round-robin over its workgroups (neighbouring tiles at the
    same time) where a round of contiguous runs would read more band lines than an XCD's
    4 MB L2 holds before a workgroup's next tile reuses them: at n = 4096, h = 12, 513
    slots (32 workgroups x 576 window rows x 256 bytes = 4.7 MB) and at 8193 slots (16
    chunks a tile); not at 257 slots (320 rows, 2.6 MB), nor on the strip split unless
    forced (dilation 3: each strip's 7 workgroups).  pv does the same for tiles of several
    chunks on the flat split only (one-chunk tiles slide their key window)."""
    monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS", raising=False)
    pl = dm.diagmm_plan("pvT", 1, 4096, 12, 64, 256, 256, 0, torch.float16)
    if pl["workgroups"] == 256:
        assert pl["interleaved"] == 1 and pl["strip_workgroups"] == 0, pl
        assert dm.diagmm_plan("pvT", 1, 32768, 12, 64, 4096, 4096, 0,
                              torch.float16)["interleaved"] == 1
        assert dm.diagmm_plan("pvT", 12, 4096, 12, 64, 256, 0, 0, torch.bfloat16,
                              torch.float32)["interleaved"] == 0
    pl3 = dm.diagmm_plan("pvT", 1, 4096, 12, 64, 256, 256, 3, torch.float16)
    if pl3["workgroups"] == 256:
        assert pl3["strip_workgroups"] == 7 and pl3["interleaved"] == 0, pl3
        monkeypatch.setenv("DIAGMM_TILE_ORDER", "interleaved")
        assert dm.diagmm_plan("pvT", 1, 4096, 12, 64, 256, 256, 3,
                              torch.float16)["interleaved"] == 1
        pv3 = dm.diagmm_plan("pv", 1, 4096, 12, 64, 256, 256, 3, torch.float16)
        assert pv3["strip_workgroups"] == 7 and pv3["interleaved"] == 0, pv3
        monkeypatch.delenv("DIAGMM_TILE_ORDER")
    # pv: one-chunk tiles slide their key window, several-chunk tiles are interleaved
    assert dm.diagmm_plan("pv", 1, 4096, 12, 64, 256, 256, 0, torch.float16)["interleaved"] == 0
    if pl["workgroups"] == 256:
        assert dm.diagmm_plan("pv", 1, 32768, 12, 64, 4096, 4096, 0,
                              torch.float16)["interleaved"] == 1
    # a grid that is not a multiple of the 8 XCDs keeps contiguous runs
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", "44")
    assert dm.diagmm_plan("pvT", 1, 4096, 12, 64, 256, 256, 0, torch.float16)["interleaved"] == 0


# (b, n, h, d, w, w_upper, dilation, in, out, workgroups): flat splits whose workgroups are
# a multiple of 8, so pv and pvT can run with each XCD's tiles dealt round-robin
ORDER_CASES = [
    (1, 2048, 3, 64, 256, 256, 0, "f16", "f16", 16),   # 96 tiles: 12 per XCD, 6 per 2 wgs
    (2, 1100, 2, 64, 128, 40, 2, "bf16", "f32", 24),   # ragged class ends, 3 wgs per XCD
    (1, 1500, 2, 128, 200, 200, 0, "f16", "f16", 8),   # d = 128 (window rows filled per tile)
    (1, 1400, 1, 32, 400, 300, 0, "bf16", "bf16", 16), # d = 32, 701 slots: 2 chunks a tile
]


@pytest.mark.gpu
@pytest.mark.parametrize("order", ["interleaved", "contiguous"])
@pytest.mark.parametrize("case", ORDER_CASES, ids=_ids)
def test_tile_orders_match_oracle(case, order, monkeypatch):
    b, n, h, d, w, wu, dil, ind, outd, wg = case
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", str(wg))
    monkeypatch.setenv("DIAGMM_TILE_ORDER", order)
    for mode in ("pv", "pvT"):
        pl = dm.diagmm_plan(mode, b, n, h, d, w, wu, dil, DT[ind], DT[outd])
        assert pl["kernel"] == mode + "_mfma" and pl["strip_workgroups"] == 0, pl
        assert pl["interleaved"] == (order == "interleaved"), pl
    g = datagen.rng(91)
    x = datagen.normal(g, (b, n, h, d), ind, 1.0 / math.sqrt(d))
    probs = datagen.softmax_rows(g, (b, n, h, w + wu + 1), ind)
    pc, xc = probs.cuda(), x.cuda()
    got = dm.diagmm_pvT(pc, xc, w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(got, oracle.pvT(probs, x, w, wu, dil, out_dtype=torch.float64), DT[ind], "pvT")
    got = dm.diagmm_pv(pc, xc, w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(got, oracle.pv(probs, x, w, wu, dil, out_dtype=torch.float64), DT[ind], "pv")


# (b, n, h, d, w, w_upper, dilation, in, out, workgroups, workgroups per strip): strip
# splits on grids of a multiple of 8 workgroups, where pvT deals each strip's tiles
# round-robin over the strip's workgroups when forced (ragged last row blocks of 29, 17,
# 16 and 18 rows)
STRIP_ORDER_CASES = [
    (1, 1081, 1, 64, 200, 200, 2, "f16", "f16", 8, 4),
    (1, 1969, 1, 64, 256, 256, 3, "f16", "f16", 16, 5),
    (1, 2080, 1, 128, 150, 100, 2, "bf16", "bf16", 16, 8),
    (1, 2006, 1, 32, 300, 0, 5, "bf16", "f32", 16, 3),
]


@pytest.mark.gpu
@pytest.mark.parametrize("order", ["interleaved", "contiguous"])
@pytest.mark.parametrize("case", STRIP_ORDER_CASES,
                         ids=lambda c: _ids(c[:10]) + f"-g{c[10]}")
def test_strip_tile_orders_match_oracle(case, order, monkeypatch):
    b, n, h, d, w, wu, dil, ind, outd, wg, per_strip = case
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", str(wg))
    monkeypatch.setenv("DIAGMM_TILE_ORDER", order)
    pl = dm.diagmm_plan("pvT", b, n, h, d, w, wu, dil, DT[ind], DT[outd])
    assert pl["kernel"] == "pvT_mfma" and pl["strip_workgroups"] == per_strip, pl
    assert pl["interleaved"] == (order == "interleaved"), pl
    g = datagen.rng(93)
    x = datagen.normal(g, (b, n, h, d), ind, 1.0 / math.sqrt(d))
    probs = datagen.softmax_rows(g, (b, n, h, w + wu + 1), ind)
    got = dm.diagmm_pvT(probs.cuda(), x.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(got, oracle.pvT(probs, x, w, wu, dil, out_dtype=torch.float64), DT[ind], "pvT")


# qk's whole-line store path (rows of more than 1000 slots, or forced with
# DIAGMM_QK_LINES=1): pieces traded between lane halves and held one step so that every
# store writes whole aligned 128-byte lines, ranges in head-fastest order.  Whole band
# against the oracle, padding slots bit for bit, both paths where forced.
# (b, n, h, w, w_upper, dilation, dtype, DIAGMM_QK_LINES (+ "nt": DIAGMM_QK_NT=1),
#  workgroups or 0 for the default)
LINE_CASES = [
    (1, 700, 2, 600, 600, 0, "f16", None, 0),       # 1201 slots: the line path by default
    (1, 2100, 1, 520, 490, 2, "bf16", None, 0),     # 1011 slots, dilation 2, ragged classes
    (1, 1000, 2, 256, 256, 0, "f16", "1", 0),       # 513 slots, forced
    (2, 500, 3, 100, 30, 3, "f16", "1", 0),         # dilation 3, two batches, forced
    (1, 300, 3, 40, 40, 0, "bf16", "1", 5),         # small grid: several ranges per workgroup
    (2, 700, 3, 100, 100, 0, "f16", "1", 16),       # 24 ranges on 16: dealt round-robin per XCD
    (1, 64, 2, 9, 0, 0, "f16", "1", 0),             # 10 slots, causal
    (1, 1300, 2, 700, 700, 1, "bf16", "0", 7),      # 1401 slots with the line path off
    # non-temporal line stores (bands over 256 MB by default), forced on small bands
    (1, 700, 2, 600, 600, 0, "f16", "1nt", 0),
    (2, 700, 3, 100, 100, 3, "bf16", "1nt", 16),    # dilation 3, ranges dealt round-robin
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", LINE_CASES,
                         ids=lambda c: f"b{c[0]}n{c[1]}h{c[2]}w{c[3]}u{c[4]}s{c[5]}-{c[6]}-L{c[7]}-wg{c[8]}")
def test_qk_stream_line_stores_match_oracle(case, monkeypatch):
    b, n, h, w, wu, dil, dt, lines, wg = case
    monkeypatch.delenv("DIAGMM_QK_NT", raising=False)
    if lines is None:
        monkeypatch.delenv("DIAGMM_QK_LINES", raising=False)
    else:
        monkeypatch.setenv("DIAGMM_QK_LINES", lines[0])
        if lines.endswith("nt"):
            monkeypatch.setenv("DIAGMM_QK_NT", "1")
    if wg:
        monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", str(wg))
    else:
        monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS", raising=False)
    assert dm.diagmm_plan("qk", b, n, h, 64, w, wu, dil, DT[dt])["kernel"] == "qk_stream"
    g = datagen.rng(123)
    q = datagen.normal(g, (b, n, h, 64), dt, 0.125)
    k = datagen.normal(g, (b, n, h, 64), dt, 0.125)
    pad = 2.5
    got = dm.diagmm_qk(q.cuda(), k.cuda(), w, wu, dil, pad).cpu()
    ref = oracle.qk(q, k, w, wu, dil, pad, out_dtype=torch.float64)
    ref_out = oracle.qk(q, k, w, wu, dil, pad, out_dtype=DT[dt])
    mask = in_range_mask(b, n, h, w, wu, dil)
    check_close(got, ref, DT[dt], "qk line stores", mask)
    assert_bits_equal(got[~mask], ref_out[~mask], "qk line stores: padding slots")
