"""GPU parity at oracle-sized shapes: every mode x dtype pair x dilation x window,
including ragged sequence lengths (edge tiles), windows wider than the sequence,
w_upper = 0, n = 1, and head dims that are not multiples of the MFMA depth.

Each case compares the C ABI (through the Python binding) with the full CPU oracle on
the same seeded inputs: in-range values within the stated tolerance, padding slots and
masked softmax slots bit for bit.
"""
import math

import pytest
import torch

import datagen
import oracle
from _util import assert_bits_equal, check_close, in_range_mask

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, d, w, w_upper, dilation, in, out)
CASES = [
    (1, 512, 1, 64, 32, 32, 0, "f32", "f32"),
    (1, 1, 1, 64, 3, 3, 0, "f16", "f16"),
    (1, 2, 2, 64, 1, 1, 0, "f16", "f16"),
    (2, 7, 3, 64, 3, 0, 0, "bf16", "f32"),
    (1, 100, 2, 64, 31, 31, 0, "f16", "f16"),
    (1, 257, 2, 64, 32, 32, 0, "f16", "f32"),
    (2, 257, 3, 64, 64, 0, 0, "bf16", "bf16"),
    (1, 1000, 2, 64, 256, 256, 0, "f16", "f16"),
    (1, 1000, 2, 64, 256, 256, 3, "f16", "f16"),
    (1, 1537, 1, 64, 100, 37, 2, "bf16", "f32"),
    (1, 300, 2, 64, 350, 350, 0, "f16", "f16"),     # window wider than the sequence
    (1, 333, 1, 64, 20, 20, 9, "f16", "f16"),
    (1, 333, 1, 64, 20, 20, 1, "f16", "f16"),       # dilation 1 == contiguous
    (1, 200, 2, 32, 16, 16, 0, "f16", "f16"),
    (1, 200, 2, 128, 48, 48, 0, "bf16", "f32"),
    (1, 129, 2, 24, 10, 5, 0, "f16", "f16"),        # d not a multiple of the MFMA depth
    (1, 70, 2, 1, 4, 4, 2, "f32", "f32"),
    (2, 96, 2, 64, 40, 40, 3, "f32", "f32"),
    (1, 64, 1, 8, 0, 0, 0, "f16", "f16"),           # K = 1: only the main diagonal
    (1, 640, 4, 64, 128, 128, 0, "bf16", "bf16"),
    (1, 5, 2, 64, 3, 3, 9, "f16", "f16"),           # dilation larger than the sequence
    (3, 130, 2, 32, 600, 0, 2, "f16", "f32"),       # several slot blocks per row
]


def _ids(c):
    b, n, h, d, w, wu, dil, i, o = c
    return f"b{b}n{n}h{h}d{d}w{w}u{wu}s{dil}-{i}-{o}"


def _inputs(case, seed):
    b, n, h, d, w, wu, dil, ind, _ = case
    g = datagen.rng(seed)
    sc = 1.0 / math.sqrt(d)
    q = datagen.normal(g, (b, n, h, d), ind, sc)
    k = datagen.normal(g, (b, n, h, d), ind, sc)
    v = datagen.normal(g, (b, n, h, d), ind, sc)
    probs = datagen.softmax_rows(g, (b, n, h, w + wu + 1), ind)
    grad = datagen.normal(g, (b, n, h, w + wu + 1), ind)
    return q, k, v, probs, grad


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_qk(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, ind, outd = case
    q, k, _, _, _ = _inputs(case, 100)
    pad = -1.5
    got = dm.diagmm_qk(q.cuda(), k.cuda(), w, wu, dil, pad, out_dtype=DT[outd]).cpu()
    ref = oracle.qk(q, k, w, wu, dil, pad, out_dtype=torch.float64)
    ref_out = oracle.qk(q, k, w, wu, dil, pad, out_dtype=DT[outd])
    mask = in_range_mask(b, n, h, w, wu, dil)
    check_close(got, ref, DT[ind], "qk", mask)
    assert_bits_equal(got[~mask], ref_out[~mask], "qk padding slots")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_pv_probabilities(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, ind, outd = case
    _, _, v, probs, _ = _inputs(case, 200)
    got = dm.diagmm_pv(probs.cuda(), v.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    ref = oracle.pv(probs, v, w, wu, dil, out_dtype=torch.float64)
    check_close(got, ref, DT[ind], "pv")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_pvT_probabilities(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, ind, outd = case
    q, _, _, probs, _ = _inputs(case, 300)
    got = dm.diagmm_pvT(probs.cuda(), q.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    ref = oracle.pvT(probs, q, w, wu, dil, out_dtype=torch.float64)
    check_close(got, ref, DT[ind], "pvT")


@pytest.mark.parametrize("case", [c for c in CASES if c[8] == "f32"], ids=_ids)
def test_pv_pvT_gradient_band_f32_out(case):
    """N(0,1) gradient bands (as in the backward pass), accumulated into f32 outputs."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, ind, outd = case
    q, k, _, _, grad = _inputs(case, 400)
    got = dm.diagmm_pv(grad.cuda(), k.cuda(), w, wu, dil, out_dtype=torch.float32).cpu()
    check_close(got, oracle.pv(grad, k, w, wu, dil, out_dtype=torch.float64), DT[ind], "pv grad")
    got = dm.diagmm_pvT(grad.cuda(), q.cuda(), w, wu, dil, out_dtype=torch.float32).cpu()
    check_close(got, oracle.pvT(grad, q, w, wu, dil, out_dtype=torch.float64), DT[ind],
                "pvT grad")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_banded_softmax(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, ind, outd = case
    g = datagen.rng(500)
    scores = datagen.normal(g, (b, n, h, w + wu + 1), ind, 3.0)
    scale = 1.0 / math.sqrt(d)
    got = dm.diagmm_banded_softmax(scores.cuda(), w, wu, dil, scale, out_dtype=DT[outd]).cpu()
    ref = oracle.softmax(scores, w, wu, dil, scale, out_dtype=torch.float64)
    mask = in_range_mask(b, n, h, w, wu, dil)
    check_close(got, ref, DT[ind], "softmax", mask)
    assert_bits_equal(got[~mask], torch.zeros_like(got[~mask]), "softmax masked slots")


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_integer_inputs_are_exact(dt):
    """Small integers make every product and partial sum exact in f32, so the GPU must
    reproduce the oracle bit for bit, at ragged shapes, with and without dilation."""
    import sliding_window_attention_diagmm_amd as dm
    odt = torch.float32 if dt == "bf16" else DT[dt]
    for (b, n, h, d, w, wu, dil) in [(1, 333, 2, 64, 40, 40, 0), (2, 301, 3, 64, 17, 0, 3),
                                     (1, 1025, 1, 64, 256, 256, 0)]:
        g = datagen.rng(600 + n)
        q = datagen.small_ints(g, (b, n, h, d), -2, 2, dt)
        k = datagen.small_ints(g, (b, n, h, d), -2, 2, dt)
        p = datagen.small_ints(g, (b, n, h, w + wu + 1), -1, 1, dt)
        got = dm.diagmm_qk(q.cuda(), k.cuda(), w, wu, dil, 7.0, out_dtype=odt).cpu()
        assert_bits_equal(got, oracle.qk(q, k, w, wu, dil, 7.0, out_dtype=odt), "qk ints")
        got = dm.diagmm_pv(p.cuda(), q.cuda(), w, wu, dil, out_dtype=odt).cpu()
        assert_bits_equal(got, oracle.pv(p, q, w, wu, dil, out_dtype=odt), "pv ints")
        got = dm.diagmm_pvT(p.cuda(), q.cuda(), w, wu, dil, out_dtype=odt).cpu()
        assert_bits_equal(got, oracle.pvT(p, q, w, wu, dil, out_dtype=odt), "pvT ints")


# (b, n, h, w, w_upper, dilation, dtype): rows long enough for a workgroup per row (more
# than 512 pieces of 16 bytes: 5 pieces per lane up to 1280 pieces, 9 up to 2304), with
# short sequences so that most rows are clipped at the sequence ends
LONG_ROW_CASES = [
    (1, 40, 2, 2100, 2100, 0, "f16"),      # 4201 slots: 526 pieces, 5 per lane
    (2, 30, 1, 4096, 4096, 0, "bf16"),     # 8193 slots
    (1, 25, 1, 1100, 1100, 0, "f32"),      # 2201 f32 slots: 551 pieces
    (1, 20, 1, 6000, 6000, 0, "f16"),      # 12001 slots: 1501 pieces, 9 per lane
    (1, 33, 3, 3000, 1500, 2, "f16"),      # 4501 slots, dilation 2, odd row starts
]


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("case", LONG_ROW_CASES,
                         ids=lambda c: f"b{c[0]}n{c[1]}h{c[2]}w{c[3]}u{c[4]}s{c[5]}-{c[6]}")
def test_banded_softmax_long_rows(case, inplace):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt = case
    g = datagen.rng(510)
    scores = datagen.normal(g, (b, n, h, w + wu + 1), dt, 3.0)
    sc = scores.cuda()
    got = dm.diagmm_banded_softmax(sc, w, wu, dil, 0.125, inplace=inplace).cpu()
    ref = oracle.softmax(scores, w, wu, dil, 0.125, out_dtype=torch.float64)
    mask = in_range_mask(b, n, h, w, wu, dil)
    check_close(got, ref, DT[dt], "softmax", mask)
    assert_bits_equal(got[~mask], torch.zeros_like(got[~mask]), "softmax masked slots")
