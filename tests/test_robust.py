"""GPU robustness: nothing is written outside the output, results are deterministic,
out-of-range band values never leak into pv / pvT, in-place softmax equals the
out-of-place one, calls honour the caller's stream, and the tiled kernels agree with
the element-per-thread kernels.
"""
import math
import os

import pytest
import torch

import datagen
from _util import assert_bits_equal, check_close, in_range_mask

pytestmark = pytest.mark.gpu

SHAPES = [  # b, n, h, d, w, wu, dil, dtype
    (1, 1000, 3, 64, 256, 256, 0, "f16"),
    (2, 777, 2, 64, 64, 0, 3, "bf16"),
    (1, 513, 2, 64, 32, 32, 2, "f32"),
]


def _inp(shape, seed=1):
    b, n, h, d, w, wu, dil, dt = shape
    g = datagen.rng(seed)
    sc = 1 / math.sqrt(d)
    q = datagen.normal(g, (b, n, h, d), dt, sc).cuda()
    k = datagen.normal(g, (b, n, h, d), dt, sc).cuda()
    p = datagen.softmax_rows(g, (b, n, h, w + wu + 1), dt).cuda()
    return q, k, p


def _guarded(shape, dtype, guard=4096):
    numel = math.prod(shape)
    buf = torch.empty(numel + 2 * guard, dtype=dtype, device="cuda")
    buf.fill_(float("nan") if dtype != torch.float32 else 12345.0)
    ref = buf.clone()
    return buf, buf[guard:guard + numel].view(shape), ref, guard, numel


def _guards_intact(buf, ref, guard, numel):
    assert_bits_equal(buf[:guard], ref[:guard], "guard before the output")
    assert_bits_equal(buf[guard + numel:], ref[guard + numel:], "guard after the output")


@pytest.mark.parametrize("shape", SHAPES)
def test_no_writes_outside_outputs(shape):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    q, k, p = _inp(shape)
    K = w + wu + 1
    buf, out, ref, g, ne = _guarded((b, n, h, K), q.dtype)
    dm.diagmm_qk(q, k, w, wu, dil, 0.0, out=out)
    torch.cuda.synchronize()
    _guards_intact(buf, ref, g, ne)
    for fn in (dm.diagmm_pv, dm.diagmm_pvT):
        buf, out, ref, g, ne = _guarded((b, n, h, d), torch.float32)
        fn(p, k, w, wu, dil, out_dtype=torch.float32, out=out)
        torch.cuda.synchronize()
        _guards_intact(buf, ref, g, ne)
    buf, out, ref, g, ne = _guarded((b, n, h, K), q.dtype)
    dm.diagmm_banded_softmax(p, w, wu, dil, 0.5, out=out)
    torch.cuda.synchronize()
    _guards_intact(buf, ref, g, ne)


@pytest.mark.parametrize("shape", SHAPES)
def test_bitwise_deterministic_reruns(shape):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    q, k, p = _inp(shape, 2)
    for fn, args in ((dm.diagmm_qk, (q, k)), (dm.diagmm_pv, (p, k)), (dm.diagmm_pvT, (p, q))):
        a = fn(*args, w, wu, dil)
        b2 = fn(*args, w, wu, dil)
        assert_bits_equal(a, b2, fn.__name__ + " rerun")
    a = dm.diagmm_banded_softmax(p, w, wu, dil, 0.7)
    assert_bits_equal(a, dm.diagmm_banded_softmax(p, w, wu, dil, 0.7), "softmax rerun")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("poison", [float("nan"), 1e30])
def test_out_of_range_band_values_are_ignored(shape, poison):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    q, k, p = _inp(shape, 3)
    mask = in_range_mask(b, n, h, w, wu, dil).cuda()
    poisoned = torch.where(mask, p, torch.tensor(poison, dtype=p.dtype, device="cuda"))
    for fn in (dm.diagmm_pv, dm.diagmm_pvT):
        assert_bits_equal(fn(poisoned, k, w, wu, dil), fn(p, k, w, wu, dil), fn.__name__)
    # the softmax never reads them either
    sm = dm.diagmm_banded_softmax
    assert_bits_equal(sm(poisoned, w, wu, dil, 0.3), sm(p, w, wu, dil, 0.3), "softmax")


@pytest.mark.parametrize("shape", SHAPES)
def test_inplace_softmax_matches_out_of_place(shape):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    q, k, p = _inp(shape, 4)
    s = dm.diagmm_qk(q, k, w, wu, dil, 0.0)
    ref = dm.diagmm_banded_softmax(s, w, wu, dil, 0.125)
    got = dm.diagmm_banded_softmax(s, w, wu, dil, 0.125, inplace=True)
    assert got.data_ptr() == s.data_ptr()
    assert_bits_equal(got, ref, "in-place softmax")


def test_calls_run_on_the_callers_stream():
    import sliding_window_attention_diagmm_amd as dm
    shape = SHAPES[0]
    b, n, h, d, w, wu, dil, dt = shape
    q, k, p = _inp(shape, 5)
    ref = dm.diagmm_qk(q, k, w, wu, dil)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = dm.diagmm_qk(q, k, w, wu, dil)
        probs = dm.diagmm_banded_softmax(got, w, wu, dil, 0.125)
        out = dm.diagmm_pv(probs, k, w, wu, dil)
    side.synchronize()
    assert_bits_equal(got, ref, "qk on a side stream")
    assert_bits_equal(out, dm.diagmm_pv(dm.diagmm_banded_softmax(ref, w, wu, dil, 0.125),
                                        k, w, wu, dil), "chain on a side stream")


@pytest.mark.parametrize("shape", SHAPES + [(1, 4096, 12, 64, 256, 256, 0, "f16"),
                                            (1, 4096, 12, 64, 256, 256, 3, "f16")])
def test_tiled_kernels_agree_with_element_kernels(shape, monkeypatch):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    q, k, p = _inp(shape, 6)
    fast = [dm.diagmm_qk(q, k, w, wu, dil, -2.0), dm.diagmm_pv(p, k, w, wu, dil),
            dm.diagmm_pvT(p, q, w, wu, dil), dm.diagmm_banded_softmax(p, w, wu, dil, 0.5)]
    monkeypatch.setenv("DIAGMM_KERNEL", "simple")
    slow = [dm.diagmm_qk(q, k, w, wu, dil, -2.0), dm.diagmm_pv(p, k, w, wu, dil),
            dm.diagmm_pvT(p, q, w, wu, dil), dm.diagmm_banded_softmax(p, w, wu, dil, 0.5)]
    monkeypatch.delenv("DIAGMM_KERNEL")
    for name, a, s in zip(("qk", "pv", "pvT", "softmax"), fast, slow):
        check_close(a.cpu(), s.cpu().double(), q.dtype, name + " tiled vs element",
                    abs_tol=None if q.dtype == torch.float32 else 2e-3)


# ---------------------------------------------------------------- the newer calls
# The softmax backward, the masked softmax, the dropout, the one-pass attention and the
# global-token attention (both entry points): nothing written outside the output, bitwise
# reruns, out-of-range band slots never read, in place = out of place.

def _band_inputs(shape, seed):
    b, n, h, d, w, wu, dil, dt = shape
    g = datagen.rng(seed)
    K = w + wu + 1
    p = datagen.softmax_rows(g, (b, n, h, K), dt).cuda()
    dp = datagen.normal(g, (b, n, h, K), dt).cuda()
    rand = datagen.uniform(g, (b, n, h, K)).cuda()
    mask = torch.ones((b, n), dtype=torch.float32)
    mask[:, ::7] = 0.0
    return p, dp, rand, mask.cuda()


def _glob(b, n):
    """Positions with a repeat and entries outside [0, n) (the set is {0, 5, n // 2, n - 1})."""
    row = [0, 5, n // 2, 5, -3, n - 1, n + 9]
    return torch.tensor([row] * b, dtype=torch.int32, device="cuda")


def _newer_calls(shape, seed):
    """(name, fn(out=None) -> tensor, output shape, output dtype) for every newer call
    the shape's dtype supports."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    p, dp, rand, mask = _band_inputs(shape, seed)
    q, k, _ = _inp(shape, seed + 1)
    v = k.flip(1).contiguous()
    K = w + wu + 1
    calls = [
        ("softmax_bwd", lambda out=None: dm.diagmm_banded_softmax_backward(
            p, dp, w, wu, dil, 0.5, out=out), (b, n, h, K), p.dtype),
        ("softmax_masked", lambda out=None: dm.diagmm_banded_softmax(
            dp, w, wu, dil, 0.5, out=out, key_mask=mask), (b, n, h, K), p.dtype),
        ("dropout", lambda out=None: dm.diagmm_banded_dropout(p, rand, w, wu, dil, 0.25, out=out),
         (b, n, h, K), p.dtype),
    ]
    if q.dtype != torch.float32:
        glob = _glob(b, n)
        gq, gk, gv = q.flip(2).contiguous(), k.flip(2).contiguous(), v.flip(2).contiguous()
        calls += [
            ("attention", lambda out=None: dm.diagmm_banded_attention(
                q, k, v, w, wu, dil, 0.125, out=out), (b, n, h, d), q.dtype),
            ("attention_global", lambda out=None: dm.diagmm_banded_attention_global(
                q, k, v, glob, w, wu, dil, 0.125, out=out, global_qkv=(gq, gk, gv)),
             (b, n, h, d), q.dtype),
            ("attention_global_noalloc", lambda out=None: dm.diagmm_banded_attention_global_noalloc(
                q, k, v, glob, w, wu, dil, 0.125, out=out, global_qkv=(gq, gk, gv)),
             (b, n, h, d), q.dtype),
        ]
    return calls


@pytest.mark.parametrize("shape", SHAPES)
def test_newer_calls_write_nothing_outside_outputs(shape):
    for name, fn, oshape, odt in _newer_calls(shape, 10):
        print(f"guard check: {name} {shape}", flush=True)
        buf, out, ref, g, ne = _guarded(oshape, odt)
        fn(out=out)
        torch.cuda.synchronize()
        _guards_intact(buf, ref, g, ne)
        assert torch.isfinite(out.float()).all(), f"{name}: an output element was not written"


@pytest.mark.parametrize("shape", SHAPES)
def test_newer_calls_bitwise_deterministic_reruns(shape):
    for name, fn, _, _ in _newer_calls(shape, 20):
        a = fn()
        b2 = fn()
        torch.cuda.synchronize()
        assert_bits_equal(a, b2, name + " rerun")


@pytest.mark.parametrize("shape", SHAPES)
def test_newer_band_calls_ignore_out_of_range_slots(shape):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    p, dp, rand, mask = _band_inputs(shape, 30)
    inr = in_range_mask(b, n, h, w, wu, dil).cuda()
    bad = torch.tensor(float("nan"), dtype=p.dtype, device="cuda")
    pp, dpp = torch.where(inr, p, bad), torch.where(inr, dp, bad)
    assert_bits_equal(dm.diagmm_banded_softmax_backward(pp, dpp, w, wu, dil, 0.5),
                      dm.diagmm_banded_softmax_backward(p, dp, w, wu, dil, 0.5), "softmax_bwd")
    assert_bits_equal(dm.diagmm_banded_softmax(dpp, w, wu, dil, 0.5, key_mask=mask),
                      dm.diagmm_banded_softmax(dp, w, wu, dil, 0.5, key_mask=mask),
                      "softmax_masked")
    assert_bits_equal(dm.diagmm_banded_dropout(pp, rand, w, wu, dil, 0.25),
                      dm.diagmm_banded_dropout(p, rand, w, wu, dil, 0.25), "dropout")


@pytest.mark.parametrize("shape", SHAPES)
def test_inplace_backward_and_dropout_match_out_of_place(shape):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    p, dp, rand, mask = _band_inputs(shape, 40)
    ref = dm.diagmm_banded_softmax_backward(p, dp, w, wu, dil, 0.5)
    for which in ("probs", "dprobs"):
        pc, dpc = p.clone(), dp.clone()
        tgt = pc if which == "probs" else dpc
        got = dm.diagmm_banded_softmax_backward(pc, dpc, w, wu, dil, 0.5, out=tgt)
        assert got.data_ptr() == tgt.data_ptr()
        assert_bits_equal(got, ref, f"softmax_bwd in place over {which}")
    ref = dm.diagmm_banded_dropout(p, rand, w, wu, dil, 0.25)
    pc = p.clone()
    got = dm.diagmm_banded_dropout(pc, rand, w, wu, dil, 0.25, out=pc)
    assert got.data_ptr() == pc.data_ptr()
    assert_bits_equal(got, ref, "dropout in place")


# Rows longer than a wavefront holds (the workgroup-per-row softmax and softmax backward
# kernels, up to 5 and 9 pieces a lane): guard regions, in place against out of place, and
# NaN in out-of-range slots (pieces holding no in-range slot are not read at all).
LONG_ROWS = [  # b, n, h, d, w, wu, dil, dtype
    (1, 40, 2, 64, 2500, 2500, 0, "bf16"),
    (1, 30, 1, 64, 4500, 4500, 0, "f32"),
    (1, 20, 2, 64, 3000, 1000, 3, "f16"),
]


@pytest.mark.parametrize("shape", LONG_ROWS)
def test_long_row_softmax_kernels_guards_inplace_and_poison(shape):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = shape
    K = w + wu + 1
    g = datagen.rng(77)
    s = datagen.normal(g, (b, n, h, K), dt, 2.0).cuda()
    p, dp, _, _ = _band_inputs(shape, 78)
    inr = in_range_mask(b, n, h, w, wu, dil).cuda()
    bad = torch.tensor(float("nan"), dtype=s.dtype, device="cuda")
    for name, fn, args, poisoned in (
            ("softmax", lambda *t, out=None: dm.diagmm_banded_softmax(
                t[0], w, wu, dil, 0.125, out=out), (s,), (torch.where(inr, s, bad),)),
            ("softmax_bwd", lambda *t, out=None: dm.diagmm_banded_softmax_backward(
                t[0], t[1], w, wu, dil, 0.5, out=out), (p, dp),
             (torch.where(inr, p, bad), torch.where(inr, dp, bad)))):
        print(f"long rows: {name} {shape}", flush=True)
        ref = fn(*args)
        buf, out, gref, gd, ne = _guarded((b, n, h, K), s.dtype)
        fn(*args, out=out)
        torch.cuda.synchronize()
        _guards_intact(buf, gref, gd, ne)
        assert_bits_equal(out, ref, f"{name} into a guarded buffer")
        assert_bits_equal(fn(*poisoned), ref, f"{name} with NaN in out-of-range slots")
        cl = [t.clone() for t in args]
        got = fn(*cl, out=cl[-1])
        assert got.data_ptr() == cl[-1].data_ptr()
        assert_bits_equal(got, ref, f"{name} in place")
