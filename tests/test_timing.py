"""The library's kernel timers (a measurement aid for the benchmark).

Host part (no GPU): argument checks of diagmm_timing_begin / _read and an empty read.
GPU part: a session records one start/end event pair per launch, tagged with the entry
point, in launch order; launches past the capacity run untimed; and the timed launch
path (hipExtLaunchKernel) gives bit-identical results to the untimed one.
"""
import ctypes
import math

import pytest
import torch

import datagen
import sliding_window_attention_diagmm_amd as dm
from _util import assert_bits_equal

ERR_NULL, ERR_SHAPE = 1, 2


def test_timing_argument_checks():
    lib = dm.load()
    assert lib.diagmm_timing_begin(0) == ERR_SHAPE
    assert lib.diagmm_timing_begin(-5) == ERR_SHAPE
    assert lib.diagmm_timing_begin((1 << 20) + 1) == ERR_SHAPE
    assert lib.diagmm_timing_end() == 0
    assert lib.diagmm_timing_read(0, None, None, None) == ERR_NULL
    assert lib.diagmm_timing_read(4, None, None, ctypes.byref(ctypes.c_int64())) == ERR_NULL


def test_timing_read_without_session_is_empty():
    lib = dm.load()
    assert lib.diagmm_timing_end() == 0
    count = ctypes.c_int64(-1)
    assert lib.diagmm_timing_read(0, None, None, ctypes.byref(count)) == 0
    assert count.value >= 0


@pytest.mark.gpu
def test_timed_launches_are_recorded_in_order_and_change_nothing():
    b, n, h, d, w, wu, dil = 1, 700, 3, 64, 64, 32, 2
    g = datagen.rng(5)
    q = datagen.normal(g, (b, n, h, d), "f16", 1 / math.sqrt(d)).cuda()
    k = datagen.normal(g, (b, n, h, d), "f16", 1 / math.sqrt(d)).cuda()

    def run():
        s = dm.diagmm_qk(q, k, w, wu, dil)
        p = dm.diagmm_banded_softmax(s, w, wu, dil, 0.125)
        o = dm.diagmm_pv(p, k, w, wu, dil)
        x = dm.diagmm_pvT(p, q, w, wu, dil)
        return s, p, o, x

    ref = run()
    torch.cuda.synchronize()
    dm.diagmm_timing_begin(6)
    timed = run()
    extra = run()                     # two of these four launches are past the capacity
    torch.cuda.synchronize()
    dm.diagmm_timing_end()
    recs = dm.diagmm_timing_read()
    assert [r[0] for r in recs] == ["qk", "softmax", "pv", "pvT", "qk", "softmax"]
    assert all(0.0 < ms < 1000.0 for _, ms in recs)
    for name, a, t, e in zip(("qk", "softmax", "pv", "pvT"), ref, timed, extra):
        assert_bits_equal(a, t, name + " timed")
        assert_bits_equal(a, e, name + " after the session filled")
