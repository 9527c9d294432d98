"""GPU parity of the banded softmax backward against the CPU oracle.

dS = scale * P * (dP - sum(P * dP)) per band row over the in-range slots, exactly +0 in
the others (the chain rule through the banded softmax; the oracle's pins are in
test_oracle.py).  Cases cover every lane layout of the kernel (1 .. 32 lanes per row,
whole wavefronts with 2 .. 8 pieces per lane, whole workgroups with 5 or 9), the row
kernel (forced, for misaligned tensors and for rows longer than 256 x 9 pieces), the three dtypes, dilation, ragged and tiny sequences, in-place
use and poisoned out-of-range slots; at the benchmark shape and the long-document shape
the probabilities come from the GPU chain itself (qk -> softmax) and the gradient from
dP = qk(dO, V), checked on sampled rows.
"""
import math
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
from _util import assert_bits_equal, check_close, in_range_mask, in_range_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, w, w_upper, dilation, dtype): the comment names the kernel layout it reaches
# (L lanes per row for rows of up to 3 L pieces of 16 bytes, then whole wavefronts, then
# whole workgroups of 256 lanes)
CASES = [
    (1, 512, 1, 32, 32, 0, "f32"),      # 65 slots, f32 (4 per piece): 8 lanes
    (1, 1, 1, 3, 3, 0, "f16"),          # one position
    (2, 7, 3, 3, 0, 0, "bf16"),         # 4 slots, causal: 1 lane per row
    (1, 100, 2, 31, 31, 0, "f16"),      # 63 slots: 4 lanes
    (1, 1000, 2, 256, 256, 0, "f16"),   # 513 slots: 32 lanes per row
    (1, 1000, 2, 256, 256, 3, "bf16"),
    (1, 300, 2, 350, 350, 0, "f16"),    # window wider than the sequence: 32 lanes
    (1, 333, 1, 20, 20, 9, "f16"),
    (1, 64, 1, 0, 0, 0, "f16"),         # K = 1
    (1, 70, 2, 4, 4, 2, "f32"),
    (2, 96, 2, 40, 40, 3, "f32"),
    (1, 40, 1, 300, 0, 0, "bf16"),      # 301 slots, causal: 16 lanes
    (1, 30, 1, 700, 700, 0, "f16"),     # 1401 slots: wave, 4 pieces per lane
    (1, 30, 1, 1200, 1200, 0, "f16"),   # 2401 slots: a wavefront, 8 pieces per lane
    (1, 12, 1, 4096, 4096, 0, "f16"),   # 8193 slots: a workgroup, up to 5 pieces per lane
    (1, 8, 1, 2500, 2500, 0, "bf16"),   # 5001 slots: a workgroup, 3 pieces per lane
    (1, 40, 1, 3000, 3000, 3, "bf16"),  # 6001 slots, dilated: a workgroup
    (1, 6, 2, 9000, 9000, 0, "f16"),    # 18001 slots: a workgroup, up to 9 pieces per lane
    (1, 10, 1, 2000, 2000, 0, "f32"),   # 4001 f32 slots: a workgroup, up to 4 pieces
    (1, 6, 1, 4500, 4500, 0, "f32"),    # 9001 f32 slots: a workgroup, up to 9 pieces
    (1, 4, 1, 10000, 10000, 0, "f16"),  # 20001 slots (2501 pieces): the row kernel
    (1, 20, 1, 150, 150, 0, "f32"),     # 301 f32 slots: 32 lanes
    (1, 20, 1, 1000, 1000, 0, "f32"),   # 2001 f32 slots: a wavefront, 8 pieces per lane
    (1, 50, 2, 16, 15, 0, "f16"),       # 32 slots: 2 lanes per row
    (1, 30, 1, 450, 450, 0, "f16"),     # 901 slots: a wavefront, 2 pieces per lane
]


def _ids(c):
    b, n, h, w, wu, dil, dt = c
    return f"b{b}n{n}h{h}w{w}u{wu}s{dil}-{dt}"


def _inputs(case, seed):
    """A probability band (the oracle's softmax of N(0,1) scores, exact zeros in masked
    slots) and an N(0,1) gradient band, both in the case's dtype."""
    b, n, h, w, wu, dil, dt = case
    g = datagen.rng(seed)
    S = datagen.normal(g, (b, n, h, w + wu + 1), "f32", 2.0)
    P = oracle.softmax(S, w, wu, dil, scale=1.0, out_dtype=DT[dt])
    dP = datagen.normal(g, (b, n, h, w + wu + 1), dt)
    return P, dP


def _check(case, P, dP, dS_gpu, scale, what):
    b, n, h, w, wu, dil, dt = case
    ref = oracle.softmax_bwd(P, dP, w, wu, dil, scale=scale, out_dtype=torch.float64)
    mask = in_range_mask(b, n, h, w, wu, dil)
    check_close(dS_gpu, ref, DT[dt], what, mask)
    masked = dS_gpu.cpu()[~mask]
    assert_bits_equal(masked, torch.zeros_like(masked), f"{what}: masked slots")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_softmax_bwd_matches_oracle(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt = case
    P, dP = _inputs(case, 300 + n + w)
    scale = 0.125
    dS = dm.diagmm_banded_softmax_backward(P.cuda(), dP.cuda(), w, wu, dil, scale)
    torch.cuda.synchronize()
    _check(case, P, dP, dS, scale, _ids(case))


@pytest.mark.parametrize("case", [CASES[4], CASES[5], CASES[13], CASES[15]], ids=_ids)
def test_softmax_bwd_in_place_and_poisoned_slots(case):
    """dS written over dP or over P equals the out-of-place result bit for bit, and
    NaN / inf in out-of-range slots of P and dP change nothing."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt = case
    P, dP = _inputs(case, 400 + n)
    Pc, dPc = P.cuda(), dP.cuda()
    ref = dm.diagmm_banded_softmax_backward(Pc, dPc, w, wu, dil, 0.5)
    x = dPc.clone()
    dm.diagmm_banded_softmax_backward(Pc, x, w, wu, dil, 0.5, out=x)
    assert_bits_equal(x, ref, "in place over dP")
    y = Pc.clone()
    dm.diagmm_banded_softmax_backward(y, dPc, w, wu, dil, 0.5, out=y)
    assert_bits_equal(y, ref, "in place over P")
    mask = in_range_mask(b, n, h, w, wu, dil).cuda()
    for poison in (float("nan"), float("inf")):
        Pp = torch.where(mask, Pc, torch.full_like(Pc, poison))
        dPp = torch.where(mask, dPc, torch.full_like(dPc, -poison))
        got = dm.diagmm_banded_softmax_backward(Pp, dPp, w, wu, dil, 0.5)
        assert_bits_equal(got, ref, f"poisoned with {poison}")


@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[5], CASES[14]], ids=_ids)
def test_softmax_bwd_row_kernel(case, monkeypatch):
    """The workgroup-per-row kernel, forced with DIAGMM_KERNEL=simple and reached by
    tensors that are not 16-byte aligned, against the oracle."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt = case
    P, dP = _inputs(case, 500 + n)
    monkeypatch.setenv("DIAGMM_KERNEL", "simple")
    dS = dm.diagmm_banded_softmax_backward(P.cuda(), dP.cuda(), w, wu, dil, 0.25)
    torch.cuda.synchronize()
    monkeypatch.delenv("DIAGMM_KERNEL")
    _check(case, P, dP, dS, 0.25, "forced row kernel")
    # one element past an aligned start: every tensor misaligned
    numel = P.numel()
    bufs = [torch.empty(numel + 8, dtype=P.dtype, device="cuda") for _ in range(3)]
    Pm, dPm, out = (t_[1:1 + numel].view(P.shape) for t_ in bufs)
    Pm.copy_(P.cuda())
    dPm.copy_(dP.cuda())
    dm.diagmm_banded_softmax_backward(Pm, dPm, w, wu, dil, 0.25, out=out)
    torch.cuda.synchronize()
    _check(case, P, dP, out, 0.25, "misaligned tensors")
    assert_bits_equal(out, dS, "misaligned vs forced row kernel")


def _flat_rows(t, rows, h, last):
    ri = torch.from_numpy(np.asarray(rows)).to(t.device)
    return t.reshape(-1, h, last).index_select(0, ri).cpu()


@pytest.mark.parametrize("dil", [0, 3])
def test_softmax_bwd_at_the_benchmark_shape(dil):
    """b=1, n=4096, h=12, 513 diagonals, f16: P from the GPU's qk -> softmax of
    N(0,1)/8 inputs, dP = qk(dO, V); 384 sampled rows (both sequence ends included)
    against the oracle on the GPU's own P and dP, and every masked slot +0."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w = 1, 4096, 12, 64, 256
    g = datagen.rng(610 + dil)
    q, k, v, do = (datagen.normal(g, (b, n, h, d), "f16", 0.125).cuda() for _ in range(4))
    P = dm.diagmm_banded_softmax(dm.diagmm_qk(q, k, w, w, dil), w, w, dil, 0.125, inplace=True)
    dP = dm.diagmm_qk(do, v, w, w, dil)
    dS = dm.diagmm_banded_softmax_backward(P, dP, w, w, dil, 0.125)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(n - 4, n),
                                     datagen.rng(620).choice(n, 376, replace=False)]))
    P_r, dP_r, dS_r = (_flat_rows(t_, rows, h, 2 * w + 1) for t_ in (P, dP, dS))
    ref = oracle.softmax_bwd(P_r, dP_r, w, w, dil, scale=0.125, out_dtype=torch.float64,
                             n=n, rows=rows)
    mask = in_range_rows(n, h, w, w, dil, rows)
    check_close(dS_r, ref, torch.float16, f"dS dilation {dil}", mask)
    full = in_range_mask(b, n, h, w, w, dil).cuda()
    assert not torch.any(dS.masked_select(~full).view(torch.int16) != 0)


def test_softmax_bwd_at_the_long_document_shape():
    """n = 32768, 8193 diagonals, h = 12, f16 (a workgroup per row, up to 5 pieces a lane):
    P and dP from the GPU chain, 64 sampled rows against the oracle."""
    import sliding_window_attention_diagmm_amd as dm
    wl = datagen.WORKLOADS["long_n32768"]
    x = datagen.make(wl, ("q", "k", "v"))
    q, k, v = x["q"].cuda(), x["k"].cuda(), x["v"].cuda()
    do = datagen.normal(datagen.rng(640), (wl.b, wl.n, wl.h, wl.d), "f16").cuda()
    P = dm.diagmm_banded_softmax(dm.diagmm_qk(q, k, wl.w, wl.w_upper, 0), wl.w, wl.w_upper,
                                 0, 0.125, inplace=True)
    del q, k
    dP = dm.diagmm_qk(do, v, wl.w, wl.w_upper, 0)
    dS = dm.diagmm_banded_softmax_backward(P, dP, wl.w, wl.w_upper, 0, 0.125)
    torch.cuda.synchronize()
    rows = datagen.sample_rows(wl.n, wl.w, 64)
    P_r, dP_r, dS_r = (_flat_rows(t_, rows, wl.h, wl.K) for t_ in (P, dP, dS))
    del P, dP, dS
    torch.cuda.empty_cache()
    ref = oracle.softmax_bwd(P_r, dP_r, wl.w, wl.w_upper, 0, scale=0.125,
                             out_dtype=torch.float64, n=wl.n, rows=rows)
    mask = in_range_rows(wl.n, wl.h, wl.w, wl.w_upper, 0, rows)
    check_close(dS_r, ref, torch.float16, "long-document dS", mask)
    assert torch.all(dS_r[~mask].view(torch.int16) == 0)
