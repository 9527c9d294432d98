"""GPU parity of the one-pass sliding-window attention against the CPU oracle.

out = softmax(scale * Q K^T over the window's in-range diagonals) V, the band never
stored (the oracle's pins are in test_oracle.py).  The kernel keeps scores in float32 and
feeds the probabilities to the second product rounded to the input dtype, as the
three-call path stores them: the bound is the 16-bit output bar plus that rounding's
effect, u * sum_k P_k |V_k| (check_attention).  Cases cover
d = 32 / 64 / 128, f16 and bf16, dilation 0 / 1 / 2 / 3 / 9, ragged and tiny
sequences (partial 64-row blocks, key blocks past the class end), windows wider than the
sequence, one-sided and one-slot windows, several workgroups per head, the benchmark
shape and the long-document shape on sampled rows.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _util import LOWP_ABS, out_ulp


def check_attention(got, q, k, v, w, wu, dil, scale, dtype, what, rows=None):
    """|gpu - oracle| <= max(2e-3, one ulp of the output) + u * sum_k P_k |V_k| per
    element: the probabilities enter the second product rounded to the input dtype
    (unit roundoff u = 2^-11 for f16, 2^-8 for bf16), which moves an output by at most
    u times the probability-weighted sum of |V| - the oracle's attention over |V|."""
    ref = oracle.attention(q, k, v, w, wu, dil, scale, out_dtype=torch.float64, rows=rows)
    mag = oracle.attention(q, k, v.abs(), w, wu, dil, scale, out_dtype=torch.float64,
                           rows=rows)
    g = got.detach().cpu().double()
    assert torch.isfinite(g).all(), f"{what}: non-finite GPU values"
    u = 2.0 ** -11 if dtype == torch.float16 else 2.0 ** -8
    tol = torch.clamp(out_ulp(ref, dtype), min=LOWP_ABS) + u * mag
    diff = (g - ref).abs()
    bad = diff > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, worst "
                           f"excess {(diff - tol).max().item():.3e}")

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, d, w, w_upper, dilation, dtype)
CASES = [
    (1, 200, 2, 64, 16, 16, 0, "f16"),
    (1, 1, 1, 64, 3, 3, 0, "f16"),        # one position
    (2, 7, 3, 32, 3, 0, 0, "bf16"),       # causal, tiny
    (1, 100, 2, 32, 31, 31, 0, "f16"),
    (1, 1000, 2, 64, 256, 256, 3, "bf16"),
    (1, 333, 1, 64, 20, 20, 9, "f16"),
    (1, 300, 2, 64, 350, 350, 0, "f16"),  # window wider than the sequence
    (2, 257, 2, 128, 40, 40, 2, "bf16"),
    (1, 130, 1, 128, 0, 0, 0, "f16"),     # one-slot window: out = V up to rounding
    (1, 515, 3, 64, 70, 5, 1, "f16"),     # dilation 1 = contiguous
    (1, 640, 2, 32, 100, 0, 0, "bf16"),   # causal, several row blocks
    (3, 77, 2, 64, 6, 90, 3, "f16"),      # right-heavy window, dilated
]


def _ids(c):
    b, n, h, d, w, wu, dil, dt = c
    return f"b{b}n{n}h{h}d{d}w{w}u{wu}s{dil}-{dt}"


def _inputs(case, seed):
    b, n, h, d, w, wu, dil, dt = case
    g = datagen.rng(seed)
    return tuple(datagen.normal(g, (b, n, h, d), dt) for _ in range(3))


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_attention_matches_oracle(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt = case
    q, k, v = _inputs(case, 1100 + n + d)
    scale = d ** -0.5
    got = dm.diagmm_banded_attention(q.cuda(), k.cuda(), v.cuda(), w, wu, dil, scale)
    torch.cuda.synchronize()
    check_attention(got, q, k, v, w, wu, dil, scale, DT[dt], _ids(case))


def test_attention_agrees_with_the_three_calls():
    """The one-pass result against qk -> softmax -> pv on the GPU (f32 scores and
    probabilities there, so only the one-pass kernel's own roundings differ)."""
    import sliding_window_attention_diagmm_amd as dm
    case = (1, 700, 2, 64, 64, 64, 2, "f16")
    b, n, h, d, w, wu, dil, dt = case
    q, k, v = (t_.cuda() for t_ in _inputs(case, 1200))
    fused = dm.diagmm_banded_attention(q, k, v, w, wu, dil, 0.125)
    S = dm.diagmm_qk(q, k, w, wu, dil, 0.0, out_dtype=torch.float32)
    P = dm.diagmm_banded_softmax(S, w, wu, dil, 0.125)
    three = dm.diagmm_pv(P.to(torch.float16), v, w, wu, dil, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (fused.float() - three).abs().max().item() <= 2e-3


def test_attention_rejects_what_it_does_not_cover():
    import sliding_window_attention_diagmm_amd as dm
    x = torch.zeros(1, 16, 1, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(dm.DiagmmError) as e:
        dm.diagmm_banded_attention(x, x, x, 4)
    assert e.value.status == 5   # DIAGMM_ERR_UNSUPPORTED
    y = torch.zeros(1, 16, 1, 48, dtype=torch.float16, device="cuda")
    with pytest.raises(dm.DiagmmError):
        dm.diagmm_banded_attention(y, y, y, 4)


@pytest.mark.parametrize("dil", [0, 3])
def test_attention_at_the_benchmark_shape(dil):
    """b=1, n=4096, h=12, d=64, 513 diagonals, f16, N(0,1) inputs: 256 sampled rows
    (both sequence ends included) against the oracle."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w = 1, 4096, 12, 64, 256
    g = datagen.rng(1300 + dil)
    q, k, v = (datagen.normal(g, (b, n, h, d), "f16") for _ in range(3))
    got = dm.diagmm_banded_attention(q.cuda(), k.cuda(), v.cuda(), w, w, dil, 0.125)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(n - 4, n),
                                     datagen.rng(1310).choice(n, 248, replace=False)]))
    ri = torch.from_numpy(rows)
    check_attention(got.cpu().reshape(n, h, d)[ri], q, k, v, w, w, dil, 0.125, torch.float16,
                    f"bench dilation {dil}", rows=rows)


def test_attention_at_the_long_document_shape():
    """n = 32768, 8193 diagonals, h = 12, d = 64, f16: 64 sampled rows."""
    import sliding_window_attention_diagmm_amd as dm
    wl = datagen.WORKLOADS["long_n32768"]
    x = datagen.make(wl, ("q", "k", "v"))
    got = dm.diagmm_banded_attention(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), wl.w,
                                     wl.w_upper, 0, 0.125)
    torch.cuda.synchronize()
    rows = datagen.sample_rows(wl.n, wl.w, 64)
    ri = torch.from_numpy(np.asarray(rows))
    check_attention(got.cpu().reshape(wl.n, wl.h, wl.d)[ri], x["q"], x["k"], x["v"], wl.w,
                    wl.w_upper, 0, 0.125, torch.float16, "long document", rows=rows)
