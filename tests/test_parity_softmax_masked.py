"""GPU parity of the banded softmax with the per-key additive attention mask (the mask
of the first fusion repro on the csarofeen/pytorch issue 2096 page) against the CPU
oracle: every group layout (1 .. 32 lanes per row), the workgroup-per-row kernel (forced,
misaligned tensors, a wider output dtype), dilation, in place, the benchmark shape with
padded key positions, and banded attention with a key mask through torch autograd."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from _util import assert_bits_equal, check_close, in_range_mask, in_range_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, w, w_upper, dilation, in, out); comment: the kernel layout it reaches
CASES = [
    (1, 64, 1, 0, 0, 0, "f16", "f16"),          # K = 1: 1 lane
    (2, 50, 2, 16, 15, 0, "f16", "f16"),        # 32 slots: 2 lanes
    (1, 100, 2, 31, 31, 0, "bf16", "bf16"),     # 63 slots: 4 lanes
    (1, 512, 1, 32, 32, 0, "f32", "f32"),       # 65 f32 slots: 8 lanes
    (1, 40, 1, 300, 0, 0, "bf16", "bf16"),      # 301 slots: 16 lanes
    (2, 1000, 2, 256, 256, 0, "f16", "f16"),    # 513 slots: 32 lanes
    (1, 1000, 2, 256, 256, 3, "f16", "f16"),
    (1, 333, 1, 20, 20, 9, "bf16", "bf16"),
    (1, 30, 1, 1200, 1200, 0, "f16", "f16"),    # 2401 slots: the row kernel
    (1, 257, 2, 64, 0, 2, "bf16", "f32"),       # wider output: the row kernel
]


def _ids(c):
    b, n, h, w, wu, dil, i, o = c
    return f"b{b}n{n}h{h}w{w}u{wu}s{dil}-{i}-{o}"


def _inputs(case, seed):
    b, n, h, w, wu, dil, ind, _ = case
    g = datagen.rng(seed)
    S = datagen.normal(g, (b, n, h, w + wu + 1), ind, 2.0)
    m = torch.from_numpy((g.random((b, n)) > 0.25).astype(np.float32))
    m[:, -max(1, n // 10):] = 0.0                      # padded positions at the end
    return S, m


def _check(case, S, m, P_gpu, scale, mv, what):
    """Against the oracle in double.  The method adds the mask term in float32 (the page's
    recipe works in Float), so a scaled score near mask_value carries a rounding error of
    up to 2^-24 (|mask_value| + max |scale S|), and every probability of its row a relative
    error of twice that: for float32 outputs that bound replaces the 1e-5 normwise bar
    where it is the larger; 16-bit outputs keep their bar (probabilities are at most 1)."""
    b, n, h, w, wu, dil, ind, outd = case
    ref = oracle.softmax_masked(S, m, w, wu, dil, scale=scale, mask_value=mv,
                                out_dtype=torch.float64)
    mask = in_range_mask(b, n, h, w, wu, dil)
    rel = 2.0 * 2.0 ** -24 * (abs(mv) + abs(scale) * S.double().abs().max().item()) * 1.25
    if DT[outd] == torch.float32 and rel > 1e-5:
        g, r = P_gpu.double().cpu()[mask], ref[mask]
        bad = (g - r).abs() > rel * r.abs() + 1e-7
        assert not bad.any(), f"{what}: {int(bad.sum())} beyond the float32 mask-term bound"
    else:
        check_close(P_gpu, ref, DT[ind] if DT[outd] == DT[ind] else torch.float32, what, mask)
    masked = P_gpu.cpu()[~mask]
    assert_bits_equal(masked, torch.zeros_like(masked), f"{what}: out-of-range slots")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_masked_softmax_matches_oracle(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, ind, outd = case
    S, m = _inputs(case, 800 + n + w)
    P = dm.diagmm_banded_softmax(S.cuda(), w, wu, dil, 0.125, out_dtype=DT[outd],
                                 key_mask=m.cuda())
    torch.cuda.synchronize()
    _check(case, S, m, P, 0.125, -10000.0, _ids(case))


@pytest.mark.parametrize("case", [CASES[3], CASES[5], CASES[6]], ids=_ids)
def test_masked_softmax_row_kernel_in_place_and_misaligned(case, monkeypatch):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, ind, outd = case
    S, m = _inputs(case, 900 + n)
    mc = m.cuda()
    ref = dm.diagmm_banded_softmax(S.cuda(), w, wu, dil, 0.5, key_mask=mc, mask_value=-30.0)
    x = S.cuda()
    dm.diagmm_banded_softmax(x, w, wu, dil, 0.5, inplace=True, key_mask=mc, mask_value=-30.0)
    assert_bits_equal(x, ref, "in place")
    monkeypatch.setenv("DIAGMM_KERNEL", "simple")
    forced = dm.diagmm_banded_softmax(S.cuda(), w, wu, dil, 0.5, key_mask=mc, mask_value=-30.0)
    torch.cuda.synchronize()
    monkeypatch.delenv("DIAGMM_KERNEL")
    _check(case, S, m, forced, 0.5, -30.0, "forced row kernel")
    numel = S.numel()
    buf_s = torch.empty(numel + 8, dtype=S.dtype, device="cuda")
    buf_p = torch.empty(numel + 8, dtype=S.dtype, device="cuda")
    Sm, Pm = buf_s[1:1 + numel].view(S.shape), buf_p[1:1 + numel].view(S.shape)
    Sm.copy_(S.cuda())
    dm.diagmm_banded_softmax(Sm, w, wu, dil, 0.5, out=Pm, key_mask=mc, mask_value=-30.0)
    torch.cuda.synchronize()
    _check(case, S, m, Pm, 0.5, -30.0, "misaligned tensors")


def test_masked_softmax_at_the_benchmark_shape():
    """b=2, n=4096, h=12, 513 diagonals, f16 scores from the GPU's qk of N(0,1)/8 inputs,
    the last 300 positions of the second sequence padded; sampled rows vs the oracle."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w = 2, 4096, 12, 64, 256
    g = datagen.rng(910)
    q, k = (datagen.normal(g, (b, n, h, d), "f16", 0.125).cuda() for _ in range(2))
    m = torch.ones(b, n)
    m[1, -300:] = 0.0
    S = dm.diagmm_qk(q, k, w, w, 0)
    S_cpu = S.cpu()
    P = dm.diagmm_banded_softmax(S, w, w, 0, 0.125, inplace=True, key_mask=m.cuda())
    rows = np.unique(np.concatenate([np.arange(0, 3), np.arange(n - 3, n), n + np.arange(0, 3),
                                     2 * n - 1 - np.arange(0, 400, 7),
                                     datagen.rng(911).choice(2 * n, 200, replace=False)]))
    ri = torch.from_numpy(rows)
    P_r = P.reshape(-1, h, 2 * w + 1).index_select(0, ri.cuda()).cpu()
    S_r = S_cpu.reshape(-1, h, 2 * w + 1).index_select(0, ri)
    ref = oracle.softmax_masked(S_r, m, w, w, 0, scale=0.125, out_dtype=torch.float64, n=n,
                                rows=rows)
    mask = in_range_rows(n, h, w, w, 0, rows)
    check_close(P_r, ref, torch.float16, "masked softmax", mask)
    assert torch.all(P_r[~mask].view(torch.int16) == 0)


def _selected(n, w, wu, s):
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    off = j - i
    return (off % s == 0) & (off >= -w * s) & (off <= wu * s)


@pytest.mark.parametrize("dil", [0, 2])
def test_masked_banded_attention_gradients(dil):
    from sliding_window_attention_diagmm_amd.attention import banded_attention
    b, n, h, d, w, wu = 2, 120, 2, 32, 10, 6
    g_ = datagen.rng(930 + dil)
    q, k, v, gout = (datagen.normal(g_, (b, n, h, d), "f32") for _ in range(4))
    m = torch.from_numpy((g_.random((b, n)) > 0.2).astype(np.float32))
    qc, kc, vc = (t_.cuda().requires_grad_(True) for t_ in (q, k, v))
    o = banded_attention(qc, kc, vc, w, wu, dil, key_mask=m.cuda())
    o.backward(gout.cuda())
    qd, kd, vd = (t_.double().requires_grad_(True) for t_ in (q, k, v))
    sel = _selected(n, w, wu, max(dil, 1))
    s = torch.einsum("bihd,bjhd->bhij", qd, kd) / math.sqrt(d)
    s = s + ((1 - m.double()) * -10000.0)[:, None, None, :]
    p = torch.softmax(s.masked_fill(~sel, float("-inf")), -1)
    od = torch.einsum("bhij,bjhd->bihd", p, vd)
    (od * gout.double()).sum().backward()
    for name, got, ref in (("out", o, od), ("dq", qc.grad, qd.grad), ("dk", kc.grad, kd.grad),
                           ("dv", vc.grad, vd.grad)):
        err = ((got.detach().double().cpu() - ref.detach()).abs().max() /
               ref.detach().abs().max()).item()
        assert err <= 1e-5, f"{name}: normwise error {err:.3e}"
