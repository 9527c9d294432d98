"""GPU parity of the banded dropout against the CPU oracle.

out = P / (1 - p) on in-range slots whose float32 random number is greater than p, +0
elsewhere (the oracle's pins are in test_oracle.py).  The keep decision is one float32
comparison on both sides, so the pattern of kept slots is compared exactly: every slot
the oracle zeroes is +0 bit for bit on the GPU, every other slot within the tolerance of
the output dtype.  Cases cover both kernel paths (16-byte pieces straddling rows, and one
element per piece for rows shorter than a piece, for misaligned tensors and under
DIAGMM_KERNEL=simple), the three dtypes, dilation, ragged tails, in-place use, poisoned
out-of-range slots, ties rand == p, p = 0 and p = 0.9, the benchmark shape in full and the
long-document shape (more than 2^32 band elements) on sampled rows.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _util import assert_bits_equal, check_close, in_range_mask, in_range_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, w, w_upper, dilation, dtype, p)
CASES = [
    (1, 512, 1, 32, 32, 0, "f32", 0.1),
    (1, 1, 1, 3, 3, 0, "f16", 0.5),       # one position, K = 7 < 8: element path
    (2, 7, 3, 3, 0, 0, "bf16", 0.25),     # K = 4, causal
    (1, 100, 2, 31, 31, 0, "f16", 0.1),   # K = 63: pieces straddle rows
    (1, 1000, 2, 256, 256, 3, "bf16", 0.1),
    (1, 333, 1, 20, 20, 9, "f16", 0.3),
    (1, 70, 2, 4, 4, 2, "f32", 0.1),      # K = 9 f32: straddles, ragged tail of 2
    (2, 96, 2, 40, 40, 3, "f32", 0.9),
    (1, 64, 1, 0, 0, 0, "f16", 0.1),      # K = 1
    (1, 300, 2, 350, 350, 0, "f16", 0.0),  # window wider than the sequence, p = 0
    (3, 77, 5, 6, 1, 1, "bf16", 0.5),     # K = 8: a piece per row
    (1, 2049, 3, 17, 30, 0, "f16", 0.2),  # several workgroups, tail of 5
]


def _ids(c):
    b, n, h, w, wu, dil, dt, p = c
    return f"b{b}n{n}h{h}w{w}u{wu}s{dil}-{dt}-p{p}"


def _inputs(case, seed):
    b, n, h, w, wu, dil, dt, p = case
    g = datagen.rng(seed)
    S = datagen.normal(g, (b, n, h, w + wu + 1), "f32", 2.0)
    P = oracle.softmax(S, w, wu, dil, scale=1.0, out_dtype=DT[dt])
    rand = datagen.uniform(g, P.shape)
    return P, rand


def _check(case, P, rand, got, what):
    b, n, h, w, wu, dil, dt, p = case
    ref = oracle.dropout(P, rand, w, wu, dil, p=p, out_dtype=torch.float64)
    zero = ref == 0
    g = got.cpu()
    assert_bits_equal(g[zero], torch.zeros_like(g[zero]), f"{what}: dropped and masked slots")
    check_close(g, ref, DT[dt], what, ~zero)
    # the kept pattern is the comparison itself
    mask = in_range_mask(b, n, h, w, wu, dil)
    assert torch.equal(~zero, mask & (rand > np.float32(p)) & (P != 0)), f"{what}: pattern"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_dropout_matches_oracle(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt, p = case
    P, rand = _inputs(case, 700 + n + w)
    got = dm.diagmm_banded_dropout(P.cuda(), rand.cuda(), w, wu, dil, p)
    torch.cuda.synchronize()
    _check(case, P, rand, got, _ids(case))


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[4], CASES[11]], ids=_ids)
def test_dropout_element_path(case, monkeypatch):
    """The element-per-piece kernel, forced with DIAGMM_KERNEL=simple and reached by
    tensors that are not 16-byte aligned, equals the oracle and the piece kernel."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt, p = case
    P, rand = _inputs(case, 800 + n)
    wide = dm.diagmm_banded_dropout(P.cuda(), rand.cuda(), w, wu, dil, p)
    monkeypatch.setenv("DIAGMM_KERNEL", "simple")
    forced = dm.diagmm_banded_dropout(P.cuda(), rand.cuda(), w, wu, dil, p)
    torch.cuda.synchronize()
    monkeypatch.delenv("DIAGMM_KERNEL")
    _check(case, P, rand, forced, "forced element path")
    assert_bits_equal(forced, wide, "element path vs piece path")
    numel = P.numel()
    bp = torch.empty(numel + 8, dtype=P.dtype, device="cuda")
    br = torch.empty(numel + 8, dtype=torch.float32, device="cuda")
    bo = torch.empty(numel + 8, dtype=P.dtype, device="cuda")
    Pm, Rm, Om = bp[1:1 + numel].view(P.shape), br[1:1 + numel].view(P.shape), \
        bo[1:1 + numel].view(P.shape)
    Pm.copy_(P.cuda())
    Rm.copy_(rand.cuda())
    dm.diagmm_banded_dropout(Pm, Rm, w, wu, dil, p, out=Om)
    torch.cuda.synchronize()
    assert_bits_equal(Om, wide, "misaligned tensors")


@pytest.mark.parametrize("case", [CASES[3], CASES[4], CASES[6], CASES[11]], ids=_ids)
def test_dropout_in_place_poisoned_slots_and_ties(case):
    """In place over P equals out of place bit for bit; NaN / inf in out-of-range slots
    of P change nothing; rand == p drops (the comparison is strict)."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, w, wu, dil, dt, p = case
    P, rand = _inputs(case, 900 + n)
    # a tenth of the random numbers exactly p
    tie = datagen.uniform(datagen.rng(901 + n), P.shape) < 0.1
    rand = torch.where(tie, torch.full_like(rand, p), rand)
    Pc, Rc = P.cuda(), rand.cuda()
    ref = dm.diagmm_banded_dropout(Pc, Rc, w, wu, dil, p)
    _check(case, P, rand, ref, "with ties")
    assert torch.all(ref.cpu()[tie] == 0)
    x = Pc.clone()
    dm.diagmm_banded_dropout(x, Rc, w, wu, dil, p, out=x)
    assert_bits_equal(x, ref, "in place")
    mask = in_range_mask(b, n, h, w, wu, dil).cuda()
    for poison in (float("nan"), float("inf")):
        Pp = torch.where(mask, Pc, torch.full_like(Pc, poison))
        assert_bits_equal(dm.diagmm_banded_dropout(Pp, Rc, w, wu, dil, p), ref,
                          f"poisoned with {poison}")


@pytest.mark.parametrize("dil", [0, 3])
def test_dropout_at_the_benchmark_shape(dil):
    """b=1, n=4096, h=12, 513 diagonals, f16, p = 0.1: P from the GPU's qk -> softmax,
    rand from torch's seeded generator on the device; the whole band against the
    oracle on the same P and rand."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w = 1, 4096, 12, 64, 256
    g = datagen.rng(710 + dil)
    q, k = (datagen.normal(g, (b, n, h, d), "f16", 0.125).cuda() for _ in range(2))
    P = dm.diagmm_banded_softmax(dm.diagmm_qk(q, k, w, w, dil), w, w, dil, 0.125, inplace=True)
    gen = torch.Generator(device="cuda").manual_seed(720 + dil)
    rand = torch.rand(P.shape, generator=gen, device="cuda", dtype=torch.float32)
    got = dm.diagmm_banded_dropout(P, rand, w, w, dil, 0.1)
    torch.cuda.synchronize()
    case = (b, n, h, w, w, dil, "f16", 0.1)
    _check(case, P.cpu(), rand.cpu(), got, f"benchmark shape, dilation {dil}")


def test_dropout_at_the_long_document_shape():
    """n = 32768, 8193 diagonals, h = 12, f16: 3.2e9 band elements (flat offsets past
    2^32); P random in [0, 1), rand from torch's seeded generator on the device; 64
    sampled rows against the oracle."""
    import sliding_window_attention_diagmm_amd as dm
    wl = datagen.WORKLOADS["long_n32768"]
    shape = (wl.b, wl.n, wl.h, wl.K)
    gen = torch.Generator(device="cuda").manual_seed(730)
    P = torch.rand(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.float16)
    rand = torch.rand(shape, generator=gen, device="cuda", dtype=torch.float32)
    got = dm.diagmm_banded_dropout(P, rand, wl.w, wl.w_upper, 0, 0.1)
    torch.cuda.synchronize()
    rows = datagen.sample_rows(wl.n, wl.w, 64)
    ri = torch.from_numpy(np.asarray(rows)).cuda()
    P_r, R_r, G_r = (t_.reshape(-1, wl.h, wl.K).index_select(0, ri).cpu()
                     for t_ in (P, rand, got))
    del P, rand, got
    torch.cuda.empty_cache()
    ref = oracle.dropout(P_r, R_r, wl.w, wl.w_upper, 0, p=0.1, out_dtype=torch.float64,
                         n=wl.n, rows=rows)
    mask = in_range_rows(wl.n, wl.h, wl.w, wl.w_upper, 0, rows)
    assert torch.equal(ref != 0, mask & (R_r > np.float32(0.1)) & (P_r != 0))
    zero = ref == 0
    assert_bits_equal(G_r[zero], torch.zeros_like(G_r[zero]), "long document: zeros")
    check_close(G_r, ref, torch.float16, "long document", ~zero)
