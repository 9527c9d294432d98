"""Pins for the CPU oracle (CPU only).

The oracle is the reference every GPU result is compared with, so it is pinned
here to things other than itself: library routines (numpy / torch conversions,
dense matrix products, torch.softmax), hand-derived tiny examples, closed-form
counts, and identities of the mathematics (adjoint, residue classes, w >= n).
Each test names the property of the pages it stands on; the pages are
TVM Discuss "Developing a faster schedule for Longformer's kernel" (posts 1-6)
and csarofeen/pytorch issue 2096 (first fusion repro).
"""
import math
import os

import numpy as np
import pytest
import torch

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- conversions

def test_half_decode_all_patterns():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    h = bits.view(torch.float16)
    got = oracle.widen(h)
    ref = h.to(torch.float64)
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], ref[~nan])


def test_bf16_decode_all_patterns():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    h = bits.view(torch.bfloat16)
    got = oracle.widen(h)
    ref = h.to(torch.float64)
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], ref[~nan])


def _edge_values():
    g = np.random.default_rng(7)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e-8, 2.0 ** -24,
            2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1e30, -1e30,
            float("inf"), float("-inf"), 3.3895313892515355e38, 3.4e38, 1e-40, 1e-45]
    # exact ties between neighbouring half / bf16 values (both parities)
    for m in range(1024, 1040):
        vals.append((m + 0.5) * 2.0 ** -10)
        vals.append(-(m + 0.5) * 2.0 ** 3)
    for m in range(128, 140):
        vals.append((m + 0.5) * 2.0 ** -7)
    rnd = g.standard_normal(20000) * np.exp(g.uniform(-30, 30, 20000))
    return np.concatenate([np.array(vals), rnd]).astype(np.float64)


def test_half_encode_matches_numpy():
    x = _edge_values()
    got = oracle.convert(torch.from_numpy(x), torch.float16).view(torch.int16).numpy()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.int16)  # numpy rounds double -> half directly, RNE
    assert np.array_equal(got, ref)


def test_bf16_encode_matches_torch_on_float32_values():
    # Values exactly representable in float32, so torch's float -> bf16 RNE applies once.
    x = _edge_values().astype(np.float32)
    x = x[np.isfinite(x) | np.isinf(x)]
    got = oracle.convert(torch.from_numpy(x.astype(np.float64)), torch.bfloat16)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_f32_encode_is_round_to_nearest():
    x = _edge_values()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32)
    got = oracle.convert(torch.from_numpy(x), torch.float32).numpy()
    assert np.array_equal(got.view(np.int32), ref.view(np.int32))


# ------------------------------------------------------------- hand examples

def test_qk_hand_example():
    """n=4, w=w_upper=1, d=2: slots (left, diagonal, right) of each row, worked by hand:
    row 0 = (pad, q0.k0, q0.k1), ..., row 3 = (q3.k2, q3.k3, pad)."""
    q = torch.tensor([[1, 0], [0, 1], [1, 1], [2, -1]], dtype=torch.float32).reshape(1, 4, 1, 2)
    k = torch.tensor([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=torch.float32).reshape(1, 4, 1, 2)
    want = torch.tensor([[-9, 1, 3], [2, 4, 6], [7, 11, 15], [4, 6, -9]], dtype=torch.float32)
    got = oracle.qk(q, k, 1, 1, 0, padding=-9.0).reshape(4, 3)
    assert torch.equal(got, want)


def test_pv_pvT_hand_example():
    """n=3, w=1, w_upper=0 (autoregressive: slots = (previous key, own key)), d=1.
    pv: out[i] = P[i,0]*V[i-1] + P[i,1]*V[i]; row 0 has no previous key.
    pvT: out[j] = G[j,1]*X[j] + G[j+1,0]*X[j+1]; the last row has no successor."""
    P = torch.tensor([[100.0, 1.0], [2.0, 3.0], [4.0, 5.0]]).reshape(1, 3, 1, 2)
    V = torch.tensor([10.0, 20.0, 30.0]).reshape(1, 3, 1, 1)
    pv = oracle.pv(P, V, 1, 0).flatten().tolist()
    assert pv == [1 * 10, 2 * 10 + 3 * 20, 4 * 20 + 5 * 30]
    pvT = oracle.pvT(P, V, 1, 0).flatten().tolist()
    assert pvT == [1 * 10 + 2 * 20, 3 * 20 + 4 * 30, 5 * 30]


def test_result_width_matches_forward_constants():
    """TVM thread post 6: for w = w_upper = 256 the result's last dimension is
    t3d3 = 2w+1 = 513, and the backward functions take a band with last dim 2w+1."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "band_width.txt"))
            if ln.strip() and not ln.startswith("#")]
    for w, wu, width in ((int(a), int(b), int(c)) for a, b, c in rows):
        q = torch.zeros(1, 2, 1, 1)
        assert oracle.qk(q, q, w, wu).shape[-1] == width
        band = torch.zeros(1, 2, 1, width)
        assert oracle.pv(band, q, w, wu).shape == (1, 2, 1, 1)


# ------------------------------------------------------ P1: dense brute force

def _selected(n, w, wu, s):
    """Mask of the selected diagonals (figures 2.b / 2.c): offset j - i is a multiple
    of s between -w*s and w_upper*s."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    off = j - i
    return (off % s == 0) & (off >= -w * s) & (off <= wu * s)


def _dense_from_band(band_row_vals, mask_row, n):
    """Place a band row's in-range values on the selected columns, in order."""
    out = np.zeros(n)
    out[np.nonzero(mask_row)[0]] = band_row_vals
    return out


CASES = [  # (n, w, wu, dil, d)
    (1, 0, 0, 0, 1), (2, 1, 1, 0, 3), (5, 1, 1, 0, 3), (5, 3, 0, 0, 2), (23, 3, 3, 0, 3),
    (23, 3, 3, 2, 3), (23, 2, 2, 3, 1), (23, 2, 0, 9, 2), (64, 5, 5, 1, 8), (64, 70, 70, 0, 4),
    (23, 30, 0, 2, 2), (40, 4, 7, 3, 5),
]


@pytest.mark.parametrize("n,w,wu,dil,d", CASES)
def test_qk_pv_pvT_match_dense_products(n, w, wu, dil, d):
    g = datagen.rng(11)
    b, h = 2, 2
    s = max(dil, 1)
    Q = datagen.normal(g, (b, n, h, d), "f32").double()
    Kt = datagen.normal(g, (b, n, h, d), "f32").double()
    G = datagen.normal(g, (b, n, h, w + wu + 1), "f32").double()
    pad = -7.5
    band = oracle.qk(Q, Kt, w, wu, dil, pad)
    pv = oracle.pv(G, Kt, w, wu, dil)
    pvT = oracle.pvT(G, Q, w, wu, dil)
    mask = _selected(n, w, wu, s)
    for bb in range(b):
        for hh in range(h):
            D = Q[bb, :, hh].numpy() @ Kt[bb, :, hh].numpy().T
            B = np.zeros((n, n))
            for i in range(n):
                row = band[bb, i, hh].numpy()
                inr = row != pad
                # in-range slots, in slot order, are the selected columns in column order
                assert inr.sum() == mask[i].sum()
                np.testing.assert_allclose(row[inr], D[i, mask[i]], rtol=1e-12, atol=1e-12)
                # the same placement turns the gradient band into a dense matrix
                gi = G[bb, i, hh].numpy()
                B[i] = _dense_from_band(gi[inr], mask[i], n)
            np.testing.assert_allclose(pv[bb, :, hh].numpy(), B @ Kt[bb, :, hh].numpy(),
                                       rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(pvT[bb, :, hh].numpy(), B.T @ Q[bb, :, hh].numpy(),
                                       rtol=1e-12, atol=1e-12)


def test_slot_order_left_diagonal_right():
    """w_upper is the window to the right of the word (TVM thread post 5): with
    w_upper = 0 no slot reaches a later key; with w = 0 none reaches an earlier one;
    slot w is the word itself."""
    n, d = 9, 1
    Q = torch.ones(1, n, 1, d)
    Kp = torch.arange(1, n + 1, dtype=torch.float32).reshape(1, n, 1, d)  # key j holds j+1
    left = oracle.qk(Q, Kp, 3, 0, padding=0.0)[0, :, 0]
    right = oracle.qk(Q, Kp, 0, 3, padding=0.0)[0, :, 0]
    for i in range(n):
        assert left[i, 3] == i + 1 and right[i, 0] == i + 1
        assert all(0 < v <= i + 1 for v in left[i].tolist() if v)
        assert all(v >= i + 1 for v in right[i].tolist() if v)
        # keys grow with the slot index
        lv = [v for v in left[i].tolist() if v]
        rv = [v for v in right[i].tolist() if v]
        assert lv == sorted(lv) and rv == sorted(rv)


# ----------------------------------------------- P2: w >= n gives the full matrix

@pytest.mark.parametrize("dil", [0, 2, 3])
def test_wide_window_reproduces_full_product(dil):
    """With w = w_upper >= n every key of the row's residue class is in range once,
    so the band's in-range slots, read in slot order, are the full row of Q.K^T
    restricted to that class (all keys when dilation is 0)."""
    n, d = 17, 5
    s = max(dil, 1)
    g = datagen.rng(3)
    Q = datagen.normal(g, (1, n, 1, d), "f32").double()
    Kt = datagen.normal(g, (1, n, 1, d), "f32").double()
    band = oracle.qk(Q, Kt, n + 4, n + 4, dil, padding=float("nan"))[0, :, 0].numpy()
    D = Q[0, :, 0].numpy() @ Kt[0, :, 0].numpy().T
    for i in range(n):
        vals = band[i][~np.isnan(band[i])]
        want = D[i, [j for j in range(n) if (j - i) % s == 0]]
        np.testing.assert_allclose(vals, want, rtol=1e-12, atol=1e-12)
    # and pv with probability rows becomes dense attention P.V
    if dil == 0:
        P = torch.softmax(torch.from_numpy(D), -1)
        Pb = torch.full((1, n, 1, 2 * (n + 4) + 1), float("nan"), dtype=torch.float64)
        for i in range(n):
            Pb[0, i, 0, ~torch.from_numpy(np.isnan(band[i]))] = P[i]
        V = Kt
        out = oracle.pv(Pb, V, n + 4, n + 4)[0, :, 0].numpy()
        np.testing.assert_allclose(out, P.numpy() @ V[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P3: adjoint

@pytest.mark.parametrize("n,w,wu,dil", [(64, 7, 7, 0), (96, 9, 0, 3), (50, 4, 6, 2), (33, 40, 40, 1)])
def test_adjoint_identity(n, w, wu, dil):
    """<qk(Q,K), G> = <pvT(G,Q), K> = <pv(G,K), Q> with padding 0: pv and pvT are the
    two backward functions of the forward qk (TVM thread post 6)."""
    g = datagen.rng(5)
    b, h, d = 2, 3, 6
    Q = datagen.normal(g, (b, n, h, d), "f32").double()
    Kt = datagen.normal(g, (b, n, h, d), "f32").double()
    G = datagen.normal(g, (b, n, h, w + wu + 1), "f32").double()
    a = (oracle.qk(Q, Kt, w, wu, dil, 0.0) * G).sum().item()
    bq = (oracle.pvT(G, Q, w, wu, dil) * Kt).sum().item()
    cq = (oracle.pv(G, Kt, w, wu, dil) * Q).sum().item()
    assert math.isclose(a, bq, rel_tol=1e-11, abs_tol=1e-9)
    assert math.isclose(a, cq, rel_tol=1e-11, abs_tol=1e-9)


def test_adjoint_at_backward_shape_fp32_output():
    """The adjoint identity at the autoregressive backward shape (one batch-head slice
    is enough: slices are independent)."""
    n, w, wu, d = 4096, 256, 0, 64
    g = datagen.rng(6)
    Q = datagen.normal(g, (1, n, 1, d), "bf16")
    Kt = datagen.normal(g, (1, n, 1, d), "bf16")
    G = datagen.normal(g, (1, n, 1, w + wu + 1), "bf16")
    a = (oracle.qk(Q, Kt, w, wu, 0, 0.0, out_dtype=torch.float64) * G.double()).sum().item()
    bq = (oracle.pvT(G, Q, w, wu, out_dtype=torch.float64) * Kt.double()).sum().item()
    cq = (oracle.pv(G, Kt, w, wu, out_dtype=torch.float64) * Q.double()).sum().item()
    assert math.isclose(a, bq, rel_tol=1e-10)
    assert math.isclose(a, cq, rel_tol=1e-10)


# -------------------------------------------------------- P4: integer exactness

@pytest.mark.parametrize("dt,odt", [("f16", torch.float16), ("bf16", torch.float32),
                                    ("f32", torch.float32), ("bf16", torch.bfloat16)])
def test_small_integers_are_exact_in_every_dtype(dt, odt):
    n, w, wu, d = 40, 5, 3, 16
    g = datagen.rng(9)
    Q = datagen.small_ints(g, (1, n, 2, d), -2, 2, dt)
    Kt = datagen.small_ints(g, (1, n, 2, d), -2, 2, dt)
    P = datagen.small_ints(g, (1, n, 2, w + wu + 1), -1, 1, dt)
    for dil in (0, 2):
        exact = oracle.qk(Q, Kt, w, wu, dil, 0.0, out_dtype=torch.float64)
        assert torch.equal(exact, exact.round())  # integer valued
        got = oracle.qk(Q, Kt, w, wu, dil, 0.0, out_dtype=odt)
        if odt == torch.bfloat16:  # |qk| <= 64 here: exact in bf16 as well
            assert exact.abs().max() <= 64
        assert torch.equal(got.double(), exact)
        e2 = oracle.pv(P, Q, w, wu, dil, out_dtype=torch.float64)
        assert torch.equal(oracle.pv(P, Q, w, wu, dil, out_dtype=odt).double(), e2)
        e3 = oracle.pvT(P, Q, w, wu, dil, out_dtype=torch.float64)
        assert torch.equal(oracle.pvT(P, Q, w, wu, dil, out_dtype=odt).double(), e3)


# ---------------------------------------------------------- P5: in-range counts

def _count_in_range(n, w, wu, s):
    # row i reaches min(w, i // s) slots to the left and min(wu, (n-1-i) // s) to the right
    return sum(min(w, i // s) + min(wu, (n - 1 - i) // s) + 1 for i in range(n))


@pytest.mark.parametrize("n,w,wu,dil,expected", [
    (4096, 256, 256, 0, 2035456),    # n*K - w(w+1)/2 - wu(wu+1)/2
    (4096, 256, 256, 3, 1903872),
    (4096, 256, 0, 0, 1019776),
    (512, 32, 32, 0, 512 * 65 - 32 * 33),
])
def test_ones_count_in_range_slots(n, w, wu, dil, expected):
    """Q = K = 1 (d = 1): every in-range slot is exactly 1, every other slot is the
    padding; the number of in-range slots has a closed form."""
    ones = torch.ones(1, n, 1, 1, dtype=torch.float16)
    band = oracle.qk(ones, ones, w, wu, dil, padding=-1.0)
    assert set(torch.unique(band).tolist()) <= {1.0, -1.0}
    cnt = int((band == 1).sum())
    assert cnt == expected == _count_in_range(n, w, wu, max(dil, 1))
    if dil <= 1 and w < n and wu < n:
        assert cnt == n * (w + wu + 1) - w * (w + 1) // 2 - wu * (wu + 1) // 2


def test_padding_slots_carry_the_rounded_constant():
    """'padding: any const' (TVM thread posts 5 and 6) - stored with one rounding."""
    n = 8
    z = torch.zeros(1, n, 1, 4, dtype=torch.float16)
    for pad in (0.0, -0.0, float("-inf"), 1e30, 0.1, -65519.0):
        band = oracle.qk(z, z, 3, 3, 0, padding=pad)
        want = torch.tensor(pad, dtype=torch.float64).to(torch.float16)  # numpy-equal RNE
        pad_slots = band[0, 0, 0, :3]
        assert torch.equal(pad_slots.view(torch.int16),
                           want.expand(3).contiguous().view(torch.int16))


# ------------------------------------------------------- P6: residue classes

@pytest.mark.parametrize("s", [2, 3, 9])
def test_dilated_band_is_undilated_band_of_each_residue_class(s):
    """Dilation s only pairs positions of one residue class mod s, as a sliding window
    with contiguous diagonals on that sub-sequence."""
    n, w, wu, d = 61, 4, 3, 5
    g = datagen.rng(13)
    Q = datagen.normal(g, (2, n, 2, d), "f32").double()
    Kt = datagen.normal(g, (2, n, 2, d), "f32").double()
    V = datagen.normal(g, (2, n, 2, d), "f32").double()
    P = datagen.normal(g, (2, n, 2, w + wu + 1), "f32").double()
    band = oracle.qk(Q, Kt, w, wu, s, 0.5)
    pv = oracle.pv(P, V, w, wu, s)
    pvT = oracle.pvT(P, V, w, wu, s)
    for r in range(s):
        sub = slice(r, None, s)
        assert torch.equal(band[:, sub], oracle.qk(Q[:, sub].contiguous(), Kt[:, sub].contiguous(),
                                                   w, wu, 0, 0.5))
        assert torch.allclose(pv[:, sub], oracle.pv(P[:, sub].contiguous(), V[:, sub].contiguous(),
                                                    w, wu, 0), rtol=0, atol=1e-13)
        assert torch.allclose(pvT[:, sub], oracle.pvT(P[:, sub].contiguous(), V[:, sub].contiguous(),
                                                      w, wu, 0), rtol=0, atol=1e-13)


# ------------------------------------------------------------ P7: one-hot band

def test_one_hot_band_gathers_rows():
    """A band that is 1 on the main diagonal slot (slot w) makes pv the identity; on
    the slot just right of it (s = 1) it shifts V up by one row, the last row getting
    nothing; pvT of the diagonal is the identity too."""
    n, w, wu, d = 30, 3, 2, 7
    g = datagen.rng(17)
    V = datagen.normal(g, (1, n, 2, d), "f32")
    eye = torch.zeros(1, n, 2, w + wu + 1)
    eye[..., w] = 1
    assert torch.equal(oracle.pv(eye, V, w, wu), V)
    assert torch.equal(oracle.pvT(eye, V, w, wu), V)
    nxt = torch.zeros(1, n, 2, w + wu + 1)
    nxt[..., w + 1] = 1
    out = oracle.pv(nxt, V, w, wu)
    assert torch.equal(out[:, :-1], V[:, 1:])
    assert torch.equal(out[:, -1], torch.zeros_like(out[:, -1]))


# ------------------------------------------------------- P8: poisoned slots

@pytest.mark.parametrize("poison", [float("nan"), 1e30, float("inf")])
def test_out_of_range_band_values_never_reach_pv_or_pvT(poison):
    n, w, wu, dil, d = 37, 6, 5, 2, 4
    g = datagen.rng(19)
    P = datagen.normal(g, (1, n, 3, w + wu + 1), "f32")
    X = datagen.normal(g, (1, n, 3, d), "f32")
    ones = torch.ones(1, n, 1, 1)
    inr = (oracle.qk(ones, ones, w, wu, dil, padding=0.0) == 1).expand_as(P)
    Pp = torch.where(inr, P, torch.tensor(poison))
    assert torch.equal(oracle.pv(Pp, X, w, wu, dil), oracle.pv(P, X, w, wu, dil))
    assert torch.equal(oracle.pvT(Pp, X, w, wu, dil), oracle.pvT(P, X, w, wu, dil))


# --------------------------------------------------------------- P9: softmax

def test_softmax_matches_torch_on_masked_dense_rows():
    """Banded softmax = torch.softmax over the full row of scale * Q.K^T with the
    unselected diagonals at -inf (recipe: scale, max, subtract, exp, sum, divide)."""
    n, w, wu, d = 29, 4, 6, 8
    for dil in (0, 2):
        s = max(dil, 1)
        g = datagen.rng(23)
        Q = datagen.normal(g, (1, n, 1, d), "f32").double()
        Kt = datagen.normal(g, (1, n, 1, d), "f32").double()
        band = oracle.qk(Q, Kt, w, wu, dil, padding=123.0)
        P = oracle.softmax(band, w, wu, dil, scale=0.125)[0, :, 0].numpy()
        D = (Q[0, :, 0] @ Kt[0, :, 0].T) * 0.125
        mask = torch.from_numpy(_selected(n, w, wu, s))
        ref = torch.softmax(D.masked_fill(~mask, float("-inf")), -1).numpy()
        inr = band[0, :, 0].numpy() != 123.0
        for i in range(n):
            np.testing.assert_allclose(P[i][inr[i]], ref[i][mask[i].numpy()], rtol=1e-13,
                                       atol=1e-15)
            assert np.all(P[i][~inr[i]] == 0.0)
            assert math.isclose(P[i].sum(), 1.0, rel_tol=1e-13)


def test_softmax_invariants_fp16():
    n, w, wu = 300, 40, 40
    g = datagen.rng(29)
    S = datagen.normal(g, (1, n, 2, w + wu + 1), "f16", 4.0)
    P = oracle.softmax(S, w, wu, 0, scale=0.125)
    P64 = oracle.softmax(S, w, wu, 0, scale=0.125, out_dtype=torch.float64)
    # one rounding: fp16 output within half an ulp of the double value
    assert torch.all((P.double() - P64).abs() <= P64.abs() * 2.0 ** -11 + 2.0 ** -25)
    sums = P.double().sum(-1)
    assert torch.all((sums - 1).abs() <= (w + wu + 1) * 2.0 ** -11)
    ones = torch.ones(1, n, 1, 1)
    inr = (oracle.qk(ones, ones, w, wu, padding=0.0) == 1).expand_as(P)
    assert torch.all(P[~inr] == 0) and not torch.any(torch.signbit(P[~inr]))
    # shift invariance (exact in double up to the rounding of scale * S)
    shifted = oracle.softmax(S.double() + 3.0, w, wu, 0, scale=0.125, out_dtype=torch.float64)
    assert torch.allclose(shifted, P64, rtol=1e-12, atol=1e-15)
    # a row of equal scores is uniform over its in-range slots
    U = oracle.softmax(torch.zeros(1, n, 1, w + wu + 1), w, wu, 0, out_dtype=torch.float64)
    cnt = inr[:, :, :1].sum(-1, keepdim=True).double()
    assert torch.allclose(U, torch.where(inr[:, :, :1], 1.0 / cnt, 0.0), rtol=1e-15, atol=0)


# ------------------------------------------------------ masked softmax pins
# The page's attention mask: a per-key mask m adds (1 - m) * (-10000) to the scaled score
# (csarofeen/pytorch issue 2096, first fusion repro).

def test_masked_softmax_with_all_ones_is_the_plain_softmax():
    n, w, wu = 50, 7, 3
    g = datagen.rng(61)
    S = datagen.normal(g, (2, n, 2, w + wu + 1), "f16", 3.0)
    ones = torch.ones(2, n)
    for dil in (0, 2):
        a = oracle.softmax_masked(S, ones, w, wu, dil, scale=0.125, out_dtype=torch.float64)
        b = oracle.softmax(S, w, wu, dil, scale=0.125, out_dtype=torch.float64)
        assert torch.equal(a, b)


def test_masked_softmax_matches_torch_on_dense_rows():
    n, w, wu, d = 31, 5, 4, 8
    for dil in (0, 3):
        s = max(dil, 1)
        g = datagen.rng(67 + dil)
        Q = datagen.normal(g, (2, n, 1, d), "f32").double()
        Kt = datagen.normal(g, (2, n, 1, d), "f32").double()
        m = torch.from_numpy((g.random((2, n)) > 0.3).astype(np.float32))
        m[:, ::7] = 0.25                                   # the term is linear in m
        band = oracle.qk(Q, Kt, w, wu, dil, padding=0.0)
        P = oracle.softmax_masked(band, m, w, wu, dil, scale=0.3, mask_value=-7.0,
                                  out_dtype=torch.float64)
        sel = torch.from_numpy(_selected(n, w, wu, s))
        for bb in range(2):
            D = (Q[bb, :, 0] @ Kt[bb, :, 0].T) * 0.3 + (1 - m[bb].double())[None, :] * -7.0
            ref = torch.softmax(D.masked_fill(~sel, float("-inf")), -1)
            for i in range(n):
                cols = torch.nonzero(sel[i]).flatten()
                ks = (cols - i) // s + w
                np.testing.assert_allclose(P[bb, i, 0, ks].numpy(), ref[i, cols].numpy(),
                                           rtol=1e-12, atol=1e-15)
                out = torch.ones(w + wu + 1, dtype=torch.bool)
                out[ks] = False
                assert torch.all(P[bb, i, 0, out] == 0)


def test_masked_softmax_closed_forms():
    n, w, wu = 40, 6, 6
    g = datagen.rng(71)
    S = datagen.normal(g, (1, n, 2, w + wu + 1), "f32").double()
    plain = oracle.softmax(S, w, wu, 0, scale=0.5, out_dtype=torch.float64)
    # every key masked: the same shift for every slot, so the plain softmax again
    zeros = torch.zeros(1, n)
    allm = oracle.softmax_masked(S, zeros, w, wu, 0, scale=0.5, out_dtype=torch.float64)
    assert torch.allclose(allm, plain, rtol=1e-9, atol=0)
    # one masked key among kept ones: its probability underflows to exactly 0, and the
    # row is the plain softmax of the other slots
    m = torch.ones(1, n)
    m[0, 20] = 0
    P = oracle.softmax_masked(S, m, w, wu, 0, scale=0.5, out_dtype=torch.float64)
    for i in range(14, 27):
        k = 20 - i + w                                     # slot of key 20 in row i
        assert P[0, i, :, k].eq(0).all()
        keep = plain[0, i].clone()
        keep[:, k] = 0
        assert torch.allclose(P[0, i], keep / keep.sum(-1, keepdim=True), rtol=1e-12, atol=0)
    # one rounding of a 16-bit output
    P16 = oracle.softmax_masked(S, m, w, wu, 0, scale=0.5, out_dtype=torch.float16)
    assert torch.equal(P16, oracle.convert(P, torch.float16))


# ------------------------------------------------------------- dropout pins

def test_dropout_keeps_by_comparison_and_scales():
    n, w, wu = 60, 8, 8
    K = w + wu + 1
    g = datagen.rng(81)
    S = datagen.normal(g, (2, n, 3, K), "f32")
    P = oracle.softmax(S, w, wu, 0, out_dtype=torch.float64)
    rand = torch.from_numpy(g.random((2, n, 3, K), dtype=np.float32))
    ones = torch.ones(1, n, 1, 1)
    inr = (oracle.qk(ones, ones, w, wu, padding=0.0) == 1).expand_as(P)
    for p in (0.1, 0.5):
        out = oracle.dropout(P, rand, w, wu, 0, p=p, out_dtype=torch.float64)
        keep = inr & (rand > torch.tensor(p, dtype=torch.float32))
        assert torch.equal(out != 0, keep & (P != 0))
        pf = float(np.float32(p))                          # p as the float the call takes
        np.testing.assert_allclose(out[keep].numpy(), (P[keep] / (1.0 - pf)).numpy(),
                                   rtol=1e-15)
        assert torch.all(out[~inr] == 0)
        # the kept share of in-range slots is 1 - p within five binomial deviations
        m = int(inr.sum())
        share = keep.sum().item() / m
        assert abs(share - (1 - p)) <= 5 * math.sqrt(p * (1 - p) / m)
    # out-of-range slots are 0 whatever the band holds there
    poisoned = torch.where(inr, P, torch.full_like(P, 7.0))
    assert torch.all(oracle.dropout(poisoned, rand, w, wu, 0, p=0.1,
                                    out_dtype=torch.float64)[~inr] == 0)
    # p = 0 keeps every in-range probability exactly; a 16-bit output is rounded once
    assert torch.equal(oracle.dropout(P, rand, w, wu, 0, p=0.0, out_dtype=torch.float64),
                       torch.where(inr, P, torch.zeros_like(P)))
    Ph = oracle.convert(P, torch.float16)
    d64 = oracle.dropout(Ph, rand, w, wu, 0, p=0.1, out_dtype=torch.float64)
    assert torch.equal(oracle.dropout(Ph, rand, w, wu, 0, p=0.1),
                       oracle.convert(d64, torch.float16))


def test_dropout_tie_drops():
    """The page keeps a slot when its uniform is strictly greater than p (`gt`), so a
    uniform equal to p, as the float32 value the call takes, drops; the float32 values
    just above keep.  Uniform float32 draws almost never hit p exactly, so the ties are
    planted: every third slot holds float32(p), the rest the next float32 up or down."""
    n, w, wu = 40, 5, 5
    K = w + wu + 1
    g = datagen.rng(82)
    S = datagen.normal(g, (1, n, 2, K), "f32")
    P = oracle.softmax(S, w, wu, 0, out_dtype=torch.float64)
    ones = torch.ones(1, n, 1, 1)
    inr = (oracle.qk(ones, ones, w, wu, padding=0.0) == 1).expand_as(P)
    for p in (0.1, 0.5):
        pf = np.float32(p)
        up = np.nextafter(pf, np.float32(1))
        dn = np.nextafter(pf, np.float32(0))
        idx = np.arange(P.numel()).reshape(P.shape) % 3
        r = np.where(idx == 0, pf, np.where(idx == 1, up, dn)).astype(np.float32)
        rand = torch.from_numpy(r)
        out = oracle.dropout(P, rand, w, wu, 0, p=p, out_dtype=torch.float64)
        tie = torch.from_numpy(idx == 0)
        above = torch.from_numpy(idx == 1)
        assert torch.all(out[tie] == 0)                    # rand == p drops
        assert torch.all(out[~above] == 0)                 # rand < p drops
        kept = above & inr
        assert int(kept.sum()) > 0
        np.testing.assert_allclose(out[kept].numpy(), (P[kept] / (1.0 - float(pf))).numpy(),
                                   rtol=1e-15)


# ---------------------------------------------------- softmax backward pins
# The gradient of the banded softmax with respect to its stored scores is not printed
# on the pages; it is the chain rule through their softmax recipe.  Three independent
# pins: torch autograd through a dense -inf-masked softmax (a library routine), central
# finite differences through the forward oracle itself, and closed forms.

def test_softmax_bwd_matches_torch_autograd_on_masked_dense_rows():
    n, w, wu, d = 23, 3, 5, 6
    for dil in (0, 2):
        s = max(dil, 1)
        g = datagen.rng(41 + dil)
        S = datagen.normal(g, (1, n, 1, w + wu + 1), "f32").double()
        dP = datagen.normal(g, (1, n, 1, w + wu + 1), "f32").double()
        P = oracle.softmax(S, w, wu, dil, scale=0.3, out_dtype=torch.float64)
        dS = oracle.softmax_bwd(P, dP, w, wu, dil, scale=0.3, out_dtype=torch.float64)
        mask = torch.from_numpy(_selected(n, w, wu, s))
        for i in range(n):
            cols = torch.nonzero(mask[i]).flatten()            # keys of the in-range slots
            ks = (cols - i) // s + w                           # their slots
            x = torch.full((n,), float("-inf"), dtype=torch.float64)
            sv = S[0, i, 0, ks].clone().requires_grad_(True)
            x = x.index_put((cols,), 0.3 * sv)
            pr = torch.softmax(x, -1)
            (gs,) = torch.autograd.grad((pr[cols] * dP[0, i, 0, ks]).sum(), sv)
            np.testing.assert_allclose(dS[0, i, 0, ks].numpy(), gs.numpy(), rtol=1e-12,
                                       atol=1e-14)
            out = torch.ones(w + wu + 1, dtype=torch.bool)
            out[ks] = False
            assert torch.all(dS[0, i, 0, out] == 0)


def test_softmax_bwd_matches_central_differences_of_the_forward_oracle():
    n, w, wu, dil, h = 17, 4, 2, 3, 2
    K = w + wu + 1
    g = datagen.rng(47)
    S = datagen.normal(g, (1, n, h, K), "f32").double()
    dP = datagen.normal(g, (1, n, h, K), "f32").double()
    P = oracle.softmax(S, w, wu, dil, scale=0.5, out_dtype=torch.float64)
    dS = oracle.softmax_bwd(P, dP, w, wu, dil, scale=0.5, out_dtype=torch.float64)
    eps = 1e-6
    ones = torch.ones(1, n, 1, 1)
    inr = (oracle.qk(ones, ones, w, wu, dil, padding=0.0) == 1)[0, :, 0]
    for i in range(0, n, 3):
        for hh in range(h):
            for k in range(K):
                Sp, Sm = S.clone(), S.clone()
                Sp[0, i, hh, k] += eps
                Sm[0, i, hh, k] -= eps
                Lp = (oracle.softmax(Sp, w, wu, dil, scale=0.5, out_dtype=torch.float64) * dP).sum()
                Lm = (oracle.softmax(Sm, w, wu, dil, scale=0.5, out_dtype=torch.float64) * dP).sum()
                fd = ((Lp - Lm) / (2 * eps)).item()
                assert abs(dS[0, i, hh, k].item() - fd) <= 1e-7, (i, hh, k)
                if not inr[i, k]:
                    assert dS[0, i, hh, k].item() == 0.0 and fd == 0.0


def test_softmax_bwd_closed_forms():
    n, w, wu = 40, 6, 6
    K = w + wu + 1
    g = datagen.rng(53)
    S = datagen.normal(g, (2, n, 3, K), "f32").double()
    P = oracle.softmax(S, w, wu, 0, scale=0.25, out_dtype=torch.float64)
    ones = torch.ones(1, n, 1, 1)
    inr = (oracle.qk(ones, ones, w, wu, padding=0.0) == 1).expand_as(P)
    # a gradient constant over the row's in-range slots (out-of-range slots hold
    # anything, NaN included) leaves the scores' gradient exactly zero in double
    dP = torch.where(inr, torch.full_like(P, 0.75), torch.full_like(P, float("nan")))
    dS = oracle.softmax_bwd(P, dP, w, wu, 0, scale=0.25, out_dtype=torch.float64)
    assert torch.all(dS.abs() <= 1e-16)
    # each row of the gradient sums to zero (the softmax is shift invariant)
    dP = datagen.normal(g, (2, n, 3, K), "f32").double()
    dS = oracle.softmax_bwd(P, dP, w, wu, 0, scale=0.25, out_dtype=torch.float64)
    assert torch.all(dS.sum(-1).abs() <= 1e-15)
    # a one-hot probability row has a zero gradient, and a two-point row is
    # scale * p (1 - p) (dP_a - dP_b) on its first point
    P1 = torch.zeros_like(P)
    P1[..., w] = 1.0
    assert torch.all(oracle.softmax_bwd(P1, dP, w, wu, 0, scale=0.25,
                                        out_dtype=torch.float64) == 0)
    P2 = torch.zeros_like(P)
    P2[..., w] = 0.375
    P2[..., w + 1] = 0.625
    dS2 = oracle.softmax_bwd(P2, dP, w, wu, 0, scale=0.25, out_dtype=torch.float64)
    want = 0.25 * 0.375 * 0.625 * (dP[..., w] - dP[..., w + 1])
    inner = inr[..., w + 1]                                   # rows where slot w+1 exists
    assert torch.allclose(dS2[..., w][inner], want[inner], rtol=1e-15, atol=0)
    # one rounding: a 16-bit output is the double value rounded once
    Ph = oracle.convert(P, torch.float16)
    dPh = oracle.convert(dP, torch.float16)
    d64 = oracle.softmax_bwd(Ph, dPh, w, wu, 0, scale=0.25, out_dtype=torch.float64)
    d16 = oracle.softmax_bwd(Ph, dPh, w, wu, 0, scale=0.25)
    assert torch.equal(d16, oracle.convert(d64, torch.float16))


# ------------------------------------------------------------ row sampling

def test_row_list_equals_full_computation():
    n, w, wu, dil, d = 70, 5, 5, 3, 4
    g = datagen.rng(31)
    Q = datagen.normal(g, (2, n, 2, d), "f16")
    Kt = datagen.normal(g, (2, n, 2, d), "f16")
    P = datagen.normal(g, (2, n, 2, w + wu + 1), "f16")
    rows = np.array([0, 1, 69, 70, 71, 100, 139])
    bi = torch.from_numpy(rows)
    full_qk = oracle.qk(Q, Kt, w, wu, dil, 2.0).reshape(2 * n, 2, -1)
    got = oracle.qk(Q.reshape(2 * n, 2, d)[bi], Kt, w, wu, dil, 2.0, rows=rows)
    assert torch.equal(got, full_qk[bi])
    full_pv = oracle.pv(P, Kt, w, wu, dil).reshape(2 * n, 2, d)
    assert torch.equal(oracle.pv(P.reshape(2 * n, 2, -1)[bi], Kt, w, wu, dil, rows=rows),
                       full_pv[bi])
    full_pvT = oracle.pvT(P, Kt, w, wu, dil).reshape(2 * n, 2, d)
    assert torch.equal(oracle.pvT(P, Kt, w, wu, dil, rows=rows), full_pvT[bi])
    full_sm = oracle.softmax(P, w, wu, dil, 0.5).reshape(2 * n, 2, -1)
    assert torch.equal(oracle.softmax(P.reshape(2 * n, 2, -1)[bi], w, wu, dil, 0.5, n=n,
                                      rows=rows), full_sm[bi])
    R = datagen.uniform(g, P.shape)
    full_dr = oracle.dropout(P, R, w, wu, dil, p=0.3).reshape(2 * n, 2, -1)
    assert torch.equal(oracle.dropout(P.reshape(2 * n, 2, -1)[bi], R.reshape(2 * n, 2, -1)[bi],
                                      w, wu, dil, p=0.3, n=n, rows=rows), full_dr[bi])


def test_sample_rows_cover_edges():
    rows = datagen.sample_rows(32768, 4096)
    assert len(rows) == 64 == len(set(rows.tolist()))
    assert {0, 4095, 32768 - 4096, 32767} <= set(rows.tolist())


# ------------------------------------------------------------ fused attention pins
# attention = the window's scores, their softmax and the weighted sum of V rows in one
# pass.  Pins: torch's float64 softmax attention over dense rows with the unselected
# diagonals at -inf (a library routine), closed forms (constant V rows, a one-slot
# window, zero queries give window means), and agreement with the three-step oracle.

def _dense_attention(q, k, v, w, wu, dil, scale):
    n = q.shape[1]
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    off = j - i
    s = max(dil, 1)
    sel = (off % s == 0) & (off >= -w * s) & (off <= wu * s)
    sc = torch.einsum("bihd,bjhd->bhij", q.double(), k.double()) * scale
    p = torch.softmax(sc.masked_fill(~sel, float("-inf")), -1)
    return torch.einsum("bhij,bjhd->bihd", p, v.double())


@pytest.mark.parametrize("shape", [(1, 40, 2, 8, 5, 5, 0), (2, 33, 1, 16, 4, 0, 0),
                                   (1, 50, 2, 8, 6, 3, 3), (1, 9, 1, 4, 20, 20, 0),
                                   (1, 61, 1, 8, 7, 2, 9), (1, 1, 1, 4, 3, 3, 0)])
def test_attention_matches_dense_softmax_attention(shape):
    b, n, h, d, w, wu, dil = shape
    g = datagen.rng(900 + n)
    q, k, v = (datagen.normal(g, (b, n, h, d), "f32") for _ in range(3))
    got = oracle.attention(q, k, v, w, wu, dil, scale=0.7, out_dtype=torch.float64)
    ref = _dense_attention(q, k, v, w, wu, dil, 0.7)
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)
    three = oracle.pv(oracle.softmax(oracle.qk(q.double(), k.double(), w, wu, dil, 0.0),
                                     w, wu, dil, 0.7), v.double(), w, wu, dil)
    assert torch.allclose(got, three, rtol=0, atol=1e-12)


def test_attention_closed_forms():
    b, n, h, d, w, wu, dil = 1, 30, 2, 8, 4, 6, 2
    g = datagen.rng(950)
    q, k = (datagen.normal(g, (b, n, h, d), "f32") for _ in range(2))
    v = datagen.normal(g, (b, n, h, d), "f32")
    # constant value rows: every output row is that row
    c = datagen.normal(g, (1, 1, h, d), "f32").expand(b, n, h, d).contiguous()
    got = oracle.attention(q, k, c, w, wu, dil, 0.5, out_dtype=torch.float64)
    assert torch.allclose(got, c.double().expand_as(got), rtol=0, atol=1e-14)
    # a one-slot window attends the diagonal only: the output is V exactly
    assert torch.equal(oracle.attention(q, k, v, 0, 0, dil, 0.5, out_dtype=torch.float64),
                       v.double())
    # zero queries: uniform weights, the mean of the in-range V rows
    z = torch.zeros_like(q)
    got = oracle.attention(z, k, v, w, wu, dil, 0.5, out_dtype=torch.float64)
    s = max(dil, 1)
    for i in range(n):
        js = [i + o * s for o in range(-w, wu + 1) if 0 <= i + o * s < n]
        assert torch.allclose(got[0, i], v[0, js].double().mean(0), rtol=0, atol=1e-14)


def test_attention_row_list_equals_full():
    b, n, h, d, w, wu, dil = 2, 40, 2, 8, 5, 3, 3
    g = datagen.rng(960)
    q, k, v = (datagen.normal(g, (b, n, h, d), "f16") for _ in range(3))
    rows = np.array([0, 1, 39, 40, 41, 79])
    full = oracle.attention(q, k, v, w, wu, dil, 0.3).reshape(b * n, h, d)
    assert torch.equal(oracle.attention(q, k, v, w, wu, dil, 0.3, rows=rows),
                       full[torch.from_numpy(rows)])


# ------------------------------------------------------------ global-token pins
# A row outside the global set attends its window and the global keys, each once; a
# global row attends every key.  Pins: torch's float64 softmax attention with that key
# set as a dense mask, no global tokens = the windowed attention, a global row = full
# dense attention, and all rows global = full dense attention everywhere.

def _dense_global(q, k, v, glob, w, wu, dil, scale, gqkv=None):
    """Dense float64 reference: the key set as a mask over all n x n pairs; the global
    rows from (GQ, GK, GV) over every key.  ``glob`` is taken as given (a clean set)."""
    b, n = q.shape[:2]
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    off = j - i
    s = max(dil, 1)
    win = (off % s == 0) & (off >= -w * s) & (off <= wu * s)
    gq, gk, gv = gqkv if gqkv is not None else (q, k, v)
    outs = []
    for bb in range(b):
        isg = torch.zeros(n, dtype=torch.bool)
        isg[glob[bb]] = True
        sel = win | isg[None, :]
        sc = torch.einsum("ihd,jhd->hij", q[bb].double(), k[bb].double()) * scale
        p = torch.softmax(sc.masked_fill(~sel, float("-inf")), -1)
        o = torch.einsum("hij,jhd->ihd", p, v[bb].double())
        gsc = torch.einsum("ihd,jhd->hij", gq[bb].double(), gk[bb].double()) * scale
        go = torch.einsum("hij,jhd->ihd", torch.softmax(gsc, -1), gv[bb].double())
        o[isg] = go[isg]
        outs.append(o)
    return torch.stack(outs)


@pytest.mark.parametrize("shape", [(2, 40, 2, 8, 3, 3, 0), (1, 50, 1, 8, 4, 0, 3),
                                   (1, 33, 2, 4, 40, 40, 0), (2, 30, 1, 8, 2, 5, 2)])
def test_attention_global_matches_dense_masked_attention(shape):
    b, n, h, d, w, wu, dil = shape
    g = datagen.rng(980 + n)
    q, k, v = (datagen.normal(g, (b, n, h, d), "f32") for _ in range(3))
    glob = torch.stack([torch.from_numpy(datagen.rng(990 + bb).choice(n, 4, replace=False))
                        for bb in range(b)])
    got = oracle.attention_global(q, k, v, glob, w, wu, dil, 0.6, out_dtype=torch.float64)
    assert torch.allclose(got, _dense_global(q, k, v, glob, w, wu, dil, 0.6), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(2, 40, 2, 8, 3, 3, 0), (1, 50, 1, 8, 4, 0, 3)])
def test_attention_global_separate_matrices(shape):
    """The global rows take Global_Q, Global_K and Global_V (onnxruntime issue 12448,
    conclusion (d)) over every key; the other rows keep Q, K and V, the global keys
    included.  A dropped global matrix, or one used on the wrong rows, fails."""
    b, n, h, d, w, wu, dil = shape
    g = datagen.rng(1960 + n)
    q, k, v, gq, gk, gv = (datagen.normal(g, (b, n, h, d), "f32") for _ in range(6))
    glob = torch.stack([torch.from_numpy(datagen.rng(1970 + bb).choice(n, 5, replace=False))
                        for bb in range(b)])
    got = oracle.attention_global(q, k, v, glob, w, wu, dil, 0.6, out_dtype=torch.float64,
                                  global_qkv=(gq, gk, gv))
    ref = _dense_global(q, k, v, glob, w, wu, dil, 0.6, gqkv=(gq, gk, gv))
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)
    # the same matrices given twice are the one-QKV form, bit for bit
    assert torch.equal(oracle.attention_global(q, k, v, glob, w, wu, dil, 0.6,
                                               out_dtype=torch.float64, global_qkv=(q, k, v)),
                       oracle.attention_global(q, k, v, glob, w, wu, dil, 0.6,
                                               out_dtype=torch.float64))


def test_attention_global_position_list_is_a_set():
    """Repeated positions count once and entries outside [0, n) name no position: the
    result equals the dense reference on the cleaned set."""
    b, n, h, d, w, wu, dil = 2, 30, 2, 8, 2, 3, 0
    g = datagen.rng(1980)
    q, k, v = (datagen.normal(g, (b, n, h, d), "f32") for _ in range(3))
    messy = torch.tensor([[4, 4, 17, -1, 30, 4, 29, 1000],
                          [0, -5, 0, 0, 12, 12, 31, 2]])
    clean = [torch.tensor([4, 17, 29]), torch.tensor([0, 12, 2])]
    got = oracle.attention_global(q, k, v, messy, w, wu, dil, 0.6, out_dtype=torch.float64)
    ref = torch.cat([_dense_global(q[bb:bb + 1], k[bb:bb + 1], v[bb:bb + 1], [clean[bb]],
                                   w, wu, dil, 0.6) for bb in range(b)])
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)
    # every entry out of range: the plain windowed attention
    junk = torch.tensor([[-3, n, n + 7], [-1, -1, 2 * n]])
    assert torch.allclose(oracle.attention_global(q, k, v, junk, w, wu, dil, 0.6,
                                                  out_dtype=torch.float64),
                          oracle.attention(q, k, v, w, wu, dil, 0.6, out_dtype=torch.float64),
                          rtol=0, atol=1e-14)


def test_attention_global_special_cases():
    b, n, h, d, w, wu, dil = 1, 36, 2, 8, 3, 2, 2
    g = datagen.rng(995)
    q, k, v = (datagen.normal(g, (b, n, h, d), "f32") for _ in range(3))
    none = torch.zeros(b, 0, dtype=torch.int64)
    assert torch.allclose(oracle.attention_global(q, k, v, none, w, wu, dil, 0.5,
                                                  out_dtype=torch.float64),
                          oracle.attention(q, k, v, w, wu, dil, 0.5, out_dtype=torch.float64),
                          rtol=0, atol=1e-14)
    dense = oracle.attention(q, k, v, n, n, 0, 0.5, out_dtype=torch.float64)   # every key
    glob = torch.tensor([[5, 17]])
    got = oracle.attention_global(q, k, v, glob, w, wu, dil, 0.5, out_dtype=torch.float64)
    assert torch.allclose(got[0, [5, 17]], dense[0, [5, 17]], rtol=0, atol=1e-14)
    every = torch.arange(n)[None, :]
    assert torch.allclose(oracle.attention_global(q, k, v, every, w, wu, dil, 0.5,
                                                  out_dtype=torch.float64), dense,
                          rtol=0, atol=1e-14)
