"""Banded attention through torch autograd (forward qk -> softmax -> pv, backward with
the softmax backward and the two transposed products) against a dense reference: the
same attention with the unselected diagonals masked to -inf, differentiated by torch
autograd in float64 on the CPU (a textbook routine).  f32 tensors are held to the f32
bar (normwise 1e-5 per tensor); f16 / bf16 runs are checked against the f32 run of the
same inputs at the spacing of their stored intermediates."""
import math

import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu


def _selected(n, w, wu, s):
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    off = j - i
    return (off % s == 0) & (off >= -w * s) & (off <= wu * s)


def _dense_grads(q, k, v, g, w, wu, dil, scale):
    q, k, v = (t_.double().requires_grad_(True) for t_ in (q, k, v))
    n = q.shape[1]
    mask = _selected(n, w, wu, max(dil, 1))
    s = torch.einsum("bihd,bjhd->bhij", q, k) * scale
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), -1)
    o = torch.einsum("bhij,bjhd->bihd", p, v)
    (o * g.double()).sum().backward()
    return o.detach(), q.grad, k.grad, v.grad


def _normwise(a, ref):
    return ((a.double().cpu() - ref).abs().max() / ref.abs().max()).item()


@pytest.mark.parametrize("shape", [(1, 200, 2, 32, 16, 16, 0), (2, 150, 2, 64, 24, 0, 0),
                                   (1, 170, 3, 32, 12, 9, 2), (1, 40, 1, 16, 60, 60, 0)])
def test_banded_attention_gradients_match_dense_autograd(shape):
    from sliding_window_attention_diagmm_amd.attention import banded_attention
    b, n, h, d, w, wu, dil = shape
    g_ = datagen.rng(700 + n)
    q, k, v = (datagen.normal(g_, (b, n, h, d), "f32") for _ in range(3))
    gout = datagen.normal(g_, (b, n, h, d), "f32")
    scale = 1.0 / math.sqrt(d)
    qc, kc, vc = (t_.cuda().requires_grad_(True) for t_ in (q, k, v))
    o = banded_attention(qc, kc, vc, w, wu, dil)
    o.backward(gout.cuda())
    ro, rq, rk, rv = _dense_grads(q, k, v, gout, w, wu, dil, scale)
    for name, got, ref in (("out", o, ro), ("dq", qc.grad, rq), ("dk", kc.grad, rk),
                           ("dv", vc.grad, rv)):
        err = _normwise(got.detach(), ref)
        assert err <= 1e-5, f"{name}: normwise error {err:.3e}"


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_banded_attention_low_precision_tracks_f32(dt):
    from sliding_window_attention_diagmm_amd.attention import banded_attention
    b, n, h, d, w, dil = 1, 1000, 4, 64, 128, 0
    g_ = datagen.rng(720)
    q, k, v, gout = (datagen.normal(g_, (b, n, h, d), "f32") for _ in range(4))
    grads = {}
    for t in (torch.float32, dt):
        qc, kc, vc = (x.to(t).cuda().requires_grad_(True) for x in (q, k, v))
        o = banded_attention(qc, kc, vc, w, w, dil)
        o.backward(gout.to(t).cuda())
        grads[t] = [x.detach().double().cpu() for x in (o, qc.grad, kc.grad, vc.grad)]
    # stored 16-bit probabilities and score gradients carry a relative error of one
    # half-ulp (2^-11 f16, 2^-8 bf16) into every product; sums of O(w) such terms
    tol = 3e-3 if dt == torch.float16 else 2.5e-2
    for name, lo, hi in zip(("out", "dq", "dk", "dv"), grads[dt], grads[torch.float32]):
        err = ((lo - hi).abs().max() / hi.abs().max()).item()
        assert err <= tol, f"{dt} {name}: normwise deviation from f32 {err:.3e}"


def _dense_keep(rand, n, w, wu, s, p):
    """Dense [b, h, n, n] dropout factors from a band of uniforms: (rand > p) / (1 - p)
    at key i + (kk - w) s of row i, 0 off the window."""
    b, _, h, K = rand.shape
    p = float(torch.tensor(p, dtype=torch.float32))   # the float32 p the kernels compare
    D = torch.zeros(b, h, n, n, dtype=torch.float64)
    i = torch.arange(n)
    for kk in range(K):
        j = i + (kk - w) * s
        ok = (j >= 0) & (j < n)
        keep = (rand[:, :, :, kk] > p).double() / (1 - p)
        D[:, :, i[ok], j[ok]] = keep.permute(0, 2, 1)[:, :, ok]
    return D


@pytest.mark.parametrize("shape", [(1, 200, 2, 32, 16, 16, 0), (1, 170, 3, 32, 12, 9, 2)])
def test_banded_attention_with_dropout_matches_dense_autograd(shape):
    """Dropout between the softmax and pv: the dense reference multiplies the masked
    softmax by the same keep factors (rand > p) / (1 - p) before the product with V."""
    from sliding_window_attention_diagmm_amd.attention import banded_attention
    b, n, h, d, w, wu, dil = shape
    p = 0.2
    g_ = datagen.rng(740 + n)
    q, k, v, gout = (datagen.normal(g_, (b, n, h, d), "f32") for _ in range(4))
    rand = datagen.uniform(g_, (b, n, h, w + wu + 1))
    scale = 1.0 / math.sqrt(d)
    qc, kc, vc = (t_.cuda().requires_grad_(True) for t_ in (q, k, v))
    o = banded_attention(qc, kc, vc, w, wu, dil, dropout_p=p, dropout_rand=rand.cuda())
    o.backward(gout.cuda())
    D = _dense_keep(rand, n, w, wu, max(dil, 1), p)
    qd, kd, vd = (t_.double().requires_grad_(True) for t_ in (q, k, v))
    mask = _selected(n, w, wu, max(dil, 1))
    sc = torch.einsum("bihd,bjhd->bhij", qd, kd) * scale
    pr = torch.softmax(sc.masked_fill(~mask, float("-inf")), -1) * D
    ro = torch.einsum("bhij,bjhd->bihd", pr, vd)
    (ro * gout.double()).sum().backward()
    for name, got, ref in (("out", o, ro.detach()), ("dq", qc.grad, qd.grad),
                           ("dk", kc.grad, kd.grad), ("dv", vc.grad, vd.grad)):
        err = _normwise(got.detach(), ref)
        assert err <= 1e-5, f"{name}: normwise error {err:.3e}"
    # p = 0 with any uniforms in (0, 1) is the attention without dropout
    o0 = banded_attention(qc.detach(), kc.detach(), vc.detach(), w, wu, dil)
    o1 = banded_attention(qc.detach(), kc.detach(), vc.detach(), w, wu, dil, dropout_p=0.0,
                          dropout_rand=rand.cuda())
    assert torch.equal(o0, o1)


def test_banded_attention_without_gradients_takes_the_one_pass_kernel():
    """Under no_grad, f16 inputs go to diagmm_banded_attention (bit for bit its output),
    which agrees with the three-call forward to the 16-bit bar."""
    import sliding_window_attention_diagmm_amd as dm
    from sliding_window_attention_diagmm_amd.attention import banded_attention
    b, n, h, d, w, dil = 1, 600, 2, 64, 40, 2
    g_ = datagen.rng(760)
    q, k, v = (datagen.normal(g_, (b, n, h, d), "f16", 0.5).cuda() for _ in range(3))
    with torch.no_grad():
        o = banded_attention(q, k, v, w, w, dil)
    assert torch.equal(o, dm.diagmm_banded_attention(q, k, v, w, w, dil))
    qg = q.clone().requires_grad_(True)
    o3 = banded_attention(qg, k, v, w, w, dil)
    assert (o.float() - o3.detach().float()).abs().max().item() <= 4e-3
