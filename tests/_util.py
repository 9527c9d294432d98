"""Comparison helpers shared by the GPU parity tests.

Tolerances (the oracle is compared before its final narrowing, i.e. in float64):
* f32 inputs: normwise relative error max|gpu - oracle| / max|oracle| <= 1e-5 per tensor
  (elementwise relative error is ill-posed where cancellation makes a value near zero);
* f16 / bf16 inputs with f32 accumulation: elementwise |gpu - oracle| <= 2e-3 for inputs
  scaled like N(0,1)/sqrt(d) (or probability bands), so the outputs are O(1).  Where a
  16-bit output's own spacing is coarser than that (bf16 above 0.5, f16 above 2), the
  bound is one unit in the last place of the output type instead;
* values with exactly one correct bit pattern (padding slots, masked softmax slots,
  integer-valued results) are compared bit for bit.
"""
import torch

import oracle

F32_NORMWISE = 1e-5
LOWP_ABS = 2e-3


def widen(t: torch.Tensor) -> torch.Tensor:
    return t.detach().cpu().double()


def out_ulp(x: torch.Tensor, dtype) -> torch.Tensor:
    """Spacing of ``dtype`` values at |x| (normal range; float64 tensor)."""
    mant = {torch.float16: 10, torch.bfloat16: 7, torch.float32: 23}[dtype]
    tiny = {torch.float16: 2.0 ** -14, torch.bfloat16: 2.0 ** -126,
            torch.float32: 2.0 ** -126}[dtype]
    e = torch.floor(torch.log2(x.abs().clamp_min(tiny)))
    return torch.pow(2.0, e - mant)


def check_close(gpu: torch.Tensor, ref64: torch.Tensor, in_dtype, what: str, mask=None,
                abs_tol=None):
    g = widen(gpu)
    r = ref64.double()
    if mask is not None:
        g, r = g[mask], r[mask]
    assert torch.isfinite(g).all(), f"{what}: non-finite GPU values"
    if not g.numel():
        return 0.0
    diff = (g - r).abs()
    if in_dtype == torch.float32 and abs_tol is None:
        scale = r.abs().max().item()
        rel = diff.max().item() / scale if scale > 0 else diff.max().item()
        assert rel <= F32_NORMWISE, f"{what}: normwise rel err {rel:.3e} > {F32_NORMWISE}"
        return rel
    tol = torch.full_like(r, LOWP_ABS if abs_tol is None else abs_tol)
    if gpu.dtype in (torch.float16, torch.bfloat16) and abs_tol is None:
        tol = torch.maximum(tol, out_ulp(r, gpu.dtype))
    bad = diff > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, worst "
                           f"{diff.max().item():.3e} (ref {r.flatten()[diff.argmax()].item():.4g})")
    return diff.max().item()


def in_range_mask(b, n, h, w, wu, dil):
    """Boolean [b, n, h, K] mask of the in-range slots, taken from the oracle itself
    (qk of all-ones operands is 1 exactly on in-range slots and the padding elsewhere)."""
    ones = torch.ones(1, n, 1, 1, dtype=torch.float32)
    m = oracle.qk(ones, ones, w, wu, dil, padding=0.0) == 1
    return m.expand(b, n, h, w + wu + 1)


def in_range_rows(n, h, w, wu, dil, rows):
    """Boolean [len(rows), h, K] in-range mask for the listed flattened positions."""
    ones = torch.ones(len(rows), 1, 1, dtype=torch.float32)
    m = oracle.qk(ones, torch.ones(1, n, 1, 1), w, wu, dil, padding=0.0, rows=[r % n for r in rows]) == 1
    return m.expand(len(rows), h, w + wu + 1)


def assert_bits_equal(a: torch.Tensor, b: torch.Tensor, what: str):
    a = a.detach().cpu().contiguous()
    b = b.detach().cpu().contiguous()
    assert a.dtype == b.dtype and a.shape == b.shape, \
        f"{what}: {a.dtype}{tuple(a.shape)} vs {b.dtype}{tuple(b.shape)}"
    iv = {2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()]
    diff = a.view(iv) != b.view(iv)
    assert not diff.any(), f"{what}: {int(diff.sum())} elements differ bitwise"
