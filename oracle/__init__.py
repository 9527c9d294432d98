"""CPU oracle for the diagonaled matmul family (qk, pv, pvT) and the banded softmax.

TEST INFRASTRUCTURE ONLY: the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may use this module; the product path (the HIP
library and its Python binding) never imports it, and it imports nothing from
there.  The arithmetic lives in ``oracle.c`` (plain loops, double accumulation,
one round-to-nearest-even at the end); this file only builds that library with
gcc and marshals torch CPU tensors into it.

Definitions (TVM Discuss, "Developing a faster schedule for Longformer's kernel",
posts 1, 3, 5 and 6): with stride ``s = max(dilation, 1)`` and ``K = w + w_upper + 1``,

* ``qk``:  band[b,i,h,k] = <Q[b,i,h,:], K[b,i+(k-w)s,h,:]>, padding where the key
  index is outside [0, n)  (the forward function, result last dim 2w+1);
* ``pv``:  out[b,i,h,:] = sum_k band[b,i,h,k] * V[b,i+(k-w)s,h,:] over in-range keys
  (backward function with transpose_t1 = 0);
* ``pvT``: out[b,j,h,:] = sum over (i,k) with i+(k-w)s = j of band[b,i,h,k] * X[b,i,h,:]
  (backward function with transpose_t1 = 1);
* ``softmax``: per band row, scale, mask out-of-range slots to -inf, max, exp, sum,
  divide (attention softmax of the first fusion repro on csarofeen/pytorch issue 2096);
* ``softmax_masked``: the same softmax with the page's additive attention mask, a per-key
  mask m adding (1 - m) * mask_value (-10000 there) before the max;
* ``dropout``: the page's dropout on the band, rand > p keeps probs / (1 - p), with the
  uniform random numbers passed in;
* ``softmax_bwd``: the derivative of that softmax with respect to the stored scores,
  scale * P * (dP - sum(P * dP)) per row over in-range slots, 0 elsewhere (not printed
  on the pages; the chain rule through the recipe above).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# dtype codes of oracle.c
F32, F16, BF16, F64 = 0, 1, 2, 3
_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.float64: F64}
_TORCH = {v: k for k, v in _CODE.items()}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            i64, vp, ci, cd = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
            lib.oracle_qk.argtypes = [vp, vp, vp] + [i64] * 7 + [cd, ci, ci, vp, i64, ci]
            lib.oracle_pv.argtypes = [vp, vp, vp] + [i64] * 7 + [ci, ci, vp, i64, ci]
            lib.oracle_pvT.argtypes = [vp, vp, vp] + [i64] * 7 + [ci, ci, vp, i64, ci]
            lib.oracle_softmax.argtypes = [vp, vp] + [i64] * 6 + [cd, ci, ci, vp, i64, ci]
            lib.oracle_softmax_bwd.argtypes = [vp, vp, vp] + [i64] * 6 + [cd, ci, ci, vp, i64, ci]
            lib.oracle_dropout.argtypes = [vp, vp, vp] + [i64] * 6 + [ctypes.c_float, ci, ci, vp, i64,
                                           ci]
            lib.oracle_attention.argtypes = [vp, vp, vp, vp] + [i64] * 7 + [cd, ci, ci, vp, i64,
                                                                              ci]
            lib.oracle_attention_global.argtypes = [vp] * 7 + [i64, vp] + [i64] * 7 + [
                cd, ci, ci, vp, i64, ci]
            lib.oracle_softmax_masked.argtypes = [vp, vp, vp] + [i64] * 6 + [cd, cd, ci, ci, vp,
                                                                                 i64, ci]
            for f in (lib.oracle_qk, lib.oracle_pv, lib.oracle_pvT, lib.oracle_softmax):
                f.restype = ci
            lib.oracle_convert.argtypes = [vp, vp, i64, ci]
            lib.oracle_convert.restype = None
            lib.oracle_widen.argtypes = [vp, vp, i64, ci]
            lib.oracle_widen.restype = None
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _check(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError(f"oracle: {name} must be a CPU tensor")
    if t.dtype not in _CODE:
        raise ValueError(f"oracle: {name} has unsupported dtype {t.dtype}")
    return t.contiguous()


def _rows(rows):
    if rows is None:
        return None, None, 0
    r = torch.as_tensor(rows, dtype=torch.int64).contiguous()
    return r, ctypes.c_void_p(r.data_ptr()), r.numel()


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def qk(q, k, w, w_upper, dilation=0, padding=0.0, out_dtype=None, rows=None, threads=None):
    """Band of Q.K^T: [b, n, h, w+w_upper+1] (or [len(rows), h, K] for a row list of
    flattened b*n+i positions; then ``q`` holds only those rows, packed)."""
    lib = _load()
    k = _check(k, "k")
    q = _check(q, "q")
    b, n, h, d = k.shape
    out_dtype = out_dtype or q.dtype
    rt, rp, nr = _rows(rows)
    K = w + w_upper + 1
    shape = (b, n, h, K) if rt is None else (nr, h, K)
    if q.dtype != k.dtype or q.shape[-2:] != (h, d):
        raise ValueError("oracle.qk: q/k mismatch")
    out = torch.empty(shape, dtype=out_dtype)
    st = lib.oracle_qk(_ptr(q), _ptr(k), _ptr(out), b, n, h, d, w, w_upper, dilation,
                       float(padding), _CODE[q.dtype], _CODE[out_dtype], rp, nr,
                       threads or default_threads())
    if st:
        raise ValueError(f"oracle.qk: bad arguments ({st})")
    return out


def _pv_like(fn, band, x, w, w_upper, dilation, out_dtype, rows, threads):
    lib = _load()
    band = _check(band, "band")
    x = _check(x, "x")
    b, n, h, d = x.shape
    out_dtype = out_dtype or x.dtype
    rt, rp, nr = _rows(rows)
    shape = (b, n, h, d) if rt is None else (nr, h, d)
    if band.dtype != x.dtype or band.shape[-1] != w + w_upper + 1:
        raise ValueError("oracle: band/x mismatch")
    out = torch.empty(shape, dtype=out_dtype)
    st = fn(_ptr(band), _ptr(x), _ptr(out), b, n, h, d, w, w_upper, dilation,
            _CODE[x.dtype], _CODE[out_dtype], rp, nr, threads or default_threads())
    if st:
        raise ValueError(f"oracle: bad arguments ({st})")
    return out


def pv(band, v, w, w_upper, dilation=0, out_dtype=None, rows=None, threads=None):
    """Banded probabilities times V: [b, n, h, d].  With a row list the band holds
    only those rows, packed; V is always the full tensor."""
    return _pv_like(_load().oracle_pv, band, v, w, w_upper, dilation, out_dtype, rows, threads)


def pvT(band, x, w, w_upper, dilation=0, out_dtype=None, rows=None, threads=None):
    """Transposed band times X: [b, n, h, d].  The band and X are always full; a row
    list selects output rows j."""
    return _pv_like(_load().oracle_pvT, band, x, w, w_upper, dilation, out_dtype, rows, threads)


def attention(q, k, v, w, w_upper, dilation=0, scale=1.0, out_dtype=None, rows=None,
              threads=None):
    """Sliding-window attention, one row at a time in double: scores on the window's
    in-range diagonals, their softmax, and the probability-weighted sum of V rows.
    q, k, v are full [b, n, h, d] tensors of one dtype; the result is [b, n, h, d], or
    [len(rows), h, d] for a list of flattened positions b * n + i."""
    lib = _load()
    q, k, v = _check(q, "q"), _check(k, "k"), _check(v, "v")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("oracle.attention: q, k, v differ in shape or dtype")
    b, n, h, d = q.shape
    out_dtype = out_dtype or q.dtype
    rt, rp, nr = _rows(rows)
    shape = (b, n, h, d) if rt is None else (nr, h, d)
    out = torch.empty(shape, dtype=out_dtype)
    st = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), b, n, h, d, w, w_upper,
                              dilation, float(scale), _CODE[q.dtype], _CODE[out_dtype], rp, nr,
                              threads or default_threads())
    if st:
        raise ValueError(f"oracle.attention: bad arguments ({st})")
    return out


def attention_global(q, k, v, glob, w, w_upper, dilation=0, scale=1.0, out_dtype=None,
                     rows=None, threads=None, global_qkv=None):
    """Sliding-window attention with global tokens: ``glob`` is an integer [b, ng] tensor
    of global positions per batch; its entries in [0, n) form the global set (a repeated
    position counts once, others name no position).  A row outside the set attends its
    window and the global keys (each key once) with q, k, v; a global row attends every
    key with ``global_qkv`` = (GQ, GK, GV) (default: q, k, v)."""
    lib = _load()
    q, k, v = _check(q, "q"), _check(k, "k"), _check(v, "v")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("oracle.attention_global: q, k, v differ in shape or dtype")
    gp = [None, None, None]
    if global_qkv is not None:
        gq, gk, gv = (_check(t, "global_qkv") for t in global_qkv)
        if not (gq.shape == gk.shape == gv.shape == q.shape
                and gq.dtype == gk.dtype == gv.dtype == q.dtype):
            raise ValueError("oracle.attention_global: global q, k, v differ from q")
        gp = [_ptr(gq), _ptr(gk), _ptr(gv)]
    b, n, h, d = q.shape
    g = torch.as_tensor(glob, dtype=torch.int64).reshape(b, -1).contiguous()
    out_dtype = out_dtype or q.dtype
    rt, rp, nr = _rows(rows)
    shape = (b, n, h, d) if rt is None else (nr, h, d)
    out = torch.empty(shape, dtype=out_dtype)
    st = lib.oracle_attention_global(_ptr(q), _ptr(k), _ptr(v), gp[0], gp[1], gp[2], _ptr(g),
                                     g.shape[1], _ptr(out), b, n, h, d, w, w_upper, dilation,
                                     float(scale), _CODE[q.dtype], _CODE[out_dtype], rp, nr,
                                     threads or default_threads())
    if st:
        raise ValueError(f"oracle.attention_global: bad arguments ({st})")
    return out


def softmax(scores, w, w_upper, dilation=0, scale=1.0, out_dtype=None, n=None, rows=None,
            threads=None):
    """Banded softmax of a band tensor [b, n, h, K] (or packed [len(rows), h, K] with the
    sequence length ``n`` given)."""
    lib = _load()
    s = _check(scores, "scores")
    out_dtype = out_dtype or s.dtype
    rt, rp, nr = _rows(rows)
    if rt is None:
        b, n, h, K = s.shape
    else:
        if n is None:
            raise ValueError("oracle.softmax: n is required with a row list")
        b = 1
        _, h, K = s.shape
    if K != w + w_upper + 1:
        raise ValueError("oracle.softmax: band width mismatch")
    out = torch.empty(s.shape, dtype=out_dtype)
    st = lib.oracle_softmax(_ptr(s), _ptr(out), b, n, h, w, w_upper, dilation, float(scale),
                            _CODE[s.dtype], _CODE[out_dtype], rp, nr,
                            threads or default_threads())
    if st:
        raise ValueError(f"oracle.softmax: bad arguments ({st})")
    return out


def softmax_masked(scores, key_mask, w, w_upper, dilation=0, scale=1.0, mask_value=-10000.0,
                   out_dtype=None, n=None, rows=None, threads=None):
    """Banded softmax with a per-key attention mask ``key_mask`` (float32 [b, n]): the
    scaled score of a slot whose key is j gains (1 - key_mask[b, j]) * mask_value."""
    lib = _load()
    s = _check(scores, "scores")
    km = key_mask.to(torch.float32).contiguous()
    out_dtype = out_dtype or s.dtype
    rt, rp, nr = _rows(rows)
    if rt is None:
        b, n, h, K = s.shape
    else:
        if n is None:
            raise ValueError("oracle.softmax_masked: n is required with a row list")
        _, h, K = s.shape
        b = km.shape[0]
    if K != w + w_upper + 1:
        raise ValueError("oracle.softmax_masked: band width mismatch")
    if tuple(km.shape) != (b, n):
        raise ValueError("oracle.softmax_masked: key_mask must be [b, n]")
    out = torch.empty(s.shape, dtype=out_dtype)
    st = lib.oracle_softmax_masked(_ptr(s), _ptr(out), _ptr(km), b, n, h, w, w_upper, dilation,
                                   float(scale), float(mask_value), _CODE[s.dtype],
                                   _CODE[out_dtype], rp, nr, threads or default_threads())
    if st:
        raise ValueError(f"oracle.softmax_masked: bad arguments ({st})")
    return out


def dropout(probs, rand, w, w_upper, dilation=0, p=0.1, out_dtype=None, n=None, rows=None,
            threads=None):
    """Dropout on a band [b, n, h, K] (or packed [len(rows), h, K] with ``n`` given):
    in-range slots with rand > p keep probs / (1 - p), the others 0 (rand: float32
    uniforms of the band's shape)."""
    lib = _load()
    pr = _check(probs, "probs")
    rd = rand.to(torch.float32).contiguous()
    if rd.shape != pr.shape:
        raise ValueError("oracle.dropout: rand must have the band's shape")
    out_dtype = out_dtype or pr.dtype
    rt, rp, nr = _rows(rows)
    if rt is None:
        b, n, h, K = pr.shape
    else:
        if n is None:
            raise ValueError("oracle.dropout: n is required with a row list")
        b = 1
        _, h, K = pr.shape
    if K != w + w_upper + 1:
        raise ValueError("oracle.dropout: band width mismatch")
    out = torch.empty(pr.shape, dtype=out_dtype)
    st = lib.oracle_dropout(_ptr(pr), _ptr(rd), _ptr(out), b, n, h, w, w_upper, dilation,
                            float(p), _CODE[pr.dtype], _CODE[out_dtype], rp, nr,
                            threads or default_threads())
    if st:
        raise ValueError(f"oracle.dropout: bad arguments ({st})")
    return out


def softmax_bwd(probs, dprobs, w, w_upper, dilation=0, scale=1.0, out_dtype=None, n=None,
                rows=None, threads=None):
    """Gradient of the banded softmax with respect to its stored scores, given its
    probabilities ``probs`` and the gradient ``dprobs`` with respect to them (both band
    tensors [b, n, h, K] of one dtype, or packed [len(rows), h, K] with ``n`` given)."""
    lib = _load()
    p = _check(probs, "probs")
    dp = _check(dprobs, "dprobs")
    if dp.dtype != p.dtype or dp.shape != p.shape:
        raise ValueError("oracle.softmax_bwd: probs and dprobs differ in dtype or shape")
    out_dtype = out_dtype or p.dtype
    rt, rp, nr = _rows(rows)
    if rt is None:
        b, n, h, K = p.shape
    else:
        if n is None:
            raise ValueError("oracle.softmax_bwd: n is required with a row list")
        b = 1
        _, h, K = p.shape
    if K != w + w_upper + 1:
        raise ValueError("oracle.softmax_bwd: band width mismatch")
    out = torch.empty(p.shape, dtype=out_dtype)
    st = lib.oracle_softmax_bwd(_ptr(p), _ptr(dp), _ptr(out), b, n, h, w, w_upper, dilation,
                                float(scale), _CODE[p.dtype], _CODE[out_dtype], rp, nr,
                                threads or default_threads())
    if st:
        raise ValueError(f"oracle.softmax_bwd: bad arguments ({st})")
    return out


def convert(x: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """Round float64 values to ``dtype`` with the oracle's own round-to-nearest-even."""
    lib = _load()
    x = x.to(torch.float64).contiguous()
    out = torch.empty(x.shape, dtype=dtype)
    lib.oracle_convert(_ptr(x), _ptr(out), x.numel(), _CODE[dtype])
    return out


def widen(x: torch.Tensor) -> torch.Tensor:
    """Widen a float tensor to float64 with the oracle's own decoders."""
    lib = _load()
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.float64)
    lib.oracle_widen(_ptr(x), _ptr(out), x.numel(), _CODE[x.dtype])
    return out
