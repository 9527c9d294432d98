"""Python binding of libdiagmm (the Longformer diagonaled matmul family on MI355X).

Argument marshalling only: every call checks the torch tensors it is given (device,
dtype, contiguity, shape), allocates the output with torch when none is passed, and
hands raw device pointers, sizes and torch's current HIP stream to the C ABI in
``libdiagmm.so`` (declared in ``include/diagmm.h``).  All arithmetic runs in the HIP
kernels of that library; there is no CPU or PyTorch fallback - if the library is
missing or fails to load, importing the ops raises.

Operations (TVM Discuss, "Developing a faster schedule for Longformer's kernel": the
banded product of post 1, parameters of post 5, forward / two backward functions of
post 6), with ``K = w + w_upper + 1`` and stride ``s = max(dilation, 1)``:

* ``diagmm_qk(q, k, w, ...)``   -> band ``[b, n, h, K]``: Q.K^T on the selected diagonals
* ``diagmm_pv(band, v, w, ...)`` -> ``[b, n, h, d]``: band times V (transpose_t1 = 0)
* ``diagmm_pvT(band, x, w, ...)``-> ``[b, n, h, d]``: transposed band times X (transpose_t1 = 1)
* ``diagmm_banded_softmax(scores, w, ...)`` -> probabilities over each band row
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["diagmm_qk", "diagmm_pv", "diagmm_pvT", "diagmm_banded_softmax",
           "diagmm_banded_softmax_backward", "diagmm_banded_dropout", "diagmm_banded_attention",
           "diagmm_banded_attention_global", "diagmm_banded_attention_global_noalloc",
           "diagmm_plan",
           "diagmm_timing_begin", "diagmm_timing_end", "diagmm_timing_read",
           "diagmm_abi_version", "library_path", "load", "DiagmmError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdiagmm.so")

_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
MODES = {"qk": 0, "pv": 1, "pvT": 2, "softmax": 3, "softmax_bwd": 4, "softmax_masked": 5,
         "dropout": 6, "attention": 7}


class DiagmmError(RuntimeError):
    """A libdiagmm call returned a status other than DIAGMM_OK."""

    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


class _Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 48), ("rows_per_tile", ctypes.c_int64),
                ("slots_per_tile", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("workgroups", ctypes.c_int64), ("threads", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int64), ("residues", ctypes.c_int64),
                ("strip_workgroups", ctypes.c_int64), ("interleaved", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libdiagmm.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libdiagmm.so not built at {_LIB_PATH}; run "
                          "`python sliding_window_attention_diagmm_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    for name in ("diagmm_qk", "diagmm_pv", "diagmm_pvT"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp] + [i64] * 7 + [f32, ci, ci, vp]
        fn.restype = ci
    lib.diagmm_banded_softmax.argtypes = [vp, vp] + [i64] * 6 + [f32, ci, ci, vp]
    lib.diagmm_banded_softmax.restype = ci
    lib.diagmm_banded_softmax_backward.argtypes = [vp, vp, vp] + [i64] * 6 + [f32, ci, vp]
    lib.diagmm_banded_softmax_backward.restype = ci
    lib.diagmm_banded_softmax_masked.argtypes = [vp, vp, vp] + [i64] * 6 + [f32, f32, ci, ci, vp]
    lib.diagmm_banded_softmax_masked.restype = ci
    lib.diagmm_banded_dropout.argtypes = [vp, vp, vp] + [i64] * 6 + [f32, ci, vp]
    lib.diagmm_banded_dropout.restype = ci
    lib.diagmm_banded_attention.argtypes = [vp, vp, vp, vp] + [i64] * 7 + [f32, ci, vp]
    lib.diagmm_banded_attention.restype = ci
    lib.diagmm_banded_attention_global.argtypes = [vp] * 8 + [i64] * 8 + [f32, ci, vp, i64, vp]
    lib.diagmm_banded_attention_global.restype = ci
    lib.diagmm_banded_attention_global_workspace.argtypes = [i64] * 8 + [ctypes.POINTER(i64)]
    lib.diagmm_banded_attention_global_workspace.restype = ci
    lib.diagmm_banded_attention_global_noalloc.argtypes = [vp] * 8 + [i64] * 8 + [f32, ci, vp]
    lib.diagmm_banded_attention_global_noalloc.restype = ci
    lib.diagmm_status_string.argtypes = [ci]
    lib.diagmm_status_string.restype = ctypes.c_char_p
    lib.diagmm_last_error.argtypes = []
    lib.diagmm_last_error.restype = ctypes.c_char_p
    lib.diagmm_abi_version.argtypes = []
    lib.diagmm_abi_version.restype = ci
    lib.diagmm_plan.argtypes = [ci] + [i64] * 7 + [ci, ci, ctypes.POINTER(_Plan)]
    lib.diagmm_plan.restype = ci
    lib.diagmm_timing_begin.argtypes = [i64]
    lib.diagmm_timing_begin.restype = ci
    lib.diagmm_timing_end.argtypes = []
    lib.diagmm_timing_end.restype = ci
    lib.diagmm_timing_read.argtypes = [i64, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.diagmm_timing_read.restype = ci
    _lib = lib
    return lib


def _raise(lib, st: int):
    text = lib.diagmm_last_error().decode() or lib.diagmm_status_string(st).decode()
    raise DiagmmError(st, text)


def diagmm_abi_version() -> int:
    return load().diagmm_abi_version()


def _dense(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype not in _DT:
        raise TypeError(f"{name} has unsupported dtype {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(out, shape, dtype, device, name="out"):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dense(out, name)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or out.device != device:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype} on {device}")
    return out


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _window(w, w_upper, dilation):
    if w_upper is None:
        w_upper = w
    for name, v in (("w", w), ("w_upper", w_upper), ("dilation", dilation)):
        if int(v) != v or v < 0:
            raise ValueError(f"{name} must be a non-negative integer (got {v})")
    return int(w), int(w_upper), int(dilation)


def diagmm_qk(q, k, w, w_upper=None, dilation=0, padding_value=0.0, out_dtype=None, out=None):
    """band[b,i,h,kk] = <q[b,i,h,:], k[b,i+(kk-w)*s,h,:]>, padding_value where that key
    position is outside [0, n).  Returns ``[b, n, h, w + w_upper + 1]``."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    q, k = _dense(q, "q"), _dense(k, "k")
    if q.shape != k.shape or q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q and k must have the same shape, dtype and device")
    b, n, h, d = q.shape
    out_dtype = out_dtype or q.dtype
    band = _out(out, (b, n, h, w + w_upper + 1), out_dtype, q.device)
    st = lib.diagmm_qk(q.data_ptr(), k.data_ptr(), band.data_ptr(), b, n, h, d, w, w_upper,
                       dilation, float(padding_value), _DT[q.dtype], _DT[out_dtype],
                       _stream(q.device))
    if st:
        _raise(lib, st)
    return band


def _pv_like(fn_name, band, x, w, w_upper, dilation, out_dtype, out):
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    band, x = _dense(band, "band"), _dense(x, "x")
    b, n, h, d = x.shape
    K = w + w_upper + 1
    if tuple(band.shape) != (b, n, h, K):
        raise ValueError(f"band must be {(b, n, h, K)}, got {tuple(band.shape)}")
    if band.dtype != x.dtype or band.device != x.device:
        raise ValueError("band and the dense operand must share dtype and device")
    out_dtype = out_dtype or x.dtype
    res = _out(out, (b, n, h, d), out_dtype, x.device)
    st = getattr(lib, fn_name)(band.data_ptr(), x.data_ptr(), res.data_ptr(), b, n, h, d, w,
                               w_upper, dilation, 0.0, _DT[x.dtype], _DT[out_dtype],
                               _stream(x.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_pv(band, v, w, w_upper=None, dilation=0, out_dtype=None, out=None):
    """out[b,i,h,:] = sum over in-range slots kk of band[b,i,h,kk] * v[b,i+(kk-w)*s,h,:]."""
    return _pv_like("diagmm_pv", band, v, w, w_upper, dilation, out_dtype, out)


def diagmm_pvT(band, x, w, w_upper=None, dilation=0, out_dtype=None, out=None):
    """out[b,j,h,:] = sum over (i, kk) with i+(kk-w)*s = j of band[b,i,h,kk] * x[b,i,h,:]."""
    return _pv_like("diagmm_pvT", band, x, w, w_upper, dilation, out_dtype, out)


def diagmm_banded_softmax(scores, w, w_upper=None, dilation=0, scale=1.0, out_dtype=None,
                          out=None, inplace=False, key_mask=None, mask_value=-10000.0):
    """Softmax of scale * scores over each band row's in-range slots; out-of-range slots
    get exactly 0.  ``inplace=True`` overwrites ``scores`` (same dtype only).  With
    ``key_mask`` (float32 [b, n] on the GPU: 1 keeps a key, 0 masks it) each slot's scaled
    score gains (1 - key_mask[b, key]) * mask_value first."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    s = _dense(scores, "scores")
    b, n, h, K = s.shape
    if K != w + w_upper + 1:
        raise ValueError(f"scores last dim {K} != w + w_upper + 1 = {w + w_upper + 1}")
    out_dtype = out_dtype or s.dtype
    if inplace:
        if out is not None or out_dtype != s.dtype:
            raise ValueError("inplace softmax writes scores itself (same dtype)")
        res = s
    else:
        res = _out(out, s.shape, out_dtype, s.device)
    if key_mask is not None:
        if (not isinstance(key_mask, torch.Tensor) or key_mask.dtype != torch.float32 or
                tuple(key_mask.shape) != (b, n) or key_mask.device != s.device or
                not key_mask.is_contiguous()):
            raise ValueError(f"key_mask must be a contiguous float32 [{b}, {n}] tensor on "
                             f"{s.device}")
        st = lib.diagmm_banded_softmax_masked(s.data_ptr(), res.data_ptr(), key_mask.data_ptr(),
                                              b, n, h, w, w_upper, dilation, float(scale),
                                              float(mask_value), _DT[s.dtype], _DT[out_dtype],
                                              _stream(s.device))
    else:
        st = lib.diagmm_banded_softmax(s.data_ptr(), res.data_ptr(), b, n, h, w, w_upper,
                                       dilation, float(scale), _DT[s.dtype], _DT[out_dtype],
                                       _stream(s.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_banded_softmax_backward(probs, dprobs, w, w_upper=None, dilation=0, scale=1.0,
                                   out=None):
    """Gradient of ``diagmm_banded_softmax`` with respect to its scores, from its output
    ``probs`` and the gradient ``dprobs`` with respect to it: per band row,
    ``scale * probs * (dprobs - sum(probs * dprobs))`` over the in-range slots, exactly 0
    elsewhere.  ``out`` may be ``probs`` or ``dprobs`` itself (in place)."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    p, dp = _dense(probs, "probs"), _dense(dprobs, "dprobs")
    if p.shape != dp.shape or p.dtype != dp.dtype or p.device != dp.device:
        raise ValueError("probs and dprobs must have the same shape, dtype and device")
    b, n, h, K = p.shape
    if K != w + w_upper + 1:
        raise ValueError(f"probs last dim {K} != w + w_upper + 1 = {w + w_upper + 1}")
    res = out if out is p or out is dp else _out(out, p.shape, p.dtype, p.device)
    st = lib.diagmm_banded_softmax_backward(p.data_ptr(), dp.data_ptr(), res.data_ptr(), b, n,
                                            h, w, w_upper, dilation, float(scale),
                                            _DT[p.dtype], _stream(p.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_banded_dropout(probs, rand, w, w_upper=None, dilation=0, p=0.1, out=None):
    """Dropout on a probability band with caller-drawn uniforms ``rand`` (float32, the
    band's shape): in-range slots with ``rand > p`` keep ``probs / (1 - p)``, the others
    are 0.  With the same ``rand`` it also maps the gradient with respect to the output to
    the gradient with respect to ``probs``.  ``out`` may be ``probs`` itself (in place)."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    pr = _dense(probs, "probs")
    rd = _dense(rand, "rand")
    if rd.dtype != torch.float32 or rd.shape != pr.shape or rd.device != pr.device:
        raise ValueError("rand must be float32 with the band's shape, on the band's device")
    b, n, h, K = pr.shape
    if K != w + w_upper + 1:
        raise ValueError(f"probs last dim {K} != w + w_upper + 1 = {w + w_upper + 1}")
    res = out if out is pr else _out(out, pr.shape, pr.dtype, pr.device)
    st = lib.diagmm_banded_dropout(pr.data_ptr(), rd.data_ptr(), res.data_ptr(), b, n, h, w,
                                   w_upper, dilation, float(p), _DT[pr.dtype],
                                   _stream(pr.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_banded_attention(q, k, v, w, w_upper=None, dilation=0, scale=None, out=None):
    """Sliding-window attention in one pass: ``softmax(scale * Q K^T)`` over the window's
    in-range diagonals times V, without writing the band ([b, n, h, d] in and out, f16 or
    bf16, d in {32, 64, 128}).  ``scale`` defaults to 1 / sqrt(d)."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    q, k, v = _dense(q, "q"), _dense(k, "k"), _dense(v, "v")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype
            and q.device == k.device == v.device):
        raise ValueError("q, k and v must have the same shape, dtype and device")
    b, n, h, d = q.shape
    if scale is None:
        scale = d ** -0.5
    res = _out(out, q.shape, q.dtype, q.device)
    st = lib.diagmm_banded_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), res.data_ptr(),
                                     b, n, h, d, w, w_upper, dilation, float(scale),
                                     _DT[q.dtype], _stream(q.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_banded_attention_global(q, k, v, global_pos, w, w_upper=None, dilation=0,
                                   scale=None, out=None, global_qkv=None):
    """``diagmm_banded_attention`` with global tokens: ``global_pos`` is int32 [b, ng] on
    the GPU; its entries in [0, n) form the global set (a repeat counts once).  Rows
    outside the set attend their window and the global keys (each key once) with q, k, v;
    global rows attend every key with ``global_qkv`` = (GQ, GK, GV) (default q, k, v).
    The call's workspace is allocated here, from torch's caching allocator."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    q, k, v = _dense(q, "q"), _dense(k, "k"), _dense(v, "v")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype
            and q.device == k.device == v.device):
        raise ValueError("q, k and v must have the same shape, dtype and device")
    gptr = [None, None, None]
    if global_qkv is not None:
        gq, gk, gv = (_dense(t, "global_qkv") for t in global_qkv)
        for t in (gq, gk, gv):
            if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
                raise ValueError("global_qkv tensors must match q in shape, dtype and device")
        gptr = [gq.data_ptr(), gk.data_ptr(), gv.data_ptr()]
    b, n, h, d = q.shape
    g = global_pos
    if (not isinstance(g, torch.Tensor) or g.dtype != torch.int32 or g.dim() != 2
            or g.shape[0] != b or g.device != q.device or not g.is_contiguous()):
        raise ValueError("global_pos must be a contiguous int32 [b, ng] tensor on q's device")
    if scale is None:
        scale = d ** -0.5
    res = _out(out, q.shape, q.dtype, q.device)
    need = ctypes.c_int64(0)
    st = lib.diagmm_banded_attention_global_workspace(b, n, h, d, w, w_upper, dilation,
                                                      g.shape[1], ctypes.byref(need))
    if st:
        _raise(lib, st)
    ws = torch.empty(need.value + 256, dtype=torch.uint8, device=q.device) if need.value else None
    ws_ptr = None if ws is None else (ws.data_ptr() + 255) // 256 * 256
    st = lib.diagmm_banded_attention_global(q.data_ptr(), k.data_ptr(), v.data_ptr(), gptr[0],
                                            gptr[1], gptr[2], res.data_ptr(), g.data_ptr(),
                                            g.shape[1], b, n, h, d, w, w_upper, dilation,
                                            float(scale), _DT[q.dtype], ws_ptr, need.value,
                                            _stream(q.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_banded_attention_global_noalloc(q, k, v, global_pos, w, w_upper=None, dilation=0,
                                           scale=None, out=None, global_qkv=None):
    """``diagmm_banded_attention_global`` through the library's allocation-free entry point:
    its workspace is the library's static per-GPU array (calls on one GPU must not overlap
    in time); only ``out`` is allocated here, and only when it is not given."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    q, k, v = _dense(q, "q"), _dense(k, "k"), _dense(v, "v")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype
            and q.device == k.device == v.device):
        raise ValueError("q, k and v must have the same shape, dtype and device")
    gptr = [None, None, None]
    if global_qkv is not None:
        gq, gk, gv = (_dense(t, "global_qkv") for t in global_qkv)
        for t in (gq, gk, gv):
            if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
                raise ValueError("global_qkv tensors must match q in shape, dtype and device")
        gptr = [gq.data_ptr(), gk.data_ptr(), gv.data_ptr()]
    b, n, h, d = q.shape
    g = global_pos
    if (not isinstance(g, torch.Tensor) or g.dtype != torch.int32 or g.dim() != 2
            or g.shape[0] != b or g.device != q.device or not g.is_contiguous()):
        raise ValueError("global_pos must be a contiguous int32 [b, ng] tensor on q's device")
    if scale is None:
        scale = d ** -0.5
    res = _out(out, q.shape, q.dtype, q.device)
    with torch.cuda.device(q.device):
        st = lib.diagmm_banded_attention_global_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), gptr[0], gptr[1], gptr[2], res.data_ptr(),
            g.data_ptr(), g.shape[1], b, n, h, d, w, w_upper, dilation, float(scale),
            _DT[q.dtype], _stream(q.device))
    if st:
        _raise(lib, st)
    return res


def diagmm_plan(mode, b, n, h, d, w, w_upper=None, dilation=0, in_dtype=torch.float16,
                out_dtype=None) -> dict:
    """The band-tile scheduler's plan for a call (host only; no GPU needed)."""
    lib = load()
    w, w_upper, dilation = _window(w, w_upper, dilation)
    out_dtype = out_dtype or in_dtype
    pl = _Plan()
    st = lib.diagmm_plan(MODES.get(mode, mode), b, n, h, d, w, w_upper, dilation,
                         _DT[in_dtype], _DT[out_dtype], ctypes.byref(pl))
    if st:
        _raise(lib, st)
    return {"kernel": pl.kernel.decode(), "rows_per_tile": pl.rows_per_tile,
            "slots_per_tile": pl.slots_per_tile, "tiles": pl.tiles,
            "workgroups": pl.workgroups, "threads": pl.threads, "lds_bytes": pl.lds_bytes,
            "residues": pl.residues, "strip_workgroups": pl.strip_workgroups,
            "interleaved": pl.interleaved}


def diagmm_timing_begin(capacity: int) -> None:
    """Start recording kernel start/end events for the next ``capacity`` launches."""
    lib = load()
    st = lib.diagmm_timing_begin(int(capacity))
    if st:
        _raise(lib, st)


def diagmm_timing_end() -> None:
    """Stop recording (launches after this run untimed)."""
    lib = load()
    st = lib.diagmm_timing_end()
    if st:
        _raise(lib, st)


def diagmm_timing_read() -> list:
    """Waits for the timed kernels; returns [(mode name, kernel ms), ...] in launch order."""
    lib = load()
    count = ctypes.c_int64(0)
    st = lib.diagmm_timing_read(0, None, None, ctypes.byref(count))
    if st:
        _raise(lib, st)
    n = count.value
    ops = (ctypes.c_int32 * max(n, 1))()
    ms = (ctypes.c_double * max(n, 1))()
    st = lib.diagmm_timing_read(n, ops, ms, ctypes.byref(count))
    if st:
        _raise(lib, st)
    names = {v: k for k, v in MODES.items()}
    return [(names.get(ops[i], str(ops[i])), ms[i]) for i in range(n)]
