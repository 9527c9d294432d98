"""Banded (sliding-window) attention with its gradient, composed from the libdiagmm calls.

TVM Discuss, "Developing a faster schedule for Longformer's kernel", post 6: the kernel
serves one forward function and two backward functions told apart by ``transpose_t1``;
with the banded softmax between them (csarofeen/pytorch issue 2096, first fusion repro)
they give attention over a (dilated) sliding window and its gradients:

    forward:   S = qk(Q, K)        P = softmax(scale * S [+ key mask term])
               Pd = dropout(P, rand)                            (when p > 0; else Pd = P)
               O = pv(Pd, V)
    backward:  dPd = qk(dO, V)     dV = pvT(Pd, dO)
               dP = dropout(dPd, rand)                          (the same keep pattern)
               dS = softmax_backward(P, dP)                     (scale included)
               dQ = pv(dS, K)      dK = pvT(dS, Q)

Without gradients (inference), f16/bf16 inputs with d in {32, 64, 128}, no key mask and no
dropout go to the one-pass kernel, which never writes the band.

Every step runs in the library's kernels; this module only orders the calls, keeps P
(and the caller's random numbers) for the backward pass, where Pd is drawn again from
them, and hands torch's autograd the results.  Tensors are contiguous ``[b, n, h, d]``
on the GPU in one dtype (f32, f16 or bf16); gradients come back in it.
"""
from __future__ import annotations

import torch

from . import (diagmm_banded_attention, diagmm_banded_dropout, diagmm_banded_softmax,
               diagmm_banded_softmax_backward, diagmm_pv, diagmm_pvT, diagmm_qk)


class BandedAttention(torch.autograd.Function):
    """O = softmax_band(scale * Q K^T) V over the window (w, w_upper, dilation)."""

    @staticmethod
    def forward(ctx, q, k, v, w, w_upper, dilation, scale, key_mask=None, mask_value=-10000.0,
                dropout_p=0.0, dropout_rand=None):
        band = diagmm_qk(q, k, w, w_upper, dilation, 0.0)
        probs = diagmm_banded_softmax(band, w, w_upper, dilation, scale, inplace=True,
                                      key_mask=key_mask, mask_value=mask_value)
        kept = probs
        if dropout_p > 0.0:
            kept = diagmm_banded_dropout(probs, dropout_rand, w, w_upper, dilation, dropout_p)
        out = diagmm_pv(kept, v, w, w_upper, dilation)
        ctx.save_for_backward(q, k, v, probs, dropout_rand if dropout_p > 0.0 else None)
        ctx.window = (w, w_upper, dilation, scale, dropout_p)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, probs, rand = ctx.saved_tensors
        w, w_upper, dilation, scale, p = ctx.window
        dout = dout.contiguous()
        dprobs = diagmm_qk(dout, v, w, w_upper, dilation, 0.0)
        if p > 0.0:
            kept = diagmm_banded_dropout(probs, rand, w, w_upper, dilation, p)
            dv = diagmm_pvT(kept, dout, w, w_upper, dilation)
            del kept
            diagmm_banded_dropout(dprobs, rand, w, w_upper, dilation, p, out=dprobs)
        else:
            dv = diagmm_pvT(probs, dout, w, w_upper, dilation)
        dscores = diagmm_banded_softmax_backward(probs, dprobs, w, w_upper, dilation, scale,
                                                 out=dprobs)
        dq = diagmm_pv(dscores, k, w, w_upper, dilation)
        dk = diagmm_pvT(dscores, q, w, w_upper, dilation)
        return dq, dk, dv, None, None, None, None, None, None, None, None


def banded_attention(q, k, v, w, w_upper=None, dilation=0, scale=None, key_mask=None,
                     mask_value=-10000.0, dropout_p=0.0, dropout_rand=None):
    """Sliding-window attention of ``q`` over ``k``/``v`` ([b, n, h, d] each): slot kk of
    row i attends key i + (kk - w) * max(dilation, 1) for kk in 0 .. w + w_upper; keys
    outside the sequence are masked.  ``scale`` defaults to 1 / sqrt(d).  ``key_mask``
    (float32 [b, n], 1 = keep) adds (1 - key_mask) * mask_value to each key's scores (the
    attention mask of the issue 2096 repro); the backward pass is unchanged by it.
    ``dropout_p`` > 0 drops attention probabilities as that repro does: ``dropout_rand``
    (float32 [b, n, h, w + w_upper + 1] on the GPU, drawn by the caller) keeps slot kk
    of row i when it is greater than ``dropout_p``, and kept probabilities are scaled by
    1 / (1 - dropout_p)."""
    if w_upper is None:
        w_upper = w
    if scale is None:
        scale = q.shape[-1] ** -0.5
    if dropout_p > 0.0 and dropout_rand is None:
        raise ValueError("dropout_p > 0 needs dropout_rand (the caller draws the uniforms)")
    needs_grad = torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v))
    if (not needs_grad and key_mask is None and dropout_p == 0.0
            and q.dtype in (torch.float16, torch.bfloat16) and q.shape[-1] in (32, 64, 128)):
        # inference: the one-pass kernel (the band is never written)
        return diagmm_banded_attention(q, k, v, int(w), int(w_upper), int(dilation),
                                       float(scale))
    return BandedAttention.apply(q, k, v, int(w), int(w_upper), int(dilation), float(scale),
                                 key_mask, float(mask_value), float(dropout_p), dropout_rand)
