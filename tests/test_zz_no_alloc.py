"""The allocation-free global-token call against the workspace call, through the C ABI.

diagmm_banded_attention_global_noalloc runs the same kernels as
diagmm_banded_attention_global on the library's static per-GPU workspace; on the same
inputs both must give the same bits.  Two calls in a row - the benchmark shape with
separate global matrices, then a smaller dilated bf16 problem - check that the second
call is not disturbed by what the first left in the shared array.
"""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import sliding_window_attention_diagmm_amd as dm

pytestmark = pytest.mark.gpu

_DT = {torch.float16: 1, torch.bfloat16: 2}

# (b, n, h, d, w, dilation, ng, dtype, seed)
CALLS = [(1, 4096, 12, 64, 256, 0, 8, "f16", 2100),
         (2, 1000, 3, 32, 40, 3, 5, "bf16", 2110)]


def _inputs(b, n, h, d, ng, dt, seed):
    g = datagen.rng(seed)
    mats = [datagen.normal(g, (b, n, h, d), dt).cuda() for _ in range(6)]
    pos = np.stack([np.concatenate([[0, n - 1], datagen.rng(seed + 1 + bb).choice(
        np.arange(1, n - 1), ng - 2, replace=False)]) for bb in range(b)])
    glob = torch.from_numpy(pos.astype(np.int32)).cuda()
    return mats, glob


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    lib = dm.load()
    for b, n, h, d, w, dil, ng, dt, seed in CALLS:
        print(f"noalloc call b={b} n={n} h={h} d={d} w={w} dil={dil} ng={ng} {dt}", flush=True)
        (q, k, v, gq, gk, gv), glob = _inputs(b, n, h, d, ng, dt, seed)
        ref = dm.diagmm_banded_attention_global(q, k, v, glob, w, w, dil, 0.125,
                                                global_qkv=(gq, gk, gv))
        out = torch.full_like(q, float("nan"))
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.diagmm_banded_attention_global_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), gq.data_ptr(), gk.data_ptr(),
            gv.data_ptr(), out.data_ptr(), glob.data_ptr(), ng, b, n, h, d, w, w, dil,
            ctypes.c_float(0.125), _DT[q.dtype], ctypes.c_void_p(stream))
        assert st == 0, lib.diagmm_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (b, n, h, d, dil, dt)
        # the Python wrapper of the same entry point
        again = dm.diagmm_banded_attention_global_noalloc(q, k, v, glob, w, w, dil, 0.125,
                                                          global_qkv=(gq, gk, gv))
        torch.cuda.synchronize()
        assert torch.equal(again, ref)
