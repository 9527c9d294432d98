"""GPU parity of the exact launches the benchmark times, against the oracle.

The benchmark's step runs pv and pvT (and qk, checked in test_parity_workloads.py) on
the forward workload of TVM Discuss "Developing a faster schedule for Longformer's
kernel" (post 6: b=1, n=4096, h=12, d=64, w=w_upper=256, 513 diagonals) in f16 in and
out, at the two dilations of post 4 (0 and 3), under the library's default plan (one
workgroup per compute unit, the strip split where the planner picks it).  Here the same
calls, on the same plan, are compared with the oracle on 256 sampled output rows per
case (all heads), including both sequence ends and both window edges, to the f16
tolerance: |gpu - oracle| <= max(2e-3, one f16 ulp of the result), the oracle taken
before its final rounding.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _util import check_close

pytestmark = pytest.mark.gpu

B, N, H, D, W, WU = 1, 4096, 12, 64, 256, 256
K = W + WU + 1


def _rows(dil):
    s = max(dil, 1)
    forced = {0, 1, 2, s, W - 1, W, W + 1, W * s - 1, W * s, N // 2,
              N - W * s - 1, N - W * s, N - W - 1, N - W, N - 3, N - 2, N - 1}
    g = np.random.RandomState(4242 + dil)
    rest = [int(p) for p in g.permutation(N) if int(p) not in forced]
    rows = sorted(forced | set(rest[: 256 - len(forced)]))
    assert len(rows) == 256
    return np.array(rows, dtype=np.int64)


@pytest.fixture(scope="module")
def inputs():
    g = datagen.rng(31)
    probs = datagen.softmax_rows(g, (B, N, H, K), "f16")
    v = datagen.normal(g, (B, N, H, D), "f16")
    x = datagen.normal(g, (B, N, H, D), "f16")
    return probs, v, x


@pytest.mark.parametrize("mode,dil", [("pv", 0), ("pv", 3), ("pvT", 0), ("pvT", 3)])
def test_bench_launch_matches_oracle(inputs, mode, dil):
    import sliding_window_attention_diagmm_amd as dm
    probs, v, x = inputs
    plan = dm.diagmm_plan(mode, B, N, H, D, W, WU, dil, torch.float16)
    assert "mfma" in plan["kernel"], plan            # the tiled kernel the bench times
    dense = v if mode == "pv" else x
    fn = dm.diagmm_pv if mode == "pv" else dm.diagmm_pvT
    out = fn(probs.cuda(), dense.cuda(), W, WU, dil).cpu()
    assert out.dtype == torch.float16 and torch.isfinite(out).all()
    rows = _rows(dil)
    ri = torch.from_numpy(rows)
    flat_out = out.reshape(N, H, D)[ri]
    if mode == "pv":
        ref = oracle.pv(probs.reshape(N, H, K)[ri], dense, W, WU, dil,
                        out_dtype=torch.float64, rows=rows)
    else:
        ref = oracle.pvT(probs, dense, W, WU, dil, out_dtype=torch.float64, rows=rows)
    check_close(flat_out, ref, torch.float16, f"{mode} dil{dil} bench launch")


def test_pvt_strip_tile_orders_agree_bitwise(inputs, monkeypatch):
    """pvT at dilation 3 on its default strip split, and with each strip's tiles dealt
    round-robin over the strip's workgroups (forced): the same bits, since a tile's sums
    do not depend on the workgroup that takes it; both against the oracle on the sampled
    rows through the test above."""
    import sliding_window_attention_diagmm_amd as dm
    probs, _, x = inputs
    monkeypatch.delenv("DIAGMM_TILE_ORDER", raising=False)
    monkeypatch.delenv("DIAGMM_MAX_WORKGROUPS", raising=False)
    plan = dm.diagmm_plan("pvT", B, N, H, D, W, WU, 3, torch.float16)
    pc, xc = probs.cuda(), x.cuda()
    base = dm.diagmm_pvT(pc, xc, W, WU, 3).cpu()
    monkeypatch.setenv("DIAGMM_TILE_ORDER", "interleaved")
    forced = dm.diagmm_plan("pvT", B, N, H, D, W, WU, 3, torch.float16)
    assert forced["interleaved"] == 1 or plan["workgroups"] % 8 != 0, (plan, forced)
    assert forced["strip_workgroups"] == plan["strip_workgroups"], (plan, forced)
    got = dm.diagmm_pvT(pc, xc, W, WU, 3).cpu()
    assert torch.equal(got, base)
