"""GPU parity with a small persistent grid (DIAGMM_MAX_WORKGROUPS): every workgroup walks
many tiles, so the continuation prefetch, the prefetch of a tile that starts a new strip,
load batches held across tiles, empty tail blocks of short residue classes and both slot
chunks of a row block all run at sizes the oracle checks in full.
"""
import math

import pytest
import torch

import datagen
import oracle
import sliding_window_attention_diagmm_amd as dm
from _util import assert_bits_equal, check_close, in_range_mask

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, d, w, w_upper, dilation, in, out, workgroups)
CASES = [
    (1, 2048, 3, 64, 256, 256, 0, "f16", "f16", 8),
    (1, 2048, 3, 64, 256, 256, 3, "f16", "f16", 8),
    (2, 1100, 2, 64, 128, 40, 2, "bf16", "f32", 5),
    (1, 1500, 2, 32, 200, 200, 0, "f16", "f16", 3),
    (1, 900, 2, 128, 96, 96, 1, "bf16", "bf16", 7),
]


def _ids(c):
    b, n, h, d, w, wu, dil, i, o, wg = c
    return f"b{b}n{n}h{h}d{d}w{w}u{wu}s{dil}-{i}-{o}-wg{wg}"


def test_grid_cap_shapes_the_plan(monkeypatch):
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", "8")
    for mode in ("qk", "pv", "pvT"):
        pl = dm.diagmm_plan(mode, 1, 2048, 3, 64, 256, 256, 0, torch.float16)
        assert pl["workgroups"] <= 8 and pl["tiles"] >= 4 * pl["workgroups"], (mode, pl)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_small_grid_matches_oracle(case, monkeypatch):
    b, n, h, d, w, wu, dil, ind, outd, wg = case
    monkeypatch.setenv("DIAGMM_MAX_WORKGROUPS", str(wg))
    g = datagen.rng(77)
    sc = 1.0 / math.sqrt(d)
    q = datagen.normal(g, (b, n, h, d), ind, sc)
    k = datagen.normal(g, (b, n, h, d), ind, sc)
    v = datagen.normal(g, (b, n, h, d), ind, sc)
    probs = datagen.softmax_rows(g, (b, n, h, w + wu + 1), ind)
    mask = in_range_mask(b, n, h, w, wu, dil)
    pad = -0.75

    s_gpu = dm.diagmm_qk(q.cuda(), k.cuda(), w, wu, dil, pad, out_dtype=DT[outd]).cpu()
    check_close(s_gpu, oracle.qk(q, k, w, wu, dil, pad, out_dtype=torch.float64), DT[ind],
                "qk", mask)
    assert_bits_equal(s_gpu[~mask], oracle.qk(q, k, w, wu, dil, pad,
                                              out_dtype=DT[outd])[~mask], "qk padding")

    pc = probs.cuda()
    o_gpu = dm.diagmm_pv(pc, v.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(o_gpu, oracle.pv(probs, v, w, wu, dil, out_dtype=torch.float64), DT[ind], "pv")
    x_gpu = dm.diagmm_pvT(pc, q.cuda(), w, wu, dil, out_dtype=DT[outd]).cpu()
    check_close(x_gpu, oracle.pvT(probs, q, w, wu, dil, out_dtype=torch.float64), DT[ind],
                "pvT")
    if ind != "f32":
        p_gpu = dm.diagmm_banded_softmax(pc, w, wu, dil, 0.5).cpu()
        check_close(p_gpu, oracle.softmax(probs, w, wu, dil, 0.5, out_dtype=torch.float64),
                    DT[ind], "softmax", mask)
