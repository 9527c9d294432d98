"""GPU parity of the one-pass attention with global tokens against the CPU oracle.

Rows outside the global set attend their window and every global key, each key once,
with Q, K, V; global rows attend every key with the global matrices (the oracle's pins
are in test_oracle.py).  The bound is the one-pass attention's: the 16-bit output bar
plus u * sum_k P_k |V_k| for the probabilities rounded to the input dtype before the
product with V.  Cases cover global tokens inside and outside the window, at both
sequence ends, more than one 64-key block of them (and more than one 64-row block of
global rows), dilation (global keys of every residue class), d = 32 / 64 / 128, f16 and
bf16, separate Global_Q / Global_K / Global_V, position lists with repeats and entries
outside [0, n), every position global, global rows merged over many key ranges, ng = 0
and a list with no position in range (the plain one-pass call, bit for bit), reruns bit
for bit, and the benchmark shape on sampled rows.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _util import LOWP_ABS, out_ulp

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}

# (b, n, h, d, w, w_upper, dilation, dtype, ng)
CASES = [
    (1, 200, 2, 64, 16, 16, 0, "f16", 3),
    (2, 300, 2, 32, 20, 5, 0, "bf16", 5),
    (1, 333, 1, 64, 20, 20, 3, "f16", 7),      # globals of every residue class
    (1, 257, 2, 128, 40, 40, 2, "bf16", 1),
    (1, 700, 1, 64, 30, 30, 0, "f16", 70),     # two blocks of global keys
    (2, 90, 3, 64, 100, 100, 0, "f16", 4),     # window wider than the sequence
    (1, 1, 1, 64, 3, 3, 0, "f16", 1),          # the only position is global
]


def _ids(c):
    b, n, h, d, w, wu, dil, dt, ng = c
    return f"b{b}n{n}h{h}d{d}w{w}u{wu}s{dil}-{dt}-g{ng}"


def _glob(b, n, ng, seed):
    """Distinct global positions per batch, both sequence ends among them when ng >= 2."""
    rows = []
    for bb in range(b):
        if ng >= 2:
            mid = datagen.rng(seed + bb).choice(np.arange(1, n - 1), ng - 2, replace=False)
            g = np.concatenate([[0, n - 1], mid])
        else:
            g = datagen.rng(seed + bb).choice(n, ng, replace=False)
        assert len(set(g.tolist())) == ng
        rows.append(np.sort(g))
    return torch.from_numpy(np.stack(rows).astype(np.int32))


def check_global(got, q, k, v, glob, w, wu, dil, scale, dtype, what, rows=None, gqkv=None):
    ref = oracle.attention_global(q, k, v, glob, w, wu, dil, scale, out_dtype=torch.float64,
                                  rows=rows, global_qkv=gqkv)
    gabs = None if gqkv is None else (gqkv[0], gqkv[1], gqkv[2].abs())
    mag = oracle.attention_global(q, k, v.abs(), glob, w, wu, dil, scale,
                                  out_dtype=torch.float64, rows=rows, global_qkv=gabs)
    g = got.detach().cpu().double()
    assert torch.isfinite(g).all(), f"{what}: non-finite GPU values"
    u = 2.0 ** -11 if dtype == torch.float16 else 2.0 ** -8
    tol = torch.clamp(out_ulp(ref, dtype), min=LOWP_ABS) + u * mag
    diff = (g - ref).abs()
    bad = diff > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, worst "
                           f"excess {(diff - tol).max().item():.3e}")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_attention_global_matches_oracle(case):
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt, ng = case
    g_ = datagen.rng(1400 + n + d)
    q, k, v = (datagen.normal(g_, (b, n, h, d), dt) for _ in range(3))
    glob = _glob(b, n, ng, 1450 + n)
    got = dm.diagmm_banded_attention_global(q.cuda(), k.cuda(), v.cuda(), glob.cuda(), w, wu,
                                            dil, d ** -0.5)
    torch.cuda.synchronize()
    check_global(got, q, k, v, glob.long(), w, wu, dil, d ** -0.5, DT[dt], _ids(case))


def test_attention_global_without_tokens_is_the_plain_call():
    import sliding_window_attention_diagmm_amd as dm
    g_ = datagen.rng(1500)
    q, k, v = (datagen.normal(g_, (1, 300, 2, 64), "f16").cuda() for _ in range(3))
    none = torch.zeros(1, 0, dtype=torch.int32, device="cuda")
    a = dm.diagmm_banded_attention_global(q, k, v, none, 20, 20, 2, 0.125)
    assert torch.equal(a, dm.diagmm_banded_attention(q, k, v, 20, 20, 2, 0.125))


@pytest.mark.parametrize("dil", [0, 3])
def test_attention_global_at_the_benchmark_shape(dil):
    """n=4096, h=12, d=64, 513 diagonals, f16, 8 global tokens: the global rows and 120
    sampled rows against the oracle."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w = 1, 4096, 12, 64, 256
    g_ = datagen.rng(1510 + dil)
    q, k, v = (datagen.normal(g_, (b, n, h, d), "f16") for _ in range(3))
    glob = _glob(b, n, 8, 1520)
    got = dm.diagmm_banded_attention_global(q.cuda(), k.cuda(), v.cuda(), glob.cuda(), w, w,
                                            dil, 0.125)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([glob[0].numpy().astype(np.int64),
                                     datagen.rng(1530).choice(n, 120, replace=False)]))
    ri = torch.from_numpy(rows)
    check_global(got.cpu().reshape(n, h, d)[ri], q, k, v, glob.long(), w, w, dil, 0.125,
                 torch.float16, f"bench dilation {dil}", rows=rows)


# (b, n, h, d, w, w_upper, dilation, dtype, ng)
QKV_CASES = [
    (1, 200, 2, 64, 16, 16, 0, "f16", 3),
    (2, 300, 2, 32, 20, 5, 2, "bf16", 5),
    (1, 257, 1, 128, 40, 40, 0, "f16", 9),
    (1, 700, 1, 64, 30, 30, 3, "bf16", 70),    # two 64-row blocks of global rows
]


@pytest.mark.parametrize("case", QKV_CASES, ids=_ids)
def test_attention_global_separate_matrices_match_oracle(case):
    """Global rows from Global_Q / Global_K / Global_V, the others from Q, K, V."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil, dt, ng = case
    g_ = datagen.rng(1600 + n + d)
    q, k, v, gq, gk, gv = (datagen.normal(g_, (b, n, h, d), dt) for _ in range(6))
    glob = _glob(b, n, ng, 1650 + n)
    got = dm.diagmm_banded_attention_global(
        q.cuda(), k.cuda(), v.cuda(), glob.cuda(), w, wu, dil, d ** -0.5,
        global_qkv=(gq.cuda(), gk.cuda(), gv.cuda()))
    torch.cuda.synchronize()
    check_global(got, q, k, v, glob.long(), w, wu, dil, d ** -0.5, DT[dt], _ids(case),
                 gqkv=(gq, gk, gv))


def test_attention_global_position_list_is_a_set():
    """Repeats count once; entries outside [0, n) name no position; and a list of such
    entries only is the plain one-pass call, bit for bit."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w, wu, dil = 2, 300, 2, 64, 20, 20, 0
    g_ = datagen.rng(1700)
    q, k, v = (datagen.normal(g_, (b, n, h, d), "f16") for _ in range(3))
    messy = torch.tensor([[5, 5, 120, -1, n, 5, 299, 1 << 30, 120, 0],
                          [0, -7, 0, 0, 150, 150, n + 3, 7, 7, 7]], dtype=torch.int32)
    got = dm.diagmm_banded_attention_global(q.cuda(), k.cuda(), v.cuda(), messy.cuda(), w, wu,
                                            dil, 0.125)
    torch.cuda.synchronize()
    check_global(got, q, k, v, messy.long(), w, wu, dil, 0.125, torch.float16, "messy list")
    junk = torch.tensor([[-1, n, -5], [n + 1, -2, 1 << 20]], dtype=torch.int32)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    a = dm.diagmm_banded_attention_global(qc, kc, vc, junk.cuda(), w, wu, dil, 0.125)
    assert torch.equal(a, dm.diagmm_banded_attention(qc, kc, vc, w, wu, dil, 0.125))


@pytest.mark.parametrize("n,ng,dil", [(150, 150, 0), (97, 97, 2)])
def test_attention_global_every_position(n, ng, dil):
    """Every position global: only global rows, each over every key (band rows store
    nothing), with separate global matrices."""
    import sliding_window_attention_diagmm_amd as dm
    b, h, d, w = 1, 2, 64, 8
    g_ = datagen.rng(1750 + n)
    q, k, v, gq, gk, gv = (datagen.normal(g_, (b, n, h, d), "f16") for _ in range(6))
    glob = torch.from_numpy(datagen.rng(1760).permutation(n).astype(np.int32))[None, :]
    got = dm.diagmm_banded_attention_global(
        q.cuda(), k.cuda(), v.cuda(), glob.contiguous().cuda(), w, w, dil, 0.125,
        global_qkv=(gq.cuda(), gk.cuda(), gv.cuda()))
    torch.cuda.synchronize()
    check_global(got, q, k, v, glob.long(), w, w, dil, 0.125, torch.float16, f"all {n}",
                 gqkv=(gq, gk, gv))


def test_attention_global_many_key_ranges_and_reruns():
    """One (batch, head) and 3 global rows at n = 5000: the global rows are merged over
    27 key ranges of 192 keys (the last one short); two calls agree bit for bit."""
    import sliding_window_attention_diagmm_amd as dm
    b, n, h, d, w = 1, 5000, 1, 64, 64
    g_ = datagen.rng(1800)
    q, k, v = (datagen.normal(g_, (b, n, h, d), "bf16") for _ in range(3))
    glob = torch.tensor([[4999, 17, 2500]], dtype=torch.int32)
    args = (q.cuda(), k.cuda(), v.cuda(), glob.cuda(), w, w, 0, 0.125)
    got = dm.diagmm_banded_attention_global(*args)
    again = dm.diagmm_banded_attention_global(*args)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    rows = np.unique(np.concatenate([[17, 2500, 4999, 0, 16, 18, 4998],
                                     datagen.rng(1810).choice(n, 40, replace=False)]))
    check_global(got.cpu().reshape(n, h, d)[torch.from_numpy(rows)], q, k, v, glob.long(), w,
                 w, 0, 0.125, torch.bfloat16, "27 ranges", rows=rows)
