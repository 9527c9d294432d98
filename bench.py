#!/usr/bin/env python3
"""Benchmark of the diagonaled-matmul hot path on one MI355X.

One step = one pass of the whole path over one batch of the forward workload of the
TVM Discuss thread "Developing a faster schedule for Longformer's kernel" (post 6: b=1,
n=4096, h=12, hidden 768 so d=64, w=w_upper=256, 513 diagonals), at both dilations the
thread asks for (post 4: 0 and 3):

    for dilation in (0, 3):
        S  = diagmm_qk(Q, K)                      band [1, 4096, 12, 513] f16
        P  = diagmm_banded_softmax(S, scale 1/8)  in place
        O  = diagmm_pv(P, V)                      [1, 4096, 12, 64] f16
        dX = diagmm_pvT(P, dO)                    [1, 4096, 12, 64] f16

Inputs are seeded synthetic tensors (Q, K, V, dO ~ N(0,1)/8 in f16), resident in HBM
before the timed region; R rotating buffer sets (> 256 MB in total) keep one step's
operands out of the Infinity Cache of the previous steps.  The value is the whole
step's algorithmic HBM bytes per second (each input read once, each output written
once; pv / pvT / softmax read only in-range band slots); useful TFLOP/s (2*d per
in-range slot of qk, pv, pvT) is reported beside it.  Per-kernel times come from the
library's kernel timers: HIP events recorded at each kernel's own start and end on the
stream it runs on, for every launch of a second run of the same steps right after the
timed one (the timers lengthen the dispatch path, so the step timing runs without them).
The roofline object is for the qk kernel at dilation 0.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense f16 MFMA

B, N, H, D, W, WU = 1, 4096, 12, 64, 256, 256
DILATIONS = (0, 3)
K = W + WU + 1
SCALE = 0.125
E = 2  # bytes per f16 element
NG = 8  # global tokens of the global-token timing (positions spread over the sequence)


def in_range_per_head(n, w, wu, dil):
    s = max(dil, 1)
    return sum(min(w, i // s) + min(wu, (n - 1 - i) // s) + 1 for i in range(n))


def op_costs(dil):
    """Algorithmic bytes and useful flops of each op at one dilation."""
    cnt = in_range_per_head(N, W, WU, dil) * B * H
    dense = B * N * H * D * E
    band = B * N * H * K * E
    return {
        "qk": {"bytes": 2 * dense + band, "flops": 2 * D * cnt},
        "softmax": {"bytes": cnt * E + band, "flops": 0},
        "pv": {"bytes": cnt * E + 2 * dense, "flops": 2 * D * cnt},
        "pvT": {"bytes": cnt * E + 2 * dense, "flops": 2 * D * cnt},
        # gradient path: P and dP read on their in-range slots, the whole band written
        "softmax_bwd": {"bytes": 2 * cnt * E + band, "flops": 0},
        # the softmax with the per-key mask: the softmax's bytes and the [b, n] f32 mask
        "softmax_masked": {"bytes": cnt * E + band + B * N * 4, "flops": 0},
        # dropout: P and its float32 random numbers on the in-range slots, the band written
        "dropout": {"bytes": cnt * (E + 4) + band, "flops": 0},
        # attention in one pass: Q, K, V read and the output written; both products' flops
        "attention": {"bytes": 4 * dense, "flops": 4 * D * cnt},
        # with NG global tokens: every row also reads the global keys (counted once per
        # launch), the global rows attend every key
        "attention_global": {"bytes": 4 * dense + B * NG * 4,
                             "flops": 4 * D * (cnt + B * H * (N * NG + NG * N))},
    }


def kernel_source_hash() -> str:
    csrc = os.path.join(ROOT, "sliding_window_attention_diagmm_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM traffic per qk launch from the committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "qk_f16_n4096_dil0_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            k_, v = ln.split(":", 1)
            vals[k_.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def practical_ceiling(torch, dev, stream):
    """Same-run reference bandwidths of the box: a 256 MiB device-to-device copy (read +
    write) and a 256 MiB fill (write only), averaged over 10 launches each."""
    nbytes = 256 << 20
    a = torch.empty(nbytes // 2, dtype=torch.float16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    res = {}
    for name, fn, moved in (("copy_256MiB", lambda: b.copy_(a), 2 * nbytes),
                            ("fill_256MiB", lambda: b.fill_(2.0), nbytes)):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        res[name] = {"us": round(us, 2), "GB/s": round(moved / (us * 1e-6) / 1e9, 1)}
    del a, b
    return res


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(target_s: float = 12.0):
    """The oracle on the host cores over a bounded sample of the same step: all 12 heads
    of a set of positions, for qk, softmax, pv and pvT at both dilations."""
    import numpy as np
    import torch

    import datagen
    import oracle

    g = datagen.rng(77)
    shape = (B, N, H, D)
    q = datagen.normal(g, shape, "f16", 0.125)
    k = datagen.normal(g, shape, "f16", 0.125)
    v = datagen.normal(g, shape, "f16", 0.125)
    do = datagen.normal(g, shape, "f16", 0.125)
    probs = datagen.softmax_rows(g, (B, N, H, K), "f16")
    threads = cpu_threads()

    def run(rows):
        qr = q.reshape(N, H, D)[torch.from_numpy(rows)]
        for dil in DILATIONS:
            s = oracle.qk(qr, k, W, WU, dil, 0.0, rows=rows, threads=threads)
            p = oracle.softmax(s, W, WU, dil, SCALE, n=N, rows=rows, threads=threads)
            oracle.pv(p, v, W, WU, dil, rows=rows, threads=threads)
            oracle.pvT(probs, do, W, WU, dil, rows=rows, threads=threads)

    probe = np.arange(0, N, N // 32, dtype=np.int64)[:32]
    t0 = time.perf_counter()
    run(probe)
    t_probe = time.perf_counter() - t0
    count = int(min(N, max(32, 32 * target_s / max(t_probe, 1e-3))))
    rows = np.linspace(0, N - 1, count).astype(np.int64)
    rows = np.unique(rows)
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    total_bytes = sum(c["bytes"] for dil in DILATIONS for c in op_costs(dil).values())
    frac = len(rows) / N
    return {
        "value": round(total_bytes * frac / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(rows)} of {N} positions (all {H} heads), qk+softmax+pv+pvT at "
                   f"dilation 0 and 3, {dt:.1f} s wall on {threads} threads; bytes scaled "
                   f"by the sampled fraction of rows"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short run for hardware counters: 3 passes of each kernel (and the softmax "
                         "backward and masked softmax) at the bench workload plus a reference copy of 64 MiB "
                         "(calibrates FETCH_SIZE / "
                         "WRITE_SIZE); prints the reference size and exits")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over batch*heads with no communication, but no multi-GPU "
              "run is part of it.", file=sys.stderr)
        sys.exit(2)

    import torch

    import datagen
    import sliding_window_attention_diagmm_amd as dm

    dm.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    sets = []
    for r in range(args.sets):
        g = datagen.rng(1000 + r)
        t = {n_: datagen.normal(g, (B, N, H, D), "f16", 0.125).to(dev) for n_ in ("q", "k", "v", "do")}
        for dil in DILATIONS:
            t[f"S{dil}"] = torch.empty((B, N, H, K), dtype=torch.float16, device=dev)
            t[f"O{dil}"] = torch.empty((B, N, H, D), dtype=torch.float16, device=dev)
            t[f"X{dil}"] = torch.empty((B, N, H, D), dtype=torch.float16, device=dev)
        sets.append(t)
    torch.cuda.synchronize()

    if args.pmc_probe:
        ref_bytes = 64 << 20
        # The reference copy reads a buffer no kernel has touched (so none of it sits in
        # L2 or the Infinity Cache) after a 512 MiB fill has flushed both caches.
        dprobs = dm.diagmm_qk(sets[0]["do"], sets[0]["v"], W, WU, 0, 0.0)
        dscores = torch.empty_like(dprobs)
        key_mask = torch.ones((B, N), dtype=torch.float32, device=dev)
        key_mask[:, -N // 10:] = 0.0
        rand = torch.rand(dprobs.shape, device=dev, dtype=torch.float32)
        flush = torch.empty(256 << 20, dtype=torch.float16, device=dev)
        src = torch.empty(ref_bytes // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        flush.fill_(0.0)
        torch.cuda.synchronize()
        dst.copy_(src)                     # the reference copy kernel: reads and writes 64 MiB
        torch.cuda.synchronize()
        del flush
        for r in range(3):
            t = sets[r % len(sets)]
            for dil in DILATIONS:
                dm.diagmm_qk(t["q"], t["k"], W, WU, dil, 0.0, out=t[f"S{dil}"])
                dm.diagmm_banded_softmax(t[f"S{dil}"], W, WU, dil, SCALE, inplace=True)
                dm.diagmm_pv(t[f"S{dil}"], t["v"], W, WU, dil, out=t[f"O{dil}"])
                dm.diagmm_pvT(t[f"S{dil}"], t["do"], W, WU, dil, out=t[f"X{dil}"])
                dm.diagmm_banded_softmax_backward(t[f"S{dil}"], dprobs, W, WU, dil, SCALE,
                                                  out=dscores)
                dm.diagmm_banded_softmax(t[f"S{dil}"], W, WU, dil, SCALE, out=dscores,
                                         key_mask=key_mask)
                dm.diagmm_banded_dropout(t[f"S{dil}"], rand, W, WU, dil, 0.1, out=dscores)
                dm.diagmm_banded_attention(t["q"], t["k"], t["v"], W, WU, dil, SCALE,
                                           out=t[f"O{dil}"])
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": True, "reference_copy_bytes": ref_bytes,
                          "qk_algorithmic_bytes": op_costs(0)["qk"]["bytes"],
                          "kernel_source_hash": kernel_source_hash()}), flush=True)
        return

    ops = [(dil, op) for dil in DILATIONS for op in ("qk", "softmax", "pv", "pvT")]

    def step(t):
        for dil in DILATIONS:
            S = t[f"S{dil}"]
            for op in ("qk", "softmax", "pv", "pvT"):
                if op == "qk":
                    dm.diagmm_qk(t["q"], t["k"], W, WU, dil, 0.0, out=S)
                elif op == "softmax":
                    dm.diagmm_banded_softmax(S, W, WU, dil, SCALE, inplace=True)
                elif op == "pv":
                    dm.diagmm_pv(S, t["v"], W, WU, dil, out=t[f"O{dil}"])
                else:
                    dm.diagmm_pvT(S, t["do"], W, WU, dil, out=t[f"X{dil}"])

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Per-kernel times: the same steps again with the library's kernel timers on (HIP events
    # recorded at each kernel's own start and end on the stream it runs on, every launch).
    # The timed launches cost a few microseconds more each on the dispatch path, so they
    # are kept out of the step timing above.
    dm.diagmm_timing_begin(args.steps * len(ops))
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    dm.diagmm_timing_end()
    recs = dm.diagmm_timing_read()
    assert len(recs) == args.steps * len(ops), (len(recs), args.steps * len(ops))
    kernel_ms = {key: [] for key in ops}
    for i, (name, ms) in enumerate(recs):
        key = ops[i % len(ops)]
        assert name == key[1], (i, name, key)
        kernel_ms[key].append(ms)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_op = {}
    step_bytes = step_flops = 0
    for (dil, op) in ops:
        ms = sum(kernel_ms[(dil, op)]) / len(kernel_ms[(dil, op)])
        c = op_costs(dil)[op]
        step_bytes += c["bytes"]
        step_flops += c["flops"]
        per_op[f"{op}_dil{dil}"] = {
            "us": round(ms * 1e3, 2),
            "GB/s": round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
            "TFLOP/s": round(c["flops"] / (ms * 1e-3) / 1e12, 2),
            "kernel": dm.diagmm_plan(op, B, N, H, D, W, WU, dil, torch.float16)["kernel"],
        }
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # The banded softmax backward, the one kernel the gradient path adds (it sits between
    # dP = qk(dO, V) and the two transposed products), timed on its own over the same
    # rotating sets: P from the step above, dP = qk(dO, V) computed once per set.
    # The softmax with the per-key attention mask (the last tenth of the positions masked)
    # is timed the same way, out of place from the step's band, and so is the dropout
    # (p = 0.1, float32 random numbers drawn once per set by torch's generator).
    extra = {}
    key_mask = torch.ones((B, N), dtype=torch.float32, device=dev)
    key_mask[:, -N // 10:] = 0.0
    gen = torch.Generator(device=dev).manual_seed(5)
    for t in sets:
        t["dP"] = dm.diagmm_qk(t["do"], t["v"], W, WU, 0, 0.0)
        t["dS"] = torch.empty_like(t["dP"])
        t["rand"] = torch.rand(t["dP"].shape, generator=gen, device=dev, dtype=torch.float32)
    glob = torch.tensor([[0] + [(j * N) // NG + 7 for j in range(1, NG - 1)] + [N - 1]],
                        dtype=torch.int32, device=dev).expand(B, NG).contiguous()
    for op in ("softmax_bwd", "softmax_masked", "dropout", "attention", "attention_global"):
        for dil in DILATIONS:
            def run(t):
                if op == "softmax_bwd":
                    dm.diagmm_banded_softmax_backward(t[f"S{dil}"], t["dP"], W, WU, dil, SCALE,
                                                      out=t["dS"])
                elif op == "softmax_masked":
                    dm.diagmm_banded_softmax(t[f"S{dil}"], W, WU, dil, SCALE, out=t["dS"],
                                             key_mask=key_mask)
                elif op == "dropout":
                    dm.diagmm_banded_dropout(t[f"S{dil}"], t["rand"], W, WU, dil, 0.1,
                                             out=t["dS"])
                elif op == "attention":
                    dm.diagmm_banded_attention(t["q"], t["k"], t["v"], W, WU, dil, SCALE,
                                               out=t[f"O{dil}"])
                else:
                    dm.diagmm_banded_attention_global(t["q"], t["k"], t["v"], glob, W, WU, dil,
                                                      SCALE, out=t[f"O{dil}"])
            for i in range(args.warmup):
                run(sets[i % len(sets)])
            torch.cuda.synchronize()
            per_call = 2 if op == "attention_global" else 1   # launches per call
            dm.diagmm_timing_begin(args.steps * per_call)
            for i in range(args.steps):
                run(sets[i % len(sets)])
            torch.cuda.synchronize()
            dm.diagmm_timing_end()
            tag = "attention" if op == "attention_global" else op
            recs = [ms for name, ms in dm.diagmm_timing_read() if name == tag]
            assert len(recs) == per_call * args.steps, (len(recs), per_call, args.steps)
            ms = sum(recs) / args.steps
            c = op_costs(dil)[op]
            extra[f"{op}_dil{dil}"] = {
                "us": round(ms * 1e3, 2),
                "GB/s": round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
                "bytes": c["bytes"],
            }
            if op in ("attention", "attention_global"):
                extra[f"{op}_dil{dil}"].update({
                    "TFLOP/s": round(c["flops"] / (ms * 1e-3) / 1e12, 2),
                    "flops": c["flops"],
                })
            if op == "attention":
                three = sum(per_op[f"{o}_dil{dil}"]["us"] for o in ("qk", "softmax", "pv"))
                extra[f"{op}_dil{dil}"]["three_calls_us"] = round(three, 2)
    for t in sets:
        del t["dP"], t["dS"], t["rand"]
    ceiling = practical_ceiling(torch, dev, stream)
    qk_us = per_op["qk_dil0"]["us"]
    qk_bytes = op_costs(0)["qk"]["bytes"]
    achieved = qk_bytes / (qk_us * 1e-6) / 1e9
    traffic = load_traffic()

    line = {
        "metric": "diagmm_qk/pv TFLOP/s + HBM GB/s (% roofline), n=4096 w=256 h=12 d=64, dil 0/3",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "longformer_fwd_n4096_w256_h12_d64_dil0+dil3",
                   "b": B, "n": N, "h": H, "d": D, "w": W, "w_upper": WU,
                   "dilations": list(DILATIONS), "ops": ["qk", "softmax", "pv", "pvT"],
                   "step_bytes": step_bytes, "step_useful_flops": step_flops,
                   "rotating_sets": args.sets},
        "tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "per_op": per_op,
        "extra_ops": extra,
        "roofline": {"kernel": per_op["qk_dil0"]["kernel"], "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": qk_bytes,
                     "avg_launch_us": qk_us},
        "practical_ceiling": ceiling,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
