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


def chain_costs(b, n, h, d, w, wu, dil, e_in=E, e_out=E):
    """Algorithmic bytes and useful flops of qk / softmax / pv / pvT on one shape: every
    input read once and every output written once; the band consumers read only the
    in-range slots; qk writes the whole band (padding included)."""
    cnt = in_range_per_head(n, w, wu, dil) * b * h
    dense_in = b * n * h * d * e_in
    dense_out = b * n * h * d * e_out
    band = b * n * h * (w + wu + 1) * e_out
    return {
        "qk": {"bytes": 2 * dense_in + band, "flops": 2 * d * cnt},
        "softmax": {"bytes": cnt * e_in + band, "flops": 0},
        "pv": {"bytes": cnt * e_in + dense_in + dense_out, "flops": 2 * d * cnt},
        "pvT": {"bytes": cnt * e_in + dense_in + dense_out, "flops": 2 * d * cnt},
    }


def op_costs(dil):
    """Algorithmic bytes and useful flops of each op at one dilation of the step's shape."""
    cnt = in_range_per_head(N, W, WU, dil) * B * H
    dense = B * N * H * D * E
    band = B * N * H * K * E
    costs = chain_costs(B, N, H, D, W, WU, dil)
    costs.update({
        # gradient path: P and dP read on their in-range slots, the whole band written
        "softmax_bwd": {"bytes": 2 * cnt * E + band, "flops": 0},
        # the softmax with the per-key mask: the softmax's bytes and the [b, n] f32 mask
        "softmax_masked": {"bytes": cnt * E + band + B * N * 4, "flops": 0},
        # the plain softmax out of place (the masked call's setting, without the mask)
        "softmax_oop": {"bytes": cnt * E + band, "flops": 0},
        # dropout: P and its float32 random numbers on the in-range slots, the band written
        "dropout": {"bytes": cnt * (E + 4) + band, "flops": 0},
        # attention in one pass: Q, K, V read and the output written; both products' flops
        "attention": {"bytes": 4 * dense, "flops": 4 * D * cnt},
        # with NG global tokens: every row also reads the global keys (counted once per
        # launch), the global rows attend every key
        "attention_global": {"bytes": 4 * dense + B * NG * 4,
                             "flops": 4 * D * (cnt + B * H * (N * NG + NG * N))},
    })
    return costs


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
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")
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


class LaunchLog:
    """The binding, with one label per library kernel launch noted in launch order: the
    bench phase, the call and its dilation.  Used only to match a profiler's kernel trace
    to the bench's phases (--launch-log); the timed runs call the binding directly."""
    _TWO = ("diagmm_banded_attention_global",)       # calls that launch two kernels

    def __init__(self, mod):
        import inspect
        self._m, self._sig, self.phase, self.log = mod, inspect.signature, "", []

    def __getattr__(self, name):
        f = getattr(self._m, name)
        if not name.startswith("diagmm_") or name in ("diagmm_plan", "diagmm_abi_version") \
                or name.startswith("diagmm_timing"):
            return f
        sig = self._sig(f)

        def call(*a, **kw):
            b = sig.bind(*a, **kw)
            b.apply_defaults()
            lbl = f"{self.phase}|{name[len('diagmm_'):]}|dil{b.arguments['dilation']}"
            self.log.extend([lbl] * (2 if name in self._TWO else 1))
            return f(*a, **kw)
        return call


def lat_stats(ms_list) -> dict:
    """Mean and nearest-rank p10 / p50 / p90 of per-launch kernel times, in microseconds."""
    us = sorted(m * 1e3 for m in ms_list)
    n_ = len(us)

    def pc(q):
        return round(us[min(n_ - 1, int(q * n_))], 2)
    return {"us": round(sum(us) / n_, 2), "p10": pc(0.1), "p50": pc(0.5), "p90": pc(0.9),
            "launches": n_}


def timed_launches(dm, torch, fn, reps, tag, per_call=1, before=None):
    """Per-launch times (ms) of the library kernels named ``tag`` over ``reps`` calls of
    fn(i), from the library's kernel timers.  ``before`` runs ahead of every call, outside
    the timed kernels (a cache flush)."""
    dm.diagmm_timing_begin(reps * per_call)
    for i in range(reps):
        if before is not None:
            before()
        fn(i)
    torch.cuda.synchronize()
    dm.diagmm_timing_end()
    recs = [ms for name, ms in dm.diagmm_timing_read() if name == tag]
    assert len(recs) == reps * per_call, (tag, len(recs), reps, per_call)
    return recs


def busy_counters():
    """MFMA-busy and CU-busy percentages per kernel from the committed rocprofv3 counter
    summary, or None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "busy_counters_n4096.txt")
    if not os.path.exists(path):
        return None
    rows, src = {}, None
    for ln in open(path):
        if ln.startswith("kernel_source_hash:"):
            src = ln.split(":", 1)[1].strip()
        elif ln.startswith("busy "):
            f = ln.split()
            rows[f[1]] = {"mfma_busy_pct": float(f[2]), "valu_busy_pct": float(f[3]),
                          "cu_busy_pct": float(f[4])}
    return rows if src == kernel_source_hash() else None


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
    ap.add_argument("--launch-log", default=None,
                    help="write a JSON list with one label (phase|call|dilation) per library "
                         "kernel launch, in launch order, for matching a profiler's trace")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short run for hardware counters: a reference copy of 64 MiB (calibrates "
                         "FETCH_SIZE / WRITE_SIZE), 3 passes of every kernel at the bench workload, "
                         "2 of the causal backward pair, 1 of the long-document chain; prints the "
                         "reference size and the launch labels and exits")
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
    log = None
    if args.launch_log:
        dm = log = LaunchLog(dm)

    def phase(name):
        if log is not None:
            log.phase = name

    def write_log():
        if log is not None:
            with open(args.launch_log, "w") as fh:
                json.dump(log.log, fh)
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
        phase("probe_setup")
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
        glob = torch.tensor([[0] + [(j * N) // NG + 7 for j in range(1, NG - 1)] + [N - 1]],
                            dtype=torch.int32, device=dev).expand(B, NG).contiguous()
        phase("probe")
        for r in range(3):
            t = sets[r % len(sets)]
            for dil in DILATIONS:
                S = t[f"S{dil}"]
                calls = (
                    ("qk", lambda: dm.diagmm_qk(t["q"], t["k"], W, WU, dil, 0.0, out=S)),
                    ("softmax", lambda: dm.diagmm_banded_softmax(S, W, WU, dil, SCALE,
                                                                 inplace=True)),
                    ("pv", lambda: dm.diagmm_pv(S, t["v"], W, WU, dil, out=t[f"O{dil}"])),
                    ("pvT", lambda: dm.diagmm_pvT(S, t["do"], W, WU, dil, out=t[f"X{dil}"])),
                    ("softmax_bwd", lambda: dm.diagmm_banded_softmax_backward(
                        S, dprobs, W, WU, dil, SCALE, out=dscores)),
                    ("softmax_masked", lambda: dm.diagmm_banded_softmax(
                        S, W, WU, dil, SCALE, out=dscores, key_mask=key_mask)),
                    ("dropout", lambda: dm.diagmm_banded_dropout(S, rand, W, WU, dil, 0.1,
                                                                 out=dscores)),
                    ("attention", lambda: dm.diagmm_banded_attention(
                        t["q"], t["k"], t["v"], W, WU, dil, SCALE, out=t[f"O{dil}"])),
                )
                for op, fn in calls:
                    fn()
                dm.diagmm_banded_attention_global(t["q"], t["k"], t["v"], glob, W, WU, dil,
                                                  SCALE, out=t[f"O{dil}"])
        # the causal backward pair (bf16 -> f32, b = 12) and the long-document chain
        phase("probe_causal")
        wl3 = datagen.WORKLOADS["bwd_n4096_causal"]
        host = datagen.make(wl3, parts=("q", "v", "band"))
        q3, v3, band3 = (host[x].to(dev) for x in ("q", "v", "band"))
        del host
        out3 = torch.empty((wl3.b, wl3.n, wl3.h, wl3.d), dtype=torch.float32, device=dev)
        for r in range(2):
            dm.diagmm_pv(band3, v3, wl3.w, wl3.w_upper, 0, out_dtype=torch.float32, out=out3)
            dm.diagmm_pvT(band3, q3, wl3.w, wl3.w_upper, 0, out_dtype=torch.float32, out=out3)
        del q3, v3, band3, out3
        wl4 = datagen.WORKLOADS["long_n32768"]
        host = datagen.make(wl4, parts=("q", "k", "v"))
        q4, k4, v4 = (host[x].to(dev) for x in ("q", "k", "v"))
        del host
        S4 = torch.empty((wl4.b, wl4.n, wl4.h, wl4.K), dtype=torch.float16, device=dev)
        O4 = torch.empty((wl4.b, wl4.n, wl4.h, wl4.d), dtype=torch.float16, device=dev)
        phase("probe_long")
        dm.diagmm_qk(q4, k4, wl4.w, wl4.w_upper, 0, 0.0, out=S4)
        dm.diagmm_banded_softmax(S4, wl4.w, wl4.w_upper, 0, SCALE, inplace=True)
        dm.diagmm_pv(S4, v4, wl4.w, wl4.w_upper, 0, out=O4)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": True, "reference_copy_bytes": ref_bytes,
                          "qk_algorithmic_bytes": op_costs(0)["qk"]["bytes"],
                          "kernel_source_hash": kernel_source_hash(),
                          "labelled_launches": None if log is None else len(log.log)}),
              flush=True)
        write_log()
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

    phase("step_warmup")
    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    phase("step_timed")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Per-kernel times: the same steps again with the library's kernel timers on (HIP events
    # recorded at each kernel's own start and end on the stream it runs on, every launch).
    # The timed launches cost a few microseconds more each on the dispatch path, so they
    # are kept out of the step timing above.
    phase("step_timers")
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
        st = lat_stats(kernel_ms[(dil, op)])
        ms = st["us"] * 1e-3
        c = op_costs(dil)[op]
        step_bytes += c["bytes"]
        step_flops += c["flops"]
        per_op[f"{op}_dil{dil}"] = dict(st, **{
            "GB/s": round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
            "TFLOP/s": round(c["flops"] / (ms * 1e-3) / 1e12, 2),
            "kernel": dm.diagmm_plan(op, B, N, H, D, W, WU, dil, torch.float16)["kernel"],
        })
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
    phase("extra_setup")
    for t in sets:
        t["dP"] = dm.diagmm_qk(t["do"], t["v"], W, WU, 0, 0.0)
        t["dS"] = torch.empty_like(t["dP"])
        t["rand"] = torch.rand(t["dP"].shape, generator=gen, device=dev, dtype=torch.float32)
    glob = torch.tensor([[0] + [(j * N) // NG + 7 for j in range(1, NG - 1)] + [N - 1]],
                        dtype=torch.int32, device=dev).expand(B, NG).contiguous()
    for op in ("softmax_bwd", "softmax_masked", "softmax_oop", "dropout", "attention",
               "attention_global"):
        for dil in DILATIONS:
            def run(t):
                if op == "softmax_bwd":
                    dm.diagmm_banded_softmax_backward(t[f"S{dil}"], t["dP"], W, WU, dil, SCALE,
                                                      out=t["dS"])
                elif op == "softmax_masked":
                    dm.diagmm_banded_softmax(t[f"S{dil}"], W, WU, dil, SCALE, out=t["dS"],
                                             key_mask=key_mask)
                elif op == "softmax_oop":
                    # the plain softmax on the masked call's inputs and output, for the ratio
                    dm.diagmm_banded_softmax(t[f"S{dil}"], W, WU, dil, SCALE, out=t["dS"])
                elif op == "dropout":
                    dm.diagmm_banded_dropout(t[f"S{dil}"], t["rand"], W, WU, dil, 0.1,
                                             out=t["dS"])
                elif op == "attention":
                    dm.diagmm_banded_attention(t["q"], t["k"], t["v"], W, WU, dil, SCALE,
                                               out=t[f"O{dil}"])
                else:
                    dm.diagmm_banded_attention_global(t["q"], t["k"], t["v"], glob, W, WU, dil,
                                                      SCALE, out=t[f"O{dil}"])
            phase("extra_warmup")
            for i in range(args.warmup):
                run(sets[i % len(sets)])
            torch.cuda.synchronize()
            per_call = 2 if op == "attention_global" else 1   # launches per call
            tag = {"attention_global": "attention", "softmax_oop": "softmax"}.get(op, op)
            phase("extra")
            recs = timed_launches(dm, torch, lambda i: run(sets[i % len(sets)]), args.steps,
                                  tag, per_call)
            # per call: the global-token form's two launches (band rows, global rows) summed
            per_call_ms = [sum(recs[i:i + per_call]) for i in range(0, len(recs), per_call)]
            st = lat_stats(per_call_ms)
            ms = st["us"] * 1e-3
            c = op_costs(dil)[op]
            extra[f"{op}_dil{dil}"] = dict(st, **{
                "GB/s": round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
                "bytes": c["bytes"],
            })
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

    # Cold launches.  In the step, softmax, pv and pvT read the band qk has just written,
    # most of which is still in the 256 MB Infinity Cache: their per_op figures are
    # warm-chain figures.  Here every kernel of the step runs right after a read of
    # 512 MiB that none of them touches (outside the timed kernels), so its operands come
    # from HBM.
    flush_src = torch.ones(256 << 20, dtype=torch.float16, device=dev)

    def flush():
        torch.amax(flush_src)

    cold = {}
    phase("cold")
    t = sets[0]
    reps_cold = max(20, args.steps // 2)
    for dil in DILATIONS:
        S = t[f"S{dil}"]
        calls = (
            ("qk", lambda i: dm.diagmm_qk(t["q"], t["k"], W, WU, dil, 0.0, out=S)),
            ("softmax", lambda i: dm.diagmm_banded_softmax(S, W, WU, dil, SCALE, inplace=True)),
            ("pv", lambda i: dm.diagmm_pv(S, t["v"], W, WU, dil, out=t[f"O{dil}"])),
            ("pvT", lambda i: dm.diagmm_pvT(S, t["do"], W, WU, dil, out=t[f"X{dil}"])),
        )
        for op, fn in calls:
            st = lat_stats(timed_launches(dm, torch, fn, reps_cold, op, before=flush))
            c = op_costs(dil)[op]
            cold[f"{op}_dil{dil}"] = dict(st, **{
                "GB/s": round(c["bytes"] / (st["us"] * 1e-6) / 1e9, 1),
                "frac": round(c["bytes"] / (st["us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    del flush_src

    # The other two workloads of the pages, each on its own: the causal backward pair
    # (TVM post 4's batch of 12, w_upper = 0: pv and pvT, bf16 in, f32 out) and the
    # long-document chain (post 3's longest sequence and widest window: n = 32768,
    # 8193 diagonals, qk -> softmax -> pv in f16).  Two rotating sets for the pair (each
    # over the Infinity Cache's size), one for the chain (its band alone is 6.4 GB).
    wl3 = datagen.WORKLOADS["bwd_n4096_causal"]
    host = datagen.make(wl3, parts=("q", "v", "band"))
    c3 = []
    for r in range(2):
        c3.append({k_: v_.to(dev) for k_, v_ in host.items()})
        c3[-1]["out"] = torch.empty((wl3.b, wl3.n, wl3.h, wl3.d), dtype=torch.float32,
                                    device=dev)
    del host
    cost3 = chain_costs(wl3.b, wl3.n, wl3.h, wl3.d, wl3.w, wl3.w_upper, 0, e_in=2, e_out=4)
    for op in ("pv", "pvT"):
        fn_ = dm.diagmm_pv if op == "pv" else dm.diagmm_pvT
        dense_ = "v" if op == "pv" else "q"

        def run3(i, fn_=fn_, dense_=dense_):
            u = c3[i % 2]
            fn_(u["band"], u[dense_], wl3.w, wl3.w_upper, 0, out_dtype=torch.float32,
                out=u["out"])
        phase("causal_warmup")
        for i in range(3):
            run3(i)
        phase("causal")
        st = lat_stats(timed_launches(dm, torch, run3, args.steps, op))
        by = cost3[op]["bytes"]
        extra[f"causal_bwd_{op}"] = dict(st, **{
            "GB/s": round(by / (st["us"] * 1e-6) / 1e9, 1), "bytes": by,
            "frac": round(by / (st["us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bound_us": round(by / (HBM_PEAK_GBS * 1e3), 2),
            "kernel": dm.diagmm_plan(op, wl3.b, wl3.n, wl3.h, wl3.d, wl3.w, wl3.w_upper, 0,
                                     torch.bfloat16, torch.float32)["kernel"],
            "shape": "b=12 n=4096 h=12 d=64 w=256 w_upper=0 bf16->f32"})
    del c3

    wl4 = datagen.WORKLOADS["long_n32768"]
    host = datagen.make(wl4, parts=("q", "k", "v"))
    q4, k4, v4 = (host[x].to(dev) for x in ("q", "k", "v"))
    del host
    S4 = torch.empty((wl4.b, wl4.n, wl4.h, wl4.K), dtype=torch.float16, device=dev)
    O4 = torch.empty((wl4.b, wl4.n, wl4.h, wl4.d), dtype=torch.float16, device=dev)

    def chain4(i):
        dm.diagmm_qk(q4, k4, wl4.w, wl4.w_upper, 0, 0.0, out=S4)
        dm.diagmm_banded_softmax(S4, wl4.w, wl4.w_upper, 0, SCALE, inplace=True)
        dm.diagmm_pv(S4, v4, wl4.w, wl4.w_upper, 0, out=O4)
    phase("long_warmup")
    chain4(0)
    torch.cuda.synchronize()
    reps4 = 5
    phase("long")
    dm.diagmm_timing_begin(3 * reps4)
    for i in range(reps4):
        chain4(i)
    torch.cuda.synchronize()
    dm.diagmm_timing_end()
    recs4 = dm.diagmm_timing_read()
    assert [nm for nm, _ in recs4] == ["qk", "softmax", "pv"] * reps4, recs4
    cost4 = chain_costs(wl4.b, wl4.n, wl4.h, wl4.d, wl4.w, wl4.w_upper, 0)
    total_us = 0.0
    for j, op in enumerate(("qk", "softmax", "pv")):
        st = lat_stats([ms for _, ms in recs4[j::3]])
        by = cost4[op]["bytes"]
        total_us += st["us"]
        extra[f"long_doc_{op}"] = dict(st, **{
            "GB/s": round(by / (st["us"] * 1e-6) / 1e9, 1), "bytes": by,
            "frac": round(by / (st["us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": dm.diagmm_plan(op, wl4.b, wl4.n, wl4.h, wl4.d, wl4.w, wl4.w_upper, 0,
                                     torch.float16)["kernel"]})
    by4 = sum(cost4[op]["bytes"] for op in ("qk", "softmax", "pv"))
    extra["long_doc_chain"] = {
        "us": round(total_us, 2), "GB/s": round(by4 / (total_us * 1e-6) / 1e9, 1),
        "bytes": by4, "frac": round(by4 / (total_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "bound_us": round(by4 / (HBM_PEAK_GBS * 1e3), 2),
        "shape": "b=1 n=32768 h=12 d=64 w=w_upper=4096 f16, qk -> softmax -> pv"}
    del q4, k4, v4, S4, O4
    ceiling = practical_ceiling(torch, dev, stream)
    qk_us = per_op["qk_dil0"]["us"]
    qk_bytes = op_costs(0)["qk"]["bytes"]
    achieved = qk_bytes / (qk_us * 1e-6) / 1e9
    traffic = load_traffic()
    busy = busy_counters()

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
        "cold_ops": cold,
        "roofline": {"kernel": per_op["qk_dil0"]["kernel"], "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": qk_bytes,
                     "avg_launch_us": qk_us,
                     "mfma_busy_pct": None if busy is None else
                     busy.get("qk_dil0", {}).get("mfma_busy_pct"),
                     "cu_busy_pct": None if busy is None else
                     busy.get("qk_dil0", {}).get("cu_busy_pct")},
        "busy_counters": busy,
        "practical_ceiling": ceiling,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)
    write_log()


if __name__ == "__main__":
    main()
