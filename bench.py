#!/usr/bin/env python3
"""Benchmark of the quantized speculative-verify path on one MI355X (gfx950).

Timed step (the JSON line's `value`): one full greedy verify step of a Qwen3-8B-shaped W8A8
verifier at M = 8 (gamma = 7 drafts + 1): for each of 36 layers, per-token activation
quantisation then the W8A8 linear for qkv (4096->6144), o (4096->4096), gate_up
(4096->24576) and down (12288->4096), each layer with its own weights; then the W8A8 LM head
(4096->151936), the vocab argmax and the accept scan against 7 drafts.  The whole step is
captured once in a HIP graph and replayed; inputs are resident in HBM before timing starts.
`value` is the step's algorithmic weight bytes (N*K int8 + 4N scale bytes per linear) per
second, in GB/s.

Also measured in the same run and reported beside it:
  * roofline   -- the step's dominant kernel (the W8A8 weight-ring GEMM that runs the
                  36 gate_up linears and the LM head), HIP events around graph replays of
                  exactly those 37 launches; the average over all 145 GEMMs is reported too;
  * w8a8_sweep -- each Qwen3-8B linear at M in {1,4,6,8,10}: latency, weight GB/s, % of peak,
                  T_v(M)/T_v(1), rotating >= 1 GB of weight copies so the 256 MB Infinity
                  Cache cannot serve them;
  * w4a16      -- Llama-3-70B-shaped int4 g128 linears at M in {1,5} (same rotation), and a
                  full 80-layer pass (35.8 GB of distinct weights) at M = 48 and M = 1 with
                  T_v(48)/T_v(1);
  * w4a8       -- the same Llama-3-70B int4 g128 weights against per-token int8 activations:
                  per linear at M in {1,5} (GEMM alone and with its quant_act launch), and the
                  80-layer pass (quant_act + linear for each) at M = 48 and M = 1;
  * verify     -- greedy acceptance of a 48-node draft tree (Llama-3 vocabulary) and the
                  step's 8-row chain verify: latency and logits GB/s;
  * prep       -- offline weight preparation from bf16: W8 (smoothed per-channel int8) of the
                  Qwen3-8B LM head and gate_up, W4 (int4 g128) of the Llama-3-70B gate_up and
                  down: GB/s of bytes read and written;
  * sample     -- speculative sampling at T = 0.8 over the step's 8 rows of 151936 logits,
                  with a drafter's 7 rows of logits and with a point-mass drafter: latency
                  and logits GB/s;
  * cpu_baseline -- the CPU oracle on the host cores, on a time-bounded sample of the step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--only step|sweep|w4a16|w4a16lin|tree|w4a8|verify|sample|prep|calib|all]
                       [--cpu-baseline on|off] [--w4a16-ms 1,5] [--no-graph]
("w4a16lin" is the W4A16 per-linear sweep alone, at the token counts of --w4a16-ms; --no-graph
launches every timed pass eagerly, for hardware-counter profiles.)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "verify-GEMM weight GB/s (% HBM peak) and T_v(M)/T_v(1), W8A8 & W4A16"
QWEN_LAYERS = 36
QWEN_VOCAB = 151936
STEP_M = 8
ROTATE_BYTES = 1 << 30  # distinct weight bytes cycled through per timed linear
MEDIAN_REPLAYS = 21  # individually timed graph replays per sweep point (the median is reported)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "step", "sweep", "w4a16", "w4a16lin", "tree", "w4a8",
                                       "verify", "sample", "prep", "calib"],
                    default="all")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--w4a16-ms", default="1,5",
                    help="token counts of the W4A16 per-linear sweep (the first is the T_v base)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every timed pass eagerly instead of replaying a HIP graph (for "
                         "hardware-counter profiles; timings then include host launch overhead)")
    return ap.parse_args()


# ----------------------------------------------------------------------------------------
# weight bytes per linear (algorithmic): what one pass must read from HBM
# ----------------------------------------------------------------------------------------
def w8a8_bytes(N, K):
    return N * K + 4 * N


def w4a16_bytes(N, K):
    return N * K // 2 + 2 * N * (K // 128) + N * (K // 128)


class Dev:
    """Seeded synthetic device tensors with the shapes and distributions of the workloads."""

    def __init__(self, torch, seed):
        self.t = torch
        self.dev = torch.device("cuda:0")
        self.g = torch.Generator(device=self.dev)
        self.g.manual_seed(seed)

    def act(self, M, K):
        return self.t.randn(M, K, device=self.dev, generator=self.g).half()

    def w8(self, N, K):
        w = self.t.randint(-127, 128, (N, K), dtype=self.t.int8, device=self.dev, generator=self.g)
        s = self.t.empty(N, device=self.dev).uniform_(1e-3, 1e-2, generator=self.g)
        return w, s

    def w4(self, N, K):
        raw = self.t.randint(0, 256, (N, K // 2), dtype=self.t.uint8, device=self.dev, generator=self.g)
        qw = raw.view(self.t.int32)
        sc = self.t.empty(N, K // 128, device=self.dev).uniform_(1e-3, 2e-2, generator=self.g).half()
        z = self.t.randint(0, 16, (N, K // 128), dtype=self.t.uint8, device=self.dev, generator=self.g)
        return qw, sc, z


class Eager:
    """Stands in for a captured graph under --no-graph: replay() launches fn's kernels
    directly on the current stream (for hardware-counter runs, where the profiler serialises
    every launch anyway)."""

    def __init__(self, fn):
        self.fn = fn

    def replay(self):
        self.fn()


NO_GRAPH = False  # set by --no-graph


def capture(torch, fn, stream):
    """Run fn once eagerly on `stream` (allocates workspaces there), then capture it."""
    torch.cuda.synchronize()  # inputs were produced on the default stream
    with torch.cuda.stream(stream):
        fn()
    stream.synchronize()
    if NO_GRAPH:
        return Eager(fn)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    stream.synchronize()
    return g


def time_graph(torch, g, stream, reps, warmup=2):
    """Mean ms per replay, from HIP events recorded on the replay stream."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def replay_times(torch, g, stream, n, warmup=2):
    """ms of each of n replays, each bracketed by its own pair of HIP events on the replay
    stream (recorded back to back, read after one synchronisation)."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for i in range(n):
            g.replay()
            ev[i + 1].record(stream)
    ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def median_ms(torch, g, stream, n=MEDIAN_REPLAYS):
    """Median ms per replay over n >= 21 individually timed replays."""
    return statistics.median(replay_times(torch, g, stream, n))


def interleaved_median(torch, graphs, stream, reps, rounds=3):
    """Median ms per replay of each graph over `rounds` rounds of `reps` individually timed
    replays that alternate between the graphs, so that a drift of the machine during the
    measurement biases none of them."""
    samples = {key: [] for key in graphs}
    for _ in range(rounds):
        for key, g in graphs.items():
            samples[key] += replay_times(torch, g, stream, reps)
    return {key: statistics.median(v) for key, v in samples.items()}


# ----------------------------------------------------------------------------------------
# the timed step: Qwen3-8B-shaped W8A8 greedy verify at M = 8
# ----------------------------------------------------------------------------------------
def build_step(torch, ops, synth, D):
    lin = synth.QWEN3_8B_LINEARS
    M = STEP_M
    layers = []
    for _ in range(QWEN_LAYERS):
        layer = {}
        for name, (K, N) in lin.items():
            w, s = D.w8(N, K)
            layer[name] = (D.act(M, K), w, s)
        layers.append(layer)
    w_lm, s_lm = D.w8(QWEN_VOCAB, 4096)
    x_lm = D.act(M, 4096)
    dev = D.dev
    xq = {K: torch.empty(M, K, dtype=torch.int8, device=dev) for K in (4096, 12288)}
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    y = {name: torch.empty(M, N, dtype=torch.float16, device=dev) for name, (K, N) in lin.items()}
    logits = torch.empty(M, QWEN_VOCAB, dtype=torch.float16, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    na = torch.empty(1, dtype=torch.int32, device=dev)
    draft = torch.zeros(M - 1, dtype=torch.int32, device=dev)

    def step():
        for layer in layers:
            for name, (x, w, s) in layer.items():
                K = x.shape[1]
                ops.quant_act(x, out=xq[K], scale_out=sx)
                ops.linear_w8a8(xq[K], sx, w, s, out=y[name])
        ops.quant_act(x_lm, out=xq[4096], scale_out=sx)
        ops.linear_w8a8(xq[4096], sx, w_lm, s_lm, out=logits)
        ops.verify_greedy(logits, draft, argmax_out=am, n_accept_out=na)

    # Drafts follow the step's argmax: each position matches with p = 0.6 until the first miss
    # (planned accept length known in advance).  The CPU leg recomputes the LM head, its argmax
    # and the accept length with the oracle on host copies of the same inputs and reports
    # whether they agree (cpu_baseline.step_check).
    step()
    torch.cuda.synchronize()
    d, planned = synth.draft_tokens(5, am.cpu().numpy(), QWEN_VOCAB)
    draft.copy_(torch.from_numpy(d))

    # Pre-quantised activations for the GEMM-only timings: all 145 linears, and the
    # dominant group (gate_up x 36 + LM head: the N >= 16384 linears, which the library runs
    # on one kernel, the LDS-staged weight ring with two 2-wave tiles per workgroup).
    gemm_args, dom_args = [], []
    for layer in layers:
        for name, (x, w, s) in layer.items():
            q, sc = ops.quant_act(x)
            gemm_args.append((q, sc, w, s, y[name]))
            if w.shape[0] >= 16384:
                dom_args.append(gemm_args[-1])
    q, sc = ops.quant_act(x_lm)
    gemm_args.append((q, sc, w_lm, s_lm, logits))
    dom_args.append(gemm_args[-1])

    def gemms(args):
        def run():
            for q, sc, w, s, out in args:
                ops.linear_w8a8(q, sc, w, s, out=out)
        return run

    nbytes = sum(w8a8_bytes(N, K) for (K, N) in lin.values()) * QWEN_LAYERS + w8a8_bytes(QWEN_VOCAB, 4096)
    dom_bytes = sum(w8a8_bytes(w.shape[0], w.shape[1]) for (_, _, w, _, _) in dom_args)
    return (step, gemms(gemm_args), len(gemm_args), nbytes, gemms(dom_args), len(dom_args),
            dom_bytes, (am, na, planned), (x_lm, w_lm, s_lm, draft))


# ----------------------------------------------------------------------------------------
# per-linear sweeps with rotated weight copies
# ----------------------------------------------------------------------------------------
def sweep_w8a8(torch, ops, synth, D, stream, reps):
    out = {}
    Ms = [1, 4, 6, 8, 10]
    layer_us = {M: 0.0 for M in Ms}
    layer_us_q = {M: 0.0 for M in Ms}
    for name, (K, N) in synth.QWEN3_8B_LINEARS.items():
        nb = w8a8_bytes(N, K)
        copies = max(2, math.ceil(ROTATE_BYTES / nb))
        ws = [D.w8(N, K) for _ in range(copies)]
        rows = {}
        for M in Ms:
            x = D.act(M, K)
            q, sc = ops.quant_act(x)
            y = torch.empty(M, N, dtype=torch.float16, device=D.dev)
            qb = torch.empty_like(q)
            sb = torch.empty_like(sc)

            def gemm_only():
                for w, s in ws:
                    ops.linear_w8a8(q, sc, w, s, out=y)

            def with_quant():
                for w, s in ws:
                    ops.quant_act(x, out=qb, scale_out=sb)
                    ops.linear_w8a8(qb, sb, w, s, out=y)

            g1 = capture(torch, gemm_only, stream)
            t1 = median_ms(torch, g1, stream) * 1e3 / copies
            g2 = capture(torch, with_quant, stream)
            t2 = median_ms(torch, g2, stream) * 1e3 / copies
            del g1, g2
            gbs = nb / (t1 * 1e-6) / 1e9
            rows[M] = {"us": round(t1, 2), "us_with_quant": round(t2, 2), "GBps": round(gbs, 1),
                       "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
            layer_us[M] += t1
            layer_us_q[M] += t2
        for M in Ms:
            rows[M]["Tv_ratio"] = round(rows[M]["us"] / rows[1]["us"], 3)
        out[name] = {"N": N, "K": K, "weight_MB": round(nb / 1e6, 2), "copies": copies, "by_M": rows}
        del ws
        torch.cuda.empty_cache()
    out["layer"] = {M: {"us": round(layer_us[M], 2), "us_with_quant": round(layer_us_q[M], 2),
                        "Tv_ratio": round(layer_us[M] / layer_us[1], 3),
                        "Tv_ratio_with_quant": round(layer_us_q[M] / layer_us_q[1], 3)} for M in Ms}
    return out


def sweep_w4a16(torch, ops, synth, D, stream, reps, Ms=(1, 5)):
    out = {}
    for name, (K, N) in synth.LLAMA3_70B_LINEARS.items():
        nb = w4a16_bytes(N, K)
        copies = max(2, math.ceil(ROTATE_BYTES / nb))
        ws = [D.w4(N, K) for _ in range(copies)]
        rows = {}
        for M in Ms:
            x = D.act(M, K)
            y = torch.empty(M, N, dtype=torch.float16, device=D.dev)

            def run():
                for qw, sc, z in ws:
                    ops.linear_w4a16(x, qw, sc, z, out=y)

            g = capture(torch, run, stream)
            t = median_ms(torch, g, stream) * 1e3 / copies
            del g
            gbs = nb / (t * 1e-6) / 1e9
            rows[M] = {"us": round(t, 2), "GBps": round(gbs, 1), "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        for M in Ms:
            if M != Ms[0]:
                rows[M]["Tv_ratio"] = round(rows[M]["us"] / rows[Ms[0]]["us"], 3)
        out[name] = {"N": N, "K": K, "weight_MB": round(nb / 1e6, 2), "copies": copies, "by_M": rows}
        del ws
        torch.cuda.empty_cache()
    return out


def w4a16_tree_pass(torch, ops, synth, D, stream, reps):
    """80 layers x 4 linears with distinct weights (35.8 GB), M = 48 vs M = 1."""
    lin = synth.LLAMA3_70B_LINEARS
    layers = [{name: D.w4(N, K) for name, (K, N) in lin.items()} for _ in range(synth.LLAMA3_70B_LAYERS)]
    nb = sum(w4a16_bytes(N, K) for (K, N) in lin.values()) * synth.LLAMA3_70B_LAYERS
    res = {"layers": synth.LLAMA3_70B_LAYERS, "weight_GB": round(nb / 1e9, 3)}
    graphs = {}
    for M in (1, 48):
        xs = {K: D.act(M, K) for (K, N) in lin.values()}
        ys = {name: torch.empty(M, N, dtype=torch.float16, device=D.dev) for name, (K, N) in lin.items()}

        def run(xs=xs, ys=ys):
            for layer in layers:
                for name, (qw, sc, z) in layer.items():
                    ops.linear_w4a16(xs[qw.shape[1] * 8], qw, sc, z, out=ys[name])

        graphs[M] = capture(torch, run, stream)
    times = interleaved_median(torch, graphs, stream, reps)
    for M, t in times.items():
        res[f"M{M}"] = {"ms": round(t, 4), "GBps": round(nb / (t * 1e-3) / 1e9, 1),
                        "pct_peak": round(100 * nb / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
    res["Tv48_over_Tv1"] = round(res["M48"]["ms"] / res["M1"]["ms"], 3)
    del graphs, layers
    torch.cuda.empty_cache()
    return res


def sweep_w4a8(torch, ops, synth, D, stream, reps):
    """W4A8 per Llama-3-70B linear at M in {1, 5}: the GEMM alone and with its quant_act."""
    out = {}
    for name, (K, N) in synth.LLAMA3_70B_LINEARS.items():
        nb = w4a16_bytes(N, K)
        copies = max(2, math.ceil(ROTATE_BYTES / nb))
        ws = [D.w4(N, K) for _ in range(copies)]
        rows = {}
        for M in (1, 5):
            x = D.act(M, K)
            xq, sx = ops.quant_act(x)
            y = torch.empty(M, N, dtype=torch.float16, device=D.dev)

            def gemm():
                for qw, sc, z in ws:
                    ops.linear_w4a8(xq, sx, qw, sc, z, out=y)

            def with_quant():
                for qw, sc, z in ws:
                    ops.quant_act(x, out=xq, scale_out=sx)
                    ops.linear_w4a8(xq, sx, qw, sc, z, out=y)

            g = capture(torch, gemm, stream)
            t = median_ms(torch, g, stream) * 1e3 / copies
            del g
            g = capture(torch, with_quant, stream)
            tq = median_ms(torch, g, stream) * 1e3 / copies
            del g
            gbs = nb / (t * 1e-6) / 1e9
            rows[M] = {"us": round(t, 2), "us_with_quant": round(tq, 2), "GBps": round(gbs, 1),
                       "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        rows[5]["Tv_ratio"] = round(rows[5]["us"] / rows[1]["us"], 3)
        out[name] = {"N": N, "K": K, "weight_MB": round(nb / 1e6, 2), "copies": copies, "by_M": rows}
        del ws
        torch.cuda.empty_cache()
    return out


def w4a8_tree_pass(torch, ops, synth, D, stream, reps):
    """80 layers x 4 linears with distinct weights (35.8 GB), each linear's input quantised
    by quant_act first; M = 48 vs M = 1."""
    lin = synth.LLAMA3_70B_LINEARS
    layers = [{name: D.w4(N, K) for name, (K, N) in lin.items()} for _ in range(synth.LLAMA3_70B_LAYERS)]
    nb = sum(w4a16_bytes(N, K) for (K, N) in lin.values()) * synth.LLAMA3_70B_LAYERS
    res = {"layers": synth.LLAMA3_70B_LAYERS, "weight_GB": round(nb / 1e9, 3)}
    graphs = {}
    for M in (1, 48):
        xs = {K: D.act(M, K) for (K, N) in lin.values()}
        qs = {K: ops.quant_act(x) for K, x in xs.items()}
        ys = {name: torch.empty(M, N, dtype=torch.float16, device=D.dev) for name, (K, N) in lin.items()}

        def run(xs=xs, qs=qs, ys=ys):
            for layer in layers:
                for name, (qw, sc, z) in layer.items():
                    K = qw.shape[1] * 8
                    xq, sx = qs[K]
                    ops.quant_act(xs[K], out=xq, scale_out=sx)
                    ops.linear_w4a8(xq, sx, qw, sc, z, out=ys[name])

        graphs[M] = capture(torch, run, stream)
    times = interleaved_median(torch, graphs, stream, reps)
    for M, t in times.items():
        res[f"M{M}"] = {"ms": round(t, 4), "GBps": round(nb / (t * 1e-3) / 1e9, 1),
                        "pct_peak": round(100 * nb / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
    res["Tv48_over_Tv1"] = round(res["M48"]["ms"] / res["M1"]["ms"], 3)
    del graphs, layers
    torch.cuda.empty_cache()
    return res


def tree_verify(torch, ops, synth, D, stream, reps):
    """Greedy acceptance of a 48-node draft tree over Llama-3 vocabulary rows (128256), and
    the chain verify of the timed step (8 rows of 151936) beside it: latency and logits
    GB/s, rotating >= 256 MB of logits copies."""
    import numpy as np

    out = {}
    for name, (M, V, tree) in {"tree_M48_V128256": (48, 128256, True),
                               "chain_M8_V151936": (8, 151936, False)}.items():
        nb = M * V * 2
        copies = max(2, math.ceil((256 << 20) / nb))
        logits = [D.act(M, V) for _ in range(copies)]
        a0 = logits[0].argmax(dim=1).to(torch.int32).cpu().numpy()
        if tree:
            parent, tokens, _ = synth.draft_tree(7, M, V, 0.8, argmax=a0)
            tok = torch.from_numpy(tokens).to(D.dev)
            par = torch.from_numpy(parent).to(D.dev)
            am = torch.empty(M, dtype=torch.int32, device=D.dev)
            path = torch.empty(M, dtype=torch.int32, device=D.dev)
            acc = torch.empty(2, dtype=torch.int32, device=D.dev)

            def run():
                for lg in logits:
                    ops.verify_tree(lg, tok, par, argmax_out=am, path_out=path, accept_out=acc)
        else:
            draft = torch.from_numpy(a0[:M - 1].copy()).to(D.dev)
            am = torch.empty(M, dtype=torch.int32, device=D.dev)
            na = torch.empty(1, dtype=torch.int32, device=D.dev)

            def run():
                for lg in logits:
                    ops.verify_greedy(lg, draft, argmax_out=am, n_accept_out=na)

        g = capture(torch, run, stream)
        t = median_ms(torch, g, stream) * 1e3 / copies
        del g
        out[name] = {"M": M, "V": V, "us": round(t, 2), "logits_MB": round(nb / 1e6, 2),
                     "GBps": round(nb / (t * 1e-6) / 1e9, 1)}
        del logits
        torch.cuda.empty_cache()
    return out


def weight_prep(torch, ops, D, stream, reps):
    """Offline preparation passes; bytes = bf16 read + codes and scales written."""
    out = {}
    cases = [("w8_lm_head_151936x4096", 151936, 4096, 8), ("w8_gate_up_24576x4096", 24576, 4096, 8),
             ("w4_gate_up_57344x8192", 57344, 8192, 4), ("w4_down_8192x28672", 8192, 28672, 4)]
    for name, N, K, bits in cases:
        w = torch.randn(N, K, device=D.dev, generator=D.g).mul_(0.02).to(torch.bfloat16)
        if bits == 8:
            inv = torch.empty(K, device=D.dev).uniform_(0.5, 2.0, generator=D.g)
            nb = 2 * N * K + N * K + 4 * N + 4 * K
            wq = ws = None

            def run():
                ops.prepare_w8(w, inv)
        else:
            nb = 2 * N * K + N * K // 2 + 3 * N * (K // 128)

            def run():
                ops.prepare_w4(w)
        g = capture(torch, run, stream)
        t = median_ms(torch, g, stream)
        del g
        out[name] = {"N": N, "K": K, "us": round(t * 1e3, 2), "MB": round(nb / 1e6, 1),
                     "GBps": round(nb / (t * 1e-3) / 1e9, 1),
                     "pct_peak": round(100 * nb / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
        del w
        torch.cuda.empty_cache()
    return out


def sample_verify(torch, ops, D, stream, reps):
    """Speculative sampling (T = 0.8) over 8 target rows of 151936 logits, with the drafter's
    7 rows of logits and with a point-mass drafter, rotating >= 256 MB of logits copies.
    Algorithmic bytes per call: every target (and drafter) row once for the statistics, plus
    the emitting row (and its drafter row) once more for the draw."""
    out = {}
    M, V, T = 8, 151936, 0.8
    u = torch.rand(M, dtype=torch.float64, device=D.dev, generator=D.g)
    draft = torch.randint(0, V, (M - 1,), dtype=torch.int32, device=D.dev, generator=D.g)
    res = torch.empty(2, dtype=torch.int32, device=D.dev)
    for name, with_dl in (("drafter_logits_M8_V151936", True), ("point_mass_M8_V151936", False)):
        rows = M + (M - 1 if with_dl else 0)
        nb = rows * V * 2 + (2 if with_dl else 1) * V * 2
        copies = max(2, math.ceil((256 << 20) / (rows * V * 2)))
        tgt = [D.act(M, V) for _ in range(copies)]
        dls = [D.act(M - 1, V) for _ in range(copies)] if with_dl else [None] * copies

        def run():
            for lg, dl in zip(tgt, dls):
                ops.verify_sample(lg, draft, u, T, draft_logits=dl, result_out=res)

        g = capture(torch, run, stream)
        t = median_ms(torch, g, stream) * 1e3 / copies
        del g
        out[name] = {"M": M, "V": V, "T": T, "us": round(t, 2), "logits_MB": round(nb / 1e6, 2),
                     "GBps": round(nb / (t * 1e-6) / 1e9, 1), "launches": 2}
        del tgt, dls
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------------------
# CPU baseline: the oracle on the host, on a time-bounded sample of the step
# ----------------------------------------------------------------------------------------
def cpu_baseline(budget_s):
    import numpy as np

    import oracle
    from quantized_weight_verification_amd import synth

    lin = synth.QWEN3_8B_LINEARS
    M = STEP_M
    # One layer's weights serve every sampled layer: the oracle's work does not depend on
    # the values, and the weights (193 MB) stream from DRAM either way.
    layer = {name: (synth.activations(5, 0, synth.LINEAR_IDS[name], M, K),) + synth.w8a8_weights(5, 0, synth.LINEAR_IDS[name], N, K)
             for name, (K, N) in lin.items()}
    x_lm = synth.activations(5, 0, synth.LINEAR_IDS["lm_head"], M, 4096)
    w_lm, s_lm = synth.w8a8_weights(5, 0, synth.LINEAR_IDS["lm_head"], QWEN_VOCAB, 4096)
    nbytes = 0
    n_layers = 0
    n_steps = 0
    t0 = time.perf_counter()
    # Whole steps (36 layers + LM head + argmax + accept) until about 10 s of work have run
    # (at least one step, at most the budget): a bounded sample of the timed workload.
    min_s = min(10.0, budget_s)
    while n_steps == 0 or time.perf_counter() - t0 < min_s:
        for _ in range(QWEN_LAYERS):
            for name, (x, w, s) in layer.items():
                q, sc = oracle.quant_act(x)
                oracle.linear_w8a8(q, sc, w, s)
                nbytes += w8a8_bytes(*w.shape)
            n_layers += 1
            if time.perf_counter() - t0 > budget_s:
                break
        q, sc = oracle.quant_act(x_lm)
        logits, _ = oracle.linear_w8a8(q, sc, w_lm, s_lm)
        am = oracle.argmax(logits)
        draft, _ = synth.draft_tokens(5, am, QWEN_VOCAB)
        oracle.accept(draft, am)
        nbytes += w8a8_bytes(QWEN_VOCAB, 4096)
        n_steps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    # The tiny W8A8 verify linear (M = 4, K = 256, N = 512) on one host thread.
    x1 = synth.activations(1, 0, 0, 4, 256)
    w1, s1 = synth.w8a8_weights(1, 0, 0, 512, 256)
    oracle.set_num_threads(1)
    try:
        reps, t1 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t1 < 0.5:
            q, sc = oracle.quant_act(x1)
            oracle.linear_w8a8(q, sc, w1, s1)
            reps += 1
        tiny_us = (time.perf_counter() - t1) / reps * 1e6
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores,
            "cpu_model": cpu_model(),
            "tiny_w8a8_M4_K256_N512_one_thread_us": round(tiny_us, 1),
            "kind": "oracle",
            "sample": f"{n_steps} verify step(s) at M={M}: {n_layers} layers (quant_act + 4 W8A8 "
                      f"linears each) and {n_steps} x (LM head 4096->151936 + argmax + accept); "
                      f"{dt:.1f} s",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


def read_ceiling(torch, ops, B, stream):
    """The practical bandwidth ceiling of a kernel that only reads: the library's read probe
    (qv_test_read_stream) over a 2 GiB buffer, in the weight-tile pattern of the GEMMs (rows of
    4096 bytes, 64 bytes from each of 16 rows per load) and as one linear run, plain and
    non-temporal loads; median of 21 individually timed replays each.  The best is the
    ceiling beside the 8.0 TB/s peak."""
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(5)
    cases = {"tiles_4096B_rows": (B.QV_READ_TILES, 4096, False, 4096),
             "tiles_4096B_rows_nt": (B.QV_READ_TILES, 4096, True, 4096),
             "linear": (B.QV_READ_LINEAR, 0, False, 8192),
             "linear_nt": (B.QV_READ_LINEAR, 0, True, 8192)}
    res = {}
    for name, (pattern, rb, nt, blocks) in cases.items():
        sink = torch.empty(blocks, 4, dtype=torch.int32, device="cuda:0")
        g = capture(torch, lambda: ops.read_stream(buf, pattern, rb, nt, blocks, sink), stream)
        res[name] = round(nbytes / (median_ms(torch, g, stream) * 1e-3) / 1e9, 1)
        del g
    del buf
    torch.cuda.empty_cache()
    return max(res.values()), res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def step_oracle_check(x_lm, w_lm, s_lm, draft, am, n_accept):
    """The oracle on the timed step's LM-head inputs (host copies): its argmax over the 8 rows
    of logits and its accept length for the step's drafts, against the step's own results.
    The drafts were built from the step's argmax; equal argmaxes make them drafts of the
    oracle's argmax as well."""
    import oracle

    q, sc = oracle.quant_act(x_lm)
    logits, _ = oracle.linear_w8a8(q, sc, w_lm, s_lm)
    am_ref = oracle.argmax(logits)
    n_ref = int(oracle.accept(draft, am_ref))
    return {"lm_head_argmax_matches_oracle": bool((am_ref == am).all()),
            "n_accept_oracle": n_ref, "n_accept_step": int(n_accept),
            "n_accept_matches_oracle": n_ref == int(n_accept)}


def traffic_from_profile():
    """HBM bytes per launch of the W8A8 GEMM from the committed counter summary, or None if
    the kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "w8a8_ring_gate_up_lm_head_counters.md")
    src = os.path.join(ROOT, "quantized_weight_verification_amd", "csrc", "w8a8.hip")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_val:
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_sha.group(1):
        return None
    return float(m_val.group(1))


def main():
    args = parse()
    global NO_GRAPH
    NO_GRAPH = args.no_graph
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the verify "
              "path has no multi-GPU mode)", file=sys.stderr)
        return 2
    import torch

    from quantized_weight_verification_amd import _binding, ops, synth

    _binding.lib()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    D = Dev(torch, 1234)
    result = {}

    if args.only == "calib":
        # A plain device copy of exactly 512 MiB, three times: the reference against which
        # the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of the kernels are scaled.
        src = torch.empty(1 << 29, dtype=torch.uint8, device=D.dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": 1 << 29, "copies": 3}), flush=True)
        return 0

    copy_gbps = None
    if args.only in ("all", "step"):
        # The practical bandwidth ceiling beside the 8.0 TB/s peak: a plain device copy of
        # 1 GiB (bytes read + written per second), timed like the kernels.
        src = torch.empty(1 << 30, dtype=torch.uint8, device=D.dev)
        src.fill_(3)
        dst = torch.empty_like(src)
        g_copy = capture(torch, lambda: dst.copy_(src), stream)
        t_copy = time_graph(torch, g_copy, stream, 10)
        copy_gbps = round(2 * (1 << 30) / (t_copy * 1e-3) / 1e9, 1)
        del g_copy, src, dst
        torch.cuda.empty_cache()
        log(f"[bench] device copy: {copy_gbps} GB/s")
        read_gbps, read_cases = read_ceiling(torch, ops, _binding, stream)
        log(f"[bench] read-only ceiling: {read_gbps} GB/s {read_cases}")
        log("[bench] building the Qwen3-8B W8A8 verify step (36 layers + LM head, M=8)")
        (step, gemms, n_gemm, step_bytes, dom, n_dom, dom_bytes,
         (am, na, planned), lm_inputs) = build_step(torch, ops, synth, D)
        g_step = capture(torch, step, stream)
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                g_step.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                g_step.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_event = e0.elapsed_time(e1) / args.steps
        ms_step = wall * 1e3 / args.steps
        n_acc = int(na.item())
        if n_acc != planned:
            raise RuntimeError(f"graph replay accepted {n_acc} drafts, planned {planned}")
        if args.cpu_baseline == "on":
            # Host copies of the LM head's inputs and the step's results, for the oracle check
            # in the CPU leg.
            step_host = tuple(t.cpu().numpy() for t in lm_inputs) + (am.cpu().numpy(), n_acc)
        log(f"[bench] step: {ms_step:.4f} ms wall, {ms_event:.4f} ms events, n_accept {n_acc}")
        reps = max(5, args.steps)
        g_all = capture(torch, gemms, stream)
        all_ms = time_graph(torch, g_all, stream, reps)
        del g_all
        g_dom = capture(torch, dom, stream)
        dom_ms = time_graph(torch, g_dom, stream, reps)
        del g_dom
        avg_launch_s = dom_ms * 1e-3 / n_dom
        per_launch_bytes = dom_bytes / n_dom
        achieved = per_launch_bytes / avg_launch_s / 1e9
        result.update({
            "metric": METRIC,
            "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "int8",
            "data": "synthetic",
            "config": {"workload": "Qwen3-8B-shaped W8A8 greedy verify step: 36 layers x "
                                   "(quant_act + qkv/o/gate_up/down W8A8 linears) + W8A8 LM head "
                                   "4096->151936 + argmax + accept scan",
                       "M": STEP_M, "gamma": STEP_M - 1, "layers": QWEN_LAYERS, "vocab": QWEN_VOCAB,
                       "weight_bytes_per_step": step_bytes,
                       "pct_hbm_peak": round(100 * step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                       "ms_per_step_events": round(ms_event, 4), "n_accept": n_acc,
                       "launch": ("eager launches (--no-graph)" if NO_GRAPH else
                                  "one HIP graph per step (290 kernels)")},
            "roofline": {"bound": "hbm",
                         "kernel": "w8a8_ring_kernel<1, 2, 2, 8> (int8 MFMA weight stream; the "
                                   "step's gate_up x 36 + LM head launches)",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_from_profile(),
                         "measured_copy_GBps": copy_gbps,
                         "measured_read_GBps": read_gbps,
                         "measured_read_cases_GBps": read_cases,
                         "frac_of_measured_read": round(achieved / read_gbps, 4),
                         "launches": n_dom, "avg_launch_us": round(avg_launch_s * 1e6, 3),
                         "bytes_per_launch": round(per_launch_bytes, 1),
                         "all_w8a8_launches": {"launches": n_gemm,
                                               "avg_launch_us": round(all_ms * 1e3 / n_gemm, 3),
                                               "GBps": round(step_bytes / (all_ms * 1e-3) / 1e9, 1)}},
        })
        del g_step, step, gemms, dom
        torch.cuda.empty_cache()

    if args.only in ("all", "sweep"):
        log("[bench] W8A8 per-linear sweep (Qwen3-8B, M in 1,4,6,8,10)")
        result["w8a8_sweep"] = sweep_w8a8(torch, ops, synth, D, stream, reps=10)
    if args.only in ("all", "w4a16", "w4a16lin"):
        ms = tuple(int(m) for m in args.w4a16_ms.split(","))
        log(f"[bench] W4A16 per-linear sweep (Llama-3-70B, M in {args.w4a16_ms})")
        result.setdefault("w4a16", {})["linears"] = sweep_w4a16(torch, ops, synth, D, stream,
                                                                reps=10, Ms=ms)
    if args.only in ("all", "w4a16", "tree"):
        log("[bench] W4A16 80-layer pass, M = 48 vs M = 1")
        result.setdefault("w4a16", {})["tree_pass"] = w4a16_tree_pass(torch, ops, synth, D, stream, reps=7)

    if args.only in ("all", "w4a8"):
        log("[bench] W4A8 per-linear sweep (Llama-3-70B, M in 1,5)")
        result.setdefault("w4a8", {})["linears"] = sweep_w4a8(torch, ops, synth, D, stream, reps=10)
        log("[bench] W4A8 80-layer pass, M = 48 vs M = 1")
        result.setdefault("w4a8", {})["tree_pass"] = w4a8_tree_pass(torch, ops, synth, D, stream, reps=7)

    if args.only in ("all", "verify"):
        log("[bench] greedy verification: 48-node draft tree and the step's 8-row chain")
        result["verify"] = tree_verify(torch, ops, synth, D, stream, reps=10)
    if args.only in ("all", "prep"):
        log("[bench] offline weight preparation (W8 Qwen3-8B, W4 Llama-3-70B)")
        result["prep"] = weight_prep(torch, ops, D, stream, reps=5)
    if args.only in ("all", "sample"):
        log("[bench] speculative sampling at T = 0.8 over the step's 8 rows")
        result["sample"] = sample_verify(torch, ops, D, stream, reps=10)

    if args.cpu_baseline == "on" and args.only in ("all", "step"):
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(args.cpu_budget)
        x_h, w_h, s_h, d_h, am_h, n_h = step_host
        result["cpu_baseline"]["step_check"] = step_oracle_check(x_h, w_h, s_h, d_h, am_h, n_h)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
