#!/usr/bin/env python3
"""Throughput of the block-hybrid attention hot path on one MI355X.

One bench step is one pass of the whole hot path over one batch of synthetic
input -- the long-prompt prefill + decode workload of one hybrid layer, all
heads: 8 requests x 32 heads x d = 128 with ragged prompts of 16k-64k tokens
(bf16, N(0,1)) folded into the fp32 state by hybrid_state_prefill (chunk
256), then 16 blocks of B = 64 tokens, each denoised by 3 hybrid_attn_step
calls and a last step fused with the block's commit
(hybrid_attn_step_commit).  Inputs are generated and
resident in HBM before timing; each step's Q/K/V are distinct tensors.

Reported value: tokens/s through the hybrid layer, where a prompt token
counts once (folded into S) and an active-block token counts once per
denoising step.  The K timed steps run back to back as replays of the step's
calls captured once as a HIP graph, in one window bracketed by
synchronisations (``--eager`` times the calls launched one by one instead).
K eager steps with HIP events around every call, on the stream the kernels
run on, give each call's achieved GB/s and TFLOP/s against the MI355X peaks
(8 TB/s HBM, 2.5 PFLOP/s dense bf16); ``roofline`` reports the call with the
largest share of the time.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample
of the same workload's (request, head) units and scales it to tokens/s.
``context`` times, for comparison only, the hybrid step against the exact
full-prefix step it replaces at the concurrent-serving shapes.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager] [--no-cpu] [--no-context]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_hybrid_linear_amd as bh  # noqa: E402
from block_hybrid_linear_amd import synth  # noqa: E402
from block_hybrid_linear_amd.workloads import BLOCK_LOOP, PREFILL_DECODE, SERVING_STEP, SINGLE_STEP  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROMPT_BLOCK = 99          # seed "block" index reserved for prompt tensors


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes / flops per call (what the method must move: Q/K/V once,
# S once or twice, O once; never the prefix keys/values it replaces)
# ---------------------------------------------------------------------------

def step_cost(units, B, d, e=2):
    return units * (4 * B * d * e + d * d * 4), units * (4 * B * B * d + 2 * B * d * d)


def commit_cost(units, B, d, e=2):
    return units * (2 * B * d * e + 2 * d * d * 4), units * (2 * B * d * d)


def step_commit_cost(units, B, d, e=2):
    """Step and commit in one pass: Q/K/V and S read once, O and S written."""
    return units * (4 * B * d * e + 2 * d * d * 4), units * (4 * B * B * d + 4 * B * d * d)


def prefill_cost(token_heads, units, d, e=2):
    return token_heads * 2 * d * e + units * d * d * 4, token_heads * 2 * d * d


def exact_cost(prefix_token_heads, units, B, d, e=2):
    """Exact full-prefix step: every prefix key/value row once, plus the block's
    Q/K/V read and O written; flops of Q K^T and P V over P_r + B keys."""
    keys = prefix_token_heads + units * B
    return prefix_token_heads * 2 * d * e + units * 4 * B * d * e, 4 * B * d * keys


# ---------------------------------------------------------------------------
# Workload builders
# ---------------------------------------------------------------------------

class Job:
    """Inputs resident in HBM plus the calls of one bench step.

    A step whose distinct inputs are smaller than ROTATE_BYTES (the serving
    step: 201 MB) gets several input sets, used in turn by successive steps,
    so that its inputs come from HBM and not from the 256 MB last-level
    cache; set 0 is the seeded workload itself."""

    ROTATE_BYTES = 1 << 30

    def __init__(self, wl, dev="cuda"):
        self.wl = wl
        self.dev = dev
        n, H, d, B = wl.n_req, wl.heads, wl.d, wl.blk
        self.slots = torch.arange(n, dtype=torch.int32, device=dev)
        self.tokens = 0
        self.cost = {}           # kind -> (bytes, flops) per call
        per_set = n * H * d * d * 4 + wl.n_blocks * wl.steps_per_block * 3 * n * B * H * d * 2
        if wl.prompt_range:
            lens = synth.uniform_int(n, *wl.prompt_range, synth.seed_of(wl.index, tensor=synth.TENSOR_LEN))
            self.prompt_lens = lens
            cu = synth.cu_from_lengths(lens)
            total = int(cu[-1])
            self.pk = synth.normal((total, H, d), synth.seed_of(wl.index, PROMPT_BLOCK, 0, synth.TENSOR_K), device=dev)
            self.pv = synth.normal((total, H, d), synth.seed_of(wl.index, PROMPT_BLOCK, 0, synth.TENSOR_V), device=dev)
            self.cu = cu.to(dev)
            self.max_len = int(lens.max())
            self.ws = torch.empty(max(1, bh.hybrid_state_prefill_workspace_bytes(n, H, d, total, self.max_len,
                                                                                  wl.chunk)),
                                  dtype=torch.uint8, device=dev)
            self.tokens += total
            self.cost["prefill"] = prefill_cost(total * H, n * H, d)
            per_set += total * H * d * 2 * 2
        self.n_sets = 1 if wl.prompt_range else max(1, min(8, -(-self.ROTATE_BYTES // per_set)))
        self.sets = []
        for r in range(self.n_sets):
            st = {"state": torch.zeros(n, H, d, d, device=dev), "q": [], "k": [], "v": [],
                  "out": torch.empty(n, B, H, d, dtype=torch.bfloat16, device=dev)}
            for b in range(wl.n_blocks):
                for t in range(wl.steps_per_block):
                    s = lambda tid: synth.seed_of(wl.index, b, t, tid) + 500_000 * r  # noqa: E731
                    for name, tid in (("q", 0), ("k", 1), ("v", 2)):
                        st[name].append(synth.normal((n, B, H, d), s(tid), std=wl.std, device=dev))
            self.sets.append(st)
        self.tokens += wl.n_blocks * wl.steps_per_block * n * B
        self.cost["step"] = step_cost(n * H, B, d)
        self.cost["step_commit"] = step_commit_cost(n * H, B, d)
        self.calls = [self.prepare(None, r) for r in range(self.n_sets)]

    def prepare(self, stream, r=0):
        """The step's calls on input set r, each validated and marshalled once
        and re-enqueued with one ctypes call (as a serving loop would), on
        `stream` (None = the current stream)."""
        wl, st = self.wl, self.sets[r]
        calls = []
        if wl.prompt_range:
            calls.append(("prefill", bh.prepare_prefill(self.pk, self.pv, self.cu, st["state"], self.slots,
                                                        max_len=self.max_len, chunk=wl.chunk, workspace=self.ws,
                                                        stream=stream)))
        commits = wl.n_blocks > 1 or wl.steps_per_block > 1
        i = 0
        for b in range(wl.n_blocks):
            for t in range(wl.steps_per_block):
                args = (st["q"][i], st["k"][i], st["v"][i], st["state"], self.slots, st["out"])
                if commits and t == wl.steps_per_block - 1:
                    # the block's last step, fused with the commit of its K, V
                    calls.append(("step_commit", bh.prepare_step_commit(*args, scale=wl.scale, stream=stream)))
                else:
                    calls.append(("step", bh.prepare_step(*args, scale=wl.scale, stream=stream)))
                i += 1
        return calls

    def reset(self):
        for st in self.sets:
            st["state"].zero_()

    def run(self, step, events=None, calls=None):
        """Enqueue one step; with `events` (pre-created (kind, start, end)
        triples, one per call) each call is bracketed by its pair."""
        for c, (kind, fn) in enumerate(calls or self.calls[step % self.n_sets]):
            if events is not None:
                events[c][1].record()
                fn()
                events[c][2].record()
            else:
                fn()

    def capture(self):
        """Each input set's whole step captured once as a HIP graph (every
        kernel of every call; no allocation, copy or memset inside)."""
        graphs = []
        for r in range(self.n_sets):
            side = torch.cuda.Stream()
            calls = self.prepare(side, r)
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.run(r, calls=calls)                 # warm-up on the capture stream
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                self.run(r, calls=calls)
            torch.cuda.synchronize()
            graphs.append(g)
        return graphs


def graph_call_us(job: Job, reps: int = 3) -> dict:
    """Per-call microseconds of each kind of call as the timed region runs it:
    the kind's calls of one step (input set 0, in step order) captured as one
    HIP graph, replayed `reps` times back to back after one warm replay."""
    side = torch.cuda.Stream()
    calls = job.prepare(side, 0)
    res = {}
    for kind in dict.fromkeys(k for k, _ in calls):
        fns = [fn for k, fn in calls if k == kind]
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for fn in fns:
                fn()                                    # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for fn in fns:
                fn()
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        res[kind] = a.elapsed_time(b) * 1e3 / (reps * len(fns))
        del g
    job.reset()
    return res


def device_copy_GBps(n_bytes: int = 1 << 30, reps: int = 5) -> float:
    """Measured device copy bandwidth, the second denominator next to the 8
    TB/s spec: read + written bytes per second of a plain device-to-device
    copy of `n_bytes`, best of `reps` timed copies after one warm-up."""
    x = torch.ones(n_bytes // 4, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        y.copy_(x)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del x, y
    return 2 * n_bytes / (best * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload's units
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(job: Job, budget_s: float) -> dict:
    """The fp64 oracle on all requests x a subset of heads of the same job,
    scaled by heads: with all the host's threads, and with one thread."""
    import numpy as np

    import oracle
    wl = job.wl
    n, H = wl.n_req, wl.heads
    multi = wl.n_blocks > 1 or wl.steps_per_block > 1

    def run(h_s: int) -> float:
        """The whole job for all requests x the first h_s heads; host copies of
        the sample are made first and are not timed."""
        hs = slice(0, h_s)
        pk = job.pk[:, hs].cpu() if wl.prompt_range else None
        pv = job.pv[:, hs].cpu() if wl.prompt_range else None
        st = job.sets[0]
        qkv = [(st["q"][i][:, :, hs].cpu(), st["k"][i][:, :, hs].cpu(), st["v"][i][:, :, hs].cpu())
               for i in range(len(st["q"]))]
        t0 = time.perf_counter()
        S = np.zeros((n, h_s, wl.d, wl.d))
        if wl.prompt_range:
            S = oracle.prefill(pk, pv, job.cu.cpu())
        i = 0
        for _ in range(wl.n_blocks):
            for _ in range(wl.steps_per_block):
                oracle.step(*qkv[i], S, scale=wl.scale)
                i += 1
            if multi:
                S = oracle.commit(qkv[i - 1][1], qkv[i - 1][2], S)
        return time.perf_counter() - t0

    def timed(budget: float) -> tuple[int, float]:
        dt1 = run(1)                               # calibration on one head
        h_s = 1
        while h_s * 2 <= H and dt1 * h_s * 2 <= budget:
            h_s *= 2
        return h_s, (run(h_s) if h_s > 1 else dt1)

    def entry(h_s: int, dt: float, cores: int) -> dict:
        return {"value": round(job.tokens * (h_s / H) / dt, 1), "unit": "tokens/s", "cores": cores,
                "kind": "oracle",
                "sample": f"all {n} requests x {h_s} of {H} heads of the same job (prefill + every step and "
                          f"commit for those units), {dt:.1f} s of fp64 oracle time on {cores} thread(s), "
                          f"scaled by {H}/{h_s}",
                "seconds": round(dt, 2)}

    threads = oracle.num_threads()
    h_s, dt = timed(budget_s)
    res = entry(h_s, dt, threads)
    oracle.set_num_threads(1)
    try:
        h1, dt1 = timed(budget_s / 2)
    finally:
        oracle.set_num_threads(threads)
    res["single_core"] = entry(h1, dt1, 1)
    res["cpu_model"] = cpu_model()
    return res


# ---------------------------------------------------------------------------
# Traffic measured by rocprofv3 counters, valid only for the kernel source it
# was taken on (profiles/traffic.md holds one line per kernel)
# ---------------------------------------------------------------------------

KERNEL_SOURCES = {"step": "step_kernels.hip", "step_commit": "step_kernels.hip", "commit": "state_kernels.hip",
                  "prefill": "state_kernels.hip",
                  "exact": "exact_kernels.hip"}


def source_digest(call: str | None = None) -> str:
    """Digest of the sources that make a call's kernels (its .hip file and the
    shared device headers), or of every kernel source when call is None."""
    csrc = os.path.join(ROOT, "block_hybrid_linear_amd", "csrc")
    names = sorted(set(KERNEL_SOURCES.values())) if call is None else [KERNEL_SOURCES[call]]
    h = hashlib.sha256()
    for name in names + ["device_common.h", "kernels.h"]:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(call: str, workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    pat = re.compile(r"^\|\s*%s\s*\|\s*%s\s*\|\s*([0-9a-f]+)\s*\|\s*([0-9.eE+]+)\s*\|" % (re.escape(workload),
                                                                                    re.escape(call)))
    for line in open(path):
        m = pat.match(line)
        if m and m.group(1) == source_digest(call):
            return float(m.group(2))
    return None


# ---------------------------------------------------------------------------
# Context: the hybrid step against the exact full-prefix step it replaces, at
# the concurrent-serving shapes (64 requests x 32 heads, d = 128, B = 32,
# prefixes uniform in [1024, 16384]: S per request for the hybrid step, a
# packed bf16 KV cache of ~9 GB for the exact step)
# ---------------------------------------------------------------------------

def time_call(fn, iters: int, warm: int = 2) -> float:
    """Average ms per call from HIP events on the current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def commit_context(dev="cuda", rotate: int = 8) -> dict:
    """hybrid_state_commit alone at the block-loop shapes (32 requests x 32
    heads, d = 128, B = 32): the calls cycle through `rotate` input sets (K/V
    and S, 84 MB each: 671 MB cycled, more than twice the 256 MB last-level
    cache and the 32 MB of L2 together), captured as one HIP graph of 40
    calls and replayed."""
    W = BLOCK_LOOP
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    sets = []
    for r in range(rotate):
        k, v = (synth.normal((n, B, H, d), synth.seed_of(W.index, 0, 0, t) + 700_000 * r, std=W.std, device=dev)
                for t in (1, 2))
        sets.append((k, v, torch.zeros(n, H, d, d, device=dev)))
    side = torch.cuda.Stream()
    runs = [bh.prepare_commit(k, v, st, slots, stream=side) for k, v, st in sets]
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in runs:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(40):
            runs[i % rotate]()
    ms = time_call(g.replay, iters=5, warm=1) / 40
    byts, flops = commit_cost(n * H, B, d)
    del g
    return {"workload": W.name, "call": "hybrid_state_commit", "n_req": n, "heads": H, "head_dim": d, "block": B,
            "input_sets": rotate, "distinct_bytes": rotate * (2 * n * B * H * d * 2 + n * H * d * d * 4),
            "us": round(ms * 1e3, 2), "alg_bytes": byts, "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)}


def exact_context(dev="cuda", rotate: int = 4) -> dict:
    """The hybrid step cycles through `rotate` distinct input sets (Q/K/V and
    S, ~201 MB each) so that its inputs come from HBM rather than from the
    256 MB last-level cache; the exact step's ~9 GB cache cannot stay there."""
    W = SERVING_STEP
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    P = synth.uniform_int(n, *W.prefix_range, synth.seed_of(W.index, tensor=synth.TENSOR_LEN))
    cu = synth.cu_from_lengths(P)
    total = int(cu[-1])
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    sets = []
    for i in range(rotate):
        S = synth.normal((n, H, d, d), synth.seed_of(W.index, i, 0, synth.TENSOR_S), dtype=torch.float32,
                         device=dev)
        S.mul_(torch.sqrt(P.double() / 2).float().to(dev).view(-1, 1, 1, 1))
        q, k, v = (synth.normal((n, B, H, d), synth.seed_of(W.index, i, 0, t), device=dev) for t in range(3))
        sets.append((q, k, v, S, torch.empty_like(q)))
    kc = synth.normal((total, H, d), synth.seed_of(W.index, PROMPT_BLOCK, 0, synth.TENSOR_K), device=dev)
    vc = synth.normal((total, H, d), synth.seed_of(W.index, PROMPT_BLOCK, 0, synth.TENSOR_V), device=dev)
    hyb = [bh.prepare_step(q, k, v, S, slots, out, scale=W.scale) for q, k, v, S, out in sets]
    q, k, v, _, out = sets[0]
    exact = bh.prepare_exact_step(q, k, v, kc, vc, cu.to(dev), out, scale=W.scale, chunk=256)
    it = iter(range(1 << 30))
    t_h = time_call(lambda: hyb[next(it) % rotate](), 48)
    t_e = time_call(exact, 10)
    hb, hf = step_cost(n * H, B, d)
    eb, ef = exact_cost(total * H, n * H, B, d)
    res = {"workload": W.name, "n_req": n, "heads": H, "head_dim": d, "block": B,
           "prefix_range": list(W.prefix_range), "prefix_tokens": total,
           "hybrid_step_us": round(t_h * 1e3, 2), "hybrid_GBps": round(hb / (t_h * 1e-3) / 1e9, 1),
           "exact_step_us": round(t_e * 1e3, 2), "exact_GBps": round(eb / (t_e * 1e-3) / 1e9, 1),
           "exact_TFLOPs": round(ef / (t_e * 1e-3) / 1e12, 2), "exact_alg_bytes": eb, "hybrid_alg_bytes": hb,
           "speedup_vs_exact": round(t_e / t_h, 2),
           "traffic": {"step": measured_traffic("step", W.name), "exact": measured_traffic("exact", W.name)}}
    del kc, vc, sets, hyb, exact
    torch.cuda.empty_cache()
    return res


def norm_context(dev="cuda", rotate: int = 4) -> dict:
    """The normalised variant (one denominator for block softmax and prefix
    linear scores, z = sum phi(k) next to S) beside the plain calls: the step
    at the serving shapes (rotating input sets, as in exact_context), the step
    and fused step + commit at the prefill + decode workload's block shape,
    and its prefill against the plain prefill."""
    res = {}
    W = SERVING_STEP
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    sets = []
    for i in range(rotate):
        S = synth.normal((n, H, d, d), synth.seed_of(W.index, i, 0, synth.TENSOR_S), dtype=torch.float32, device=dev)
        z = synth.normal((n, H, d), synth.seed_of(W.index, i, 1, synth.TENSOR_S), dtype=torch.float32,
                         device=dev).abs_().mul_(1000.0)
        q, k, v = (synth.normal((n, B, H, d), synth.seed_of(W.index, i, 0, t), device=dev) for t in range(3))
        sets.append((q, k, v, S, z, torch.empty_like(q)))
    plain = [bh.prepare_step(q, k, v, S, slots, out, scale=W.scale) for q, k, v, S, z, out in sets]
    norm = [bh.prepare_step_norm(q, k, v, S, z, slots, out, scale=W.scale) for q, k, v, S, z, out in sets]
    it = iter(range(1 << 30))
    t_p = time_call(lambda: plain[next(it) % rotate](), 48)
    t_n = time_call(lambda: norm[next(it) % rotate](), 48)
    hb, _ = step_cost(n * H, B, d)
    res["serving_step"] = {"workload": W.name, "plain_us": round(t_p * 1e3, 2), "norm_us": round(t_n * 1e3, 2),
                           "norm_GBps": round((hb + n * H * d * 4) / (t_n * 1e-3) / 1e9, 1)}
    del sets, plain, norm
    W = PREFILL_DECODE
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    S = torch.zeros((n, H, d, d), dtype=torch.float32, device=dev)
    z = torch.zeros((n, H, d), dtype=torch.float32, device=dev)
    q, k, v = (synth.normal((n, B, H, d), synth.seed_of(W.index, 0, 0, t), device=dev) for t in range(3))
    out = torch.empty_like(q)
    calls = {"step": (bh.prepare_step(q, k, v, S, slots, out), bh.prepare_step_norm(q, k, v, S, z, slots, out)),
             "step_commit": (bh.prepare_step_commit(q, k, v, S, slots, out),
                             bh.prepare_step_commit_norm(q, k, v, S, z, slots, out))}
    for name, (fp, fn) in calls.items():
        res[f"decode_{name}"] = {"plain_us": round(time_call(fp, 48) * 1e3, 2),
                                 "norm_us": round(time_call(fn, 48) * 1e3, 2)}
    lens = synth.uniform_int(n, *W.prompt_range, synth.seed_of(W.index, tensor=synth.TENSOR_LEN))
    cu = synth.cu_from_lengths(lens)
    total = int(cu[-1])
    kp = synth.normal((total, H, d), synth.seed_of(W.index, PROMPT_BLOCK, 0, synth.TENSOR_K), device=dev)
    vp = synth.normal((total, H, d), synth.seed_of(W.index, PROMPT_BLOCK, 0, synth.TENSOR_V), device=dev)
    cud = cu.to(dev)
    fp = bh.prepare_prefill(kp, vp, cud, S, slots, chunk=W.chunk)
    fn = bh.prepare_prefill_norm(kp, vp, cud, S, z, slots, chunk=W.chunk)
    t_p, t_n = time_call(fp, 5), time_call(fn, 5)
    pb, _ = prefill_cost(total * H, n * H, d)
    res["prefill"] = {"workload": W.name, "plain_us": round(t_p * 1e3, 1), "norm_us": round(t_n * 1e3, 1),
                      "norm_GBps": round(pb / (t_n * 1e-3) / 1e9, 1)}
    del kp, vp
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# The other workloads, each timed as the calls it is made of
# ---------------------------------------------------------------------------

def _graph_ms(fns, side, reps: int = 3) -> float:
    """ms per replay of the calls `fns` captured (in order) as one HIP graph on
    `side`, the stream they enqueue on, after one warm replay."""
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for fn in fns:
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / reps


def _rate(byts: float, flops: float, us: float) -> dict:
    gbs = byts / (us * 1e-6) / 1e9
    tfs = flops / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "alg_bytes": int(byts), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "TFLOPs": round(tfs, 2),
            "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 5)}


def launch_floor_us(calls: int = 200) -> float:
    """us per launch of an (almost) empty kernel replayed in a HIP graph: the
    floor under every call of the step."""
    side = torch.cuda.Stream()
    return _graph_ms([lambda: torch.cuda._sleep(0)] * calls, side) * 1e3 / calls


def single_step_context(dev="cuda", calls: int = 200) -> dict:
    """The single-denoising-step workload (1 request x 16 heads, d = 64,
    B = 32; a 4096-token prefix folded into S, drawn as N(0, 4096 / 2) fp32):
    one call moves 0.52 MB, so it is launch-bound; timed as `calls` calls
    replayed in a HIP graph and launched one by one."""
    W = SINGLE_STEP
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    S = synth.normal((n, H, d, d), synth.seed_of(W.index, 0, 0, synth.TENSOR_S), dtype=torch.float32, device=dev)
    S.mul_((W.prefix_fixed / 2) ** 0.5)
    q, k, v = (synth.normal((n, B, H, d), synth.seed_of(W.index, 0, 0, t), device=dev) for t in range(3))
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    fn = bh.prepare_step(q, k, v, S, slots, out, scale=W.scale, stream=side)
    us_graph = _graph_ms([fn] * calls, side) * 1e3 / calls
    fe = bh.prepare_step(q, k, v, S, slots, out, scale=W.scale)
    us_eager = time_call(fe, calls) * 1e3
    byts, flops = step_cost(n * H, B, d)
    floor = launch_floor_us()
    return {"workload": W.name, "n_req": n, "heads": H, "head_dim": d, "block": B,
            "graph": _rate(byts, flops, us_graph), "eager": _rate(byts, flops, us_eager),
            "launch_floor_us": round(floor, 2), "hbm_floor_us": round(byts / (HBM_PEAK_GBS * 1e3), 3),
            "note": "0.52 MB per call: launch-bound (graph time minus the empty-kernel floor is the kernel's own)"}


def block_loop_context(dev="cuda") -> dict:
    """The full block loop (32 requests x 32 heads, d = 128, 32 blocks of
    B = 32, 8 denoising steps per block with Q/K/V ~ N(0, 0.5^2) drawn anew
    for every step, all 6.4 GB resident before timing): each block's 8
    hybrid_attn_step calls and then one hybrid_state_commit of its last
    step's K, V -- 288 calls -- captured as one HIP graph and replayed; the
    same loop with each block's last step fused with its commit
    (hybrid_attn_step_commit: 256 calls); and each kind of call alone."""
    W = BLOCK_LOOP
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    state = torch.zeros(n, H, d, d, device=dev)
    out = torch.empty(n, B, H, d, dtype=torch.bfloat16, device=dev)
    qkv = [[synth.normal((n, B, H, d), synth.seed_of(W.index, b, t, tid), std=W.std, device=dev)
            for tid in range(3)] for b in range(W.n_blocks) for t in range(W.steps_per_block)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    steps = [bh.prepare_step(q, k, v, state, slots, out, scale=W.scale, stream=side) for q, k, v in qkv]
    T = W.steps_per_block
    last = [qkv[b * T + T - 1] for b in range(W.n_blocks)]
    commits = [bh.prepare_commit(k, v, state, slots, stream=side) for _, k, v in last]
    fused = [bh.prepare_step_commit(q, k, v, state, slots, out, scale=W.scale, stream=side) for q, k, v in last]
    plain_loop, fused_loop = [], []
    for b in range(W.n_blocks):
        plain_loop += steps[b * T:(b + 1) * T] + [commits[b]]
        fused_loop += steps[b * T:(b + 1) * T - 1] + [fused[b]]
    sb, sf = step_cost(n * H, B, d)
    cb, cf = commit_cost(n * H, B, d)
    fb, ff = step_commit_cost(n * H, B, d)
    nb = W.n_blocks
    loop_bytes, loop_flops = nb * T * sb + nb * cb, nb * T * sf + nb * cf
    fused_bytes, fused_flops = nb * (T - 1) * sb + nb * fb, nb * (T - 1) * sf + nb * ff
    res = {"workload": W.name, "n_req": n, "heads": H, "head_dim": d, "block": B, "blocks": nb,
           "steps_per_block": T, "qkv_std": W.std, "calls": len(plain_loop)}
    state.zero_()
    ms = _graph_ms(plain_loop, side)
    tok = nb * T * n * B                      # active-block token-steps of the loop
    res["loop"] = {"ms": round(ms, 3), "alg_bytes": loop_bytes, "GBps": round(loop_bytes / (ms * 1e-3) / 1e9, 1),
                   "hbm_frac": round(loop_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "hbm_floor_ms": round(loop_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 3),
                   "token_steps_per_s": round(tok / (ms * 1e-3), 1),
                   "committed_tokens_per_s": round(nb * n * B / (ms * 1e-3), 1)}
    state.zero_()
    ms = _graph_ms(fused_loop, side)
    res["fused_loop"] = {"ms": round(ms, 3), "alg_bytes": fused_bytes,
                         "GBps": round(fused_bytes / (ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(fused_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "hbm_floor_ms": round(fused_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 3),
                         "token_steps_per_s": round(tok / (ms * 1e-3), 1)}
    state.zero_()
    res["step"] = _rate(sb, sf, _graph_ms(steps, side) * 1e3 / len(steps))
    res["commit"] = _rate(cb, cf, _graph_ms(commits, side) * 1e3 / len(commits))
    res["step_commit"] = _rate(fb, ff, _graph_ms(fused, side) * 1e3 / len(fused))
    del qkv, steps, commits, fused, plain_loop, fused_loop
    torch.cuda.empty_cache()
    return res


def cold_decode_context(dev="cuda", rotate: int = 40) -> dict:
    """The prefill + decode workload's decode calls (8 requests x 32 heads,
    d = 128, B = 64) with cold state: `rotate` sets of state and Q/K/V
    (33.5 MB each: 1.3 GB between two uses of one set, against 256 MB of
    last-level cache and 32 MB of L2), `rotate` calls per HIP graph."""
    W = PREFILL_DECODE
    n, H, d, B = W.n_req, W.heads, W.d, W.blk
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    sets = []
    for i in range(rotate):
        S = synth.normal((n, H, d, d), synth.seed_of(W.index, 50 + i, 0, synth.TENSOR_S), dtype=torch.float32,
                         device=dev)
        q, k, v = (synth.normal((n, B, H, d), synth.seed_of(W.index, 50 + i, 0, t), device=dev) for t in range(3))
        sets.append((q, k, v, S, torch.empty_like(q)))
    side = torch.cuda.Stream()
    st = [bh.prepare_step(q, k, v, S, slots, o, scale=W.scale, stream=side) for q, k, v, S, o in sets]
    sc = [bh.prepare_step_commit(q, k, v, S, slots, o, scale=W.scale, stream=side) for q, k, v, S, o in sets]
    sb, sf = step_cost(n * H, B, d)
    fb, ff = step_commit_cost(n * H, B, d)
    res = {"workload": W.name, "input_sets": rotate, "distinct_bytes": rotate * sb,
           "step": _rate(sb, sf, _graph_ms(st, side) * 1e3 / rotate),
           "step_commit": _rate(fb, ff, _graph_ms(sc, side) * 1e3 / rotate)}
    del sets, st, sc
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# Layer-stack timing: one denoising step of a 20-layer stand-in stack (random
# bf16 weights; RMSNorm, Q/K/V projections, attention, output projection,
# SwiGLU MLP per layer) with every layer's attention exact over its KV cache
# against the same stack with 6 of the 20 layers hybrid (the pages' LLaDA 2.1
# model converts 6 of its 20 attention layers).  Timing only: the pages give
# no architecture beyond the layer counts, so the widths are assumptions, and
# the exact layers share one KV cache buffer (its 9-43 GB cannot stay in any
# cache, so sharing it changes no traffic).

STACK = {"layers": 20, "hybrid_layers": 6, "n_req": 64, "heads": 32, "head_dim": 128, "block": 32,
         "mlp_inter": 11008, "prefix_ranges": [[1024, 16384], [16384, 65536]]}


def _fill_normal_(x: torch.Tensor, seed: int, chunk: int = 1 << 28) -> torch.Tensor:
    """Fills a large bf16 tensor with N(0, 1) values piece by piece (no fp32
    copy of the whole tensor)."""
    flat = x.view(-1)
    g = torch.Generator(device=x.device)
    g.manual_seed(seed)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n].copy_(torch.randn(n, generator=g, device=x.device))
    return x


class LayerStack:
    """A stand-in decoder stack for one denoising step of the active block:
    per layer RMSNorm, Q/K/V projections, attention, output projection and a
    SwiGLU MLP, with seeded random bf16 weights.  Layers in `hybrid_at` run
    hybrid_attn_step over a per-layer fp32 state (entries ~ N(0, P_r / 2)),
    the others hybrid_exact_step over a packed bf16 KV cache of the requests'
    prefixes (one cache buffer shared by the exact layers: at 9-43 GB it
    cannot stay in any cache, so sharing it changes no traffic)."""

    def __init__(self, cfg: dict, prefix_range, dev="cuda", base: int = 7_000_000):
        L, LH = cfg["layers"], cfg["hybrid_layers"]
        self.n, self.H, self.d, self.B, self.F = (cfg["n_req"], cfg["heads"], cfg["head_dim"], cfg["block"],
                                                  cfg["mlp_inter"])
        n, H, d, B, F = self.n, self.H, self.d, self.B, self.F
        self.hid = hid = H * d
        self.hybrid_at = {(2 * i + 1) * L // (2 * LH) for i in range(LH)}   # spread over the stack
        assert len(self.hybrid_at) == LH
        wsc = lambda fan_in: fan_in ** -0.5                 # noqa: E731
        self.weights = []
        for l in range(L):
            w = [synth.normal((hid, hid), base + 100 * l + t, std=wsc(hid), device=dev) for t in range(4)]  # qkvo
            w.append(synth.normal((hid, 2 * F), base + 100 * l + 4, std=wsc(hid), device=dev))            # gate|up
            w.append(synth.normal((F, hid), base + 100 * l + 5, std=wsc(F), device=dev))                  # down
            self.weights.append(w)
        self.x0 = synth.normal((n * B, hid), base + 99_000, device=dev)
        self.slots = torch.arange(n, dtype=torch.int32, device=dev)
        lo, hi = prefix_range
        P = synth.uniform_int(n, lo, hi, base + 98_000 + lo)
        cu = synth.cu_from_lengths(P)
        self.cu = cu
        self.total = total = int(cu[-1])
        self.cud = cu.to(dev)
        self.kc = _fill_normal_(torch.empty((total, H, d), dtype=torch.bfloat16, device=dev), base + 1)
        self.vc = _fill_normal_(torch.empty((total, H, d), dtype=torch.bfloat16, device=dev), base + 2)
        self.states = {l: synth.normal((n, H, d, d), base + 200 + l, dtype=torch.float32, device=dev)
                       .mul_(torch.sqrt(P.double() / 2).float().to(dev).view(-1, 1, 1, 1)) for l in self.hybrid_at}
        self.ws = torch.empty(bh.hybrid_exact_step_workspace_bytes(n, H, B, d), dtype=torch.uint8, device=dev)
        self.attn_out = torch.empty((n, B, H, d), dtype=torch.bfloat16, device=dev)

    def forward(self, hybrid: bool, attn_ms=None, capture=None):
        """One denoising step through the stack.  `attn_ms` collects (layer,
        start event, end event) around each attention call; `capture` (a
        dict) receives each layer's q, k, v and attention output."""
        n, H, d, B, F, hid = self.n, self.H, self.d, self.B, self.F, self.hid
        x = self.x0.clone()
        for l, (wq, wk, wv, wo, wgu, wd) in enumerate(self.weights):
            h = torch.nn.functional.rms_norm(x, (hid,))
            q, k, v = ((h @ w).view(n, B, H, d) for w in (wq, wk, wv))
            e0 = e1 = None
            if attn_ms is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            if hybrid and l in self.hybrid_at:
                bh.hybrid_attn_step(q, k, v, self.states[l], self.slots, out=self.attn_out)
            else:
                bh.hybrid_exact_step(q, k, v, self.kc, self.vc, self.cud, out=self.attn_out, chunk=256,
                                     workspace=self.ws)
            if attn_ms is not None:
                e1.record()
                attn_ms.append((l, e0, e1))
            if capture is not None:
                capture[l] = (q.clone(), k.clone(), v.clone(), self.attn_out.clone())
            x = x + self.attn_out.view(n * B, hid) @ wo
            h = torch.nn.functional.rms_norm(x, (hid,))
            g, u = (h @ wgu).split(F, dim=1)
            x = x + (torch.nn.functional.silu(g) * u) @ wd
        return x


def layer_stack(dev="cuda", steps: int = 3) -> dict:
    L, LH = STACK["layers"], STACK["hybrid_layers"]
    out = {"config": dict(STACK), "results": []}
    for lo, hi in STACK["prefix_ranges"]:
        stk = LayerStack(STACK, (lo, hi), dev)
        out["hybrid_layer_indices"] = sorted(stk.hybrid_at)
        res = {"prefix_range": [lo, hi], "prefix_tokens": stk.total,
               "kv_cache_GB": round(2 * stk.kc.numel() * 2 / 1e9, 2)}
        for mode in ("exact", "hybrid"):
            hyb = mode == "hybrid"
            for _ in range(2):
                stk.forward(hyb)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                stk.forward(hyb)
            b.record()
            torch.cuda.synchronize()
            step_ms = a.elapsed_time(b) / steps
            evs = []
            stk.forward(hyb, evs)
            torch.cuda.synchronize()
            att = [(l, e0.elapsed_time(e1)) for l, e0, e1 in evs]
            res[f"{mode}_step_ms"] = round(step_ms, 3)
            res[f"{mode}_attention_ms"] = round(sum(t for _, t in att), 3)
            if hyb:
                res["hybrid_layer_attention_ms"] = round(sum(t for l, t in att if l in stk.hybrid_at) / LH, 4)
            res["exact_layer_attention_ms"] = round(sum(t for l, t in att if not (hyb and l in stk.hybrid_at)) /
                                                    (L - (LH if hyb else 0)), 4)
            log(f"[stack] prefixes {lo}-{hi}: {mode} stack {step_ms:.2f} ms per step")
        res["speedup"] = round(res["exact_step_ms"] / res["hybrid_step_ms"], 3)
        out["results"].append(res)
        del stk
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------

WORKLOADS = {w.name: w for w in (PREFILL_DECODE, BLOCK_LOOP, SERVING_STEP)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=PREFILL_DECODE.name, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true",
                    help="time the eager calls instead of replays of the step captured as a HIP graph")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the hybrid-vs-exact step timing at the serving shapes")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="target seconds of oracle time")
    ap.add_argument("--stack", action="store_true",
                    help="only time the 20-layer stand-in stack, every layer exact vs 6 hybrid layers, and print "
                         "that result as the JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (5 times): the known-size kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.calibrate_copy:
        n = 1 << 28                                   # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
        x = torch.ones(n, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 5 copies of 1 GiB")
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark runs on one GPU "
              "(every (request, head) unit is independent, so the work shards across GPUs with no "
              "exchange; only the one-GPU share is measured)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    bh.load_library()
    if args.stack:
        res = layer_stack(steps=args.steps)
        print(json.dumps({"metric": "decode-step time of a 20-layer stack, exact vs 6 hybrid layers", **res}))
        return
    wl = WORKLOADS[args.workload]
    log(f"[bench] building inputs for {wl.name}")
    job = Job(wl)
    torch.cuda.synchronize()
    log(f"[bench] {len(job.calls[0])} calls per step, {job.tokens} tokens per step, {job.n_sets} input set(s); "
        f"warmup {args.warmup}")
    for w in range(args.warmup):
        job.reset()
        job.run(w)
    torch.cuda.synchronize()

    # ---- per-call timings: K eager steps back to back with HIP events around
    # every call, on the stream the kernels run on.  The events are created
    # beforehand, the garbage collector is paused, and a spin kernel is queued
    # first (50 us per call, at least 20 ms), so that the host has enqueued
    # the steps before the GPU reaches them: the intervals time the kernels,
    # not host-side gaps.
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    plan = [[(kind, ev(), ev()) for kind, _ in job.calls[s % job.n_sets]] for s in range(args.steps)]
    n_calls = sum(len(p) for p in plan)
    gc.collect()
    gc.disable()
    job.reset()
    a, b = ev(), ev()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * max(0.02, 50e-6 * n_calls)))
    a.record()
    for s in range(args.steps):
        job.run(s, plan[s])
    b.record()
    torch.cuda.synchronize()
    events = [e for p in plan for e in p]
    eager_ms = [a.elapsed_time(b) / args.steps] * args.steps
    log(f"[bench] {args.steps} eager steps: {a.elapsed_time(b):.3f} ms")
    step_ms = eager_ms
    mode = "eager"
    total_ms = sum(step_ms)
    if not args.eager:
        # the K steps back to back (input sets in turn; the state is reset
        # once, before the window), bracketed by synchronisations
        graphs = job.capture()
        for w in range(args.warmup):
            graphs[w % job.n_sets].replay()
        job.reset()
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for s in range(args.steps):
            graphs[s % job.n_sets].replay()
        b.record()
        torch.cuda.synchronize()
        total_ms = a.elapsed_time(b)
        mode = "hip_graph"
        log(f"[bench] {args.steps} graph steps: {total_ms:.3f} ms")
        del graphs
    gc.enable()
    ms_per_step = total_ms / args.steps
    eager_ms_per_step = sum(eager_ms) / args.steps

    kernels = {}
    for kind in job.cost:
        ts = [e0.elapsed_time(e1) for k, e0, e1 in events if k == kind]
        if not ts:
            continue
        avg_ms = sum(ts) / len(ts)
        byts, flops = job.cost[kind]
        gbs = byts / (avg_ms * 1e-3) / 1e9
        tfs = flops / (avg_ms * 1e-3) / 1e12
        kernels[kind] = {"calls_per_step": len(ts) // args.steps, "avg_us": round(avg_ms * 1e3, 2),
                         "alg_bytes": byts, "alg_flops": flops, "GBps": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "TFLOPs": round(tfs, 2),
                         "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 5),
                         "share_of_step": round(avg_ms * len(ts) / args.steps / eager_ms_per_step, 4)}
    # the same calls as they run in the timed region: each kind's calls of one
    # step (input set 0, step order) captured as a HIP graph and replayed back
    # to back; per call = replay time / calls
    for kind, us in graph_call_us(job, reps=3).items():
        if kind in kernels:
            byts = job.cost[kind][0]
            gbs = byts / (us * 1e-6) / 1e9
            kernels[kind].update({"graph_us": round(us, 2), "graph_GBps": round(gbs, 1),
                                  "graph_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    # the denoising calls alone: per bench step, each block's steps and fused
    # last step (one denoising step of the hybrid layer for all requests and
    # heads per call), at their in-graph per-call times
    dec_kinds = [k for k in ("step", "step_commit") if k in kernels]
    denoise = None
    if dec_kinds:
        calls = sum(kernels[k]["calls_per_step"] for k in dec_kinds)
        dec_us = sum(kernels[k]["calls_per_step"] * kernels[k]["graph_us"] for k in dec_kinds)
        tok = wl.n_blocks * wl.steps_per_block * wl.n_req * wl.blk
        denoise = {"calls_per_step": calls, "token_steps_per_step": tok, "us_per_step": round(dec_us, 2),
                   "token_steps_per_s": round(tok / (dec_us * 1e-6), 1),
                   "denoising_steps_per_s": round(calls / (dec_us * 1e-6), 1),
                   "from": "graph_us of the step and step_commit calls (state as the bench step leaves it)"}
    copy_gbs = device_copy_GBps()
    for kd in kernels.values():
        kd["of_copy"] = round(kd["GBps"] / copy_gbs, 4)
        if "graph_GBps" in kd:
            kd["graph_of_copy"] = round(kd["graph_GBps"] / copy_gbs, 4)
    dom = max(kernels, key=lambda k: kernels[k]["share_of_step"])
    kd = kernels[dom]
    traffic = measured_traffic(dom, wl.name)
    roofline = {"bound": "hbm", "achieved": kd["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kd["hbm_frac"], "traffic": traffic, "kernel": dom}

    value = job.tokens * args.steps / (total_ms * 1e-3)
    result = {
        "metric": "hybrid-attn denoising steps/s (tokens/s) + % HBM peak; commit/prefill % MFMA",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "n_req": wl.n_req, "heads": wl.heads, "head_dim": wl.d,
                   "block": wl.blk, "blocks": wl.n_blocks, "steps_per_block": wl.steps_per_block,
                   "prompt_range": list(wl.prompt_range) or None, "chunk": wl.chunk if wl.prompt_range else None,
                   "qkv_std": wl.std, "tokens_per_step": job.tokens, "input_sets": job.n_sets,
                   "parallelism": "single_gpu",
                   "source_digest": source_digest()},
        "roofline": roofline,
        "timing": {"mode": mode, "eager_ms_per_step": round(eager_ms_per_step, 4),
                   "kernels_from": "HIP events around each call of the eager steps; graph_* from each "
                                   "kind's calls of one step replayed back to back in a HIP graph"},
        "kernels": kernels,
        "denoise": denoise,
        "device_copy": {"GBps": round(copy_gbs, 1), "bytes_per_copy": 2 << 30,
                        "what": "read + written bytes per second of a 1 GiB device-to-device copy (best of 5); "
                                "the kernels' of_copy fractions use it as the denominator (streams that only "
                                "read can exceed it)"},
    }
    if not args.no_context:
        log("[bench] context: hybrid step vs exact full-prefix step at the serving shapes")
        result["context"] = exact_context()
        log("[bench] context: the normalised variant beside the plain calls")
        result["context"]["norm"] = norm_context()
        log("[bench] context: the commit alone at the block-loop shapes (cold)")
        result["context"]["commit"] = commit_context()
        if wl is PREFILL_DECODE:
            log("[bench] context: the decode calls with cold state")
            cold = cold_decode_context()
            result["context"]["cold_decode"] = cold
            if denoise is not None:
                cs, cc = cold["step"]["us"], cold["step_commit"]["us"]
                dec_us = kernels["step"]["calls_per_step"] * cs + kernels["step_commit"]["calls_per_step"] * cc
                denoise["cold"] = {"us_per_step": round(dec_us, 2),
                                   "token_steps_per_s": round(denoise["token_steps_per_step"] / (dec_us * 1e-6), 1),
                                   "denoising_steps_per_s": round(denoise["calls_per_step"] / (dec_us * 1e-6), 1)}
        log("[bench] context: the single-step workload")
        result["context"]["single_step"] = single_step_context()
        log("[bench] context: the block-loop workload end to end")
        result["context"]["block_loop"] = block_loop_context()
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(job, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
