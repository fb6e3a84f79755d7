"""Parity at the workloads' full sizes, through the same C-ABI calls and
kernels the benchmark times.

Where the fp64 oracle finishes in seconds (single step, serving step) the
whole output of the call is compared; for the block loop and the prefill +
decode workload the GPU runs the full job and sampled (request, head) units
are recomputed by the oracle from the identical inputs, at every step for
the block loop, and the tolerance rule is applied over the sampled outputs.
Large inputs are drawn with the seeded device generator and copied back for
the sampled units (the oracle never sees GPU-computed values).
"""
import numpy as np
import pytest
import torch

import block_hybrid_linear_amd as bh
import oracle
from block_hybrid_linear_amd import synth
from block_hybrid_linear_amd.workloads import BLOCK_LOOP, PREFILL_DECODE, SERVING_STEP, SINGLE_STEP
from parity import assert_parity, state_from_oracle, state_to_oracle, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


def test_single_step_full():
    """1 request x 16 heads, d = 64, B = 32; S = oracle prefill of 4096 seeded
    tokens, rounded to fp32 and given to both sides."""
    W = SINGLE_STEP
    pk = synth.normal((W.prefix_fixed, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_K))
    pv = synth.normal((W.prefix_fixed, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_V))
    S = oracle.prefill(pk, pv, [0, W.prefix_fixed]).astype(np.float32).astype(np.float64)
    state = state_from_oracle(S)
    q, k, v = (synth.normal((1, W.blk, W.heads, W.d), synth.seed_of(W.index, 0, 0, t)).to(DEV) for t in range(3))
    slots = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = bh.hybrid_attn_step(q, k, v, state, slots, scale=W.scale)
    out0 = bh.hybrid_attn_step(q, k, v, torch.zeros_like(state), slots, scale=W.scale)
    torch.cuda.synchronize()
    e = assert_parity(out, oracle.step(q, k, v, S, scale=W.scale), torch.bfloat16, "single step")
    e0 = assert_parity(out0, oracle.step(q, k, v, 0 * S, scale=W.scale), torch.bfloat16, "single step, S = 0")
    log(f"single step: rel err {e:.2e}, softmax part {e0:.2e}")


def test_serving_step_full():
    """64 requests x 32 heads, d = 128, B = 32, per-request fp32 S with entries
    ~ N(0, P_r / 2) for prefixes P_r uniform in [1024, 16384]; whole output
    compared, and the two parts isolated."""
    W = SERVING_STEP
    P = synth.uniform_int(W.n_req, *W.prefix_range, synth.seed_of(W.index, tensor=synth.TENSOR_LEN))
    S = synth.normal((W.n_req, W.heads, W.d, W.d), synth.seed_of(W.index, tensor=synth.TENSOR_S),
                     dtype=torch.float32, device=DEV)
    S.mul_(torch.sqrt(P.double() / 2).float().to(DEV).view(-1, 1, 1, 1))
    q, k, v = (synth.normal((W.n_req, W.blk, W.heads, W.d), synth.seed_of(W.index, 0, 0, t), device=DEV)
               for t in range(3))
    slots = torch.arange(W.n_req, dtype=torch.int32, device=DEV)
    out = bh.hybrid_attn_step(q, k, v, S, slots, scale=W.scale)
    out_s = bh.hybrid_attn_step(q, k, v, torch.zeros_like(S), slots, scale=W.scale)
    out_l = bh.hybrid_attn_step(q, k, torch.zeros_like(v), S, slots, scale=W.scale)
    torch.cuda.synchronize()
    S64 = state_to_oracle(S)
    e = assert_parity(out, oracle.step(q, k, v, S64, scale=W.scale), torch.bfloat16, "serving step")
    es = assert_parity(out_s, oracle.step(q, k, v, 0 * S64, scale=W.scale), torch.bfloat16, "softmax part")
    el = assert_parity(out_l, oracle.step(q, k, np.zeros(v.shape), S64, scale=W.scale), torch.bfloat16,
                       "linear part")
    log(f"serving step: rel err {e:.2e} (softmax part {es:.2e}, linear part {el:.2e})")


def test_serving_exact_step_sampled():
    """The exact full-prefix step at the serving shapes (64 requests x 32 heads,
    d = 128, B = 32, prefixes uniform in [1024, 16384] held as a packed bf16
    KV cache of ~9 GB); 6 sampled units against the oracle's softmax over
    [prefix; block]."""
    W = SERVING_STEP
    P = synth.uniform_int(W.n_req, *W.prefix_range, synth.seed_of(W.index, tensor=synth.TENSOR_LEN))
    cu = synth.cu_from_lengths(P)
    total = int(cu[-1])
    kc = synth.normal((total, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_K), device=DEV)
    vc = synth.normal((total, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_V), device=DEV)
    q, k, v = (synth.normal((W.n_req, W.blk, W.heads, W.d), synth.seed_of(W.index, 0, 0, t), device=DEV)
               for t in range(3))
    out = bh.hybrid_exact_step(q, k, v, kc, vc, cu.to(DEV), scale=W.scale)
    units = _units(W.n_req, W.heads, 6, 303)
    log(f"exact step: {total} cache rows; sampled units {units}")
    got, ref = [], []
    for r, h in units:
        s0, s1 = int(cu[r]), int(cu[r + 1])
        sl = lambda t: t[r:r + 1, :, h:h + 1].cpu()  # noqa: E731
        ref.append(oracle.exact_step(sl(q), sl(k), sl(v), kc[s0:s1, h:h + 1].cpu(), vc[s0:s1, h:h + 1].cpu(),
                                     [0, s1 - s0], scale=W.scale))
        got.append(sl(out))
    torch.cuda.synchronize()
    e = assert_parity(np.stack([to64(g) for g in got]), np.stack(ref), torch.bfloat16, "exact step")
    log(f"serving exact step: rel err {e:.2e}")


def _units(n_req, heads, count, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(n_req * heads, size=count, replace=False)
    return sorted((int(i) // heads, int(i) % heads) for i in idx)


def _gather(t, units):
    """[n, T, H, d] device tensor -> [len(units), T, 1, d] host copy of the sampled units."""
    return torch.stack([t[r, :, h:h + 1] for r, h in units]).cpu()


def test_block_loop_sampled():
    """32 requests x 32 heads, d = 128: 32 blocks of 32 tokens, 8 steps per
    block (fresh N(0, 0.5^2) Q/K/V each step), the block's last step fused
    with its commit (hybrid_attn_step_commit), as the benchmark runs it.
    Every step's output and the final state are compared on 6 sampled units
    against the oracle's fp64 chain."""
    W = BLOCK_LOOP
    units = _units(W.n_req, W.heads, 6, 404)
    state = torch.zeros(W.n_req, W.heads, W.d, W.d, device=DEV)
    slots = torch.arange(W.n_req, dtype=torch.int32, device=DEV)
    S_ref = np.zeros((len(units), 1, W.d, W.d))
    worst = 0.0
    for b in range(W.n_blocks):
        for t in range(W.steps_per_block):
            q, k, v = (synth.normal((W.n_req, W.blk, W.heads, W.d), synth.seed_of(W.index, b, t, i), std=W.std,
                                    device=DEV) for i in range(3))
            step = bh.hybrid_attn_step_commit if t == W.steps_per_block - 1 else bh.hybrid_attn_step
            out = step(q, k, v, state, slots, scale=W.scale)
            qs, ks, vs, os_ = _gather(q, units), _gather(k, units), _gather(v, units), _gather(out, units)
            ref = oracle.step(qs, ks, vs, S_ref, scale=W.scale)
            worst = max(worst, assert_parity(os_, ref, torch.bfloat16, f"block {b} step {t}"))
        S_ref = oracle.commit(ks, vs, S_ref)
    torch.cuda.synchronize()
    got = np.stack([state_to_oracle(state)[r, h:h + 1] for r, h in units])
    es = assert_parity(got, S_ref, torch.bfloat16, "final state")
    log(f"block loop: worst step rel err {worst:.2e}, final state rel err {es:.2e}")


def test_prefill_decode_sampled():
    """8 requests x 32 heads, d = 128, prompts uniform in [16384, 65536]
    (packed, chunk 256) prefilled, then 16 blocks of 64 tokens x 4 steps, the
    last one fused with the block's commit, as the benchmark runs it.  4
    sampled units: prefilled state, every step's output and the final state
    against the oracle."""
    W = PREFILL_DECODE
    lens = synth.uniform_int(W.n_req, *W.prompt_range, synth.seed_of(W.index, tensor=synth.TENSOR_LEN))
    cu = synth.cu_from_lengths(lens)
    total = int(cu[-1])
    pk = synth.normal((total, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_K), device=DEV)
    pv = synth.normal((total, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_V), device=DEV)
    state = torch.full((W.n_req, W.heads, W.d, W.d), 3.0, device=DEV)
    slots = torch.arange(W.n_req, dtype=torch.int32, device=DEV)
    bh.hybrid_state_prefill(pk, pv, cu.to(DEV), state, slots, max_len=int(lens.max()), chunk=W.chunk)
    units = _units(W.n_req, W.heads, 4, 505)
    log(f"prefill: {total} tokens; sampled units {units}")
    # the sampled units' prompts, packed as one oracle call (one unit per "request")
    ks_ = [pk[int(cu[r]):int(cu[r + 1]), h:h + 1].cpu() for r, h in units]
    vs_ = [pv[int(cu[r]):int(cu[r + 1]), h:h + 1].cpu() for r, h in units]
    S_ref = oracle.prefill(torch.cat(ks_), torch.cat(vs_), synth.cu_from_lengths([x.shape[0] for x in ks_]))
    torch.cuda.synchronize()
    got = np.stack([state_to_oracle(state)[r, h:h + 1] for r, h in units])
    ep = assert_parity(got, S_ref, torch.bfloat16, "prefilled state")
    worst = 0.0
    for b in range(W.n_blocks):
        for t in range(W.steps_per_block):
            q, k, v = (synth.normal((W.n_req, W.blk, W.heads, W.d), synth.seed_of(W.index, b, t, i), device=DEV)
                       for i in range(3))
            step = bh.hybrid_attn_step_commit if t == W.steps_per_block - 1 else bh.hybrid_attn_step
            out = step(q, k, v, state, slots, scale=W.scale)
            qs, ks, vs, os_ = _gather(q, units), _gather(k, units), _gather(v, units), _gather(out, units)
            worst = max(worst, assert_parity(os_, oracle.step(qs, ks, vs, S_ref, scale=W.scale), torch.bfloat16,
                                             f"block {b} step {t}"))
        S_ref = oracle.commit(ks, vs, S_ref)
    torch.cuda.synchronize()
    got = np.stack([state_to_oracle(state)[r, h:h + 1] for r, h in units])
    es = assert_parity(got, S_ref, torch.bfloat16, "final state")
    log(f"prefill + decode: prefill rel err {ep:.2e}, worst step {worst:.2e}, final state {es:.2e}")


def test_prefill_decode_parts_isolated():
    """The prefill + decode workload's decode calls at their full size (8
    requests x 32 heads, d = 128, B = 64), each part of the output isolated:
    S = 0 (softmax part only) and V = 0 (linear part only), for the step and
    for the fused step + commit.  Compared on every head of the request with
    the shortest prompt and one head of each other request, whose states are
    the oracle's prefill of their prompts (the other units get random states).
    At these prefix lengths the linear part dominates the output, so the
    whole-output rule alone would not see an error in the softmax part."""
    W = PREFILL_DECODE
    lens = synth.uniform_int(W.n_req, *W.prompt_range, synth.seed_of(W.index, tensor=synth.TENSOR_LEN))
    cu = synth.cu_from_lengths(lens)
    total = int(cu[-1])
    pk = synth.normal((total, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_K), device=DEV)
    pv = synth.normal((total, W.heads, W.d), synth.seed_of(W.index, 99, 0, synth.TENSOR_V), device=DEV)
    r0 = int(torch.argmin(lens))
    units = sorted({(r0, h) for h in range(W.heads)} | {(r, (7 * r + 3) % W.heads) for r in range(W.n_req)})
    log(f"isolation: {len(units)} units, all heads of request {r0} ({int(lens[r0])} prompt tokens)")
    ks_ = [pk[int(cu[r]):int(cu[r + 1]), h:h + 1].cpu() for r, h in units]
    vs_ = [pv[int(cu[r]):int(cu[r + 1]), h:h + 1].cpu() for r, h in units]
    S_ref = oracle.prefill(torch.cat(ks_), torch.cat(vs_), synth.cu_from_lengths([x.shape[0] for x in ks_]))
    del pk, pv
    state = synth.normal((W.n_req, W.heads, W.d, W.d), synth.seed_of(W.index, 98, 0, synth.TENSOR_S),
                         dtype=torch.float32, device=DEV).mul_(150.0)
    Sl = state_from_oracle(S_ref)                               # [units, 1, d, d], library layout
    for i, (r, h) in enumerate(units):
        state[r, h] = Sl[i, 0]
    slots = torch.arange(W.n_req, dtype=torch.int32, device=DEV)
    q, k, v = (synth.normal((W.n_req, W.blk, W.heads, W.d), synth.seed_of(W.index, 0, 0, t), device=DEV)
               for t in range(3))
    qs, ks, vs = _gather(q, units), _gather(k, units), _gather(v, units)
    zv = torch.zeros_like(v)
    for name, call in (("step", bh.hybrid_attn_step), ("fused step + commit", bh.hybrid_attn_step_commit)):
        out_s = call(q, k, v, torch.zeros_like(state), slots, scale=W.scale)
        out_l = call(q, k, zv, state.clone(), slots, scale=W.scale)
        torch.cuda.synchronize()
        es = assert_parity(_gather(out_s, units), oracle.step(qs, ks, vs, 0 * S_ref, scale=W.scale), torch.bfloat16,
                           f"{name}: softmax part (S = 0)")
        el = assert_parity(_gather(out_l, units), oracle.step(qs, ks, np.zeros(vs.shape), S_ref, scale=W.scale),
                           torch.bfloat16, f"{name}: linear part (V = 0)")
        log(f"{name}: softmax part rel err {es:.2e}, linear part rel err {el:.2e}")


def test_block_loop_linear_part_isolated():
    """The block loop's calls at full size (32 requests x 32 heads, d = 128,
    B = 32) with V = 0 over a state of 31 committed blocks' magnitude, for the
    step and the fused step + commit, compared on every head of one request
    and one head of each other (the loop itself starts from S = 0, which
    isolates the softmax part of its first block)."""
    W = BLOCK_LOOP
    units = sorted({(5, h) for h in range(W.heads)} | {(r, (11 * r + 1) % W.heads) for r in range(W.n_req)})
    S = synth.normal((W.n_req, W.heads, W.d, W.d), synth.seed_of(W.index, 97, 0, synth.TENSOR_S),
                     dtype=torch.float32, device=DEV).mul_(4.0)
    slots = torch.arange(W.n_req, dtype=torch.int32, device=DEV)
    q, k = (synth.normal((W.n_req, W.blk, W.heads, W.d), synth.seed_of(W.index, 31, 7, t), std=W.std, device=DEV)
            for t in range(2))
    zv = torch.zeros_like(q)
    S_units = np.stack([state_to_oracle(S)[r, h:h + 1] for r, h in units])
    qs, ks = _gather(q, units), _gather(k, units)
    ref = oracle.step(qs, ks, np.zeros(qs.shape), S_units, scale=W.scale)
    for name, call in (("step", bh.hybrid_attn_step), ("fused step + commit", bh.hybrid_attn_step_commit)):
        out = call(q, k, zv, S.clone(), slots, scale=W.scale)
        torch.cuda.synchronize()
        e = assert_parity(_gather(out, units), ref, torch.bfloat16, f"{name}: linear part (V = 0)")
        log(f"block loop {name}: linear part rel err {e:.2e}")
