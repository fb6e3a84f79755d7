"""GPU path vs the fp64 oracle on identical seeded inputs, through the C ABI.

Sizes span several 32-row tiles with ragged tails, every supported head dim,
both dtypes, slot indirection, and the degenerate cases (one valid row, empty
prompts, invalid slots).  Each step is also checked with its two parts
isolated (S = 0: softmax only; V = 0: linear only), because at long prefixes
the linear term dominates the output's magnitude and the whole-output rule
alone would hide softmax errors.
"""
import numpy as np
import pytest
import torch

import block_hybrid_linear_amd as bh
import oracle
from block_hybrid_linear_amd import synth
from block_hybrid_linear_amd.workloads import WORKED_EXAMPLE
from parity import assert_parity, rows_mask, state_from_oracle, state_to_oracle, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = -1024.0  # exact in bf16 and fp32


def gen(shape, seed, dtype, std=1.0):
    return synth.normal(shape, seed, std=std, dtype=dtype).to(DEV)


def check_step(q, k, v, state, slots, blk_lens, scale, what):
    n_req, blk = q.shape[:2]
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step(q, k, v, state, slots, out=out, blk_lens=blk_lens, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.step(q, k, v, state_to_oracle(state), slots=slots, blk_lens=blk_lens, scale=scale)
    mask = rows_mask(blk_lens, n_req, blk)
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL), f"{what}: rows past B_r were written"
    return assert_parity(o[mask], ref[mask], q.dtype, what)


# --------------------------------------------------------------------------
# The worked example end to end (fp32, L = 10, B = 4, blocks 4/4/2, H = 2, d = 16)
# --------------------------------------------------------------------------

def test_worked_example_generation():
    W = WORKED_EXAMPLE
    state = torch.zeros(1, W.heads, W.d, W.d, device=DEV)
    slots = torch.zeros(1, dtype=torch.int32, device=DEV)
    S_ref = np.zeros((1, W.heads, W.d, W.d))
    for b, n in enumerate(W.block_lens):
        q, k, v = (gen((1, W.blk, W.heads, W.d), synth.seed_of(W.index, b, 0, t), torch.float32) for t in range(3))
        lens = torch.tensor([n], dtype=torch.int32, device=DEV)
        out = bh.hybrid_attn_step(q, k, v, state, slots, blk_lens=lens, scale=W.scale)
        ref = oracle.step(q, k, v, S_ref, blk_lens=[n], scale=W.scale)
        assert_parity(out[:, :n], ref[:, :n], torch.float32, f"block {b + 1} output", f32_absolute=True)
        bh.hybrid_state_commit(k, v, state, slots, blk_lens=lens)
        S_ref = oracle.commit(k, v, S_ref, blk_lens=[n])
        torch.cuda.synchronize()
        assert_parity(state_to_oracle(state), S_ref, torch.float32, f"S after block {b + 1}", f32_absolute=True)


# --------------------------------------------------------------------------
# Step
# --------------------------------------------------------------------------

STEP_CASES = [  # (d, blk)
    (128, 32), (128, 64), (128, 100), (128, 128), (128, 1), (128, 5), (128, 200), (128, 256),
    (64, 32), (64, 33), (64, 128), (64, 256), (32, 17), (32, 64), (32, 96), (32, 200),
    (16, 4), (16, 32), (16, 128), (16, 256),
]


@pytest.mark.parametrize("d,blk", STEP_CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_step_parity(d, blk, dtype):
    n_req, H, n_slots = 3, 5, 4
    seed = 7000 + 100 * d + blk
    q, k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(3))
    # ragged: one full block, one mid, one single row
    blk_lens = torch.tensor([blk, max(1, (blk * 2) // 3), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([3, 0, 2], dtype=torch.int32, device=DEV)
    std = 30.0 if dtype == torch.bfloat16 else 1.0
    state = synth.normal((n_slots, H, d, d), seed + 3, std=std, dtype=torch.float32).to(DEV)
    scale = d ** -0.5
    check_step(q, k, v, state, slots, blk_lens, scale, "full")
    check_step(q, k, v, torch.zeros_like(state), slots, blk_lens, scale, "softmax part (S = 0)")
    check_step(q, k, torch.zeros_like(v), state, slots, blk_lens, scale, "linear part (V = 0)")


def test_step_no_blk_lens_and_scale():
    """blk_lens = NULL means every row is valid; the scale is honoured."""
    n_req, blk, H, d = 2, 48, 3, 128
    q, k, v = (gen((n_req, blk, H, d), 8100 + t, torch.bfloat16, std=2.0) for t in range(3))
    state = synth.normal((n_req, H, d, d), 8103, std=5.0, dtype=torch.float32).to(DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    for scale in (0.0, 0.02, 0.3):
        check_step(q, k, v, torch.zeros_like(state), slots, None, scale, f"scale {scale}")


def test_step_large_logits():
    """Logits of several hundred: the max-subtracted softmax stays finite."""
    n_req, blk, H, d = 1, 32, 2, 64
    q, k = (gen((n_req, blk, H, d), 8200 + t, torch.bfloat16, std=6.0) for t in range(2))
    v = gen((n_req, blk, H, d), 8202, torch.bfloat16)
    state = torch.zeros(1, H, d, d, device=DEV)
    slots = torch.zeros(1, dtype=torch.int32, device=DEV)
    check_step(q, k, v, state, slots, None, 1.0, "large logits")


def test_step_invalid_slot_and_empty_rows_skip():
    """A request with an out-of-range slot or B_r = 0 writes nothing."""
    n_req, blk, H, d = 4, 32, 2, 128
    q, k, v = (gen((n_req, blk, H, d), 8300 + t, torch.bfloat16) for t in range(3))
    state = synth.normal((2, H, d, d), 8303, dtype=torch.float32).to(DEV)
    slots = torch.tensor([0, -1, 2, 1], dtype=torch.int32, device=DEV)
    lens = torch.tensor([32, 32, 32, 0], dtype=torch.int32, device=DEV)
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step(q, k, v, state, slots, out=out, blk_lens=lens)
    torch.cuda.synchronize()
    o = to64(out)
    assert np.all(o[1:] == SENTINEL)
    ref = oracle.step(q[:1], k[:1], v[:1], state_to_oracle(state)[:1], scale=d ** -0.5)
    assert_parity(o[:1], ref, torch.bfloat16, "valid request")


def _bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significand bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("d,blk", [(128, 32), (128, 64), (64, 64), (32, 64), (128, 1), (64, 20), (128, 200),
                                   (64, 256)])
def test_step_outputs_correctly_rounded(d, blk, fused):
    """The matrix-core step keeps fp32 S and P at ~16 significand bits (hi + lo
    bf16), so every bf16 output is within one bf16 ulp of the exact value plus
    fp32 accumulation error (1e-5 of the output's scale).  A dropped lo term
    or a stale accumulator register shows up here while staying inside the
    whole-output rule."""
    n_req, H = 3, 4
    seed = 8500 + 100 * d + blk
    q, k, v = (gen((n_req, blk, H, d), seed + t, torch.bfloat16) for t in range(3))
    lens = torch.tensor([blk, max(1, blk // 2), 1], dtype=torch.int32, device=DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    state = synth.normal((n_req, H, d, d), seed + 3, std=10.0, dtype=torch.float32).to(DEV)
    S0 = state_to_oracle(state)
    call = bh.hybrid_attn_step_commit if fused else bh.hybrid_attn_step
    out = call(q, k, v, state, slots, blk_lens=lens)
    torch.cuda.synchronize()
    ref = oracle.step(q, k, v, S0, blk_lens=lens, scale=d ** -0.5)
    mask = rows_mask(lens, n_req, blk)
    o, r = to64(out)[mask], ref[mask]
    bound = _bf16_ulp(r) + 1e-5 * np.abs(r).max()
    bad = np.abs(o - r) > bound
    assert not bad.any(), f"{bad.sum()} outputs off by more than one bf16 ulp, worst {np.abs(o - r)[bad].max():.3e}"


def test_step_deterministic():
    n_req, blk, H, d = 4, 64, 4, 128
    q, k, v = (gen((n_req, blk, H, d), 8400 + t, torch.bfloat16) for t in range(3))
    state = synth.normal((n_req, H, d, d), 8403, std=40.0, dtype=torch.float32).to(DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    a = bh.hybrid_attn_step(q, k, v, state, slots)
    b = bh.hybrid_attn_step(q, k, v, state, slots)
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# Commit
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d,blk", [(128, 32), (128, 20), (128, 33), (128, 64), (128, 100), (128, 128), (128, 1),
                                   (128, 200), (128, 256), (64, 32), (64, 9), (64, 77), (64, 256), (32, 32), (32, 5),
                                   (32, 200), (16, 4), (16, 64), (16, 256)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_commit_parity(d, blk, dtype):
    n_req, H, n_slots = 3, 4, 5
    seed = 9000 + 100 * d + blk
    k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(2))
    lens = torch.tensor([blk, max(1, blk // 2), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([4, 1, 2], dtype=torch.int32, device=DEV)
    state = synth.normal((n_slots, H, d, d), seed + 3, dtype=torch.float32).to(DEV)
    S0 = state_to_oracle(state)
    bh.hybrid_state_commit(k, v, state, slots, blk_lens=lens)
    torch.cuda.synchronize()
    ref = oracle.commit(k, v, S0, slots=slots, blk_lens=lens)
    got = state_to_oracle(state)
    assert np.array_equal(got[[0, 3]], S0[[0, 3]]), "slots not named were modified"
    assert_parity(got, ref, dtype, "state after commit")
    # not idempotent: a second identical commit adds the block again
    bh.hybrid_state_commit(k, v, state, slots, blk_lens=lens)
    torch.cuda.synchronize()
    ref2 = oracle.commit(k, v, ref, slots=slots, blk_lens=lens)
    assert_parity(state_to_oracle(state), ref2, dtype, "state after second commit")


# --------------------------------------------------------------------------
# Fused last step + commit
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d,blk", [(128, 32), (128, 64), (128, 33), (128, 1), (128, 100), (128, 200), (128, 256),
                                   (64, 64), (64, 17), (64, 256), (32, 64), (32, 5), (32, 256), (16, 32)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_step_commit_parity(d, blk, dtype):
    """Output from the old state and the updated state both match the oracle's
    step then commit; slots not named are untouched; on the matrix-core path
    the output is bit-identical to hybrid_attn_step's."""
    n_req, H, n_slots = 3, 5, 4
    seed = 17000 + 100 * d + blk
    q, k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(3))
    lens = torch.tensor([blk, max(1, (blk * 2) // 3), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([2, 0, 3], dtype=torch.int32, device=DEV)
    state = synth.normal((n_slots, H, d, d), seed + 3, std=10.0, dtype=torch.float32).to(DEV)
    S0 = state_to_oracle(state)
    plain = bh.hybrid_attn_step(q, k, v, state, slots, blk_lens=lens)
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_commit(q, k, v, state, slots, out=out, blk_lens=lens)
    torch.cuda.synchronize()
    mask = rows_mask(lens, n_req, blk)
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL), "rows past B_r were written"
    ref = oracle.step(q, k, v, S0, slots=slots, blk_lens=lens, scale=d ** -0.5)
    assert_parity(o[mask], ref[mask], dtype, "fused step output")
    S1 = oracle.commit(k, v, S0, slots=slots, blk_lens=lens)
    got = state_to_oracle(state)
    assert np.array_equal(got[1], S0[1]), "a slot not named was modified"
    assert_parity(got, S1, dtype, "state after fused commit")
    if dtype == torch.bfloat16 and d >= 32 and blk <= 64:
        assert torch.equal(out[torch.from_numpy(mask).to(DEV)], plain[torch.from_numpy(mask).to(DEV)])


def test_step_commit_skips_invalid_slot_and_empty_rows():
    n_req, blk, H, d = 3, 64, 2, 128
    q, k, v = (gen((n_req, blk, H, d), 17500 + t, torch.bfloat16) for t in range(3))
    state = synth.normal((2, H, d, d), 17503, dtype=torch.float32).to(DEV)
    before = state.clone()
    slots = torch.tensor([7, 0, 1], dtype=torch.int32, device=DEV)       # request 0: invalid slot
    lens = torch.tensor([64, 40, 0], dtype=torch.int32, device=DEV)       # request 2: no rows
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_commit(q, k, v, state, slots, out=out, blk_lens=lens)
    torch.cuda.synchronize()
    o = to64(out)
    assert np.all(o[0] == SENTINEL) and np.all(o[2] == SENTINEL) and np.all(o[1, 40:] == SENTINEL)
    assert torch.equal(state[1], before[1]), "slot of the empty request was modified"
    S1 = oracle.commit(k[1:2], v[1:2], state_to_oracle(before[0:1]), blk_lens=[40])
    assert_parity(state_to_oracle(state[0:1]), S1, torch.bfloat16, "state of request 1")
    ref = oracle.step(q[1:2], k[1:2], v[1:2], state_to_oracle(before[0:1]), blk_lens=[40])
    assert_parity(o[1:2, :40], ref[:, :40], torch.bfloat16, "output of request 1")


def test_step_commit_block_loop_matches_separate_calls():
    """A block loop with the last step fused into the commit tracks the loop
    with separate calls: outputs within the rule, states within fp32 rounding."""
    n_req, blk, H, d = 4, 64, 4, 128
    s_a = torch.zeros(n_req, H, d, d, device=DEV)
    s_b = torch.zeros_like(s_a)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    S_ref = np.zeros((n_req, H, d, d))
    for b in range(6):
        for t in range(3):
            q, k, v = (gen((n_req, blk, H, d), 18000 + 100 * b + 10 * t + i, torch.bfloat16) for i in range(3))
            last = t == 2
            out_a = bh.hybrid_attn_step(q, k, v, s_a, slots)
            if last:
                bh.hybrid_state_commit(k, v, s_a, slots)
                out_b = bh.hybrid_attn_step_commit(q, k, v, s_b, slots)
            else:
                out_b = bh.hybrid_attn_step(q, k, v, s_b, slots)
            ref = oracle.step(q, k, v, S_ref)
            assert_parity(out_b, ref, torch.bfloat16, f"block {b} step {t}")
            assert_parity(out_a, ref, torch.bfloat16, f"block {b} step {t} (separate)")
        S_ref = oracle.commit(k, v, S_ref)
    torch.cuda.synchronize()
    assert_parity(state_to_oracle(s_b), S_ref, torch.bfloat16, "final state (fused)")
    rel = float((s_b - s_a).abs().max() / s_a.abs().max())
    assert rel < 1e-5, rel


def test_commit_order_independent():
    """Commits of several blocks in any order give the same state (fp32
    reassociation only), equal to the oracle's sum."""
    H, d, blk = 4, 128, 32
    blocks = [tuple(gen((2, blk, H, d), 9500 + 10 * i + t, torch.bfloat16) for t in range(2)) for i in range(4)]
    slots = torch.arange(2, dtype=torch.int32, device=DEV)
    finals = []
    for order in ([0, 1, 2, 3], [3, 1, 0, 2], [2, 3, 1, 0]):
        state = torch.zeros(2, H, d, d, device=DEV)
        for i in order:
            bh.hybrid_state_commit(blocks[i][0], blocks[i][1], state, slots)
        finals.append(state.clone())
    torch.cuda.synchronize()
    ref = np.zeros((2, H, d, d))
    for kk, vv in blocks:
        ref = oracle.commit(kk, vv, ref)
    for f in finals:
        assert_parity(state_to_oracle(f), ref, torch.bfloat16, "commit order")


# --------------------------------------------------------------------------
# Prefill
# --------------------------------------------------------------------------

def prefill_case(lengths, H, d, dtype, seed, chunk=256, n_slots=None, slots=None):
    lengths = list(lengths)
    n_req = len(lengths)
    cu = synth.cu_from_lengths(lengths)
    total = int(cu[-1])
    k, v = (synth.normal((total, H, d), seed + t, dtype=dtype) for t in range(2))
    n_slots = n_slots or n_req
    slots = slots if slots is not None else list(range(n_req))
    state = torch.full((n_slots, H, d, d), 77.0, device=DEV)
    before = to64(state)
    bh.hybrid_state_prefill(k.to(DEV), v.to(DEV), cu.to(DEV), state,
                            torch.tensor(slots, dtype=torch.int32, device=DEV),
                            max_len=max(lengths) if lengths else 0, chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.prefill(k, v, cu, S=state_to_oracle(torch.from_numpy(before).float()), slots=slots)
    return state, ref, before, slots


@pytest.mark.parametrize("d", [128, 64, 32, 16])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_parity(d, dtype):
    lengths = [0, 1, 31, 4096, 4097, 9000] if dtype == torch.bfloat16 else [0, 1, 31, 700]
    state, ref, before, slots = prefill_case(lengths, 2, d, dtype, 10000 + d)
    assert_parity(state_to_oracle(state), ref, dtype, "prefilled state")
    assert np.all(state_to_oracle(state)[slots[0]] == 0.0), "empty prompt must reset the slot"


@pytest.mark.parametrize("chunk", [1, 7, 64, 256, 9000])
def test_prefill_chunk_independent(chunk):
    lengths = [9000, 300, 4100]
    state, ref, _, _ = prefill_case(lengths, 2, 128, torch.bfloat16, 11000, chunk=chunk)
    assert_parity(state_to_oracle(state), ref, torch.bfloat16, f"chunk {chunk}")


def test_prefill_slot_indirection():
    lengths = [500, 0, 1200]
    state, ref, before, slots = prefill_case(lengths, 3, 64, torch.bfloat16, 11500, n_slots=6, slots=[5, 0, 2])
    got = state_to_oracle(state)
    assert np.array_equal(got[[1, 3, 4]], state_to_oracle(torch.from_numpy(before))[[1, 3, 4]])
    assert_parity(got, ref, torch.bfloat16, "prefill with slots")


def test_prefill_equals_commits_and_resume_bitwise():
    """Prefill of a prompt = commits of its blocks (within tolerance); and a
    state saved after block k, restored, continues bit-identically."""
    H, d, blk, nb = 4, 128, 32, 6
    k, v = (synth.normal((nb * blk, H, d), 12000 + t) for t in range(2))
    slots = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = torch.zeros(1, H, d, d, device=DEV)
    bh.hybrid_state_prefill(k.to(DEV), v.to(DEV), torch.tensor([0, nb * blk], device=DEV), sp, slots,
                            max_len=nb * blk)
    sc = torch.zeros(1, H, d, d, device=DEV)
    saved = None
    kb, vb = k.view(nb, 1, blk, H, d).to(DEV), v.view(nb, 1, blk, H, d).to(DEV)
    for b in range(nb):
        bh.hybrid_state_commit(kb[b], vb[b], sc, slots)
        if b == 2:
            saved = sc.clone()
    torch.cuda.synchronize()
    ref = oracle.prefill(k, v, [0, nb * blk])
    assert_parity(state_to_oracle(sp), ref, torch.bfloat16, "prefill")
    assert_parity(state_to_oracle(sc), ref, torch.bfloat16, "commits")
    resumed = saved.clone()
    for b in range(3, nb):
        bh.hybrid_state_commit(kb[b], vb[b], resumed, slots)
    torch.cuda.synchronize()
    assert torch.equal(resumed, sc)


def test_state_layout_row_is_value_dim():
    """The state block is stored as S^T: state[slot][h][c][f] = S[f][c] (row =
    value dim, column = feature of phi(k)).  Committing one token whose key
    has a single positive feature f0 writes v into column f0 and nothing else;
    a step with V = 0 then gives relu(q) @ S, which differs from relu(q) @ S^T
    by far more than the tolerance (so the other orientation fails here)."""
    n_req, blk, H, d = 2, 32, 2, 128
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    k1 = torch.full((n_req, 1, H, d), -1.0, dtype=torch.bfloat16, device=DEV)
    f0 = [5, 77]
    for r in range(n_req):
        k1[r, 0, :, f0[r]] = 1.0
    v1 = gen((n_req, 1, H, d), 12490, torch.bfloat16)
    state = torch.zeros(n_req, H, d, d, device=DEV)
    bh.hybrid_state_commit(k1, v1, state, slots)
    torch.cuda.synchronize()
    St = to64(state)
    for r in range(n_req):
        expect = np.zeros((H, d, d))
        expect[:, :, f0[r]] = to64(v1)[r, 0]
        assert np.array_equal(St[r], expect), f"request {r}: commit did not write column f0 = v"

    q, k, v = (gen((n_req, blk, H, d), 12500 + t, torch.bfloat16) for t in range(3))
    S = np.random.default_rng(5).standard_normal((n_req, H, d, d)) * 10
    S[..., :d // 2, d // 2:] += 40.0                      # far from symmetric
    state = state_from_oracle(S)
    out = bh.hybrid_attn_step(q, k, torch.zeros_like(v), state, slots)
    torch.cuda.synchronize()
    Sd = state_to_oracle(state)                           # S[f][c]
    qr = np.maximum(to64(q), 0.0)
    ref = np.einsum("rihf,rhfc->rihc", qr, Sd)
    ref_t = np.einsum("rihf,rhcf->rihc", qr, Sd)
    assert_parity(out, ref, torch.bfloat16, "relu(q) @ S")
    assert np.abs(ref - ref_t).max() > 10 * 2e-2 * np.abs(ref).max()
    assert_parity(out, oracle.step(q, k, np.zeros(v.shape), Sd, scale=d ** -0.5), torch.bfloat16, "oracle")


@pytest.mark.parametrize("d,H", [(64, 2), (32, 2), (16, 2), (128, 2), (128, 3)])
def test_prefill_many_ragged_requests(d, H):
    """Hundreds of prompts (more than the 256 runs each slice workgroup's
    planning scan covers, so every run holds two), many shorter than a chunk,
    some empty: the balanced split crosses request and head boundaries inside
    workgroups, prompts lie inside one slice or span several.  Every
    workgroup size of the slice kernels: 64 threads (d = 32), 256 (d = 16, 64,
    one head of d = 128), 512 (head pairs)."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 700, size=300)]
    lengths[5] = 0
    lengths[6] = 1
    lengths[7] = 5000
    state, ref, _, _ = prefill_case(lengths, H, d, torch.bfloat16, 13000 + d + H, chunk=64)
    assert_parity(state_to_oracle(state), ref, torch.bfloat16, "many prompts")


@pytest.mark.parametrize("H", [1, 3, 6])
def test_prefill_head_groups(H):
    """d = 128 in bf16 streams adjacent head pairs when the head count is even
    and single heads otherwise; ragged prompts with small chunks put pieces of
    both heads of a pair, and of several prompts, in one workgroup."""
    rng = np.random.default_rng(78 + H)
    lengths = [int(x) for x in rng.integers(0, 400, size=40)]
    lengths[3] = 0
    lengths[4] = 1
    lengths[9] = 3000
    state, ref, _, _ = prefill_case(lengths, H, 128, torch.bfloat16, 13200 + H, chunk=64)
    assert_parity(state_to_oracle(state), ref, torch.bfloat16, f"{H} heads")


@pytest.mark.parametrize("H,d", [(600, 128), (520, 64), (2100, 32)])
def test_prefill_more_head_groups_than_workgroups(H, d):
    """More head groups than the usual number of slice workgroups: every head
    group then gets one workgroup (and its own partial slot)."""
    lengths = [70, 5, 0, 33]
    state, ref, _, _ = prefill_case(lengths, H, d, torch.bfloat16, 13300 + d, chunk=16)
    assert_parity(state_to_oracle(state), ref, torch.bfloat16, f"{H} heads, d = {d}")


def test_prefill_malformed_offsets_are_empty():
    """Offsets running backwards or past total_tokens count as empty prompts
    (S = 0) instead of reading out of bounds."""
    H, d, total = 2, 128, 300
    k, v = (synth.normal((total, H, d), 13500 + t) for t in range(2))
    cu = torch.tensor([0, 100, 50, 300, 400], dtype=torch.int64)
    state = torch.full((4, H, d, d), 5.0, device=DEV)
    slots = torch.arange(4, dtype=torch.int32, device=DEV)
    bh.hybrid_state_prefill(k.to(DEV), v.to(DEV), cu.to(DEV), state, slots)
    torch.cuda.synchronize()
    got = state_to_oracle(state)
    assert np.all(got[1] == 0.0) and np.all(got[3] == 0.0)
    ref = oracle.prefill(k[:100], v[:100], [0, 100])
    assert_parity(got[:1], ref, torch.bfloat16, "valid prompt 0")
    ref2 = oracle.prefill(k[50:300], v[50:300], [0, 250])
    assert_parity(got[2:3], ref2, torch.bfloat16, "valid prompt 2")


def test_prefill_deterministic():
    lengths = [20000, 3000, 17]
    a, _, _, _ = prefill_case(lengths, 4, 128, torch.bfloat16, 14000)
    b, _, _, _ = prefill_case(lengths, 4, 128, torch.bfloat16, 14000)
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [128, 64, 16])
def test_prefill_workspace_reused_with_stale_contents(d):
    """One workspace, filled with 0xFF bytes, serves calls of different shapes
    in a row (its contents on entry do not matter): prompts inside one slice
    and prompts spanning several, empty prompts, and requests whose slot is
    out of range (skipped: no slot is written for them)."""
    H = 4
    cases = [([9000, 0, 4100, 33], [0, 1, 2, 3]),
             ([20000, 50, 7000], [2, -1, 0]),
             ([15000, 300, 0], [-1, 1, 3])]
    n_slots = 4
    big = max(bh.hybrid_state_prefill_workspace_bytes(len(l), H, d, sum(l), 0, 256) for l, _ in cases)
    ws = torch.full((big,), 255, dtype=torch.uint8, device=DEV)
    for i, (lengths, slots) in enumerate(cases):
        cu = synth.cu_from_lengths(lengths)
        k, v = (synth.normal((int(cu[-1]), H, d), 15000 + 10 * i + t) for t in range(2))
        state = torch.full((n_slots, H, d, d), 9.0, device=DEV)
        before = to64(state)
        bh.hybrid_state_prefill(k.to(DEV), v.to(DEV), cu.to(DEV), state,
                                torch.tensor(slots, dtype=torch.int32, device=DEV), workspace=ws)
        torch.cuda.synchronize()
        got = state_to_oracle(state)
        valid = [s for s in slots if s >= 0]
        untouched = [s for s in range(n_slots) if s not in valid]
        assert np.array_equal(got[untouched], state_to_oracle(torch.from_numpy(before))[untouched]), \
            f"call {i}: a slot not named (or named by an out-of-range request) was written"
        keep = [r for r, s in enumerate(slots) if s >= 0]
        ref = oracle.prefill(k, v, cu, slots=list(range(len(lengths))))
        assert_parity(got[[slots[r] for r in keep]], ref[keep], torch.bfloat16, f"call {i}")


def test_prepared_calls_match_and_rerun():
    """Prepared calls give bit-identical results to the regular calls and
    pick up new contents of the same buffers when re-run."""
    n_req, blk, H, d = 4, 32, 8, 128
    q, k, v = (gen((n_req, blk, H, d), 15000 + t, torch.bfloat16) for t in range(3))
    state = synth.normal((n_req, H, d, d), 15003, std=20.0, dtype=torch.float32).to(DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    ref = bh.hybrid_attn_step(q, k, v, state, slots)
    out = torch.empty_like(q)
    run = bh.prepare_step(q, k, v, state, slots, out)
    run()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    q.copy_(gen((n_req, blk, H, d), 15010, torch.bfloat16))
    ref2 = bh.hybrid_attn_step(q, k, v, state, slots)
    run()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    s2 = state.clone()
    bh.hybrid_state_commit(k, v, s2, slots)
    c = bh.prepare_commit(k, v, state, slots)
    c()
    torch.cuda.synchronize()
    assert torch.equal(state, s2)


def test_graph_capture_replays_match_eager():
    """A step + commit captured in a graph, replayed several times with eager
    work between replays, matches the eager result bit for bit each time."""
    n_req, blk, H, d = 8, 64, 4, 128
    q, k, v = (gen((n_req, blk, H, d), 16000 + t, torch.bfloat16) for t in range(3))
    state0 = synth.normal((n_req, H, d, d), 16003, std=20.0, dtype=torch.float32).to(DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    s_e = state0.clone()
    out_e = bh.hybrid_attn_step(q, k, v, s_e, slots)
    bh.hybrid_state_commit(k, v, s_e, slots)
    torch.cuda.synchronize()

    s_g = state0.clone()
    out_g = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside capture
        bh.hybrid_attn_step(q, k, v, s_g, slots, out=out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bh.hybrid_attn_step(q, k, v, s_g, slots, out=out_g)
        bh.hybrid_state_commit(k, v, s_g, slots)
    for rep in range(3):
        s_g.copy_(state0)
        out_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: output differs"
        assert torch.equal(s_g, s_e), f"replay {rep}: state differs"
        _ = (q.float() * 2).sum().item()   # unrelated eager work between replays


def test_side_stream_calls():
    """Calls enqueued on a stream other than the current one, with the output
    and the prefill workspace allocated by the binding: they are allocated
    and filled on that stream, so the results match the oracle."""
    n_req, blk, H, d = 2, 48, 4, 128
    q, k, v = (gen((n_req, blk, H, d), 19000 + t, torch.bfloat16) for t in range(3))
    lens = [900, 2500]
    cu = synth.cu_from_lengths(lens)
    kp = gen((int(cu[-1]), H, d), 19010, torch.bfloat16)
    vp = gen((int(cu[-1]), H, d), 19011, torch.bfloat16)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    state = torch.full((n_req, H, d, d), 7.0, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda._sleep(50_000_000)                 # keep the current stream busy meanwhile
    bh.hybrid_state_prefill(kp, vp, cu.to(DEV), state, slots, stream=side)
    out = bh.hybrid_attn_step(q, k, v, state, slots, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    S = oracle.prefill(kp, vp, cu)
    assert_parity(state_to_oracle(state), S, torch.bfloat16, "prefill on a side stream")
    assert_parity(out, oracle.step(q, k, v, S, scale=d ** -0.5), torch.bfloat16, "step on a side stream")
