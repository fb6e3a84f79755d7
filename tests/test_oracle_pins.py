"""Pins of the CPU oracle to things other than itself (CPU only).

Each test names what pins which part of the oracle:
  * a hand-derived example with exact rational values (tests/golden);
  * library routines (torch scaled_dot_product_attention in fp64, numpy matmul,
    numpy outer) on special cases that reduce to them;
  * closed forms (one valid row, zero queries, a single prompt token);
  * invariants (associativity of the two forms of the linear term, order and
    split independence of the state, linearity, permutations);
  * brute force over all tiny sizes.
A plausible slip in the oracle -- ReLU on the wrong operand, S transposed, the
scale applied to the linear term, a missing max-subtraction, a dropped term,
the wrong rows for a ragged block -- fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20260806)


def rnd(*shape):
    return RNG.standard_normal(shape)


def relu(x):
    return np.maximum(x, 0.0)


def sdpa64(q, k, v, scale):
    """torch's non-causal scaled-dot-product attention in fp64 on the CPU,
    per (request, head); q/k/v as [n, T, H, d]."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


# --------------------------------------------------------------------------
# Hand-derived worked example (exact rationals)
# --------------------------------------------------------------------------

def test_hand_worked_example_exact():
    """Pins step + commit chain, ReLU placement, S orientation, the sum, the
    ragged last block and S_{1,2} against values derived by hand."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    d, blk = g["d"], g["blk"]
    scale = math.log(2.0)
    S = np.zeros((1, 1, d, d))
    for b in g["blocks"]:
        n = len(b["Q"])
        q = np.zeros((1, blk, 1, d)); k = np.zeros_like(q); v = np.zeros_like(q)
        q[0, :n, 0] = b["Q"]; k[0, :n, 0] = b["K"]; v[0, :n, 0] = b["V"]
        # rows past the valid length hold junk that must not be read
        q[0, n:, 0] = 1e6; k[0, n:, 0] = 1e6; v[0, n:, 0] = -1e6
        exp_S0 = np.array([[float(Fraction(x)) for x in r] for r in b["S_before"]])
        np.testing.assert_allclose(S[0, 0], exp_S0, rtol=0, atol=1e-12)
        lens = np.array([n], dtype=np.int32)
        o = oracle.step(q, k, v, S, blk_lens=lens, scale=scale)
        exp_O = np.array([[float(Fraction(x)) for x in r] for r in b["O"]])
        np.testing.assert_allclose(o[0, :n, 0], exp_O, rtol=1e-13, atol=1e-13)
        assert np.all(o[0, n:] == 0.0)  # never written
        S = oracle.commit(k, v, S, blk_lens=lens)
        exp_S1 = np.array([[float(Fraction(x)) for x in r] for r in b["S_after"]])
        np.testing.assert_allclose(S[0, 0], exp_S1, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Special cases reducing to library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("blk,d", [(1, 3), (4, 16), (7, 5), (32, 64)])
def test_empty_prefix_is_sdpa(blk, d):
    """S = 0: the step is textbook non-causal softmax attention over the block
    (block 1 of the worked example uses only softmax attention)."""
    n, H = 2, 3
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    scale = 0.37
    o = oracle.step(q, k, v, np.zeros((n, H, d, d)), scale=scale)
    np.testing.assert_allclose(o, sdpa64(q, k, v, scale), rtol=1e-12, atol=1e-12)


def test_large_logits_need_max_subtraction():
    """Logits of several hundred overflow a naive exp; the textbook routine
    does not, and neither may the oracle."""
    n, blk, H, d = 1, 8, 1, 4
    q, k, v = 30 * rnd(n, blk, H, d), 30 * rnd(n, blk, H, d), rnd(n, blk, H, d)
    o = oracle.step(q, k, v, np.zeros((n, H, d, d)), scale=1.0)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, sdpa64(q, k, v, 1.0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [2, 16, 64])
def test_zero_values_is_phiQ_times_S(d):
    """V_a = 0: only the linear term remains, relu(Q_a) @ S (numpy matmul);
    pins the orientation of S (rows = feature of phi, columns = value dim)
    and that the scale does not touch the linear term."""
    n, blk, H = 2, 5, 2
    q, k = rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    o = oracle.step(q, k, np.zeros_like(q), S, scale=0.1)
    for r in range(n):
        for h in range(H):
            np.testing.assert_allclose(o[r, :, h], relu(q[r, :, h]) @ S[r, h], rtol=1e-12, atol=1e-12)


def test_single_token_commit_is_outer_product():
    """One committed token: S = relu(k) outer v (numpy outer).  ReLU acts on
    the key, not the value."""
    d = 6
    k, v = rnd(1, 1, 1, d), rnd(1, 1, 1, d)
    k[0, 0, 0, :3] = -np.abs(k[0, 0, 0, :3]); v[0, 0, 0, ::2] = -np.abs(v[0, 0, 0, ::2])
    S = oracle.commit(k, v, np.zeros((1, 1, d, d)))
    np.testing.assert_allclose(S[0, 0], np.outer(relu(k[0, 0, 0]), v[0, 0, 0]), rtol=0, atol=1e-15)


def test_prefill_is_matmul_of_blocks():
    """Prefill of a prompt: relu(K)^T V over all its tokens (numpy matmul)."""
    H, d = 2, 8
    lens = [0, 1, 13, 40]
    cu = np.concatenate([[0], np.cumsum(lens)])
    k, v = rnd(cu[-1], H, d), rnd(cu[-1], H, d)
    S = oracle.prefill(k, v, cu, S=np.full((4, H, d, d), 7.0))
    for r in range(4):
        for h in range(H):
            kk, vv = k[cu[r]:cu[r + 1], h], v[cu[r]:cu[r + 1], h]
            np.testing.assert_allclose(S[r, h], relu(kk).T @ vv, rtol=1e-12, atol=1e-12)
    assert np.all(S[0] == 0.0)  # empty prompt resets the slot


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def test_single_valid_row_closed_form():
    """B_r = 1: the only softmax weight is 1, so O = v + relu(q) S."""
    n, blk, H, d = 3, 4, 2, 8
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    o = oracle.step(q, k, v, S, blk_lens=np.ones(n, np.int32))
    for r in range(n):
        for h in range(H):
            exp = v[r, 0, h] + relu(q[r, 0, h]) @ S[r, h]
            np.testing.assert_allclose(o[r, 0, h], exp, rtol=1e-13, atol=1e-13)
    assert np.all(o[:, 1:] == 0.0)


def test_zero_queries_closed_form():
    """Q_a = 0: uniform weights over the B_r valid keys and phi(0) = 0, so
    O = column mean of the first B_r value rows."""
    n, blk, H, d = 2, 6, 2, 5
    k, v = rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    lens = np.array([6, 3], np.int32)
    o = oracle.step(np.zeros_like(k), k, v, S, blk_lens=lens)
    for r in range(n):
        m = v[r, :lens[r]].mean(axis=0)  # [H, d]
        for i in range(lens[r]):
            np.testing.assert_allclose(o[r, i], m, rtol=1e-13, atol=1e-13)


def test_identical_keys_closed_form():
    """All keys equal: weights uniform whatever Q is."""
    n, blk, H, d = 1, 5, 1, 4
    q, v = rnd(n, blk, H, d), rnd(n, blk, H, d)
    k = np.repeat(rnd(n, 1, H, d), blk, axis=1)
    o = oracle.step(q, k, v, np.zeros((n, H, d, d)))
    np.testing.assert_allclose(o[0, :, 0], np.repeat(v[0, :, 0].mean(0, keepdims=True), blk, 0),
                               rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def test_state_form_equals_formula_form_bruteforce():
    """phi(Q)(phi(K_p)^T V_p) == (phi(Q) phi(K_p)^T) V_p: the state form of
    the linear term equals the pages' formula evaluated from the retained
    prefix, over every tiny size."""
    H = 1
    worst = 0.0
    for blk, d, P in itertools.product(range(1, 5), (1, 2, 3, 5, 8), (0, 1, 2, 5, 12)):
        q, k, v = rnd(1, blk, H, d), rnd(1, blk, H, d), rnd(1, blk, H, d)
        kp, vp = rnd(P, H, d), rnd(P, H, d)
        cu = np.array([0, P])
        S = oracle.prefill(kp, vp, cu)
        a = oracle.step(q, k, v, S)
        b = oracle.step_recompute(q, k, v, kp, vp, cu)
        err = np.abs(a - b).max() / max(1.0, np.abs(b).max())
        worst = max(worst, err)
    assert worst <= 1e-12, worst


def test_commit_order_independent():
    """S after k commits equals the sum of per-block outer products in any
    order (all permutations of 4 blocks), and equals one prefill of the
    blocks' concatenation (S_{1,2} = phi(K_1)^T V_1 + phi(K_2)^T V_2)."""
    H, d, blk = 2, 6, 5
    blocks = [(rnd(1, blk, H, d), rnd(1, blk, H, d)) for _ in range(4)]
    S0 = rnd(1, H, d, d)
    results = []
    for perm in itertools.permutations(range(4)):
        S = S0
        for i in perm:
            S = oracle.commit(blocks[i][0], blocks[i][1], S)
        results.append(S)
    for S in results[1:]:
        np.testing.assert_allclose(S, results[0], rtol=1e-12, atol=1e-12)
    kcat = np.concatenate([b[0][0] for b in blocks], 0)
    vcat = np.concatenate([b[1][0] for b in blocks], 0)
    Sp = oracle.prefill(kcat, vcat, np.array([0, 4 * blk]))
    np.testing.assert_allclose(results[0] - S0, Sp, rtol=1e-12, atol=1e-12)


def test_prefill_additive_over_splits():
    """Prefill of a prompt equals the sum of prefills of any split of it."""
    H, d, L = 2, 4, 50
    k, v = rnd(L, H, d), rnd(L, H, d)
    whole = oracle.prefill(k, v, np.array([0, L]))
    for cuts in ([7], [1, 2, 3], [49], [10, 20, 30, 40]):
        edges = [0] + cuts + [L]
        parts = oracle.prefill(k, v, np.array(edges))  # one "request" per piece
        np.testing.assert_allclose(parts.sum(0, keepdims=True), whole, rtol=1e-12, atol=1e-12)


def test_linearity():
    """O(S + dS) - O(S) = relu(Q) dS, and O is linear in V_a."""
    n, blk, H, d = 1, 6, 2, 7
    q, k, v, v2 = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    S, dS = rnd(n, H, d, d), rnd(n, H, d, d)
    o1 = oracle.step(q, k, v, S)
    o2 = oracle.step(q, k, v, S + dS)
    for h in range(H):
        np.testing.assert_allclose(o2[0, :, h] - o1[0, :, h], relu(q[0, :, h]) @ dS[0, h],
                                   rtol=1e-11, atol=1e-11)
    z = np.zeros((n, H, d, d))
    a = oracle.step(q, k, 2.0 * v - 3.0 * v2, z)
    b = 2.0 * oracle.step(q, k, v, z) - 3.0 * oracle.step(q, k, v2, z)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_permutations():
    """Permuting active key/value rows jointly leaves O unchanged; permuting
    query rows permutes O; permuting prompt tokens leaves S unchanged."""
    n, blk, H, d = 1, 7, 2, 5
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    o = oracle.step(q, k, v, S)
    p = RNG.permutation(blk)
    np.testing.assert_allclose(oracle.step(q, k[:, p], v[:, p], S), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.step(q[:, p], k, v, S), o[:, p], rtol=1e-12, atol=1e-12)
    kp, vp = rnd(30, H, d), rnd(30, H, d)
    t = RNG.permutation(30)
    np.testing.assert_allclose(oracle.prefill(kp[t], vp[t], np.array([0, 30])),
                               oracle.prefill(kp, vp, np.array([0, 30])), rtol=1e-12, atol=1e-12)


def test_ragged_rows_match_truncated_block():
    """A block with B_r valid rows gives the same rows as a block of length
    B_r; rows past B_r are not written."""
    n, blk, H, d = 3, 8, 2, 6
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    lens = np.array([8, 3, 1], np.int32)
    o = oracle.step(q, k, v, S, blk_lens=lens)
    S2 = oracle.commit(k, v, S, blk_lens=lens)
    for r in range(n):
        b = lens[r]
        sub = oracle.step(q[r:r + 1, :b], k[r:r + 1, :b], v[r:r + 1, :b], S[r:r + 1])
        np.testing.assert_allclose(o[r:r + 1, :b], sub, rtol=1e-13, atol=1e-13)
        assert np.all(o[r, b:] == 0.0)
        sub2 = oracle.commit(k[r:r + 1, :b], v[r:r + 1, :b], S[r:r + 1])
        np.testing.assert_allclose(S2[r:r + 1], sub2, rtol=1e-13, atol=1e-13)


def test_slot_indirection():
    """Request r reads and writes state slot slots[r]; other slots untouched."""
    n, blk, H, d = 3, 4, 1, 3
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    store = rnd(5, H, d, d)
    slots = np.array([4, 0, 2], np.int32)
    o = oracle.step(q, k, v, store, slots=slots)
    np.testing.assert_allclose(o, oracle.step(q, k, v, store[slots]), rtol=0, atol=0)
    s2 = oracle.commit(k, v, store, slots=slots)
    np.testing.assert_array_equal(s2[[1, 3]], store[[1, 3]])
    np.testing.assert_allclose(s2[slots], oracle.commit(k, v, store[slots]), rtol=0, atol=0)


# --------------------------------------------------------------------------
# Exact full-prefix step (the comparator the method replaces)
# --------------------------------------------------------------------------

def test_exact_step_is_sdpa_over_prefix_and_block():
    """Exact step = textbook softmax attention of Q_a over [K_p; K_a]."""
    H, d, blk = 2, 8, 4
    P = [0, 3, 17]
    cu = np.concatenate([[0], np.cumsum(P)])
    kp, vp = rnd(cu[-1], H, d), rnd(cu[-1], H, d)
    q, k, v = rnd(3, blk, H, d), rnd(3, blk, H, d), rnd(3, blk, H, d)
    o = oracle.exact_step(q, k, v, kp, vp, cu, scale=0.3)
    for r in range(3):
        kk = np.concatenate([kp[cu[r]:cu[r + 1]][None], k[r:r + 1]], 1)
        vv = np.concatenate([vp[cu[r]:cu[r + 1]][None], v[r:r + 1]], 1)
        np.testing.assert_allclose(o[r:r + 1], sdpa64(q[r:r + 1], kk, vv, 0.3), rtol=1e-12, atol=1e-12)
    # no prefix: identical to the hybrid step with an empty state
    z = oracle.step(q[:1], k[:1], v[:1], np.zeros((1, H, d, d)), scale=0.3)
    np.testing.assert_allclose(o[:1], z, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# The worked example's schedule at its own shape (L=10, B=4, H=2, d=16, fp32)
# --------------------------------------------------------------------------

def test_worked_example_schedule():
    """Blocks 4/4/2 generated in turn: block 1 is pure softmax attention;
    block b's linear term uses S built from blocks < b; the state form agrees
    with the formula form from the retained keys/values at every block."""
    from block_hybrid_linear_amd import synth
    from block_hybrid_linear_amd.workloads import WORKED_EXAMPLE as W
    S = np.zeros((1, W.heads, W.d, W.d))
    kept_k, kept_v = [], []
    for b, n in enumerate(W.block_lens):
        q = synth.normal((1, W.blk, W.heads, W.d), synth.seed_of(W.index, b, 0, 0), dtype=torch.float32)
        k = synth.normal((1, W.blk, W.heads, W.d), synth.seed_of(W.index, b, 0, 1), dtype=torch.float32)
        v = synth.normal((1, W.blk, W.heads, W.d), synth.seed_of(W.index, b, 0, 2), dtype=torch.float32)
        lens = np.array([n], np.int32)
        o = oracle.step(q, k, v, S, blk_lens=lens, scale=W.scale)
        qn, kn, vn = (x.double().numpy()[:, :n] for x in (q, k, v))
        if b == 0:
            np.testing.assert_allclose(o[:, :n], sdpa64(qn, kn, vn, W.scale), rtol=1e-12, atol=1e-12)
        kp = np.concatenate(kept_k, 0) if kept_k else np.zeros((0, W.heads, W.d))
        vp = np.concatenate(kept_v, 0) if kept_v else np.zeros((0, W.heads, W.d))
        o2 = oracle.step_recompute(q, k, v, kp, vp, np.array([0, kp.shape[0]]), blk_lens=lens, scale=W.scale)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
        S = oracle.commit(k, v, S, blk_lens=lens)
        kept_k.append(kn[0]); kept_v.append(vn[0])
        for h in range(W.heads):
            ref = sum(relu(kk[:, h]).T @ vv[:, h] for kk, vv in zip(kept_k, kept_v))
            np.testing.assert_allclose(S[0, h], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Normalised variant: block softmax scores and prefix linear scores share one
# denominator (z = sum phi(k_p) next to S)
# --------------------------------------------------------------------------

def _prefix_state(kp, vp, P):
    cu = np.array([0, P])
    return oracle.prefill(kp, vp, cu), oracle.znorm_prefill(kp, cu), cu


@pytest.mark.parametrize("blk,d", [(1, 3), (4, 16), (7, 5), (32, 64)])
def test_norm_empty_prefix_is_sdpa(blk, d):
    """S = 0 and z = 0 (no previous block): plain softmax attention over the
    block (torch, fp64)."""
    n, H = 2, 3
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    o = oracle.step_norm(q, k, v, np.zeros((n, H, d, d)), np.zeros((n, H, d)), scale=0.37)
    np.testing.assert_allclose(o, sdpa64(q, k, v, 0.37), rtol=1e-12, atol=1e-12)


def test_norm_nonpositive_queries_is_sdpa():
    """phi(q) = 0 when every query entry is <= 0: the prefix drops out of the
    numerator AND the denominator, whatever S and z hold."""
    n, blk, H, d = 2, 6, 2, 8
    q = -np.abs(rnd(n, blk, H, d))
    k, v = rnd(n, blk, H, d), rnd(n, blk, H, d)
    S, z = rnd(n, H, d, d), np.abs(rnd(n, H, d)) * 50
    o = oracle.step_norm(q, k, v, S, z, scale=0.5)
    np.testing.assert_allclose(o, sdpa64(q, k, v, 0.5), rtol=1e-12, atol=1e-12)


def test_norm_state_form_equals_recompute_bruteforce():
    """The state form (S, z) equals one weight per key -- exp(l) for block
    keys, phi(q).phi(k_t) for each retained prefix token -- over every tiny
    size."""
    H = 1
    worst = 0.0
    for blk, d, P in itertools.product(range(1, 5), (1, 2, 3, 5, 8), (0, 1, 2, 5, 12)):
        q, k, v = rnd(1, blk, H, d), rnd(1, blk, H, d), rnd(1, blk, H, d)
        kp, vp = rnd(P, H, d), rnd(P, H, d)
        S, z, cu = _prefix_state(kp, vp, P)
        a = oracle.step_norm(q, k, v, S, z)
        b = oracle.step_norm_recompute(q, k, v, kp, vp, cu)
        worst = max(worst, np.abs(a - b).max() / max(1.0, np.abs(b).max()))
    assert worst <= 1e-12, worst


def test_norm_constant_values_give_that_value():
    """When every block value and every prefix value is the same vector u the
    output is u for every query: the weights sum to one.  A term missing from
    the numerator or the denominator (or exp(-m) on one side only) breaks it."""
    blk, H, d, P = 6, 2, 7, 40
    u = rnd(d)
    q, k = 2 * rnd(1, blk, H, d), 2 * rnd(1, blk, H, d)
    v = np.broadcast_to(u, (1, blk, H, d)).copy()
    kp = rnd(P, H, d)
    vp = np.broadcast_to(u, (P, H, d)).copy()
    S, z, _ = _prefix_state(kp, vp, P)
    o = oracle.step_norm(q, k, v, S, z, scale=0.8)
    np.testing.assert_allclose(o, np.broadcast_to(u, o.shape), rtol=1e-12, atol=1e-12)


def test_norm_output_in_convex_hull_of_values():
    """All weights are >= 0, so each output entry lies between the smallest
    and largest value entry over block and prefix."""
    blk, H, d, P = 9, 2, 6, 30
    q, k, v = rnd(1, blk, H, d), rnd(1, blk, H, d), rnd(1, blk, H, d)
    kp, vp = rnd(P, H, d), rnd(P, H, d)
    S, z, _ = _prefix_state(kp, vp, P)
    o = oracle.step_norm(q, k, v, S, z)
    for h in range(H):
        vals = np.concatenate([v[0, :, h], vp[:, h]], 0)
        lo, hi = vals.min(0), vals.max(0)
        assert np.all(o[0, :, h] >= lo - 1e-12) and np.all(o[0, :, h] <= hi + 1e-12)


def test_norm_large_logits_are_finite():
    """Logits of several hundred: the block maximum is factored out of both
    sides, so nothing overflows, and against such scores the prefix's linear
    scores are negligible (softmax of the block, torch fp64)."""
    n, blk, H, d, P = 1, 8, 1, 4, 20
    q, k, v = 30 * rnd(n, blk, H, d), 30 * rnd(n, blk, H, d), rnd(n, blk, H, d)
    q[..., 0] = np.abs(q[..., 0]) + 30          # a positive feature, so phi(q).z > 0
    k[..., 0] = np.abs(k[..., 0]) + 30
    kp, vp = rnd(P, H, d), rnd(P, H, d)
    S, z, _ = _prefix_state(kp, vp, P)
    o = oracle.step_norm(q, k, v, S, z, scale=1.0)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, sdpa64(q, k, v, 1.0), rtol=1e-9, atol=1e-9)


def test_znorm_is_sum_of_relu_keys_in_any_order():
    """z after prefill = numpy's column sum of relu(K) per request; commits of
    blocks in any order add up to the prefill of their concatenation."""
    H, d, blk = 2, 5, 4
    lens = [0, 3, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = rnd(int(cu[-1]), H, d)
    z = oracle.znorm_prefill(k, cu)
    for r in range(3):
        np.testing.assert_allclose(z[r], relu(k[cu[r]:cu[r + 1]]).sum(0), rtol=1e-13, atol=1e-13)
    blocks = [rnd(1, blk, H, d) for _ in range(3)]
    z0 = rnd(1, H, d)
    res = []
    for perm in itertools.permutations(range(3)):
        zz = z0
        for i in perm:
            zz = oracle.znorm_commit(blocks[i], zz)
        res.append(zz)
    for zz in res[1:]:
        np.testing.assert_allclose(zz, res[0], rtol=1e-13, atol=1e-13)
    cat = np.concatenate([b[0] for b in blocks], 0)
    np.testing.assert_allclose(res[0] - z0, oracle.znorm_prefill(cat, np.array([0, 3 * blk])), rtol=1e-12,
                               atol=1e-12)
    lens = np.array([2], dtype=np.int32)                 # ragged block: rows past B_r are not read
    zr = oracle.znorm_commit(blocks[0], np.zeros((1, H, d)), blk_lens=lens)
    np.testing.assert_allclose(zr[0], relu(blocks[0][0, :2]).sum(0), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# The ELU + 1 feature map (phi(x) = x + 1 for x > 0, e^x otherwise), pinned to
# torch's ELU (a library routine), closed forms and the same invariants
# --------------------------------------------------------------------------

def elu1_lib(x):
    """torch.nn.functional.elu(x) + 1 in fp64 (the library's ELU, alpha = 1)."""
    return torch.nn.functional.elu(torch.from_numpy(np.asarray(x, dtype=np.float64))).numpy() + 1.0


def test_elu1_map_closed_forms():
    """phi(0) = 1 (ReLU: 0), phi(x) = x + 1 above 0, e^x below: one query row
    against a state whose row f is e_f scaled, so the linear part reads phi
    back feature by feature."""
    d = 6
    q = np.array([0.0, 2.5, -1.0, -40.0, 1e-9, -1e-9]).reshape(1, 1, 1, d)
    S = np.eye(d).reshape(1, 1, d, d) * 3.0
    o = oracle.step(q, q, np.zeros_like(q), S, phi="elu1")
    expect = 3.0 * np.array([1.0, 3.5, math.exp(-1.0), math.exp(-40.0), 1.0 + 1e-9, math.exp(-1e-9)])
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=1e-15, atol=0)
    o_relu = oracle.step(q, q, np.zeros_like(q), S, phi="relu")
    np.testing.assert_allclose(o_relu[0, 0, 0], 3.0 * np.maximum(q[0, 0, 0], 0.0), rtol=1e-15, atol=0)


@pytest.mark.parametrize("d", [2, 16, 64])
def test_elu1_zero_values_is_library_elu_times_S(d):
    """V_a = 0 with phi = ELU + 1: the linear term is (elu(Q_a) + 1) @ S
    (torch ELU, numpy matmul); the scale does not touch it."""
    n, blk, H = 2, 5, 2
    q, k = rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    o = oracle.step(q, k, np.zeros_like(q), S, scale=0.1, phi="elu1")
    for r in range(n):
        for h in range(H):
            np.testing.assert_allclose(o[r, :, h], elu1_lib(q[r, :, h]) @ S[r, h], rtol=1e-12, atol=1e-12)


def test_elu1_zero_queries_give_column_sums_of_S():
    """Q_a = 0: phi(0) = 1 for every feature, so the linear part is the sum of
    S's rows (and the softmax part the mean of the valid values)."""
    n, blk, H, d = 1, 6, 2, 5
    k, v = rnd(n, blk, H, d), rnd(n, blk, H, d)
    S = rnd(n, H, d, d)
    o = oracle.step(np.zeros((n, blk, H, d)), k, v, S, phi="elu1")
    for h in range(H):
        expect = v[0, :, h].mean(axis=0) + S[0, h].sum(axis=0)
        np.testing.assert_allclose(o[0, :, h], np.broadcast_to(expect, (blk, d)), rtol=1e-12, atol=1e-12)


def test_elu1_empty_prefix_is_sdpa():
    """The map does not touch the softmax part: S = 0 gives SDPA."""
    n, blk, H, d = 2, 7, 3, 8
    q, k, v = rnd(n, blk, H, d), rnd(n, blk, H, d), rnd(n, blk, H, d)
    o = oracle.step(q, k, v, np.zeros((n, H, d, d)), scale=0.3, phi="elu1")
    np.testing.assert_allclose(o, sdpa64(q, k, v, 0.3), rtol=1e-12, atol=1e-12)


def test_elu1_commit_and_prefill_are_library_products():
    """One committed token: S += outer(elu(k) + 1, v); a prefill is
    (elu(K) + 1)^T V over the prompt (torch ELU, numpy outer/matmul)."""
    d, H = 6, 2
    k, v = rnd(1, 1, H, d), rnd(1, 1, H, d)
    S0 = rnd(1, H, d, d)
    S = oracle.commit(k, v, S0, phi="elu1")
    for h in range(H):
        np.testing.assert_allclose(S[0, h], S0[0, h] + np.outer(elu1_lib(k[0, 0, h]), v[0, 0, h]),
                                   rtol=1e-13, atol=1e-13)
    lens = [0, 1, 9, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    kp, vp = rnd(cu[-1], H, d), rnd(cu[-1], H, d)
    Sp = oracle.prefill(kp, vp, cu, phi="elu1")
    for r in range(4):
        for h in range(H):
            kk, vv = kp[cu[r]:cu[r + 1], h], vp[cu[r]:cu[r + 1], h]
            np.testing.assert_allclose(Sp[r, h], elu1_lib(kk).T @ vv, rtol=1e-12, atol=1e-12)
    assert np.all(Sp[0] == 0.0)


def test_elu1_state_form_equals_formula_form_all_tiny_sizes():
    """The method's associativity with phi = ELU + 1: phi(Q)(phi(K_p)^T V_p) ==
    (phi(Q) phi(K_p)^T) V_p, for every B <= 3, d <= 3 and prefix <= 5, with the
    prefix folded by prefill and by commits in any order."""
    worst = 0.0
    for blk, d, P in itertools.product(range(1, 4), range(1, 4), range(0, 6)):
        H = 2
        q, k, v = rnd(1, blk, H, d), rnd(1, blk, H, d), rnd(1, blk, H, d)
        kp, vp = rnd(P, H, d), rnd(P, H, d)
        S = oracle.prefill(kp, vp, [0, P], phi="elu1")
        a = oracle.step(q, k, v, S, phi="elu1")
        b = oracle.step_recompute(q, k, v, kp, vp, [0, P], phi="elu1")
        worst = max(worst, float(np.abs(a - b).max()) / max(1.0, float(np.abs(b).max())))
        Sc = np.zeros((1, H, d, d))
        for t in RNG.permutation(P):
            Sc = oracle.commit(kp[None, t:t + 1], vp[None, t:t + 1], Sc, phi="elu1")
        np.testing.assert_allclose(Sc, S, rtol=1e-12, atol=1e-12)
    assert worst <= 1e-12


def test_elu1_normalised_variant():
    """Normalised with phi = ELU + 1: z is sum(elu(k) + 1) over the prompt
    (torch ELU); the state form equals the per-key form over all tiny sizes;
    phi > 0, so the denominator stays positive for all-negative inputs."""
    H, d = 2, 4
    lens = [0, 3, 11]
    cu = np.concatenate([[0], np.cumsum(lens)])
    kp, vp = rnd(cu[-1], H, d), rnd(cu[-1], H, d)
    z = oracle.znorm_prefill(kp, cu, phi="elu1")
    for r in range(3):
        np.testing.assert_allclose(z[r], elu1_lib(kp[cu[r]:cu[r + 1]]).sum(axis=0), rtol=1e-13, atol=1e-13)
    z1 = oracle.znorm_commit(kp[None, :5], np.zeros((1, H, d)), phi="elu1")
    np.testing.assert_allclose(z1[0], elu1_lib(kp[:5]).sum(axis=0), rtol=1e-13, atol=1e-13)
    for blk, dd, P in itertools.product(range(1, 4), range(1, 4), range(0, 5)):
        q, k, v = rnd(1, blk, 1, dd), rnd(1, blk, 1, dd), rnd(1, blk, 1, dd)
        kk, vv = rnd(P, 1, dd), rnd(P, 1, dd)
        S = oracle.prefill(kk, vv, [0, P], phi="elu1")
        zz = oracle.znorm_prefill(kk, [0, P], phi="elu1")
        a = oracle.step_norm(q, k, v, S, zz, phi="elu1")
        b = oracle.step_norm_recompute(q, k, v, kk, vv, [0, P], phi="elu1")
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    qn = -np.abs(rnd(1, 4, 1, 3)) - 5.0
    kn = -np.abs(rnd(6, 1, 3)) - 5.0
    S = oracle.prefill(kn, rnd(6, 1, 3), [0, 6], phi="elu1")
    zz = oracle.znorm_prefill(kn, [0, 6], phi="elu1")
    assert np.all(zz > 0)
    o = oracle.step_norm(qn, qn, rnd(1, 4, 1, 3), S, zz, phi="elu1")
    assert np.all(np.isfinite(o))
