"""The normalised variant on the GPU vs the fp64 oracle, through the C ABI.

The block's softmax scores and the prefix's linear scores share one
denominator, with z = sum phi(k) [n_slots, H, d] next to S.  States come from
an oracle prefill of a seeded prefix (rounded to fp32 and fed to both sides),
so S and z are consistent and the prefix carries real weight in the output.
Outputs are convex combinations of values, O(1), so the whole-output rule
also checks the softmax part; the matrix-core shapes are additionally held to
one bf16 ulp of the exact value.  Fused step + commit must reproduce the
plain normalised step bit for bit and update S and z as the oracle does.
"""
import numpy as np
import pytest
import torch

import block_hybrid_linear_amd as bh
import oracle
from block_hybrid_linear_amd import synth
from parity import assert_parity, rows_mask, state_from_oracle, state_to_oracle, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = -1024.0


def gen(shape, seed, dtype, std=1.0):
    return synth.normal(shape, seed, std=std, dtype=dtype).to(DEV)


def prefix_states(n_slots, H, d, P, seed):
    """S and z of a seeded N(0, 1) prefix of P tokens per slot (oracle prefill,
    rounded to fp32): returns (S fp32 device in the library layout, z fp32
    device, S fp64 oracle layout, z fp64)."""
    kp = synth.normal((n_slots * P, H, d), seed, dtype=torch.bfloat16)
    vp = synth.normal((n_slots * P, H, d), seed + 1, dtype=torch.bfloat16)
    cu = np.arange(n_slots + 1) * P
    S = oracle.prefill(kp, vp, cu).astype(np.float32).astype(np.float64)
    z = oracle.znorm_prefill(kp, cu).astype(np.float32).astype(np.float64)
    return state_from_oracle(S), torch.from_numpy(z).float().to(DEV), S, z


def bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


NORM_CASES = [  # (d, blk): matrix-core shapes first, then the fp32-arithmetic ones
    (128, 32), (128, 64), (128, 1), (128, 20), (128, 33), (64, 32), (64, 64), (64, 17), (32, 32), (32, 9),
    (128, 100), (32, 64), (16, 16),
]


@pytest.mark.parametrize("d,blk", NORM_CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_step_norm_parity(d, blk, dtype):
    n_req, H, P = 3, 4, 300
    seed = 30000 + 100 * d + blk
    q, k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(3))
    lens = torch.tensor([blk, max(1, blk // 2), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([2, 0, 1], dtype=torch.int32, device=DEV)
    state, z, S0, z0 = prefix_states(3, H, d, P, seed + 10)
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_norm(q, k, v, state, z, slots, out=out, blk_lens=lens)
    torch.cuda.synchronize()
    ref = oracle.step_norm(q, k, v, S0, z0, slots=slots, blk_lens=lens, scale=d ** -0.5)
    mask = rows_mask(lens, n_req, blk)
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL), "rows past B_r were written"
    assert_parity(o[mask], ref[mask], dtype, "normalised step")
    if dtype == torch.bfloat16 and d >= 32 and (blk <= 32 or (blk <= 64 and d >= 64)):
        r = ref[mask]
        bad = np.abs(o[mask] - r) > bf16_ulp(r) + 1e-5 * np.abs(r).max()
        assert not bad.any(), f"{bad.sum()} outputs off by more than one bf16 ulp"


@pytest.mark.parametrize("d,blk", [(128, 32), (128, 64), (64, 48)])
def test_step_norm_reduces_to_softmax_without_prefix(d, blk):
    """S = 0 and z = 0: the normalised step is the plain step with S = 0
    (softmax attention over the block)."""
    n_req, H = 2, 3
    q, k, v = (gen((n_req, blk, H, d), 31000 + d + t, torch.bfloat16) for t in range(3))
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    state = torch.zeros(n_req, H, d, d, device=DEV)
    z = torch.zeros(n_req, H, d, device=DEV)
    a = bh.hybrid_attn_step_norm(q, k, v, state, z, slots)
    b = bh.hybrid_attn_step(q, k, v, state, slots)
    torch.cuda.synchronize()
    ref = oracle.step(q, k, v, np.zeros((n_req, H, d, d)), scale=d ** -0.5)
    assert_parity(a, ref, torch.bfloat16, "no prefix")
    assert torch.allclose(a.float(), b.float(), rtol=0, atol=float(to64(ref).__abs__().max()) * 2 ** -8)


@pytest.mark.parametrize("d,blk", [(128, 32), (128, 64), (64, 64), (32, 32), (128, 100), (32, 48), (16, 8)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_step_commit_norm_parity(d, blk, dtype):
    n_req, H, P = 3, 5, 200
    seed = 32000 + 100 * d + blk
    q, k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(3))
    lens = torch.tensor([blk, max(1, (2 * blk) // 3), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([3, 0, 1], dtype=torch.int32, device=DEV)
    state, z, S0, z0 = prefix_states(4, H, d, P, seed + 10)
    plain = bh.hybrid_attn_step_norm(q, k, v, state, z, slots, blk_lens=lens)
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_commit_norm(q, k, v, state, z, slots, out=out, blk_lens=lens)
    torch.cuda.synchronize()
    mask = rows_mask(lens, n_req, blk)
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL)
    ref = oracle.step_norm(q, k, v, S0, z0, slots=slots, blk_lens=lens, scale=d ** -0.5)
    assert_parity(o[mask], ref[mask], dtype, "fused normalised step")
    assert torch.equal(out[torch.from_numpy(mask).to(DEV)], plain[torch.from_numpy(mask).to(DEV)])
    S1 = oracle.commit(k, v, S0, slots=slots, blk_lens=lens)
    z1 = oracle.znorm_commit(k, z0, slots=slots, blk_lens=lens)
    got_S, got_z = state_to_oracle(state), to64(z)
    assert np.array_equal(got_S[2], S0[2]) and np.array_equal(got_z[2], z0[2]), "a slot not named was modified"
    assert_parity(got_S, S1, dtype, "S after fused commit")
    assert_parity(got_z, z1, dtype, "z after fused commit")


@pytest.mark.parametrize("d,blk", [(128, 64), (64, 32), (32, 17), (16, 4)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_commit_norm_parity(d, blk, dtype):
    n_req, H = 3, 4
    seed = 33000 + 100 * d + blk
    k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(2))
    lens = torch.tensor([blk, max(1, blk // 2), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([4, 1, 2], dtype=torch.int32, device=DEV)
    state, z, S0, z0 = prefix_states(5, H, d, 50, seed + 10)
    bh.hybrid_state_commit_norm(k, v, state, z, slots, blk_lens=lens)
    torch.cuda.synchronize()
    got_S, got_z = state_to_oracle(state), to64(z)
    assert np.array_equal(got_z[[0, 3]], z0[[0, 3]]), "slots not named were modified"
    assert_parity(got_S, oracle.commit(k, v, S0, slots=slots, blk_lens=lens), dtype, "S after commit")
    assert_parity(got_z, oracle.znorm_commit(k, z0, slots=slots, blk_lens=lens), dtype, "z after commit")


@pytest.mark.parametrize("d,H", [(128, 2), (128, 3), (64, 2), (32, 2), (16, 2)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_norm_parity(d, H, dtype):
    lengths = [0, 1, 31, 4096, 4097, 900] if dtype == torch.bfloat16 else [0, 1, 31, 300]
    n_req = len(lengths)
    cu = synth.cu_from_lengths(lengths)
    total = int(cu[-1])
    k, v = (synth.normal((total, H, d), 34000 + d + t, dtype=dtype) for t in range(2))
    state = torch.full((n_req, H, d, d), 77.0, device=DEV)
    z = torch.full((n_req, H, d), 77.0, device=DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    bh.hybrid_state_prefill_norm(k.to(DEV), v.to(DEV), cu.to(DEV), state, z, slots, max_len=max(lengths), chunk=64)
    torch.cuda.synchronize()
    assert_parity(state_to_oracle(state), oracle.prefill(k, v, cu), dtype, "S after prefill")
    zr = oracle.znorm_prefill(k, cu)
    assert_parity(to64(z), zr, dtype, "z after prefill")
    assert np.all(to64(z)[0] == 0.0), "an empty prompt must reset z"


def test_prefill_norm_many_ragged_prompts():
    """Hundreds of prompts with head pairs: pieces of several prompts and both
    heads of a pair share workgroups; z is summed from the same partial slots
    as S."""
    rng = np.random.default_rng(79)
    lengths = [int(x) for x in rng.integers(0, 600, size=200)]
    lengths[3] = 0
    lengths[8] = 4000
    H, d = 4, 128
    cu = synth.cu_from_lengths(lengths)
    total = int(cu[-1])
    k, v = (synth.normal((total, H, d), 34500 + t) for t in range(2))
    state = torch.zeros(len(lengths), H, d, d, device=DEV)
    z = torch.zeros(len(lengths), H, d, device=DEV)
    slots = torch.arange(len(lengths), dtype=torch.int32, device=DEV)
    bh.hybrid_state_prefill_norm(k.to(DEV), v.to(DEV), cu.to(DEV), state, z, slots, chunk=64)
    torch.cuda.synchronize()
    assert_parity(state_to_oracle(state), oracle.prefill(k, v, cu), torch.bfloat16, "S")
    assert_parity(to64(z), oracle.znorm_prefill(k, cu), torch.bfloat16, "z")


def test_norm_generation_chain():
    """Prompt prefill, then blocks of steps with each block's last step fused
    with its commit, all normalised, against the oracle's own chain of S and z."""
    n_req, H, d, blk = 2, 4, 128, 64
    lengths = [700, 1500]
    cu = synth.cu_from_lengths(lengths)
    kp, vp = (synth.normal((int(cu[-1]), H, d), 35000 + t) for t in range(2))
    state = torch.zeros(n_req, H, d, d, device=DEV)
    z = torch.zeros(n_req, H, d, device=DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    bh.hybrid_state_prefill_norm(kp.to(DEV), vp.to(DEV), cu.to(DEV), state, z, slots)
    S_ref, z_ref = oracle.prefill(kp, vp, cu), oracle.znorm_prefill(kp, cu)
    for b in range(3):
        for t in range(3):
            q, k, v = (gen((n_req, blk, H, d), 35100 + 100 * b + 10 * t + i, torch.bfloat16) for i in range(3))
            if t == 2:
                out = bh.hybrid_attn_step_commit_norm(q, k, v, state, z, slots)
            else:
                out = bh.hybrid_attn_step_norm(q, k, v, state, z, slots)
            ref = oracle.step_norm(q, k, v, S_ref, z_ref, scale=d ** -0.5)
            torch.cuda.synchronize()
            assert_parity(out, ref, torch.bfloat16, f"block {b} step {t}")
        S_ref = oracle.commit(k, v, S_ref)
        z_ref = oracle.znorm_commit(k, z_ref)
    assert_parity(state_to_oracle(state), S_ref, torch.bfloat16, "final S")
    assert_parity(to64(z), z_ref, torch.bfloat16, "final z")
