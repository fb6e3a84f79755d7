"""The ELU + 1 feature map through the C ABI's *_phi calls against the oracle
with phi = ELU + 1: step (plain and normalised, with the softmax and linear
parts isolated), commit, the fused step + commit and prefill, on the
matrix-core shapes (d = 64, 128; blocks of 32 and 64 rows) and on shapes
that take the fp32 kernels.  States come from the oracle's own prefill of a
seeded prefix (so S and z agree), stored in the library's layout.  With
phi = ReLU the *_phi calls must give bit-identical results to the plain
calls."""
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
MAT_CASES = [(128, 32), (128, 64), (64, 32), (64, 64), (128, 17), (64, 50), (128, 100), (64, 200), (128, 256),
             (32, 130)]
FALLBACK_CASES = [(32, 40), (16, 32)]


def gen(shape, seed, dtype=torch.bfloat16, std=1.0):
    return synth.normal(shape, seed, std=std, dtype=dtype).to(DEV)


def prefix_state(n_slots, H, d, P, seed, dtype):
    """S and z of a seeded P-token prefix per slot, from the oracle (ELU + 1)."""
    kp = synth.normal((n_slots * P, H, d), seed, dtype=dtype)
    vp = synth.normal((n_slots * P, H, d), seed + 1, dtype=dtype)
    cu = synth.cu_from_lengths([P] * n_slots)
    S = oracle.prefill(kp, vp, cu, phi="elu1").astype(np.float32).astype(np.float64)
    z = oracle.znorm_prefill(kp, cu, phi="elu1").astype(np.float32).astype(np.float64)
    return S, z


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("d,blk", MAT_CASES + FALLBACK_CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_step_elu1(d, blk, dtype, norm):
    n_req, H, n_slots = 3, 4, 4
    seed = 31000 + 100 * d + blk + (50 if norm else 0)
    q, k, v = (gen((n_req, blk, H, d), seed + t, dtype) for t in range(3))
    lens = torch.tensor([blk, max(1, blk // 2), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([3, 0, 2], dtype=torch.int32, device=DEV)
    S, z = prefix_state(n_slots, H, d, 300, seed + 10, dtype)
    mask = rows_mask(lens, n_req, blk)
    scale = d ** -0.5
    parts = (("full", v, S, z), ("softmax part", v, 0 * S, 0 * z), ("linear part", torch.zeros_like(v), S, z))
    for what, vv, SS, zz in parts:
        out = torch.full_like(q, SENTINEL)
        st = state_from_oracle(SS)
        zt = torch.from_numpy(zz).float().to(DEV) if norm else None
        bh.hybrid_attn_step_phi(q, k, vv, st, slots, "elu1", z=zt, out=out, blk_lens=lens)
        torch.cuda.synchronize()
        if norm:
            ref = oracle.step_norm(q, k, vv, SS, zz, slots=slots, blk_lens=lens, scale=scale, phi="elu1")
        else:
            ref = oracle.step(q, k, vv, SS, slots=slots, blk_lens=lens, scale=scale, phi="elu1")
        o = to64(out)
        assert np.all(o[~mask] == SENTINEL), f"{what}: rows past B_r were written"
        assert_parity(o[mask], ref[mask], dtype, f"{what} (norm={norm})")


def _bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("d,blk", [(128, 64), (128, 32), (64, 64), (64, 32), (128, 200)])
def test_step_elu1_correctly_rounded(d, blk, fused):
    """phi(Q) as hi + lo bf16 on the matrix cores: every bf16 output within one
    ulp of the exact value (plus fp32 accumulation error)."""
    n_req, H = 3, 4
    seed = 32000 + 100 * d + blk
    q, k, v = (gen((n_req, blk, H, d), seed + t) for t in range(3))
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    state = synth.normal((n_req, H, d, d), seed + 3, std=10.0, dtype=torch.float32).to(DEV)
    S0 = state_to_oracle(state)
    call = bh.hybrid_attn_step_commit_phi if fused else bh.hybrid_attn_step_phi
    out = call(q, k, v, state, slots, "elu1")
    torch.cuda.synchronize()
    r = oracle.step(q, k, v, S0, scale=d ** -0.5, phi="elu1")
    o = to64(out)
    bound = _bf16_ulp(r) + 1e-5 * np.abs(r).max()
    bad = np.abs(o - r) > bound
    assert not bad.any(), f"{bad.sum()} outputs off by more than one bf16 ulp, worst {np.abs(o - r)[bad].max():.3e}"


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("d,blk", [(128, 32), (128, 64), (64, 32), (64, 64), (32, 48), (16, 20), (128, 200),
                                   (128, 21), (64, 9)])
def test_commit_and_fused_elu1(d, blk, norm):
    """Commit, and the fused step + commit (output bit-identical to the step's
    on the matrix-core shapes), against the oracle's commit with ELU + 1."""
    n_req, H, n_slots = 3, 4, 5
    seed = 33000 + 100 * d + blk + (50 if norm else 0)
    q, k, v = (gen((n_req, blk, H, d), seed + t) for t in range(3))
    lens = torch.tensor([blk, max(1, blk // 2), 1], dtype=torch.int32, device=DEV)
    slots = torch.tensor([4, 1, 2], dtype=torch.int32, device=DEV)
    S0, z0 = prefix_state(n_slots, H, d, 120, seed + 10, torch.bfloat16)
    S1 = oracle.commit(k, v, S0, slots=slots, blk_lens=lens, phi="elu1")
    z1 = oracle.znorm_commit(k, z0, slots=slots, blk_lens=lens, phi="elu1")
    zt = (lambda: torch.from_numpy(z0).float().to(DEV)) if norm else (lambda: None)
    # commit alone
    st, zz = state_from_oracle(S0), zt()
    bh.hybrid_state_commit_phi(k, v, st, slots, "elu1", z=zz, blk_lens=lens)
    torch.cuda.synchronize()
    got = state_to_oracle(st)
    assert np.array_equal(got[[0, 3]], S0[[0, 3]].astype(np.float32)), "slots not named were modified"
    assert_parity(got, S1, torch.bfloat16, "commit state")
    if norm:
        assert_parity(to64(zz), z1, torch.bfloat16, "commit z")
    # fused
    st, zz = state_from_oracle(S0), zt()
    plain = bh.hybrid_attn_step_phi(q, k, v, state_from_oracle(S0), slots, "elu1", z=zt(), blk_lens=lens)
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_commit_phi(q, k, v, st, slots, "elu1", z=zz, out=out, blk_lens=lens)
    torch.cuda.synchronize()
    mask = rows_mask(lens, n_req, blk)
    if norm:
        ref = oracle.step_norm(q, k, v, S0, z0, slots=slots, blk_lens=lens, scale=d ** -0.5, phi="elu1")
    else:
        ref = oracle.step(q, k, v, S0, slots=slots, blk_lens=lens, scale=d ** -0.5, phi="elu1")
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL)
    assert_parity(o[mask], ref[mask], torch.bfloat16, "fused output")
    assert_parity(state_to_oracle(st), S1, torch.bfloat16, "fused commit state")
    if norm:
        assert_parity(to64(zz), z1, torch.bfloat16, "fused commit z")
    if d >= 32 and blk <= 64:
        m = torch.from_numpy(mask).to(DEV)
        assert torch.equal(out[m], plain[m]), "fused output differs from the step's"


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("H,d", [(4, 128), (3, 128), (2, 64), (2, 32), (2, 16)])
@pytest.mark.parametrize("chunk", [64, 256])
def test_prefill_elu1(H, d, chunk, norm):
    """Prefill with ELU + 1 (head pairs at d = 128 with an even head count,
    single heads otherwise) against the oracle: ragged prompts, one empty."""
    lens = [700, 0, 1, 2300, 129]
    cu = synth.cu_from_lengths(lens)
    seed = 34000 + 10 * H + d + chunk
    k = gen((int(cu[-1]), H, d), seed)
    v = gen((int(cu[-1]), H, d), seed + 1)
    n_slots = len(lens) + 1
    slots = torch.arange(1, n_slots, dtype=torch.int32, device=DEV)
    state = torch.full((n_slots, H, d, d), 5.0, device=DEV)
    z = torch.full((n_slots, H, d), 5.0, device=DEV) if norm else None
    bh.hybrid_state_prefill_phi(k, v, cu.to(DEV), state, slots, "elu1", z=z, chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.prefill(k, v, cu, phi="elu1")
    got = state_to_oracle(state)
    assert np.all(got[0] == 5.0), "slot 0 was written"
    assert np.all(got[2] == 0.0), "the empty prompt did not reset its slot"
    assert_parity(got[1:], ref, torch.bfloat16, "prefill state")
    if norm:
        zr = oracle.znorm_prefill(k, cu, phi="elu1")
        assert_parity(to64(z)[1:], zr, torch.bfloat16, "prefill z")


def test_relu_map_is_the_plain_calls():
    """phi = ReLU through the *_phi calls runs the plain calls' kernels:
    bit-identical outputs and states."""
    n_req, blk, H, d = 2, 64, 4, 128
    q, k, v = (gen((n_req, blk, H, d), 35000 + t) for t in range(3))
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    state = synth.normal((n_req, H, d, d), 35003, std=20.0, dtype=torch.float32).to(DEV)
    a = bh.hybrid_attn_step(q, k, v, state, slots)
    b = bh.hybrid_attn_step_phi(q, k, v, state, slots, "relu")
    s1, s2 = state.clone(), state.clone()
    bh.hybrid_state_commit(k, v, s1, slots)
    bh.hybrid_state_commit_phi(k, v, s2, slots, "relu")
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(s1, s2)


def test_unknown_map_rejected():
    n_req, blk, H, d = 1, 8, 1, 64
    q = gen((n_req, blk, H, d), 35100)
    state = torch.zeros(1, H, d, d, device=DEV)
    slots = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(bh.HybridAttnError, match="feature map"):
        bh.hybrid_attn_step_phi(q, q, q, state, slots, 7)
