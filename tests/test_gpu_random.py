"""Seeded random configurations through every call, against the oracle.

Each case draws its shapes from a fixed seed: the head dim, the head count
(odd and even, so both prefill unit widths run), the number of requests, the
block length (1..128, the range of every step kernel), ragged valid lengths
(zero included), an injective slot map into a larger store, the dtype, the
scale, the prompt lengths (empty ones included) and the prefill chunk.  The
step, the fused step + commit, the commit and the prefill, plain and
normalised, and the exact comparator are compared with the oracle under the
tolerance rule of the other parity tests; rows past a request's valid length
and slots no request names must be left untouched.
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
SENTINEL = -1024.0  # exact in bf16 and fp32


def draw(case):
    rng = np.random.default_rng(91000 + case)
    d = int(rng.choice([128, 128, 64, 32, 16]))
    dtype = torch.float32 if (d == 16 or rng.random() < 0.2) else torch.bfloat16
    H = int(rng.integers(1, 6))
    n_req = int(rng.integers(1, 5))
    blk = int(rng.choice([1, 7, 32, 33, 48, 64, 65, 100, 128]))
    lens = [int(rng.integers(0, blk + 1)) for _ in range(n_req)]
    lens[int(rng.integers(0, n_req))] = blk                # at least one full block
    n_slots = n_req + int(rng.integers(1, 4))
    slots = rng.permutation(n_slots)[:n_req].astype(np.int32)
    scale = float(rng.choice([d ** -0.5, 0.05, 0.3]))
    prompts = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 1500, size=n_req)]
    chunk = int(rng.choice([1, 13, 64, 256, 1000]))
    return dict(d=d, dtype=dtype, H=H, n_req=n_req, blk=blk, lens=lens, n_slots=n_slots, slots=slots,
                scale=scale, prompts=prompts, chunk=chunk, seed=92000 + 100 * case)


def consistent_state(c):
    """S and z of a short seeded prefix per slot (oracle prefill, rounded to
    fp32 for both sides), so the normalised calls see z that matches S."""
    n_slots, H, d = c["n_slots"], c["H"], c["d"]
    plens = [17 + 5 * s for s in range(n_slots)]
    cu = synth.cu_from_lengths(plens)
    kp, vp = (synth.normal((int(cu[-1]), H, d), c["seed"] + 50 + t) for t in range(2))
    S = oracle.prefill(kp, vp, cu).astype(np.float32).astype(np.float64)
    z = oracle.znorm_prefill(kp, cu).astype(np.float32).astype(np.float64)
    return S, z


def block_inputs(c, salt):
    shape = (c["n_req"], c["blk"], c["H"], c["d"])
    return [synth.normal(shape, c["seed"] + salt + t, dtype=c["dtype"]).to(DEV) for t in range(3)]


def unnamed(c):
    return np.setdiff1d(np.arange(c["n_slots"]), c["slots"])


CASES = list(range(20))


@pytest.mark.parametrize("case", CASES)
def test_random_step_and_commits(case):
    c = draw(case)
    print(f"case {case}: d={c['d']} H={c['H']} n_req={c['n_req']} blk={c['blk']} lens={c['lens']} "
          f"dtype={c['dtype']}", flush=True)
    q, k, v = block_inputs(c, 0)
    S0, _ = consistent_state(c)
    state = state_from_oracle(S0)
    slots = torch.from_numpy(c["slots"]).to(DEV)
    lens = torch.tensor(c["lens"], dtype=torch.int32, device=DEV)
    mask = rows_mask(lens, c["n_req"], c["blk"])
    ref = oracle.step(q, k, v, S0, slots=c["slots"], blk_lens=c["lens"], scale=c["scale"])

    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step(q, k, v, state, slots, out=out, blk_lens=lens, scale=c["scale"])
    torch.cuda.synchronize()
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL), "step: rows past B_r were written"
    assert_parity(o[mask], ref[mask], c["dtype"], "step")

    out2 = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_commit(q, k, v, state, slots, out=out2, blk_lens=lens, scale=c["scale"])
    torch.cuda.synchronize()
    o2 = to64(out2)
    assert np.all(o2[~mask] == SENTINEL), "fused step: rows past B_r were written"
    assert_parity(o2[mask], ref[mask], c["dtype"], "fused step output")
    S1 = oracle.commit(k, v, S0, slots=c["slots"], blk_lens=c["lens"])
    got = state_to_oracle(state)
    assert np.array_equal(got[unnamed(c)], S0[unnamed(c)]), "fused commit touched an unnamed slot"
    assert_parity(got, S1, c["dtype"], "state after the fused commit")

    k2, v2, _ = block_inputs(c, 10)
    bh.hybrid_state_commit(k2, v2, state, slots, blk_lens=lens)
    torch.cuda.synchronize()
    S2 = oracle.commit(k2, v2, S1, slots=c["slots"], blk_lens=c["lens"])
    got = state_to_oracle(state)
    assert np.array_equal(got[unnamed(c)], S0[unnamed(c)]), "commit touched an unnamed slot"
    assert_parity(got, S2, c["dtype"], "state after the commit")


@pytest.mark.parametrize("case", CASES)
def test_random_prefill(case):
    c = draw(case)
    print(f"case {case}: d={c['d']} H={c['H']} prompts={c['prompts']} chunk={c['chunk']} dtype={c['dtype']}",
          flush=True)
    cu = synth.cu_from_lengths(c["prompts"])
    total = int(cu[-1])
    k, v = (synth.normal((total, c["H"], c["d"]), c["seed"] + 30 + t, dtype=c["dtype"]) for t in range(2))
    S0, z0 = consistent_state(c)
    state = state_from_oracle(S0)
    z = torch.from_numpy(z0).float().to(DEV)
    slots = torch.from_numpy(c["slots"]).to(DEV)
    bh.hybrid_state_prefill(k.to(DEV), v.to(DEV), cu.to(DEV), state, slots, chunk=c["chunk"])
    torch.cuda.synchronize()
    Sref = oracle.prefill(k, v, cu, S=S0, slots=c["slots"])
    got = state_to_oracle(state)
    assert np.array_equal(got[unnamed(c)], S0[unnamed(c)]), "prefill touched an unnamed slot"
    assert_parity(got, Sref, c["dtype"], "state after the prefill")

    state = state_from_oracle(S0)
    bh.hybrid_state_prefill_norm(k.to(DEV), v.to(DEV), cu.to(DEV), state, z, slots, chunk=c["chunk"])
    torch.cuda.synchronize()
    zref = oracle.znorm_prefill(k, cu, z=z0, slots=c["slots"])
    assert_parity(state_to_oracle(state), Sref, c["dtype"], "state after the normalised prefill")
    gz = to64(z)
    assert np.array_equal(gz[unnamed(c)], z0[unnamed(c)]), "normalised prefill touched an unnamed z"
    assert_parity(gz, zref, c["dtype"], "z after the normalised prefill")


@pytest.mark.parametrize("case", CASES)
def test_random_normalised_calls(case):
    c = draw(case)
    print(f"case {case}: d={c['d']} H={c['H']} n_req={c['n_req']} blk={c['blk']} lens={c['lens']} "
          f"dtype={c['dtype']}", flush=True)
    q, k, v = block_inputs(c, 20)
    S0, z0 = consistent_state(c)
    state = state_from_oracle(S0)
    z = torch.from_numpy(z0).float().to(DEV)
    slots = torch.from_numpy(c["slots"]).to(DEV)
    lens = torch.tensor(c["lens"], dtype=torch.int32, device=DEV)
    mask = rows_mask(lens, c["n_req"], c["blk"])
    ref = oracle.step_norm(q, k, v, S0, z0, slots=c["slots"], blk_lens=c["lens"], scale=c["scale"])

    out = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_norm(q, k, v, state, z, slots, out=out, blk_lens=lens, scale=c["scale"])
    torch.cuda.synchronize()
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL), "normalised step: rows past B_r were written"
    assert_parity(o[mask], ref[mask], c["dtype"], "normalised step")

    out2 = torch.full_like(q, SENTINEL)
    bh.hybrid_attn_step_commit_norm(q, k, v, state, z, slots, out=out2, blk_lens=lens, scale=c["scale"])
    torch.cuda.synchronize()
    assert_parity(to64(out2)[mask], ref[mask], c["dtype"], "normalised fused step output")
    S1 = oracle.commit(k, v, S0, slots=c["slots"], blk_lens=c["lens"])
    z1 = oracle.znorm_commit(k, z0, slots=c["slots"], blk_lens=c["lens"])
    assert_parity(state_to_oracle(state), S1, c["dtype"], "state after the normalised fused commit")
    assert_parity(to64(z), z1, c["dtype"], "z after the normalised fused commit")

    k2, v2, _ = block_inputs(c, 40)
    bh.hybrid_state_commit_norm(k2, v2, state, z, slots, blk_lens=lens)
    torch.cuda.synchronize()
    S2 = oracle.commit(k2, v2, S1, slots=c["slots"], blk_lens=c["lens"])
    z2 = oracle.znorm_commit(k2, z1, slots=c["slots"], blk_lens=c["lens"])
    gz = to64(z)
    assert np.array_equal(gz[unnamed(c)], z0[unnamed(c)]), "normalised commit touched an unnamed z"
    assert_parity(state_to_oracle(state), S2, c["dtype"], "state after the normalised commit")
    assert_parity(gz, z2, c["dtype"], "z after the normalised commit")


@pytest.mark.parametrize("case", CASES[:12])
def test_random_exact_step(case):
    """The exact comparator on the same random shapes, over random prefix
    lengths (empty ones included) and key chunks."""
    c = draw(case)
    rng = np.random.default_rng(93000 + case)
    prefixes = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(1, 2500, size=c["n_req"])]
    chunk = int(rng.choice([1, 32, 100, 256, 3000]))
    print(f"case {case}: d={c['d']} H={c['H']} blk={c['blk']} lens={c['lens']} prefixes={prefixes} "
          f"chunk={chunk} dtype={c['dtype']}", flush=True)
    q, k, v = block_inputs(c, 60)
    cu = synth.cu_from_lengths(prefixes)
    kc, vc = (synth.normal((int(cu[-1]), c["H"], c["d"]), c["seed"] + 70 + t, dtype=c["dtype"]).to(DEV)
              for t in range(2))
    lens = torch.tensor(c["lens"], dtype=torch.int32, device=DEV)
    out = torch.full_like(q, SENTINEL)
    bh.hybrid_exact_step(q, k, v, kc, vc, cu.to(DEV), out=out, blk_lens=lens, scale=c["scale"], chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.exact_step(q, k, v, kc, vc, cu, blk_lens=c["lens"], scale=c["scale"])
    mask = rows_mask(lens, c["n_req"], c["blk"])
    o = to64(out)
    assert np.all(o[~mask] == SENTINEL), "exact step: rows past B_r were written"
    assert_parity(o[mask], ref[mask], c["dtype"], "exact step")
