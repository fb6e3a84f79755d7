"""Degenerate cases of the method, where the result is known without the
oracle's general path (summary page, "core formula": ReLU feature map, a
softmax inside the block, a linear term phi(Q) S over the prefix):

* queries <= 0: phi(Q) = 0, so the linear term vanishes whatever S holds and
  the output equals the same call with S = 0, bit for bit;
* keys <= 0: phi(K) = 0, so a commit leaves S unchanged and a prefill writes
  exact zeros;
* identical keys: every logit of a query is the same, so the softmax is
  uniform and the softmax part is the mean of the valid V rows.

Every kernel family is covered: 32-row blocks, 33..64-row blocks (head-pair
kernel) and 65..128-row blocks, head dims 64 and 128, plain and fused calls.
"""
import numpy as np
import pytest
import torch

import block_hybrid_linear_amd as bh
import oracle
from block_hybrid_linear_amd import synth
from parity import assert_parity, state_to_oracle, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPES = [(64, 32), (128, 32), (64, 64), (128, 48), (128, 64), (128, 100)]


def block(shape, seed, std=1.0):
    return synth.normal(shape, seed, std=std, dtype=torch.bfloat16).to(DEV)


@pytest.mark.parametrize("d,blk", SHAPES)
def test_nonpositive_queries_drop_the_linear_term(d, blk):
    n_req, H = 3, 2
    shape = (n_req, blk, H, d)
    q = -block(shape, 610).abs()                      # every query feature <= 0
    k, v = block(shape, 611), block(shape, 612)
    state = synth.normal((n_req, H, d, d), 613, dtype=torch.float32).to(DEV) * 3.0
    zero = torch.zeros_like(state)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    lens = torch.tensor([blk, blk // 2, 1], dtype=torch.int32, device=DEV)
    out_s = bh.hybrid_attn_step(q, k, v, state, slots, blk_lens=lens)
    out_0 = bh.hybrid_attn_step(q, k, v, zero, slots, blk_lens=lens)
    torch.cuda.synchronize()
    a, b = to64(out_s), to64(out_0)
    assert np.array_equal(a, b), f"d={d} blk={blk}: S changed the output although phi(Q) = 0"
    ref = oracle.step(q, k, v, np.zeros((n_req, H, d, d)), blk_lens=lens.cpu())
    mask = np.arange(blk)[None, :] < lens.cpu().numpy()[:, None]
    assert_parity(a[mask], ref[mask], torch.bfloat16, f"softmax-only output d={d} blk={blk}")


@pytest.mark.parametrize("d,blk", SHAPES)
def test_nonpositive_keys_commit_nothing(d, blk):
    n_req, H = 3, 2
    shape = (n_req, blk, H, d)
    q, v = block(shape, 620), block(shape, 621)
    k = -block(shape, 622).abs()                      # every key feature <= 0
    S0 = synth.normal((n_req, H, d, d), 623, dtype=torch.float32).to(DEV)
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    state = S0.clone()
    bh.hybrid_state_commit(k, v, state, slots)
    torch.cuda.synchronize()
    assert torch.equal(state, S0), f"d={d} blk={blk}: the commit of phi(K) = 0 changed S"
    if blk <= 64:
        state = S0.clone()
        out = bh.hybrid_attn_step_commit(q, k, v, state, slots)
        ref = bh.hybrid_attn_step(q, k, v, S0, slots)
        torch.cuda.synchronize()
        assert torch.equal(state, S0), f"d={d} blk={blk}: the fused commit of phi(K) = 0 changed S"
        assert torch.equal(out, ref), f"d={d} blk={blk}: fused output differs from the step's"


@pytest.mark.parametrize("d", [64, 128])
def test_nonpositive_keys_prefill_to_zero(d):
    H = 4
    lens = [0, 1, 300, 1000]
    cu = synth.cu_from_lengths(lens)
    total = int(cu[-1])
    k = -synth.normal((total, H, d), 630, dtype=torch.bfloat16).abs().to(DEV)
    v = synth.normal((total, H, d), 631, dtype=torch.bfloat16).to(DEV)
    state = torch.full((len(lens), H, d, d), 7.0, device=DEV)
    slots = torch.arange(len(lens), dtype=torch.int32, device=DEV)
    bh.hybrid_state_prefill(k, v, cu.to(DEV), state, slots, chunk=128)
    torch.cuda.synchronize()
    assert torch.count_nonzero(state).item() == 0, f"d={d}: prefill of phi(K) = 0 is not exactly zero"


@pytest.mark.parametrize("d,blk", SHAPES)
def test_identical_keys_give_uniform_attention(d, blk):
    n_req, H = 2, 2
    shape = (n_req, blk, H, d)
    q, v = block(shape, 640), block(shape, 641)
    k = block((n_req, 1, H, d), 642).expand(shape).contiguous()   # one key row repeated
    S = synth.normal((n_req, H, d, d), 643, dtype=torch.float32).to(DEV) * 0.1
    slots = torch.arange(n_req, dtype=torch.int32, device=DEV)
    lens = torch.tensor([blk, max(1, blk - 7)], dtype=torch.int32, device=DEV)
    out = bh.hybrid_attn_step(q, k, v, S, slots, blk_lens=lens)
    torch.cuda.synchronize()
    o = to64(out)
    S64 = state_to_oracle(S)
    q64, v64 = to64(q), to64(v)
    for r in range(n_req):
        n = int(lens[r])
        mean_v = v64[r, :n].mean(axis=0)                                  # [H, d]
        lin = np.einsum("ihf,hfc->ihc", np.maximum(q64[r, :n], 0.0), S64[r])
        ref = mean_v[None] + lin
        assert_parity(o[r, :n], ref, torch.bfloat16, f"uniform attention d={d} blk={blk} request {r}")
