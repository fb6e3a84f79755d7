"""Offsets past 2^31 elements.

Every index into the state store, the block tensors and the packed prompts is
64-bit.  These cases place the checked units where a 32-bit element offset
would wrap: a state store of 16400 slots x 32 heads x 128 x 128 fp32 (34 GB,
2^32 floats), block tensors of 2.15e9 bf16 elements (4.3 GB each) at block
lengths 32, 64 and 100 (one kernel each), and 524,800 packed prompt tokens
whose last prompt ends past element 2^31.  Units that are not checked hold
zeros or the values an earlier case left; every unit is independent, so
only the checked ones need seeded data, and the oracle sees just those.
"""
import numpy as np
import pytest
import torch

import block_hybrid_linear_amd as bh
import oracle
from block_hybrid_linear_amd import synth
from parity import assert_parity, state_from_oracle, state_to_oracle, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = -1024.0
H, D = 32, 128
N_SLOTS = 16400
FLAT = 16400 * 32 * H * D          # 2,149,580,800 elements per block tensor
assert FLAT > 2 ** 31 and N_SLOTS * H * D * D > 2 ** 32


@pytest.fixture(scope="module")
def big():
    free, _ = torch.cuda.mem_get_info()
    need = N_SLOTS * H * D * D * 4 + 4 * FLAT * 2
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 1e9:.0f} GB of device memory ({free / 1e9:.0f} GB free)")
    bufs = {"state": torch.zeros((N_SLOTS, H, D, D), dtype=torch.float32, device=DEV)}
    for name in ("q", "k", "v", "out"):
        bufs[name] = torch.zeros(FLAT, dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    yield bufs
    bufs.clear()
    torch.cuda.empty_cache()


def seeded_rows(buf, shape, idx, seed):
    """Writes seeded N(0, 1) bf16 values into buf.view(shape)[idx]; returns them."""
    view = buf.view(shape)
    x = synth.normal((len(idx),) + shape[1:], seed, dtype=torch.bfloat16)
    view[torch.as_tensor(idx, device=DEV)] = x.to(DEV)
    return x


@pytest.mark.parametrize("blk", [32, 64, 100])
def test_large_offsets_step_and_commits(big, blk):
    n_req = FLAT // (blk * H * D)
    shape = (n_req, blk, H, D)
    assert n_req * blk * H * D > 2 ** 31
    checked = [0, n_req // 2, n_req - 1]                   # the last one's rows sit past element 2^31
    print(f"blk={blk} n_req={n_req} checked={checked}", flush=True)
    q, k, v = (seeded_rows(big[t], shape, checked, 81000 + 10 * blk + i) for i, t in enumerate("qkv"))
    qd, kd, vd, out = (big[t].view(shape) for t in ("q", "k", "v", "out"))
    state = big["state"]
    slots_all = torch.arange(N_SLOTS - 1, N_SLOTS - 1 - n_req, -1, dtype=torch.int32, device=DEV)
    slots = slots_all[checked].long()                       # the checked units' slots, top slot first
    lens_all = torch.full((n_req,), blk, dtype=torch.int32, device=DEV)
    lens_all[checked[1]] = blk - 5                          # one ragged block
    lens = [blk, blk - 5, blk]
    S0 = synth.normal((3, H, D, D), 82000 + blk).double().numpy()
    state[slots] = state_from_oracle(S0)
    spare = None
    if n_req < N_SLOTS:                                     # highest unnamed slot, just below the named ones
        spare = N_SLOTS - 1 - n_req
        state[spare] = synth.normal((H, D, D), 83000 + blk).to(DEV)
        spare_before = state[spare].clone()
    scale = D ** -0.5
    mask = np.arange(blk)[None, :] < np.array(lens)[:, None]

    ref = oracle.step(q, k, v, S0, blk_lens=lens, scale=scale)
    out.fill_(SENTINEL)
    bh.hybrid_attn_step(qd, kd, vd, state, slots_all, out=out, blk_lens=lens_all, scale=scale)
    torch.cuda.synchronize()
    o = to64(out[torch.as_tensor(checked, device=DEV)])
    assert np.all(o[~mask] == SENTINEL), "step: rows past B_r were written"
    assert_parity(o[mask], ref[mask], torch.bfloat16, f"step at blk={blk}")

    out.fill_(SENTINEL)
    bh.hybrid_attn_step_commit(qd, kd, vd, state, slots_all, out=out, blk_lens=lens_all, scale=scale)
    torch.cuda.synchronize()
    o = to64(out[torch.as_tensor(checked, device=DEV)])
    assert np.all(o[~mask] == SENTINEL), "fused step: rows past B_r were written"
    assert_parity(o[mask], ref[mask], torch.bfloat16, f"fused step output at blk={blk}")
    S1 = oracle.commit(k, v, S0, blk_lens=lens)
    assert_parity(state_to_oracle(state[slots]), S1, torch.bfloat16, f"state after the fused commit at blk={blk}")

    k2, v2 = (seeded_rows(big[t], shape, checked, 84000 + 10 * blk + i) for i, t in enumerate("kv"))
    bh.hybrid_state_commit(kd, vd, state, slots_all, blk_lens=lens_all)
    torch.cuda.synchronize()
    S2 = oracle.commit(k2, v2, S1, blk_lens=lens)
    assert_parity(state_to_oracle(state[slots]), S2, torch.bfloat16, f"state after the commit at blk={blk}")
    if spare is not None:
        assert torch.equal(state[spare], spare_before), "an unnamed slot was written"


def test_large_offsets_prefill(big):
    lens = [300000, 204800, 20000]                          # 524,800 tokens; the last prompt ends past 2^31
    total = sum(lens)
    assert total * H * D == FLAT
    cu = synth.cu_from_lengths(lens)
    shape = (total, H, D)
    kd, vd = big["k"].view(shape), big["v"].view(shape)
    checked = [(2, 0), (2, 17), (2, 31), (1, 9)]            # (prompt, head)
    data = {}
    for i, (r, h) in enumerate(checked):
        s0, s1 = int(cu[r]), int(cu[r + 1])
        kx = synth.normal((s1 - s0, 1, D), 85000 + 2 * i, dtype=torch.bfloat16)
        vx = synth.normal((s1 - s0, 1, D), 85001 + 2 * i, dtype=torch.bfloat16)
        kd[s0:s1, h:h + 1] = kx.to(DEV)
        vd[s0:s1, h:h + 1] = vx.to(DEV)
        data[(r, h)] = (kx, vx)
    slots = torch.tensor([5, 9000, N_SLOTS - 1], dtype=torch.int32, device=DEV)
    state = big["state"]
    print(f"prefill: lens={lens} slots={slots.tolist()} checked={checked}", flush=True)
    bh.hybrid_state_prefill(kd, vd, cu.to(DEV), state, slots)
    torch.cuda.synchronize()
    for (r, h), (kx, vx) in data.items():
        ref = oracle.prefill(kx, vx, torch.tensor([0, kx.shape[0]], dtype=torch.int64))
        slot = int(slots[r])
        got = state_to_oracle(state[slot:slot + 1, h:h + 1])
        assert_parity(got, ref, torch.bfloat16, f"prefill of prompt {r}, head {h}")
