"""hybrid_state_prefill_noalloc (the prefill whose workspace is the library's
own device scratch) against hybrid_state_prefill with a caller workspace,
through the C ABI: two calls in a row on one GPU, the second smaller than the
first, so the second runs over the first one's leftovers in the scratch.  Both
calls run the same kernels, so the states must be bit-identical; each is also
held to the oracle's tolerance rule."""
import numpy as np
import pytest
import torch

import block_hybrid_linear_amd as bh
import oracle
from block_hybrid_linear_amd import synth
from parity import assert_parity, state_to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(lens, H, d, seed, dtype=torch.bfloat16):
    cu = synth.cu_from_lengths(torch.tensor(lens, dtype=torch.int64))
    total = int(cu[-1])
    k = synth.normal((total, H, d), seed, dtype=dtype).to(DEV)
    v = synth.normal((total, H, d), seed + 1, dtype=dtype).to(DEV)
    return k, v, cu


@pytest.mark.parametrize("calls", [
    # (prompt lengths, heads, d, slots of the store) -- first large, then small
    ([(3000, 1, 777, 4100, 0, 2600), 32, 128, 9], [(5, 300), 4, 64, 3]),
    ([(9000, 12), 6, 128, 4], [(70,), 3, 32, 2]),
])
def test_noalloc_prefill_matches_workspace_prefill(calls):
    print(f"[noalloc] calls {[(len(c[0]), c[1], c[2]) for c in calls]}", flush=True)
    for i, (lens, H, d, n_slots) in enumerate(calls):
        k, v, cu = _case(list(lens), H, d, 91_000 + 100 * i + d)
        n_req = len(lens)
        slots = torch.arange(n_slots - n_req, n_slots, dtype=torch.int32, device=DEV)   # the top slots
        cud = cu.to(DEV)
        fill = float(3 + i)
        st_ref = torch.full((n_slots, H, d, d), fill, device=DEV)
        st_na = torch.full((n_slots, H, d, d), fill, device=DEV)
        ws = torch.empty(bh.hybrid_state_prefill_workspace_bytes(n_req, H, d, k.shape[0], 0, 256),
                         dtype=torch.uint8, device=DEV)
        bh.hybrid_state_prefill(k, v, cud, st_ref, slots, chunk=256, workspace=ws)
        bh.hybrid_state_prefill_noalloc(k, v, cud, st_na, slots, chunk=256)
        torch.cuda.synchronize()
        assert torch.equal(st_na, st_ref), f"call {i}: states differ from the workspace call's"
        S = state_to_oracle(st_na)
        assert np.all(S[: n_slots - n_req] == fill), f"call {i}: unnamed slots written"
        ref = oracle.prefill(k, v, cu)
        assert_parity(S[n_slots - n_req:], ref, k.dtype, f"noalloc prefill call {i}")
