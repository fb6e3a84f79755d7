"""The layer-stack timing harness of the benchmark (``bench.py --stack``) at a
small size.  The attention output of a layer, taken from inside the stack's
forward pass, is checked against the oracle wherever the layer's inputs come
from the harness alone (the first layer: projections of the seeded input):
a one-layer stack whose layer is hybrid against the step (its state drawn by
the harness), and the first layer of a two-layer stack, exact, against the
exact step over the harness's prefix cache.  A later layer's inputs depend
on the library's outputs, so there the test only checks that the hybrid mode
changes the hybrid layer and nothing before it.  This pins what the stack
timing measures to the method."""
import os
import sys

import pytest
import torch

import oracle
from parity import assert_parity, state_to_oracle

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CFG = {"layers": 2, "hybrid_layers": 1, "n_req": 3, "heads": 4, "head_dim": 64, "block": 32, "mlp_inter": 512}
SCALE = CFG["head_dim"] ** -0.5


def test_hybrid_layer_of_the_stack_is_the_step():
    import bench
    stk = bench.LayerStack(dict(CFG, layers=1), (50, 700), dev="cuda", base=7_400_000)
    assert stk.hybrid_at == {0}
    cap = {}
    stk.forward(True, capture=cap)
    torch.cuda.synchronize()
    q, k, v, out = (t.cpu() for t in cap[0])
    ref = oracle.step(q, k, v, state_to_oracle(stk.states[0]), scale=SCALE)
    e = assert_parity(out, ref, torch.bfloat16, "hybrid layer")
    print(f"[stack] hybrid layer: rel err {e:.2e}", flush=True)


def test_exact_layer_of_the_stack_is_the_exact_step():
    import bench
    stk = bench.LayerStack(CFG, (50, 700), dev="cuda", base=7_500_000)
    assert stk.hybrid_at == {1}
    cap_h, cap_e = {}, {}
    stk.forward(True, capture=cap_h)
    stk.forward(False, capture=cap_e)
    torch.cuda.synchronize()
    q, k, v, out = (t.cpu() for t in cap_h[0])
    ref = oracle.exact_step(q, k, v, stk.kc.cpu(), stk.vc.cpu(), stk.cu, scale=SCALE)
    e = assert_parity(out, ref, torch.bfloat16, "exact layer 0")
    print(f"[stack] exact layer 0: rel err {e:.2e}", flush=True)
    assert torch.equal(cap_h[0][3], cap_e[0][3]), "layer 0 differs between the modes"
    diff = (cap_h[1][3].float() - cap_e[1][3].float()).abs().max().item()
    assert diff > 1e-2, "the hybrid layer ran the exact step"
