"""The five synthetic workloads, named by what they are.

Sizes follow the block-hybrid attention setting: blockwise semi-autoregressive
decoding (blocks generated one after another, each block denoised for a few
steps with all its tokens in parallel), the hybrid layer's active-block softmax
plus a linear term over the fp32 prefix state, and a prompt folded into that
state by prefill.  The worked example of the paper summary page ("technical
details in action": L = 10, B = 4, blocks 4/4/2, phi = ReLU) is the first.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    index: int                 # seed base (synth.seed_of)
    name: str
    n_req: int
    heads: int
    d: int
    blk: int
    dtype: str                 # "f32" | "bf16"
    std: float = 1.0           # std of the Q/K/V draws
    block_lens: tuple = ()     # block schedule of a generation (worked example)
    n_blocks: int = 1
    steps_per_block: int = 1
    prefix_range: tuple = ()   # (lo, hi) inclusive, prefix tokens already in S
    prompt_range: tuple = ()   # (lo, hi) inclusive, prompt tokens prefilled
    prefix_fixed: int = 0      # fixed prefix length folded into S
    chunk: int = 256
    notes: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return self.d ** -0.5


WORKED_EXAMPLE = Workload(1, "worked_example_L10_B4_d16_f32", n_req=1, heads=2, d=16, blk=4,
                          dtype="f32", block_lens=(4, 4, 2), n_blocks=3)
SINGLE_STEP = Workload(2, "single_step_b1_h16_d64_B32_prefix4096", n_req=1, heads=16, d=64,
                       blk=32, dtype="bf16", prefix_fixed=4096)
SERVING_STEP = Workload(3, "serving_step_b64_h32_d128_B32_prefix1k-16k", n_req=64, heads=32,
                        d=128, blk=32, dtype="bf16", prefix_range=(1024, 16384))
BLOCK_LOOP = Workload(4, "block_loop_b32_h32_d128_32x32blocks_8steps", n_req=32, heads=32,
                      d=128, blk=32, dtype="bf16", std=0.5, n_blocks=32, steps_per_block=8)
PREFILL_DECODE = Workload(5, "prefill16k-64k_decode_b8_h32_d128_16x64blocks_4steps", n_req=8,
                          heads=32, d=128, blk=64, dtype="bf16", n_blocks=16, steps_per_block=4,
                          prompt_range=(16384, 65536), chunk=256)

ALL = (WORKED_EXAMPLE, SINGLE_STEP, SERVING_STEP, BLOCK_LOOP, PREFILL_DECODE)
