"""Block-hybrid attention for MI355X (gfx950).

For each head, the active denoising block gets exact softmax attention over
itself plus a linear-attention term ReLU(Q_a) S over all previous blocks, where
S = sum of ReLU(K_p)^T V_p is an fp32 d x d prefix state ("Retrofitting Linear
Attention into Diffusion Language Models").  The hot path is three calls of
the C-ABI library libhybrid_attn.so (hand-written HIP kernels), exposed here
with the same names:

    hybrid_attn_step      one denoising step of a hybrid layer
    hybrid_state_commit   S += ReLU(K_blk)^T V_blk when a block is finished
    hybrid_state_prefill  S = sum over a prompt of ReLU(k)^T v
    hybrid_attn_step_commit  a block's last step fused with its commit

the normalised variant (block softmax scores and prefix linear scores over one
denominator, with z = sum ReLU(k) next to S):

    hybrid_attn_step_norm, hybrid_attn_step_commit_norm,
    hybrid_state_commit_norm, hybrid_state_prefill_norm

the same calls with the feature map as an argument (ReLU, the worked
example's, or ELU + 1), plain or normalised by whether z is given:

    hybrid_attn_step_phi, hybrid_attn_step_commit_phi,
    hybrid_state_commit_phi, hybrid_state_prefill_phi

the prefill for callers that cannot allocate (its workspace is the library's
own device scratch):

    hybrid_state_prefill_noalloc

and, for comparison, the exact step the method replaces:

    hybrid_exact_step     softmax attention of the active block over its
                          whole prefix KV cache and itself

PyTorch only provides device memory and streams.
"""
from .binding import (HybridAttnError, abi_version, hybrid_attn_step, hybrid_attn_step_commit,
                      hybrid_attn_step_commit_norm, hybrid_attn_step_commit_phi, hybrid_attn_step_norm,
                      hybrid_attn_step_phi, hybrid_exact_step, hybrid_state_commit_phi, hybrid_state_prefill_phi,
                      hybrid_exact_step_workspace_bytes, hybrid_state_commit, hybrid_state_commit_norm,
                      hybrid_state_prefill, hybrid_state_prefill_noalloc, hybrid_state_prefill_norm,
                      hybrid_state_prefill_workspace_bytes,
                      load_library, prepare_commit, prepare_exact_step, prepare_prefill, prepare_prefill_norm,
                      prepare_step, prepare_step_commit, prepare_step_commit_norm, prepare_step_norm)

__all__ = ["HybridAttnError", "abi_version", "hybrid_attn_step", "hybrid_attn_step_commit",
           "hybrid_attn_step_commit_norm", "hybrid_attn_step_commit_phi", "hybrid_attn_step_norm",
           "hybrid_attn_step_phi", "hybrid_exact_step", "hybrid_state_commit_phi", "hybrid_state_prefill_phi",
           "hybrid_exact_step_workspace_bytes", "hybrid_state_commit", "hybrid_state_commit_norm",
           "hybrid_state_prefill", "hybrid_state_prefill_noalloc", "hybrid_state_prefill_norm",
           "hybrid_state_prefill_workspace_bytes",
           "load_library", "prepare_commit", "prepare_exact_step", "prepare_prefill", "prepare_prefill_norm",
           "prepare_step", "prepare_step_commit", "prepare_step_commit_norm", "prepare_step_norm"]
