// Kernel argument blocks and launchers of libhybrid_attn (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ha {

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* state;
    const int32_t* slots;
    void* out;
    const int32_t* blk_lens;
    int32_t n_req, n_slots, heads, blk, d;
    float scale;
    bool dtype_bf16;
};

// phi(K)^T V over token rows, shared by the block commit and prompt prefill.
//   commit : rows of request r are r*blk + [0, B_r); the result is added to
//            the state slot in place.
//   prefill: rows of request r are cu[r] + [g*G, min((g+1)*G, L_r)) for group
//            g; the result is written as a partial state into the workspace.
struct PhiKVArgs {
    const void* k;
    const void* v;
    float* state;               // commit: state store
    const int32_t* slots;       // commit
    const int32_t* blk_lens;    // commit (may be NULL)
    const int64_t* cu;          // prefill
    float* partial;             // prefill: [n_req][groups][heads][d][d]
    int64_t total_tokens;       // prefill
    int64_t group_tokens;       // prefill: G
    int32_t groups;             // prefill: groups per request
    int32_t n_req, n_slots, heads, blk, d;
    bool dtype_bf16;
};

struct ReduceArgs {
    const float* partial;
    const int64_t* cu;
    float* state;
    const int32_t* slots;
    int64_t total_tokens;
    int64_t group_tokens;
    int32_t groups;
    int32_t n_req, n_slots, heads, d;
};

hipError_t launch_step(const StepArgs& a, hipStream_t stream);
hipError_t launch_commit(const PhiKVArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PhiKVArgs& a, const ReduceArgs& r, hipStream_t stream);

}  // namespace ha
