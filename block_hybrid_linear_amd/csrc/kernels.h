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
    float* state_rw;            // fused step + commit: the same store, updated in place
    const int32_t* slots;
    void* out;
    const int32_t* blk_lens;
    float* z;                   // normalised variant: z = sum phi(k) [n_slots][heads][d]
                                // (read by the step, updated by the fused commit); NULL: plain sum
    int32_t n_req, n_slots, heads, blk, d;
    float scale;
    bool dtype_bf16;
    int32_t phi;                // feature map: 0 = ReLU, 1 = ELU + 1
};

// ReLU(K)^T V over token rows, shared by the block commit and prompt prefill.
//   commit : rows of request r are r*blk + [0, B_r); the result is added to
//            the state slot in place.
//   prefill: the (request, head, chunk) list is split into `slices` equal
//            ranges; each slice workgroup writes partial states into the
//            workspace and a reduction sums them per (request, head).
struct PhiKVArgs {
    const void* k;
    const void* v;
    float* state;               // state store (commit: updated; prefill: overwritten)
    const int32_t* slots;
    const int32_t* blk_lens;    // commit (may be NULL)
    const int64_t* cu;          // prefill: [n_req + 1]
    int64_t* plan;              // prefill workspace: [n_req + 2], written by the slice kernel for the reduce
    float* partial;             // prefill workspace: [slices + n_req * heads][d][d]
    float* z;                   // normalised variant: z = sum phi(k) [n_slots][heads][d] (prefill: overwritten);
                                // NULL: plain
    float* zpartial;            // prefill workspace, normalised variant: [slices + n_req * heads][d]
    int64_t total_tokens;       // prefill
    int32_t chunk;              // prefill
    int32_t slices;             // prefill: slice workgroups, spu per unit
    int32_t spu;                // prefill: slices per unit
    int32_t hp;                 // prefill: heads per unit (1 or 2, divides heads)
    int32_t n_req, n_slots, heads, blk, d;
    bool dtype_bf16;
    int32_t phi;                // feature map: 0 = ReLU, 1 = ELU + 1
};

// Heads per prefill unit: bf16 with d = 128 and an even head count streams two
// adjacent heads per workgroup (512 contiguous bytes per token row).
inline int prefill_group(int d, int heads, bool bf16) { return bf16 && d == 128 && heads % 2 == 0 ? 2 : 1; }

// Prefill slice workgroups per unit for head dim d, hp heads per unit and
// upr units per request: about (d == 32 ? 2048 : 512) / hp workgroups in all
// (two 4-wave or one 8-wave workgroup per compute unit of an MI355X), the same
// number for every unit, at least one.  Fixed per shape, so results do not
// depend on the device.  The workgroups' partial states, upr * spu * hp, never
// exceed max(2048 or 512, heads).
inline int prefill_base_slices(int d) { return d == 32 ? 2048 : 512; }
inline int prefill_spu(int d, int hp, int upr)
{
    const int per = prefill_base_slices(d) / hp / upr;
    return per > 0 ? per : 1;
}

// Exact softmax attention of the active block over [prefix; block] (the step
// without linearisation).  The (request, head, key chunk) list is split into
// `slices` equal ranges; each slice workgroup writes, per (request, head) it
// touches, an unnormalised partial output with its running max and sum, and
// a combine kernel merges them per (request, head).
struct ExactArgs {
    const void* q;
    const void* k;
    const void* v;              // active block [n_req][blk][heads][d]
    const void* kc;
    const void* vc;             // prefix cache [total_prefix][heads][d]
    const int64_t* cu;          // [n_req + 1] prefix offsets into the cache
    int64_t total_prefix;
    void* out;
    const int32_t* blk_lens;
    int64_t* plan;              // workspace: [n_req + 2]
    float* partial;             // workspace: [slices + n_req * heads][exact_slot_floats]
    int32_t chunk, slices, n_req, heads, blk, d;
    float scale;
    bool dtype_bf16;
};

// Slice workgroups of the exact step: as many as the 256 compute units of an
// MI355X hold at once for the matrix-core variant of (d, blk), so the
// balanced split runs in one round.  Per compute unit that is the smaller of
// 4 SIMDs x waves per SIMD (3, 2, 1 for one, two, four query tiles) / (d / 32)
// waves per workgroup and what its LDS footprint allows out of 160 KB.
// Fixed per (d, blk), so results do not depend on the device.
inline int exact_slices(int d, int blk)
{
    const int t = blk <= 32 ? 0 : (blk <= 64 ? 1 : 2);
    static const int per_cu[3][3] = {{9, 6, 4},      // d = 32
                                     {5, 4, 2},      // d = 64
                                     {3, 2, 1}};     // d = 128
    if (d != 32 && d != 64 && d != 128) return 1024;
    return 256 * per_cu[d == 32 ? 0 : (d == 64 ? 1 : 2)][t];
}

// Rows of one partial slot: the query rows of the kernel that runs for blk
// (one, two or four 32-row tiles).  A slot holds rows x d unnormalised
// outputs, then the running max and the running sum of each row.
__host__ __device__ inline int exact_slot_rows(int blk) { return blk <= 32 ? 32 : (blk <= 64 ? 64 : 128); }
inline int exact_slot_floats(int blk, int d) { return exact_slot_rows(blk) * (d + 2); }

hipError_t launch_step(const StepArgs& a, hipStream_t stream);
hipError_t launch_step_commit(const StepArgs& a, hipStream_t stream);
hipError_t launch_znorm_commit(const StepArgs& a, hipStream_t stream);
hipError_t launch_commit(const PhiKVArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PhiKVArgs& a, hipStream_t stream);

hipError_t launch_exact(const ExactArgs& a, hipStream_t stream);

}  // namespace ha
