/*
 * hybrid_attn.h -- C ABI of the block-hybrid attention library for MI355X
 * (gfx950), libhybrid_attn.so.
 *
 * Block-hybrid attention (paper "Retrofitting Linear Attention into Diffusion
 * Language Models": abstract; paper-daily summary page, sections "core
 * formula" and "technical details in action") keeps exact softmax attention
 * inside the active denoising block and replaces attention over previous
 * blocks by linear attention with the feature map phi(x) = ReLU(x):
 *
 *     O = Softmax(scale * Q_a K_a^T) V_a + phi(Q_a) S,
 *     S = sum over committed tokens of phi(k)^T v          (d x d, fp32)
 *
 * and after a block is finished S += phi(K_blk)^T V_blk (the worked example's
 * S_1 = phi(K_1)^T V_1, S_{1,2} = phi(K_1)^T V_1 + phi(K_2)^T V_2).  A prompt
 * folds into S the same way (prefill).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers are DEVICE pointers unless stated otherwise.  `stream` is a
 * hipStream_t passed as void* (NULL = the default stream).  Every call is
 * asynchronous: it validates its host arguments, enqueues kernels on `stream`
 * and returns; device faults surface at the caller's next synchronisation.
 *
 * Ownership: the caller owns all memory.  The library allocates nothing and
 * keeps no state between calls apart from a thread-local error string.
 *
 * Element types (ha_dtype): HA_F32 (float) or HA_BF16 (bfloat16 bits in
 * uint16).  q/k/v/out share one dtype; the state is always fp32.  All
 * accumulation is fp32; a bf16 output is rounded to nearest even once.
 *
 * Layouts (row-major, innermost dimension contiguous, no other strides):
 *   active block  q, k, v, out  [n_req][blk][heads][d]
 *   packed prompt k, v          [total_tokens][heads][d], request r owns rows
 *                               cu_seqlens[r] .. cu_seqlens[r+1]-1
 *   state store   state         [n_slots][heads][d][d] fp32.  Each d x d block
 *                               holds S TRANSPOSED: state[s][h][c][f] =
 *                               S[f][c] = sum phi(k)_f v_c, i.e. row = value
 *                               dimension c, column = feature f of phi(k).
 *                               The step contracts S over f; stored this way,
 *                               the 8 consecutive f a lane's matrix-core
 *                               operand holds are 32 contiguous bytes (one
 *                               16-byte load pair, or one 16-byte LDS read),
 *                               where row = f would make them a column.
 *   slots         int32[n_req]  request r uses state slot slots[r].
 *   blk_lens      int32[n_req]  valid rows B_r of request r's block, or NULL
 *                               for "all blk rows valid".
 *
 * Ragged blocks: only the first B_r rows of q/k/v are read and only the first
 * B_r rows of out are written; rows B_r..blk-1 of out are left untouched.
 * Device data is never read for validation on the host.  On the device a
 * request whose slot lies outside [0, n_slots) or whose B_r <= 0 is skipped
 * (nothing read or written for it); B_r > blk is treated as blk.
 *
 * Errors: a non-OK status other than HA_ERR_HIP is returned BEFORE anything
 * is enqueued, so outputs and the state are untouched.  hybrid_last_error()
 * gives a message for the calling thread's last non-OK status.
 *   HA_ERR_INVALID_ARG  NULL pointer, negative or zero size, blk > 256
 *                       (blk > 128 for hybrid_exact_step),
 *                       non-finite scale, chunk < 1, workspace too small,
 *                       a q/k/v/out/state/cache pointer not 16-byte aligned
 *                       or a workspace not 256-byte aligned (allocations
 *                       from hipMalloc or torch satisfy both).
 *   HA_ERR_UNSUPPORTED  d not in {16, 32, 64, 128} or unknown dtype.
 *   HA_ERR_HIP          the kernel launch failed (hipGetLastError).
 * A call with n_req == 0 does nothing and returns HA_OK (pointers unused).
 *
 * Aliasing: out must not overlap q, k, v or state; the state store must not
 * overlap any input.  Calls that write the same state slots must be ordered
 * on one stream.
 */
#ifndef HYBRID_ATTN_H
#define HYBRID_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYBRID_ATTN_ABI_VERSION 2
#define HYBRID_ATTN_MAX_BLK 256         /* rows of an active block */
#define HYBRID_ATTN_EXACT_MAX_BLK 128   /* rows of an active block in hybrid_exact_step */

typedef enum {
    HA_OK = 0,
    HA_ERR_INVALID_ARG = 1,
    HA_ERR_UNSUPPORTED = 2,
    HA_ERR_HIP = 3
} ha_status;

typedef enum { HA_F32 = 0, HA_BF16 = 1 } ha_dtype;

/*
 * One denoising step of a hybrid layer ("core formula"; worked example:
 * "block 2's output is the sum of the softmax result and phi(Q_2) S_1"):
 *
 *   out[r, i, h, :] = sum_{j < B_r} P_ij v_j  +  phi(q_i) S_{slots[r], h}
 *   P_ij = exp(scale q_i.k_j - m_i) / sum_{j' < B_r} exp(scale q_i.k_j' - m_i)
 *
 * for i < B_r, with no mask inside the block (all tokens of the active block
 * are denoised in parallel).  `scale` multiplies the logits only; pass
 * 1/sqrtf(d) for the usual scaling.  The state is read-only here.
 */
ha_status hybrid_attn_step(const void* q, const void* k, const void* v,
                           const float* state, const int32_t* slots,
                           void* out, const int32_t* blk_lens,
                           int32_t n_req, int32_t n_slots, int32_t heads,
                           int32_t blk, int32_t d, float scale,
                           ha_dtype dtype, void* stream);

/*
 * Commit a finished block into the prefix state (worked example:
 * S_{1,2} = S_1 + phi(K_2)^T V_2):
 *
 *   S_{slots[r], h} += sum_{j < B_r} phi(k_j)^T v_j        (in place, fp32)
 *
 * Not idempotent: committing the same block twice adds it twice.  Requests
 * of one call must use distinct slots (two requests committing into one slot
 * in the same call race).
 */
ha_status hybrid_state_commit(const void* k, const void* v, float* state,
                              const int32_t* slots, const int32_t* blk_lens,
                              int32_t n_req, int32_t n_slots, int32_t heads,
                              int32_t blk, int32_t d, ha_dtype dtype,
                              void* stream);

/*
 * The last denoising step of a block fused with its commit (worked example:
 * block 2's output uses S_1, then S_{1,2} = S_1 + phi(K_2)^T V_2):
 *
 *   out = hybrid_attn_step(q, k, v, state)            (from the OLD state)
 *   S_{slots[r], h} += sum_{j < B_r} phi(k_j)^T v_j    (in place)
 *
 * with the same arguments, rules and results as hybrid_attn_step followed by
 * hybrid_state_commit on the same k, v (up to fp32 rounding of the state),
 * but in one launch that reads q, k and v once and writes the state once.
 * At d = 128 with 33..64 rows it also reads the state once; shorter blocks
 * read the old tiles a second time for the commit, mostly from the caches.
 * Requests of one call must use distinct slots (as for hybrid_state_commit).
 */
ha_status hybrid_attn_step_commit(const void* q, const void* k, const void* v,
                                  float* state, const int32_t* slots,
                                  void* out, const int32_t* blk_lens,
                                  int32_t n_req, int32_t n_slots,
                                  int32_t heads, int32_t blk, int32_t d,
                                  float scale, ha_dtype dtype, void* stream);

/*
 * Fold whole prompts into the state, OVERWRITING each request's slot:
 *
 *   S_{slots[r], h} = sum_{t in prompt r} phi(k_t)^T v_t
 *
 * (the prefix summary of the worked example, taken over prompt tokens).  A
 * request with an empty prompt gets S = 0, which is also the reset path.
 *
 * cu_seqlens: device int64[n_req + 1], non-decreasing, cu_seqlens[0] = 0,
 *   cu_seqlens[n_req] = total_tokens.  A request whose rows fall outside
 *   [0, total_tokens] (or run backwards) is treated as an empty prompt.
 * total_tokens: HOST scalar, rows of k and v.
 * max_len: HOST scalar >= 0, an upper bound of the prompt lengths; the
 *   current kernels do not need it (kept for ABI stability).
 * slots: the requests of one call must use distinct slots (two requests
 *   writing one slot in the same call would leave either one's sum there).
 * chunk: prompts are cut into chunks of `chunk` tokens; for every head (or
 *   pair of adjacent heads) the chunks of all prompts form one list, which is
 *   split into the same number of equal ranges, one per workgroup, so the
 *   work is balanced whatever the prompt lengths and all heads are cut at
 *   the same token positions.  Two kernel launches: the workgroups (each
 *   working out its range from cu_seqlens) write a (request, head) whose
 *   chunks lie in one range straight into the state, and one fp32 partial
 *   state per range into `workspace` for one that spans several; a second
 *   kernel sums those partials in ascending range order (deterministic: the
 *   same inputs give bit-identical states).  The result does not depend on
 *   chunk beyond fp32 rounding.
 * workspace: device scratch of at least
 *   hybrid_state_prefill_workspace_bytes(...) bytes (non-NULL when
 *   n_req > 0); its contents on entry do not matter.  Calls sharing one
 *   workspace must be ordered on one stream.
 */
ha_status hybrid_state_prefill(const void* k, const void* v,
                               const int64_t* cu_seqlens,
                               int64_t total_tokens, int64_t max_len,
                               float* state, const int32_t* slots,
                               int32_t n_req, int32_t n_slots, int32_t heads,
                               int32_t d, int32_t chunk,
                               void* workspace, size_t workspace_bytes,
                               ha_dtype dtype, void* stream);

/* Workspace size for hybrid_state_prefill and hybrid_state_prefill_norm with
 * the same arguments (host): the plan ((n_req + 2) int64, padded to 256
 * bytes) and (max(W, heads) + n_req * heads) fp32 partial states of d x d + d
 * floats (S and z), W = 2048 for d = 32 and 512 otherwise; 0 when n_req,
 * heads, d or chunk is <= 0. */
size_t hybrid_state_prefill_workspace_bytes(int32_t n_req, int32_t heads,
                                            int32_t d, int64_t total_tokens,
                                            int64_t max_len, int32_t chunk);

/*
 * hybrid_state_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call, the same kernels and the same results, but the
 * workspace is the library's own scratch array instead of an argument.  The
 * array is a fixed HYBRID_ATTN_NOALLOC_SCRATCH_BYTES (128 MiB) of device
 * memory, one copy per GPU the library runs on, held until the process ends;
 * its address on a device is looked up once, on the first call on that
 * device (the device of `stream`; NULL = the current device).  The call
 * itself allocates and frees nothing.
 *
 * A call whose hybrid_state_prefill_workspace_bytes(...) exceeds the maximum
 * returns HA_ERR_INVALID_ARG before anything is enqueued (e.g. d = 128 and
 * 32 heads allow up to 47 requests per call).  HA_ERR_HIP: the scratch
 * array's address could not be obtained on the stream's device.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race and
 * give undefined results; order them on one stream.  The array keeps the last
 * call's contents, which no call depends on.
 */
#define HYBRID_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
ha_status hybrid_state_prefill_noalloc(const void* k, const void* v,
                                       const int64_t* cu_seqlens,
                                       int64_t total_tokens, int64_t max_len,
                                       float* state, const int32_t* slots,
                                       int32_t n_req, int32_t n_slots,
                                       int32_t heads, int32_t d, int32_t chunk,
                                       ha_dtype dtype, void* stream);

/*
 * Normalised variant.  The pages say the retrofit largely follows LoLCATs
 * (summary page, sections "problem solving" and "method"; abstract page) and
 * print no formula for a normaliser; the reading implemented here is that
 * method's hybrid attention with one shared denominator: for query i of the
 * active block,
 *
 *   O_i = (sum_j exp(l_ij) v_j + phi(q_i) S) / (sum_j exp(l_ij) + phi(q_i) . z)
 *
 * over the B_r valid block keys j (l_ij = scale <q_i, k_j>), with a second
 * per-(slot, head) state z = sum over committed / prompt tokens of phi(k)
 * next to S.  With S = 0 and z = 0 (no previous block) it is plain softmax
 * attention over the block.
 *
 * z: device fp32 [n_slots][heads][d], 16-byte aligned.  The calls below take
 * the arguments of their plain counterparts plus z and keep their
 * conventions (slots, blk_lens, alignment, errors); z is required (NULL is
 * HA_ERR_INVALID_ARG).  Per query, both sides are divided by
 * exp(max(m_i, ln(phi(q_i) . z))) (m_i the block's largest logit), so the
 * denominator's larger part is one; results are undefined only when both
 * parts underflow fp32.
 *
 * hybrid_attn_step_norm: the output above; reads S and z.
 * hybrid_attn_step_commit_norm: the same output from the old S and z, then
 *   S += phi(K)^T V and z += sum_j phi(k_j) over the block's valid rows.
 * hybrid_state_commit_norm: S += phi(K)^T V and z += sum_j phi(k_j).
 * hybrid_state_prefill_norm: S and z of each request's slot overwritten by
 *   the sums over its prompt (an empty prompt gives S = 0, z = 0); the
 *   workspace is hybrid_state_prefill_workspace_bytes(...).
 */
ha_status hybrid_attn_step_norm(const void* q, const void* k, const void* v,
                                const float* state, const float* z,
                                const int32_t* slots, void* out,
                                const int32_t* blk_lens, int32_t n_req,
                                int32_t n_slots, int32_t heads, int32_t blk,
                                int32_t d, float scale, ha_dtype dtype,
                                void* stream);

ha_status hybrid_attn_step_commit_norm(const void* q, const void* k,
                                       const void* v, float* state, float* z,
                                       const int32_t* slots, void* out,
                                       const int32_t* blk_lens, int32_t n_req,
                                       int32_t n_slots, int32_t heads,
                                       int32_t blk, int32_t d, float scale,
                                       ha_dtype dtype, void* stream);

ha_status hybrid_state_commit_norm(const void* k, const void* v, float* state,
                                   float* z, const int32_t* slots,
                                   const int32_t* blk_lens, int32_t n_req,
                                   int32_t n_slots, int32_t heads, int32_t blk,
                                   int32_t d, ha_dtype dtype, void* stream);

ha_status hybrid_state_prefill_norm(const void* k, const void* v,
                                    const int64_t* cu_seqlens,
                                    int64_t total_tokens, int64_t max_len,
                                    float* state, float* z,
                                    const int32_t* slots, int32_t n_req,
                                    int32_t n_slots, int32_t heads, int32_t d,
                                    int32_t chunk, void* workspace,
                                    size_t workspace_bytes, ha_dtype dtype,
                                    void* stream);

/*
 * The feature map as an explicit argument.  The pages' worked example uses
 * phi = ReLU (every call above); the summary page names phi only as a
 * kernel-function map ("core formula") of linear attention ("technical
 * approach").  HA_PHI_ELU1 is ELU + 1, phi(x) = x + 1 for x > 0 and e^x
 * otherwise: positive everywhere, so the normalised variant's denominator
 * never vanishes.  The state S, z and every rule of the calls above are
 * unchanged; a state must be built and read with one map.
 *
 * The calls below are the calls above with the map as an argument, and z
 * optional: z == NULL gives the plain sum (hybrid_attn_step and its kin),
 * z != NULL the normalised variant (the *_norm calls).  With HA_PHI_RELU
 * they run the same kernels as those calls.  ELU + 1 is not exact in bf16:
 * on the matrix cores phi of a bf16 input is formed in fp32 and split into
 * hi + lo bf16 (one more pass per product); it runs on the matrix cores for
 * every bf16 shape with d >= 32 (blocks of up to 256 rows), and in plain fp32
 * kernels otherwise.
 *   HA_ERR_UNSUPPORTED  unknown feature map.
 */
typedef enum { HA_PHI_RELU = 0, HA_PHI_ELU1 = 1 } ha_feature_map;

ha_status hybrid_attn_step_phi(const void* q, const void* k, const void* v,
                               const float* state, const float* z,
                               const int32_t* slots, void* out,
                               const int32_t* blk_lens, int32_t n_req,
                               int32_t n_slots, int32_t heads, int32_t blk,
                               int32_t d, float scale, ha_feature_map phi,
                               ha_dtype dtype, void* stream);

ha_status hybrid_attn_step_commit_phi(const void* q, const void* k,
                                      const void* v, float* state, float* z,
                                      const int32_t* slots, void* out,
                                      const int32_t* blk_lens, int32_t n_req,
                                      int32_t n_slots, int32_t heads,
                                      int32_t blk, int32_t d, float scale,
                                      ha_feature_map phi, ha_dtype dtype,
                                      void* stream);

ha_status hybrid_state_commit_phi(const void* k, const void* v, float* state,
                                  float* z, const int32_t* slots,
                                  const int32_t* blk_lens, int32_t n_req,
                                  int32_t n_slots, int32_t heads, int32_t blk,
                                  int32_t d, ha_feature_map phi,
                                  ha_dtype dtype, void* stream);

ha_status hybrid_state_prefill_phi(const void* k, const void* v,
                                   const int64_t* cu_seqlens,
                                   int64_t total_tokens, int64_t max_len,
                                   float* state, float* z,
                                   const int32_t* slots, int32_t n_req,
                                   int32_t n_slots, int32_t heads, int32_t d,
                                   int32_t chunk, void* workspace,
                                   size_t workspace_bytes, ha_feature_map phi,
                                   ha_dtype dtype, void* stream);

/*
 * The exact step that block-hybrid attention replaces (paper abstract: without
 * linearisation every denoising step attends to all previous blocks through
 * the KV cache), for comparison at the same shapes:
 *
 *   out[r, i, h, :] = sum_{j < P_r + B_r} P_ij w_j,
 *   P_ij = softmax_j(scale q_i . u_j)
 *
 * over the keys u = [prefix keys of request r; its B_r active keys] and the
 * values w likewise, for i < B_r.  No state is involved.
 *
 * q, k, v, out: the active block as in hybrid_attn_step.
 * k_cache, v_cache: the prefix KV cache, packed [total_prefix][heads][d] in
 *   the dtype of q; request r's prefix is rows cu_prefix[r] ..
 *   cu_prefix[r+1]-1 (device int64[n_req + 1]).  A request whose rows fall
 *   outside [0, total_prefix] (or run backwards) has an empty prefix.  The
 *   cache pointers may be NULL when total_prefix == 0.
 * total_prefix: HOST scalar >= 0.
 * chunk: keys are cut into chunks of `chunk` and the (request, head, chunk)
 *   list is split into a fixed number of equal ranges, one per workgroup;
 *   each writes an unnormalised partial output with its running max and sum
 *   per (request, head) into `workspace`, and a second kernel merges the
 *   partials of each (request, head) in a fixed order (deterministic).
 * workspace: device scratch of at least hybrid_exact_step_workspace_bytes()
 *   bytes (non-NULL when n_req > 0); contents on entry do not matter; calls
 *   sharing one workspace must be ordered on one stream.
 * Errors as for hybrid_attn_step, plus chunk < 1, total_prefix < 0, a NULL
 * cache when total_prefix > 0, or a small workspace (HA_ERR_INVALID_ARG).
 */
ha_status hybrid_exact_step(const void* q, const void* k, const void* v,
                            const void* k_cache, const void* v_cache,
                            const int64_t* cu_prefix, int64_t total_prefix,
                            void* out, const int32_t* blk_lens,
                            int32_t n_req, int32_t heads, int32_t blk,
                            int32_t d, float scale, int32_t chunk,
                            void* workspace, size_t workspace_bytes,
                            ha_dtype dtype, void* stream);

/* Workspace size for hybrid_exact_step (host): a 256-byte-padded plan of
 * n_req + 2 int64, then (W + n_req * heads) partials of R * (d + 2) floats,
 * R = 32, 64 or 128 for blk <= 32, <= 64 or <= 128, and W the number of
 * slice workgroups, 256 x (9, 6, 4 | 5, 4, 2 | 3, 2, 1) for d = 32 | 64 | 128
 * and the same blk ranges, 1024 for d = 16.  0 for empty or invalid sizes. */
size_t hybrid_exact_step_workspace_bytes(int32_t n_req, int32_t heads,
                                         int32_t blk, int32_t d);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* hybrid_last_error(void);

/* HYBRID_ATTN_ABI_VERSION of the loaded library. */
int32_t hybrid_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_ATTN_H */
