// C ABI of libhybrid_attn: host-side argument validation and kernel dispatch.
// Every check runs before anything is enqueued, so a rejected call leaves the
// outputs and the state store untouched.  The library allocates nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/hybrid_attn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

ha_status fail(ha_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

ha_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return HA_OK;
    return fail(HA_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
}

bool supported_d(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// The kernels move data in 16-byte vectors and address the workspace's
// partial slots with 256-byte-aligned offsets.
bool aligned(const void* p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }

ha_status check_aligned(const char* fn, std::initializer_list<const void*> data, const void* workspace)
{
    for (const void* p : data)
        if (!aligned(p, 16)) return fail(HA_ERR_INVALID_ARG, "%s: data pointers must be 16-byte aligned", fn);
    if (!aligned(workspace, 256)) return fail(HA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    return HA_OK;
}
bool known_dtype(ha_dtype t) { return t == HA_F32 || t == HA_BF16; }

// Prefill and exact-step workspaces: the plan (n_req + 2 int64, padded to 256
// bytes), then one fp32 partial per (slice, unit) slot.
size_t plan_bytes(int32_t n_req) { return ((size_t)(n_req + 2) * sizeof(int64_t) + 255) / 256 * 256; }


// Checks shared by step and commit.  Returns HA_OK or the failure status.
ha_status check_block_call(const char* fn, int32_t n_req, int32_t n_slots, int32_t heads,
                           int32_t blk, int32_t d, ha_dtype dtype, int32_t max_blk = HYBRID_ATTN_MAX_BLK)
{
    if (n_req < 0) return fail(HA_ERR_INVALID_ARG, "%s: n_req must be >= 0 (got %d)", fn, n_req);
    if (n_slots <= 0) return fail(HA_ERR_INVALID_ARG, "%s: n_slots must be > 0 (got %d)", fn, n_slots);
    if (heads <= 0) return fail(HA_ERR_INVALID_ARG, "%s: heads must be > 0 (got %d)", fn, heads);
    if (blk <= 0 || blk > max_blk)
        return fail(HA_ERR_INVALID_ARG, "%s: blk must be in [1, %d] (got %d)", fn, max_blk, blk);
    if (!known_dtype(dtype)) return fail(HA_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
    if (!supported_d(d)) return fail(HA_ERR_UNSUPPORTED, "%s: head dim d=%d not in {16, 32, 64, 128}", fn, d);
    if ((int64_t)n_req * heads > 0x7fffffffLL)
        return fail(HA_ERR_INVALID_ARG, "%s: n_req * heads too large", fn);
    return HA_OK;
}

}  // namespace

extern "C" {

const char* hybrid_last_error(void) { return g_last_error.c_str(); }

int32_t hybrid_abi_version(void) { return HYBRID_ATTN_ABI_VERSION; }

}  // extern "C"

namespace {

// The step, the fused step + commit, the commit and the prefill, with z =
// NULL for the plain sum and z non-NULL for the normalised variant.
bool known_map(int phi) { return phi == HA_PHI_RELU || phi == HA_PHI_ELU1; }

ha_status step_impl(const char* fn, const void* q, const void* k, const void* v, const float* state, float* z,
                    const int32_t* slots, void* out, const int32_t* blk_lens, int32_t n_req, int32_t n_slots,
                    int32_t heads, int32_t blk, int32_t d, float scale, ha_dtype dtype, void* stream, bool norm,
                    int phi = HA_PHI_RELU)
{
    ha_status st = check_block_call(fn, n_req, n_slots, heads, blk, d, dtype);
    if (st != HA_OK) return st;
    if (!known_map(phi)) return fail(HA_ERR_UNSUPPORTED, "%s: unknown feature map %d", fn, phi);
    if (!std::isfinite(scale)) return fail(HA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    if (n_req == 0) return HA_OK;
    if (!q || !k || !v || !state || !slots || !out || (norm && !z))
        return fail(HA_ERR_INVALID_ARG, "%s: q, k, v, state%s, slots and out must be non-NULL", fn,
                    norm ? ", z" : "");
    if ((st = check_aligned(fn, {q, k, v, state, out, z}, nullptr)) != HA_OK) return st;
    ha::StepArgs a{q, k, v, state, nullptr, slots, out, blk_lens, z, n_req, n_slots, heads, blk, d, scale,
                   dtype == HA_BF16, phi};
    return hip_status(ha::launch_step(a, static_cast<hipStream_t>(stream)), fn);
}

ha_status step_commit_impl(const char* fn, const void* q, const void* k, const void* v, float* state, float* z,
                           const int32_t* slots, void* out, const int32_t* blk_lens, int32_t n_req,
                           int32_t n_slots, int32_t heads, int32_t blk, int32_t d, float scale, ha_dtype dtype,
                           void* stream, bool norm, int phi = HA_PHI_RELU)
{
    ha_status st = check_block_call(fn, n_req, n_slots, heads, blk, d, dtype);
    if (st != HA_OK) return st;
    if (!known_map(phi)) return fail(HA_ERR_UNSUPPORTED, "%s: unknown feature map %d", fn, phi);
    if (!std::isfinite(scale)) return fail(HA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    if (n_req == 0) return HA_OK;
    if (!q || !k || !v || !state || !slots || !out || (norm && !z))
        return fail(HA_ERR_INVALID_ARG, "%s: q, k, v, state%s, slots and out must be non-NULL", fn,
                    norm ? ", z" : "");
    if ((st = check_aligned(fn, {q, k, v, state, out, z}, nullptr)) != HA_OK) return st;
    ha::StepArgs a{q, k, v, state, state, slots, out, blk_lens, z, n_req, n_slots, heads, blk, d, scale,
                   dtype == HA_BF16, phi};
    return hip_status(ha::launch_step_commit(a, static_cast<hipStream_t>(stream)), fn);
}

ha_status commit_impl(const char* fn, const void* k, const void* v, float* state, float* z, const int32_t* slots,
                      const int32_t* blk_lens, int32_t n_req, int32_t n_slots, int32_t heads, int32_t blk,
                      int32_t d, ha_dtype dtype, void* stream, bool norm, int phi = HA_PHI_RELU)
{
    ha_status st = check_block_call(fn, n_req, n_slots, heads, blk, d, dtype);
    if (st != HA_OK) return st;
    if (!known_map(phi)) return fail(HA_ERR_UNSUPPORTED, "%s: unknown feature map %d", fn, phi);
    if (n_req == 0) return HA_OK;
    if (!k || !v || !state || !slots || (norm && !z))
        return fail(HA_ERR_INVALID_ARG, "%s: k, v, state%s and slots must be non-NULL", fn, norm ? ", z" : "");
    if ((st = check_aligned(fn, {k, v, state, z}, nullptr)) != HA_OK) return st;
    ha::PhiKVArgs a{};
    a.k = k;
    a.v = v;
    a.state = state;
    a.slots = slots;
    a.blk_lens = blk_lens;
    a.n_req = n_req;
    a.n_slots = n_slots;
    a.heads = heads;
    a.blk = blk;
    a.d = d;
    a.dtype_bf16 = dtype == HA_BF16;
    a.phi = phi;
    hipError_t e = ha::launch_commit(a, static_cast<hipStream_t>(stream));
    if (e == hipSuccess && norm) {
        ha::StepArgs zc{nullptr, k, v, nullptr, nullptr, slots, nullptr, blk_lens, z, n_req, n_slots, heads, blk,
                        d, 0.f, dtype == HA_BF16, phi};
        e = ha::launch_znorm_commit(zc, static_cast<hipStream_t>(stream));
    }
    return hip_status(e, fn);
}

size_t prefill_slots(int32_t n_req, int32_t heads, int32_t d)
{
    return (size_t)std::max(ha::prefill_base_slices(d), (int)heads) + (size_t)n_req * (size_t)heads;
}

// Argument checks of the prefill calls that do not involve the workspace.
ha_status prefill_check(const char* fn, const void* k, const void* v, const int64_t* cu_seqlens,
                        int64_t total_tokens, int64_t max_len, float* state, float* z, const int32_t* slots,
                        int32_t n_req, int32_t n_slots, int32_t heads, int32_t d, int32_t chunk, ha_dtype dtype,
                        bool norm, int phi = HA_PHI_RELU)
{
    if (!known_map(phi)) return fail(HA_ERR_UNSUPPORTED, "%s: unknown feature map %d", fn, phi);
    if (n_req < 0) return fail(HA_ERR_INVALID_ARG, "%s: n_req must be >= 0 (got %d)", fn, n_req);
    if (n_slots <= 0) return fail(HA_ERR_INVALID_ARG, "%s: n_slots must be > 0 (got %d)", fn, n_slots);
    if (heads <= 0) return fail(HA_ERR_INVALID_ARG, "%s: heads must be > 0 (got %d)", fn, heads);
    if (chunk <= 0) return fail(HA_ERR_INVALID_ARG, "%s: chunk must be > 0 (got %d)", fn, chunk);
    if (total_tokens < 0 || max_len < 0)
        return fail(HA_ERR_INVALID_ARG, "%s: total_tokens and max_len must be >= 0", fn);
    if (!known_dtype(dtype)) return fail(HA_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
    if (!supported_d(d)) return fail(HA_ERR_UNSUPPORTED, "%s: head dim d=%d not in {16, 32, 64, 128}", fn, d);
    if (n_req > 65535 || heads > 65535)
        return fail(HA_ERR_INVALID_ARG, "%s: n_req and heads must be <= 65535", fn);
    if (n_req == 0) return HA_OK;
    if (!cu_seqlens || !state || !slots || (norm && !z))
        return fail(HA_ERR_INVALID_ARG, "%s: cu_seqlens, state%s and slots must be non-NULL", fn,
                    norm ? ", z" : "");
    if (total_tokens > 0 && (!k || !v))
        return fail(HA_ERR_INVALID_ARG, "%s: k and v must be non-NULL when total_tokens > 0", fn);
    return HA_OK;
}

ha_status prefill_impl(const char* fn, const void* k, const void* v, const int64_t* cu_seqlens,
                       int64_t total_tokens, int64_t max_len, float* state, float* z, const int32_t* slots,
                       int32_t n_req, int32_t n_slots, int32_t heads, int32_t d, int32_t chunk, void* workspace,
                       size_t workspace_bytes, ha_dtype dtype, void* stream, bool norm, int phi = HA_PHI_RELU)
{
    if (ha_status st = prefill_check(fn, k, v, cu_seqlens, total_tokens, max_len, state, z, slots, n_req, n_slots,
                                     heads, d, chunk, dtype, norm, phi);
        st != HA_OK || n_req == 0)
        return st;
    const size_t need = hybrid_state_prefill_workspace_bytes(n_req, heads, d, total_tokens, max_len, chunk);
    if (workspace_bytes < need || !workspace)
        return fail(HA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed (got %zu%s)", fn, need,
                    workspace_bytes, workspace ? "" : ", NULL");
    if (ha_status st = check_aligned(fn, {k, v, state, z}, workspace); st != HA_OK) return st;
    ha::PhiKVArgs a{};
    a.k = k;
    a.v = v;
    a.state = state;
    a.z = z;
    a.slots = slots;
    a.cu = cu_seqlens;
    a.plan = static_cast<int64_t*>(workspace);
    a.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan_bytes(n_req));
    a.zpartial = a.partial + prefill_slots(n_req, heads, d) * (size_t)d * (size_t)d;
    a.total_tokens = total_tokens;
    a.chunk = chunk;
    a.hp = ha::prefill_group(d, heads, dtype == HA_BF16);
    a.spu = ha::prefill_spu(d, a.hp, heads / a.hp);
    a.slices = heads / a.hp * a.spu;
    a.n_req = n_req;
    a.n_slots = n_slots;
    a.heads = heads;
    a.d = d;
    a.dtype_bf16 = dtype == HA_BF16;
    a.phi = phi;
    return hip_status(ha::launch_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

ha_status hybrid_attn_step(const void* q, const void* k, const void* v, const float* state,
                           const int32_t* slots, void* out, const int32_t* blk_lens,
                           int32_t n_req, int32_t n_slots, int32_t heads, int32_t blk, int32_t d,
                           float scale, ha_dtype dtype, void* stream)
{
    return step_impl("hybrid_attn_step", q, k, v, state, nullptr, slots, out, blk_lens, n_req, n_slots, heads, blk,
                     d, scale, dtype, stream, false);
}

ha_status hybrid_attn_step_commit(const void* q, const void* k, const void* v, float* state,
                                  const int32_t* slots, void* out, const int32_t* blk_lens,
                                  int32_t n_req, int32_t n_slots, int32_t heads, int32_t blk, int32_t d,
                                  float scale, ha_dtype dtype, void* stream)
{
    return step_commit_impl("hybrid_attn_step_commit", q, k, v, state, nullptr, slots, out, blk_lens, n_req,
                            n_slots, heads, blk, d, scale, dtype, stream, false);
}

ha_status hybrid_state_commit(const void* k, const void* v, float* state, const int32_t* slots,
                              const int32_t* blk_lens, int32_t n_req, int32_t n_slots,
                              int32_t heads, int32_t blk, int32_t d, ha_dtype dtype, void* stream)
{
    return commit_impl("hybrid_state_commit", k, v, state, nullptr, slots, blk_lens, n_req, n_slots, heads, blk, d,
                       dtype, stream, false);
}

size_t hybrid_state_prefill_workspace_bytes(int32_t n_req, int32_t heads, int32_t d,
                                            int64_t total_tokens, int64_t max_len, int32_t chunk)
{
    (void)total_tokens;
    (void)max_len;
    if (n_req <= 0 || heads <= 0 || d <= 0 || chunk <= 0) return 0;
    return plan_bytes(n_req) + prefill_slots(n_req, heads, d) * ((size_t)d * (size_t)d + (size_t)d) * sizeof(float);
}

ha_status hybrid_state_prefill(const void* k, const void* v, const int64_t* cu_seqlens,
                               int64_t total_tokens, int64_t max_len, float* state,
                               const int32_t* slots, int32_t n_req, int32_t n_slots,
                               int32_t heads, int32_t d, int32_t chunk, void* workspace,
                               size_t workspace_bytes, ha_dtype dtype, void* stream)
{
    return prefill_impl("hybrid_state_prefill", k, v, cu_seqlens, total_tokens, max_len, state, nullptr, slots,
                        n_req, n_slots, heads, d, chunk, workspace, workspace_bytes, dtype, stream, false);
}

}  // extern "C"

namespace {

// Device scratch of the prefill entry point that allocates nothing: one copy
// of this array per GPU the library runs on, held until the process ends.
// Host code never uses the array's name as an address (on the host it is only
// a stand-in); the device address is looked up once per device and kept in
// g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[HYBRID_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the device that runs `stream`.
ha_status scratch_address(const char* fn, void* stream, void** out)
{
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(HA_ERR_HIP, "%s: cannot find the stream's device: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(HA_ERR_HIP, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(HA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(HA_ERR_HIP, "%s: hipSetDevice(%d) failed: %s", fn, dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return fail(HA_ERR_HIP, "%s: scratch address on device %d: %s", fn, dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return HA_OK;
}

}  // namespace

extern "C" {

ha_status hybrid_state_prefill_noalloc(const void* k, const void* v, const int64_t* cu_seqlens,
                                       int64_t total_tokens, int64_t max_len, float* state,
                                       const int32_t* slots, int32_t n_req, int32_t n_slots,
                                       int32_t heads, int32_t d, int32_t chunk, ha_dtype dtype, void* stream)
{
    static const char* fn = "hybrid_state_prefill_noalloc";
    if (ha_status st = prefill_check(fn, k, v, cu_seqlens, total_tokens, max_len, state, nullptr, slots, n_req,
                                     n_slots, heads, d, chunk, dtype, false);
        st != HA_OK || n_req == 0)
        return st;
    const size_t need = hybrid_state_prefill_workspace_bytes(n_req, heads, d, total_tokens, max_len, chunk);
    if (need > HYBRID_ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(HA_ERR_INVALID_ARG, "%s: needs %zu bytes of scratch, more than the %zu available", fn, need,
                    (size_t)HYBRID_ATTN_NOALLOC_SCRATCH_BYTES);
    if (ha_status st = check_aligned(fn, {k, v, state}, nullptr); st != HA_OK) return st;
    void* ws = nullptr;
    if (ha_status st = scratch_address(fn, stream, &ws); st != HA_OK) return st;
    return prefill_impl(fn, k, v, cu_seqlens, total_tokens, max_len, state, nullptr, slots, n_req, n_slots, heads,
                        d, chunk, ws, HYBRID_ATTN_NOALLOC_SCRATCH_BYTES, dtype, stream, false);
}

ha_status hybrid_attn_step_norm(const void* q, const void* k, const void* v, const float* state, const float* z,
                                const int32_t* slots, void* out, const int32_t* blk_lens,
                                int32_t n_req, int32_t n_slots, int32_t heads, int32_t blk, int32_t d,
                                float scale, ha_dtype dtype, void* stream)
{
    // the step only reads z; the argument block carries it as a writable
    // pointer because the fused commit updates it
    return step_impl("hybrid_attn_step_norm", q, k, v, state, const_cast<float*>(z), slots, out, blk_lens, n_req,
                     n_slots, heads, blk, d, scale, dtype, stream, true);
}

ha_status hybrid_attn_step_commit_norm(const void* q, const void* k, const void* v, float* state, float* z,
                                       const int32_t* slots, void* out, const int32_t* blk_lens,
                                       int32_t n_req, int32_t n_slots, int32_t heads, int32_t blk, int32_t d,
                                       float scale, ha_dtype dtype, void* stream)
{
    return step_commit_impl("hybrid_attn_step_commit_norm", q, k, v, state, z, slots, out, blk_lens, n_req,
                            n_slots, heads, blk, d, scale, dtype, stream, true);
}

ha_status hybrid_state_commit_norm(const void* k, const void* v, float* state, float* z, const int32_t* slots,
                                   const int32_t* blk_lens, int32_t n_req, int32_t n_slots,
                                   int32_t heads, int32_t blk, int32_t d, ha_dtype dtype, void* stream)
{
    return commit_impl("hybrid_state_commit_norm", k, v, state, z, slots, blk_lens, n_req, n_slots, heads, blk, d,
                       dtype, stream, true);
}

ha_status hybrid_state_prefill_norm(const void* k, const void* v, const int64_t* cu_seqlens,
                                    int64_t total_tokens, int64_t max_len, float* state, float* z,
                                    const int32_t* slots, int32_t n_req, int32_t n_slots,
                                    int32_t heads, int32_t d, int32_t chunk, void* workspace,
                                    size_t workspace_bytes, ha_dtype dtype, void* stream)
{
    return prefill_impl("hybrid_state_prefill_norm", k, v, cu_seqlens, total_tokens, max_len, state, z, slots,
                        n_req, n_slots, heads, d, chunk, workspace, workspace_bytes, dtype, stream, true);
}

ha_status hybrid_attn_step_phi(const void* q, const void* k, const void* v, const float* state, const float* z,
                               const int32_t* slots, void* out, const int32_t* blk_lens, int32_t n_req,
                               int32_t n_slots, int32_t heads, int32_t blk, int32_t d, float scale,
                               ha_feature_map phi, ha_dtype dtype, void* stream)
{
    return step_impl("hybrid_attn_step_phi", q, k, v, state, const_cast<float*>(z), slots, out, blk_lens, n_req,
                     n_slots, heads, blk, d, scale, dtype, stream, z != nullptr, (int)phi);
}

ha_status hybrid_attn_step_commit_phi(const void* q, const void* k, const void* v, float* state, float* z,
                                      const int32_t* slots, void* out, const int32_t* blk_lens, int32_t n_req,
                                      int32_t n_slots, int32_t heads, int32_t blk, int32_t d, float scale,
                                      ha_feature_map phi, ha_dtype dtype, void* stream)
{
    return step_commit_impl("hybrid_attn_step_commit_phi", q, k, v, state, z, slots, out, blk_lens, n_req, n_slots,
                            heads, blk, d, scale, dtype, stream, z != nullptr, (int)phi);
}

ha_status hybrid_state_commit_phi(const void* k, const void* v, float* state, float* z, const int32_t* slots,
                                  const int32_t* blk_lens, int32_t n_req, int32_t n_slots, int32_t heads,
                                  int32_t blk, int32_t d, ha_feature_map phi, ha_dtype dtype, void* stream)
{
    return commit_impl("hybrid_state_commit_phi", k, v, state, z, slots, blk_lens, n_req, n_slots, heads, blk, d,
                       dtype, stream, z != nullptr, (int)phi);
}

ha_status hybrid_state_prefill_phi(const void* k, const void* v, const int64_t* cu_seqlens, int64_t total_tokens,
                                   int64_t max_len, float* state, float* z, const int32_t* slots, int32_t n_req,
                                   int32_t n_slots, int32_t heads, int32_t d, int32_t chunk, void* workspace,
                                   size_t workspace_bytes, ha_feature_map phi, ha_dtype dtype, void* stream)
{
    return prefill_impl("hybrid_state_prefill_phi", k, v, cu_seqlens, total_tokens, max_len, state, z, slots, n_req,
                        n_slots, heads, d, chunk, workspace, workspace_bytes, dtype, stream, z != nullptr, (int)phi);
}

size_t hybrid_exact_step_workspace_bytes(int32_t n_req, int32_t heads, int32_t blk, int32_t d)
{
    if (n_req <= 0 || heads <= 0 || blk <= 0 || blk > HYBRID_ATTN_EXACT_MAX_BLK || d <= 0) return 0;
    return plan_bytes(n_req) + ((size_t)ha::exact_slices(d, blk) + (size_t)n_req * (size_t)heads) *
                                   (size_t)ha::exact_slot_floats(blk, d) * sizeof(float);
}

ha_status hybrid_exact_step(const void* q, const void* k, const void* v, const void* k_cache,
                            const void* v_cache, const int64_t* cu_prefix, int64_t total_prefix,
                            void* out, const int32_t* blk_lens, int32_t n_req, int32_t heads,
                            int32_t blk, int32_t d, float scale, int32_t chunk, void* workspace,
                            size_t workspace_bytes, ha_dtype dtype, void* stream)
{
    static const char* fn = "hybrid_exact_step";
    ha_status st = check_block_call(fn, n_req, 1, heads, blk, d, dtype, HYBRID_ATTN_EXACT_MAX_BLK);
    if (st != HA_OK) return st;
    if (!std::isfinite(scale)) return fail(HA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    if (chunk <= 0) return fail(HA_ERR_INVALID_ARG, "%s: chunk must be > 0 (got %d)", fn, chunk);
    if (total_prefix < 0) return fail(HA_ERR_INVALID_ARG, "%s: total_prefix must be >= 0", fn);
    if (n_req == 0) return HA_OK;
    if (!q || !k || !v || !out || !cu_prefix)
        return fail(HA_ERR_INVALID_ARG, "%s: q, k, v, out and cu_prefix must be non-NULL", fn);
    if (total_prefix > 0 && (!k_cache || !v_cache))
        return fail(HA_ERR_INVALID_ARG, "%s: k_cache and v_cache must be non-NULL when total_prefix > 0", fn);
    const size_t need = hybrid_exact_step_workspace_bytes(n_req, heads, blk, d);
    if (workspace_bytes < need || !workspace)
        return fail(HA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed (got %zu%s)", fn, need,
                    workspace_bytes, workspace ? "" : ", NULL");
    if ((st = check_aligned(fn, {q, k, v, k_cache, v_cache, out}, workspace)) != HA_OK) return st;
    ha::ExactArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kc = k_cache;
    a.vc = v_cache;
    a.cu = cu_prefix;
    a.total_prefix = total_prefix;
    a.out = out;
    a.blk_lens = blk_lens;
    a.plan = static_cast<int64_t*>(workspace);
    a.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan_bytes(n_req));
    a.chunk = chunk;
    a.slices = ha::exact_slices(d, blk);
    a.n_req = n_req;
    a.heads = heads;
    a.blk = blk;
    a.d = d;
    a.scale = scale;
    a.dtype_bf16 = dtype == HA_BF16;
    return hip_status(ha::launch_exact(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
