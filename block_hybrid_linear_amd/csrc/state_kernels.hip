// Prefix-state kernels: block commit S += ReLU(K)^T V and prompt prefill
// S = sum_t ReLU(k_t)^T v_t ("Retrofitting Linear Attention into Diffusion
// Language Models", paper-daily summary page, section "technical details in
// action": S_1 = phi(K_1)^T V_1, S_{1,2} = phi(K_1)^T V_1 + phi(K_2)^T V_2).
// The state is stored transposed: state[c][f] = S[f][c].
#include "device_common.h"
#include "kernels.h"

namespace ha {

// ---------------------------------------------------------------------------
// bf16 matrix-core reduction of ReLU(K)^T V over a token range.
//
//   dS^T[c][f] = sum_j V[j][c] * ReLU(K[j][f])      (A = V^T, B = ReLU(K), k = token)
//
// The reduction runs over tokens, which are the strided dimension of the
// token-major inputs, so K and V go through LDS transposed: each thread loads
// an 8-token x 8-column block with eight coalesced 16-byte loads (a wave
// instruction covers whole 256-byte rows), transposes it in registers and
// writes eight 16-byte rows of K^T / V^T.  Matrix-core operands are then one
// 16-byte LDS read each.  Stages of T tokens are double-buffered: the next
// stage's global loads are in flight while the current one is multiplied,
// with one barrier per stage.
//
// Output tiles are 32 x 32; wave w owns value-row tile ct and the feature
// tiles listed by tile_of().  Accumulator register r of lane l holds
// c = 32 ct + 8 (r/4) + 4 (l/32) + r%4 and f = 32 ft + l%32, so every register
// of a wave is two 128-byte runs of one state row: coalesced read-modify-write.
// ---------------------------------------------------------------------------
template <int D> struct PhiKVShape;
template <> struct PhiKVShape<128> { static constexpr int NW = 4, T = 64; };
template <> struct PhiKVShape<64> { static constexpr int NW = 4, T = 128; };
template <> struct PhiKVShape<32> { static constexpr int NW = 1, T = 64; };

template <int D, bool kCommit>
__global__ __launch_bounds__(PhiKVShape<D>::NW * kWave) void phikv_bf16_mfma(PhiKVArgs a)
{
    constexpr int NW = PhiKVShape<D>::NW, T = PhiKVShape<D>::T;
    constexpr int NT = D / 32;                   // tiles per dimension
    constexpr int TPW = NT * NT / NW;            // tiles per wave
    constexpr int PITCH = T + 8;                 // LDS row pitch in bf16 (16 B pad)
    constexpr int CG = D / 8;                    // 8-column groups per token row
    static_assert(2 * (T / 8) * CG == NW * kWave, "one 8x8 block per thread per stage");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][D * PITCH];  // [buf][K^T, V^T]

    // ---- token range of this workgroup
    int r, h, slot = 0;
    int64_t row0, nrows;
    if (kCommit) {
        r = blockIdx.x / a.heads;
        h = blockIdx.x % a.heads;
        int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
        Br = Br > a.blk ? a.blk : Br;
        slot = a.slots[r];
        if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;
        row0 = (int64_t)r * a.blk;
        nrows = Br;
    } else {
        const int g = blockIdx.x;
        h = blockIdx.y;
        r = blockIdx.z;
        const int64_t s0 = a.cu[r], s1 = a.cu[r + 1];
        if (s0 < 0 || s1 > a.total_tokens || s1 < s0) return;     // malformed: treated as empty
        row0 = s0 + (int64_t)g * a.group_tokens;
        const int64_t end = (s1 - row0 < a.group_tokens) ? s1 : row0 + a.group_tokens;
        if (row0 >= end) return;                                   // beyond this prompt
        nrows = end - row0;
    }
    const int64_t rs = (int64_t)a.heads * D;
    const uint16_t* kb = static_cast<const uint16_t*>(a.k) + row0 * rs + (int64_t)h * D;
    const uint16_t* vb = static_cast<const uint16_t*>(a.v) + row0 * rs + (int64_t)h * D;

    const int tid = threadIdx.x;
    const int lane = tid % kWave, w = tid / kWave;
    const int l32 = lane % 32, hh = lane / 32;

    // ---- this thread's 8x8 staging block: tensor (K or V), token group, column group
    const int blocks_per_tensor = (T / 8) * CG;
    const int tensor = tid / blocks_per_tensor;          // 0 = K, 1 = V
    const int bidx = tid % blocks_per_tensor;
    const int tg = bidx / CG, cg = bidx % CG;
    const uint16_t* src = (tensor == 0 ? kb : vb) + (int64_t)(tg * 8) * rs + cg * 8;

    auto load_stage = [&](int64_t t0, u32x4 (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t t = t0 + tg * 8 + e;
            x[e] = u32x4{0, 0, 0, 0};
            if (t < nrows) x[e] = *reinterpret_cast<const u32x4*>(src + t0 * rs + (int64_t)e * rs);
        }
    };
    // transpose the 8x8 bf16 block and write eight 16-byte rows (one per column)
    auto store_stage = [&](int buf, const u32x4 (&x)[8]) {
        uint16_t* dst = &lds[buf][tensor][(cg * 8) * PITCH + tg * 8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 y;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = x[2 * p][c / 2], hi = x[2 * p + 1][c / 2];
                y[p] = (c % 2 == 0) ? ((lo & 0xffffu) | (hi << 16)) : ((lo >> 16) | (hi & 0xffff0000u));
            }
            *reinterpret_cast<u32x4*>(dst + c * PITCH) = y;
        }
    };

    f32x16 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};

    const int nstages = (int)((nrows + T - 1) / T);
    u32x4 x[8];
    load_stage(0, x);

    // commit: the state tiles are read while the first stage is in flight
    float sold[TPW][16];
    float* st = nullptr;
    if (kCommit) {
        st = a.state + ((int64_t)slot * a.heads + h) * D * D;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = w * TPW + u, ct = t / NT, ft = t % NT;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int c = ct * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
                sold[u][rr] = st[(int64_t)c * D + ft * 32 + l32];
            }
        }
    }

    for (int sg = 0; sg < nstages; ++sg) {
        const int buf = sg & 1;
        store_stage(buf, x);
        __syncthreads();
        if (sg + 1 < nstages) load_stage((int64_t)(sg + 1) * T, x);
        const uint16_t* kt = lds[buf][0];
        const uint16_t* vt = lds[buf][1];
#pragma unroll
        for (int s = 0; s < T / 16; ++s) {
            const int j = 16 * s + 8 * hh;
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int t = w * TPW + u, ct = t / NT, ft = t % NT;
                const u16x8 av = *reinterpret_cast<const u16x8*>(vt + (ct * 32 + l32) * PITCH + j);
                const u16x8 bk = *reinterpret_cast<const u16x8*>(kt + (ft * 32 + l32) * PITCH + j);
                acc[u] = mfma32(as_bf16x8(av), as_bf16x8(relu_bf16x8(bk)), acc[u]);
            }
        }
    }

    // ---- epilogue
    float* dstp;
    if (kCommit) {
        dstp = st;
    } else {
        dstp = a.partial + (((int64_t)r * a.groups + blockIdx.x) * a.heads + h) * D * D;
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = w * TPW + u, ct = t / NT, ft = t % NT;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int c = ct * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
            float val = acc[u][rr];
            if (kCommit) val = sold[u][rr] + val;
            dstp[(int64_t)c * D + ft * 32 + l32] = val;
        }
    }
}

// ---------------------------------------------------------------------------
// Plain fp32-arithmetic reduction (fp32 inputs, and bf16 with d = 16): one
// thread per state element, looping over the token range.
// ---------------------------------------------------------------------------
template <typename T, bool kCommit>
__global__ __launch_bounds__(256) void phikv_generic(PhiKVArgs a)
{
    const int D = a.d;
    int r, h, slot = 0;
    int64_t row0, nrows;
    if (kCommit) {
        r = blockIdx.x / a.heads;
        h = blockIdx.x % a.heads;
        int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
        Br = Br > a.blk ? a.blk : Br;
        slot = a.slots[r];
        if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;
        row0 = (int64_t)r * a.blk;
        nrows = Br;
    } else {
        const int g = blockIdx.x;
        h = blockIdx.y;
        r = blockIdx.z;
        const int64_t s0 = a.cu[r], s1 = a.cu[r + 1];
        if (s0 < 0 || s1 > a.total_tokens || s1 < s0) return;
        row0 = s0 + (int64_t)g * a.group_tokens;
        const int64_t end = (s1 - row0 < a.group_tokens) ? s1 : row0 + a.group_tokens;
        if (row0 >= end) return;
        nrows = end - row0;
    }
    const int64_t rs = (int64_t)a.heads * D;
    const T* kb = static_cast<const T*>(a.k) + row0 * rs + (int64_t)h * D;
    const T* vb = static_cast<const T*>(a.v) + row0 * rs + (int64_t)h * D;
    float* dstp = kCommit ? a.state + ((int64_t)slot * a.heads + h) * D * D
                          : a.partial + (((int64_t)r * a.groups + blockIdx.x) * a.heads + h) * D * D;
    for (int e = threadIdx.x; e < D * D; e += blockDim.x) {
        const int c = e / D, f = e % D;
        float acc = 0.f;
        for (int64_t t = 0; t < nrows; ++t)
            acc = fmaf(Elem<T>::load(vb, t * rs + c), relu(Elem<T>::load(kb, t * rs + f)), acc);
        dstp[e] = kCommit ? dstp[e] + acc : acc;
    }
}

// ---------------------------------------------------------------------------
// Deterministic reduction of prefill partials: S[slot] = sum_g partial[g] in
// ascending group order (0 if the prompt is empty).  Each thread owns four
// consecutive floats of one (request, head) state.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_reduce(ReduceArgs a)
{
    const int h = blockIdx.y, r = blockIdx.z;
    const int slot = a.slots[r];
    if (slot < 0 || slot >= a.n_slots) return;
    const int64_t n4 = (int64_t)a.d * a.d / 4;
    const int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e4 >= n4) return;
    const int64_t s0 = a.cu[r], s1 = a.cu[r + 1];
    int64_t ng = 0;
    if (s0 >= 0 && s1 <= a.total_tokens && s1 > s0) ng = (s1 - s0 + a.group_tokens - 1) / a.group_tokens;
    if (ng > a.groups) ng = a.groups;
    const int64_t dd = (int64_t)a.d * a.d;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int64_t g = 0; g < ng; ++g) {
        const f32x4* p = reinterpret_cast<const f32x4*>(a.partial + ((r * (int64_t)a.groups + g) * a.heads + h) * dd);
        sum += p[e4];
    }
    reinterpret_cast<f32x4*>(a.state + ((int64_t)slot * a.heads + h) * dd)[e4] = sum;
}

// ---------------------------------------------------------------------------
template <bool kCommit>
static void launch_phikv(const PhiKVArgs& a, dim3 grid, hipStream_t stream)
{
    if (a.dtype_bf16 && a.d >= 32) {
        switch (a.d) {
        case 32: phikv_bf16_mfma<32, kCommit><<<grid, PhiKVShape<32>::NW * kWave, 0, stream>>>(a); break;
        case 64: phikv_bf16_mfma<64, kCommit><<<grid, PhiKVShape<64>::NW * kWave, 0, stream>>>(a); break;
        default: phikv_bf16_mfma<128, kCommit><<<grid, PhiKVShape<128>::NW * kWave, 0, stream>>>(a); break;
        }
    } else if (a.dtype_bf16) {
        phikv_generic<uint16_t, kCommit><<<grid, 256, 0, stream>>>(a);
    } else {
        phikv_generic<float, kCommit><<<grid, 256, 0, stream>>>(a);
    }
}

hipError_t launch_commit(const PhiKVArgs& a, hipStream_t stream)
{
    launch_phikv<true>(a, dim3(a.n_req * a.heads), stream);
    return hipGetLastError();
}

hipError_t launch_prefill(const PhiKVArgs& a, const ReduceArgs& ra, hipStream_t stream)
{
    if (a.groups > 0) {
        launch_phikv<false>(a, dim3(a.groups, a.heads, a.n_req), stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n4 = (int64_t)ra.d * ra.d / 4;
    prefill_reduce<<<dim3((unsigned)((n4 + 255) / 256), ra.heads, ra.n_req), 256, 0, stream>>>(ra);
    return hipGetLastError();
}

}  // namespace ha
