// Hybrid step kernels: O = Softmax(scale Q_a K_a^T) V_a + ReLU(Q_a) S per
// (request, head) ("Retrofitting Linear Attention into Diffusion Language
// Models", paper-daily summary page, section "core formula"; the worked
// example's "block output = softmax result + phi(Q_2) S_1").
#include "device_common.h"
#include "kernels.h"

namespace ha {

// ---------------------------------------------------------------------------
// bf16 matrix-core step, head dim D in {32, 64, 128}, blk <= 128.
//
// One workgroup per (request, head); wave w owns value columns [32w, 32w+32).
// Everything is computed transposed so that each lane ends up holding one
// query row:
//   L^T = K Q^T          (keys x queries): lane l holds query i = l % 32 and
//                        16 of its 32 keys per key tile, the other 16 sit in
//                        lane l ^ 32 -> row max / sum need one exchange.
//   O^T = V^T P^T + S^T phi(Q)^T
//                        both terms go into ONE accumulator, so the sum of
//                        the two parts costs nothing.
// S^T (the stored orientation) is an A operand read straight from HBM: lane l
// loads 8 contiguous fp32 of row c per k-step.  fp32 S and fp32 P enter the
// bf16 matrix cores as hi + lo bf16 pairs (two passes), which keeps ~16
// mantissa bits; Q, K, V are bf16 already, so their products are exact.
// V^T operands are gathered with 2-byte loads: per load instruction lanes
// 0..31 read 64 contiguous bytes of one row and lanes 32..63 another.
// No LDS and no barriers: waves of a unit only share L1/L2 lines of Q and K.
//
// Value-column permutation: the A-operand row m of wave w maps to column
//   c(m) = 32w + 16 * ((m / 4) % 2) + 4 * (m / 8) + m % 4,
// chosen so that accumulator register r of lane half hh holds column
// 32w + 16 hh + r: each lane stores 16 contiguous output columns (32 bytes).
// ---------------------------------------------------------------------------
template <int D, int NKT>
__global__ __launch_bounds__(D / 32 * kWave) void step_bf16_mfma(StepArgs a)
{
    constexpr int KS = D / 16;              // k-steps over the head dimension
    const int unit = blockIdx.x;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;   // uniform per workgroup

    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int l32 = lane % 32, hh = lane / 32;
    const int64_t rs = (int64_t)a.heads * D;                 // token row stride
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + base;
    uint16_t* out = static_cast<uint16_t*>(a.out) + base;
    const float* st = a.state + ((int64_t)slot * a.heads + h) * D * D;

    const int cA = 32 * w + 16 * ((l32 / 4) % 2) + 4 * (l32 / 8) + l32 % 4;  // A row -> column
    const int nkt = (Br + 31) / 32;                          // <= NKT
    const float sl2 = a.scale * 1.4426950408889634f;         // logits in log2 units

    bf16x8 shi[KS], slo[KS];                                 // S^T operands, kept across query tiles

    for (int qt = 0; qt < nkt; ++qt) {
        // ---- Q operand (B of L^T and, ReLU'd, B of S^T phi(Q)^T): row i, k-step s
        const int i = qt * 32 + l32;
        u16x8 qv[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qv[s] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (i < Br) qv[s] = *reinterpret_cast<const u16x8*>(q + i * rs + 16 * s + 8 * hh);
        }
        // ---- L^T tiles and V^T operands for every key tile
        f32x16 lt[NKT];
        u16x8 vop[NKT][2];
#pragma unroll
        for (int jt = 0; jt < NKT; ++jt) {
            lt[jt] = f32x16{};
            if (jt < nkt) {
                const int j = jt * 32 + l32;
                f32x16 acc = {};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    u16x8 kv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                    if (j < Br) kv = *reinterpret_cast<const u16x8*>(k + j * rs + 16 * s + 8 * hh);
                    acc = mfma32(as_bf16x8(kv), as_bf16x8(qv[s]), acc);
                }
                lt[jt] = acc;
                // V^T operand for k-step (jt, gp): key j = jt*32 + 16gp + 8(e/4) + 4hh + e%4,
                // matching accumulator registers 8gp .. 8gp+7 of L^T.
#pragma unroll
                for (int gp = 0; gp < 2; ++gp) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int jj = jt * 32 + 16 * gp + 8 * (e / 4) + 4 * hh + e % 4;
                        vop[jt][gp][e] = jj < Br ? v[jj * rs + cA] : uint16_t(0);
                    }
                }
            }
        }
        // ---- S^T row cA: 8 contiguous fp32 per k-step, streamed once per unit
        if (qt == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const f32x4* sp = reinterpret_cast<const f32x4*>(st + (int64_t)cA * D + 16 * s + 8 * hh);
                const f32x4 s0 = sp[0], s1 = sp[1];
                const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                split_hi_lo(sv, shi[s], slo[s]);
            }
        }
        // ---- row softmax over the Br valid keys (one query per lane pair)
        float m = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < NKT; ++jt) {
            if (jt < nkt) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int j = jt * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
                    const float x = j < Br ? lt[jt][rr] * sl2 : -INFINITY;
                    lt[jt][rr] = x;
                    m = fmaxf(m, x);
                }
            }
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        float sum = 0.f;
#pragma unroll
        for (int jt = 0; jt < NKT; ++jt) {
            if (jt < nkt) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const float p = exp2f(lt[jt][rr] - m);
                    lt[jt][rr] = p;
                    sum += p;
                }
            }
        }
        sum += __shfl_xor(sum, 32);
        const float inv = 1.0f / sum;

        // ---- O^T = V^T P^T (P as hi + lo bf16)
        f32x16 o = {};
#pragma unroll
        for (int jt = 0; jt < NKT; ++jt) {
            if (jt < nkt) {
#pragma unroll
                for (int gp = 0; gp < 2; ++gp) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) p[e] = lt[jt][8 * gp + e] * inv;
                    bf16x8 phi, plo;
                    split_hi_lo(p, phi, plo);
                    o = mfma32(as_bf16x8(vop[jt][gp]), phi, o);
                    o = mfma32(as_bf16x8(vop[jt][gp]), plo, o);
                }
            }
        }
        // ---- O^T += S^T phi(Q)^T (S as hi + lo bf16)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 pq = as_bf16x8(relu_bf16x8(qv[s]));
            o = mfma32(shi[s], pq, o);
            o = mfma32(slo[s], pq, o);
        }
        // ---- store: lane holds query i, columns 32w + 16hh + 0..15
        if (i < Br) {
            u16x8 o0, o1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o0[e] = f32_to_bf16_bits(o[e]);
                o1[e] = f32_to_bf16_bits(o[8 + e]);
            }
            u16x8* op = reinterpret_cast<u16x8*>(out + i * rs + 32 * w + 16 * hh);
            op[0] = o0;
            op[1] = o1;
        }
    }
}

// ---------------------------------------------------------------------------
// Plain fp32-arithmetic step for fp32 inputs (any supported d) and for bf16
// with d = 16.  One workgroup of 256 threads per (request, head); the B_r x B_r
// softmax matrix lives in LDS, everything else is read from global memory.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void step_generic(StepArgs a)
{
    extern __shared__ float P[];                  // [Br][Br]
    const int D = a.d;
    const int unit = blockIdx.x;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;
    const int64_t rs = (int64_t)a.heads * D;
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const T* q = static_cast<const T*>(a.q) + base;
    const T* k = static_cast<const T*>(a.k) + base;
    const T* v = static_cast<const T*>(a.v) + base;
    T* out = static_cast<T*>(a.out) + base;
    const float* st = a.state + ((int64_t)slot * a.heads + h) * D * D;

    for (int idx = threadIdx.x; idx < Br * Br; idx += blockDim.x) {
        const int i = idx / Br, j = idx % Br;
        float dot = 0.f;
        for (int c = 0; c < D; ++c) dot = fmaf(Elem<T>::load(q, i * rs + c), Elem<T>::load(k, j * rs + c), dot);
        P[idx] = a.scale * dot;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < Br; i += blockDim.x) {
        float m = -INFINITY;
        for (int j = 0; j < Br; ++j) m = fmaxf(m, P[i * Br + j]);
        float sum = 0.f;
        for (int j = 0; j < Br; ++j) {
            const float p = expf(P[i * Br + j] - m);
            P[i * Br + j] = p;
            sum += p;
        }
        const float inv = 1.f / sum;
        for (int j = 0; j < Br; ++j) P[i * Br + j] *= inv;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Br * D; idx += blockDim.x) {
        const int i = idx / D, c = idx % D;
        float acc = 0.f;
        for (int j = 0; j < Br; ++j) acc = fmaf(P[i * Br + j], Elem<T>::load(v, j * rs + c), acc);
        for (int f = 0; f < D; ++f) acc = fmaf(relu(Elem<T>::load(q, i * rs + f)), st[(int64_t)c * D + f], acc);
        Elem<T>::store(out, i * rs + c, acc);
    }
}

// ---------------------------------------------------------------------------
template <int D>
static void launch_step_d(const StepArgs& a, int units, hipStream_t stream)
{
    if (a.blk <= 32) step_bf16_mfma<D, 1><<<units, D / 32 * kWave, 0, stream>>>(a);
    else if (a.blk <= 64) step_bf16_mfma<D, 2><<<units, D / 32 * kWave, 0, stream>>>(a);
    else step_bf16_mfma<D, 4><<<units, D / 32 * kWave, 0, stream>>>(a);
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream)
{
    const int units = a.n_req * a.heads;
    if (a.dtype_bf16 && a.d >= 32) {
        switch (a.d) {
        case 32: launch_step_d<32>(a, units, stream); break;
        case 64: launch_step_d<64>(a, units, stream); break;
        default: launch_step_d<128>(a, units, stream); break;
        }
    } else {
        const size_t lds = sizeof(float) * (size_t)a.blk * a.blk;
        if (a.dtype_bf16) step_generic<uint16_t><<<units, 256, lds, stream>>>(a);
        else step_generic<float><<<units, 256, lds, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace ha
