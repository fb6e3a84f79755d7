// Device-side helpers for the gfx950 kernels of libhybrid_attn.
//
// Matrix-core conventions used throughout (CDNA3/CDNA4 MFMA, wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A operand, lane l: row m = l % 32, k = 8 * (l / 32) + e,  e = 0..7
//     B operand, lane l: col n = l % 32, k = 8 * (l / 32) + e,  e = 0..7
//     D/C,       lane l: col n = l % 32, row m = 8 * (r / 4) + 4 * (l / 32) + r % 4,
//                        r = 0..15 the accumulator register.
// The reduction index k of one MFMA may be any permutation of the 16 values
// shared by A and B, which the kernels use to keep loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxBlk = 128;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ReLU on 8 packed bf16: a bf16 is <= 0 exactly when its sign bit is set or it
// is +0, so max as signed 16-bit integers against 0 maps every value with the
// sign bit set (including -0) to +0 and keeps the rest.
__device__ __forceinline__ u16x8 relu_bf16x8(u16x8 x) {
    u16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (static_cast<int16_t>(x[e]) > 0) ? x[e] : uint16_t(0);
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 x) { return __builtin_bit_cast(bf16x8, x); }



// Split 8 fp32 values into bf16 hi + lo with hi + lo == x to about 2^-17
// relative (hi = RNE(x), lo = RNE(x - hi)); bf16 x bf16 products are exact in
// fp32, so two matrix-core passes reproduce fp32 operands to ~16 bits.
__device__ __forceinline__ void split_hi_lo(const float* x, bf16x8& hi, bf16x8& lo) {
    u16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = f32_to_bf16_bits(x[e]);
        l[e] = f32_to_bf16_bits(x[e] - bf16_bits_to_f32(h[e]));
    }
    hi = as_bf16x8(h);
    lo = as_bf16x8(l);
}

// Feature maps phi (the ha_feature_map values): 0 = ReLU, the worked
// example's map; 1 = ELU + 1, phi(x) = x + 1 for x > 0 and e^x otherwise.
template <int M>
__device__ __forceinline__ float phi_of(float x)
{
    if constexpr (M == 1) return x > 0.f ? x + 1.f : expf(x);
    else return x > 0.f ? x : 0.f;
}

__device__ __forceinline__ float phi_rt(int map, float x) { return map == 1 ? phi_of<1>(x) : phi_of<0>(x); }

// phi of 8 packed bf16 as a matrix-core operand: ReLU of a bf16 is a bf16
// (hi only, kExact); ELU + 1 is computed in fp32 and split into hi + lo bf16
// (the caller adds the lo pass), and f keeps the fp32 values for sums.
template <int M>
struct PhiOp {
    static constexpr bool kExact = M == 0;
    bf16x8 hi, lo;
    float f[8];
};

template <int M>
__device__ __forceinline__ PhiOp<M> phi_op(u16x8 x)
{
    PhiOp<M> r;
    if constexpr (M == 0) {
        const u16x8 y = relu_bf16x8(x);
        r.hi = as_bf16x8(y);
#pragma unroll
        for (int e = 0; e < 8; ++e) r.f[e] = bf16_bits_to_f32(y[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.f[e] = phi_of<1>(bf16_bits_to_f32(x[e]));
        split_hi_lo(r.f, r.hi, r.lo);
    }
    return r;
}

// The same split for two floats, each result packed as a bf16 pair (element 0
// in the low half).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_hi_lo2(f32x2 x, uint32_t& hi, uint32_t& lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    const f32x2 hf = {__uint_as_float(h << 16), __uint_as_float(h & 0xffff0000u)};
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - hf, bf16x2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16_bits(x); }
};

__device__ __forceinline__ float relu(float x) { return x > 0.f ? x : 0.f; }

// In-place prefix sum over part[1..256] by a workgroup of 256 threads, thread
// t owning part[t + 1] (already written by it): afterwards part[0] = 0 and
// part[i] is the sum of the first i elements.  Log-step (8 rounds of read,
// barrier, add) instead of one thread walking the array, whose 256 dependent
// LDS round trips were most of a plan kernel's time.
__device__ __forceinline__ void scan256(int64_t* part, int tid)
{
    if (tid == 0) part[0] = 0;
    for (int off = 1; off < 256; off <<= 1) {
        __syncthreads();
        const int64_t v = tid >= off ? part[tid + 1 - off] : 0;
        __syncthreads();
        part[tid + 1] += v;
    }
    __syncthreads();
}

// Max and sum of x over lane pairs (i, i + 32), returned in both lanes.  The
// permlane32 swap hands every lane the value of lanes 0-31 and of lanes 32-63
// in one VALU op (no LDS round trip); both halves add the two operands in the
// same order, so the result is the same in the pair.
__device__ __forceinline__ float half_pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Read of a small per-request array (offsets, plans, lengths) at an index that
// is the same in every lane, through the scalar cache.  The data is written
// by the host or by an earlier kernel, never by the reading kernel, and a
// scalar load does not count against the vector-memory counter, so cursor
// updates in a streaming loop never wait for the key/value loads in flight.
template <typename T>
__device__ __forceinline__ T uniform_load(const T* p, int64_t i)
{
    typedef const __attribute__((address_space(4))) T* const_ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)i);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)i >> 32));
    return ((const_ptr)p)[(int64_t)(((uint64_t)hi << 32) | lo)];
}

// The same read where the index differs between lanes.
template <typename T>
__device__ __forceinline__ T lane_load(const T* p, int64_t i) { return p[i]; }

}  // namespace ha
