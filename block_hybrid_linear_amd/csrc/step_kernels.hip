// Hybrid step kernels: O = Softmax(scale Q_a K_a^T) V_a + ReLU(Q_a) S per
// (request, head) ("Retrofitting Linear Attention into Diffusion Language
// Models", paper-daily summary page, section "core formula"; the worked
// example's "block output = softmax result + phi(Q_2) S_1").
#include "device_common.h"
#include "kernels.h"

namespace ha {

// ---------------------------------------------------------------------------
// bf16 matrix-core step, head dim D in {32, 64, 128}, blk <= 32 * NKT.
//
// One workgroup per (request, head, 32-query tile) with D/32 waves; wave ct
// owns value columns [32 ct, 32 ct + 32) of the tile's queries, so each wave
// reads its S^T tile once and splits it into hi/lo bf16 once.  A block of
// more than 32 rows is split over NKT workgroups (one per query tile) so that
// small batches still put several workgroups on every compute unit; the
// workgroups of one (request, head) are numbered so that they land on the
// same XCD (workgroups are dealt to the 8 XCDs round-robin), where the second
// read of the unit's S, K and V hits that XCD's L2.
//
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
//
// The query tile and all key/value rows are staged once per workgroup in LDS
// (row-major, 16-byte pad) with 16-byte coalesced loads.  Matrix-core operands
// of Q and K are then one 16-byte LDS read each; V^T operands use the gfx950
// transposing LDS read (ds_read_b64_tr_b16), which hands each lane four
// consecutive rows of one column.  Rows past B_r are clamped to row B_r - 1
// (masked out of the softmax), so every global load is unconditional; they
// are issued in the order Q/K/V, then the wave's S tile, and the scheduler is
// fenced so the S stream -- most of the bytes -- is in flight while the
// softmax part is computed.
//
// Value-column permutation: the A-operand row m of tile ct maps to column
//   c(m) = 32 ct + 16 * ((m / 4) % 2) + 4 * (m / 8) + m % 4,
// chosen so that accumulator register r of lane half hh holds column
// 32 ct + 16 hh + r: each lane stores 16 contiguous output columns (32 bytes).
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

// Four consecutive rows of one column per lane: within each 16-lane group,
// lane j' supplies the address of 4 bf16 at (row0 + j'/4, col(j'%4)) and lane
// i receives element i%4 of the rows supplied by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr4(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Normalised variant (one denominator for the block's softmax scores and the
// prefix's linear scores, z = sum phi(k) next to S): the output of a query is
//   (sum_j 2^(l_j) v_j + phi(q) S) / (sum_j 2^(l_j) + phi(q).z)
// with l_j its logits in log2 units.  Both sides are divided by 2^c,
// c = max(m, log2(phi(q).z)), m the logits' maximum, so that the larger part
// of the denominator is one and nothing overflows; given m, the block's sum
// A = sum_j 2^(l_j - m) and qz = phi(q).z, alpha scales the probabilities
// 2^(l_j - m) and beta the linear term phi(q) S.  (c is kept above -100, so
// 2^-c stays finite; below that both parts would underflow anyway.)
__device__ __forceinline__ void norm_weights(float m, float A, float qz, float& alpha, float& beta)
{
    float c = m;
    if (qz > 0.f) c = fmaxf(c, __builtin_amdgcn_logf(qz));   // log2
    c = fmaxf(c, -100.f);
    const float ws = __builtin_amdgcn_exp2f(m - c), wl = __builtin_amdgcn_exp2f(-c);
    const float inv = __builtin_amdgcn_rcpf(fmaf(ws, A, wl * qz));
    alpha = ws * inv;
    beta = wl * inv;
}

// phi(q).z for the query whose staged row starts at qrow (pitch D + 8 bf16)
// against z staged in LDS: lane half hh sums features [hh D/2, hh D/2 + D/2),
// then the halves are added (every lane returns its query's full sum).
template <int D, int M = 0>
__device__ __forceinline__ float query_dot_z(const uint16_t* qrow, const float* zl, int hh)
{
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const int f0 = hh * (D / 2) + 8 * c;
        const u16x8 qv = *reinterpret_cast<const u16x8*>(qrow + f0);
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zl + f0), z1 = *reinterpret_cast<const f32x4*>(zl + f0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(phi_of<M>(bf16_bits_to_f32(qv[e])), z0[e], acc);
            acc = fmaf(phi_of<M>(bf16_bits_to_f32(qv[4 + e])), z1[e], acc);
        }
    }
    return half_pair_sum(acc);
}

// Stages the unit's z (D floats) in LDS; threads 0 .. D/4 - 1 each copy 16 bytes.
template <int D>
__device__ __forceinline__ void stage_z(float* zl, const float* zg, int tid)
{
    if (tid < D / 4) reinterpret_cast<f32x4*>(zl)[tid] = reinterpret_cast<const f32x4*>(zg)[tid];
}

// z += sum over the block's first Br staged key rows (pitch PK bf16, row
// major) of phi(k): thread f < D owns feature f.
template <int D, int PK = D + 8, int M = 0>
__device__ __forceinline__ void commit_z(float* zg, const uint16_t* sk, int Br, int tid)
{
    if (tid < D) {
        float acc = 0.f;
        for (int j = 0; j < Br; ++j) acc += phi_of<M>(bf16_bits_to_f32(sk[j * PK + tid]));
        zg[tid] += acc;
    }
}

// One k-step of the linear part, S^T (hi + lo bf16) times phi(Q)^T: two
// matrix-core passes for ReLU (exact in bf16), three for ELU + 1 (phi(Q) as
// hi + lo as well; the lo x lo product, ~2^-18 of the term, is dropped).
template <int M>
__device__ __forceinline__ f32x16 linear_mfma(f32x16 acc, bf16x8 shi, bf16x8 slo, u16x8 qv)
{
    const PhiOp<M> pq = phi_op<M>(qv);
    acc = mfma32(shi, pq.hi, acc);
    acc = mfma32(slo, pq.hi, acc);
    if constexpr (!PhiOp<M>::kExact) acc = mfma32(shi, pq.lo, acc);
    return acc;
}

// Softmax part of one 32-query tile whose rows start at qtile in LDS:
// L^T = K Q^T over the key tiles, row softmax over the Br valid keys (one
// query per lane pair), O^T = V^T P^T with P as hi + lo bf16.  Returns the
// wave's accumulator (value columns of tile ct, transposed).  Contraction of
// the scaling and the max subtraction into one fma is switched off so that
// every kernel that inlines this computes bit-identical probabilities.
template <int D, int NKT, bool kNorm = false, int PK = D + 8, int PV = D + 8>
__device__ __forceinline__ f32x16 softmax_tile(const uint16_t* qtile, const uint16_t* sk, const uint16_t* sv,
                                               int Br, float sl2, int ct, int lane, float qz = 0.f,
                                               float* beta = nullptr)
{
#pragma clang fp contract(off)
    constexpr int KS = D / 16, P = D + 8;
    const int l32 = lane % 32, hh = lane / 32;
    const int g = lane / 16, jl = lane % 16;
    const int vcol = 32 * ct + 16 * ((jl % 4) % 2) + 8 * (g % 2) + 4 * ((jl % 4) / 2);
    f32x16 o = {};
    const uint16_t* qr = qtile + l32 * P + 8 * hh;
    f32x16 lt[NKT];
#pragma unroll
    for (int jt = 0; jt < NKT; ++jt) {
        f32x16 acc = {};
        const uint16_t* kr = sk + (jt * 32 + l32) * PK + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = mfma32(as_bf16x8(*reinterpret_cast<const u16x8*>(kr + 16 * s)),
                         as_bf16x8(*reinterpret_cast<const u16x8*>(qr + 16 * s)), acc);
        lt[jt] = acc;
    }
    float m = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < NKT; ++jt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int j = jt * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
            const float x = j < Br ? lt[jt][rr] * sl2 : -INFINITY;
            lt[jt][rr] = x;
            m = fmaxf(m, x);
        }
    }
    m = half_pair_max(m);
    float sum = 0.f;
#pragma unroll
    for (int jt = 0; jt < NKT; ++jt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float p = __builtin_amdgcn_exp2f(lt[jt][rr] - m);   // exp2(-inf) = 0 for masked keys
            lt[jt][rr] = p;
            sum += p;
        }
    }
    sum = half_pair_sum(sum);
    float inv;
    if constexpr (kNorm) norm_weights(m, sum, qz, inv, *beta);   // probabilities over the shared denominator
    else inv = __builtin_amdgcn_rcpf(sum);
    // V^T operand of k-step (jt, gp): keys jt*32 + 16gp + 4hh + {0..3} and the
    // same + 8, matching registers 8gp .. 8gp+7 of L^T; the column of lane i in
    // 16-lane group g is 32ct + 16(q%2) + 8(g%2) + 4(q/2) + i%4, q = i/4 (= cA).
#pragma unroll
    for (int jt = 0; jt < NKT; ++jt) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            const int row0 = jt * 32 + 16 * gp + 4 * hh + jl / 4;
            const s16x4 v0 = lds_read_tr4(sv + row0 * PV + vcol);
            const s16x4 v1 = lds_read_tr4(sv + (row0 + 8) * PV + vcol);
            u16x8 vop;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vop[e] = static_cast<uint16_t>(v0[e]);
                vop[4 + e] = static_cast<uint16_t>(v1[e]);
            }
            float pp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pp[e] = lt[jt][8 * gp + e] * inv;
            bf16x8 phi, plo;
            split_hi_lo(pp, phi, plo);
            o = mfma32(as_bf16x8(vop), phi, o);
            o = mfma32(as_bf16x8(vop), plo, o);
        }
    }
    return o;
}

// Writes a wave's output accumulator (query l32, columns 32 ct + 16 hh + r)
// as bf16 into a row-major LDS tile of 32 rows (pitch D + 8).
template <int D>
__device__ __forceinline__ void store_tile_lds(uint16_t* tile, const f32x16& o, int l32, int hh, int ct)
{
    u16x8 o0, o1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o0[e] = f32_to_bf16_bits(o[e]);
        o1[e] = f32_to_bf16_bits(o[8 + e]);
    }
    u16x8* op = reinterpret_cast<u16x8*>(tile + l32 * (D + 8) + 32 * ct + 16 * hh);
    op[0] = o0;
    op[1] = o1;
}

// Writes a wave's output accumulator (query l32, columns 32 ct + 16 hh + r)
// as bf16 straight to its output row (two 16-byte stores per lane; the four
// waves of a query tile fill the row's 256 bytes between them).  Non-temporal
// stores: the workgroup never reads them back, and a step measured 1.6 %
// faster with them than with ordinary stores.
template <int D>
__device__ __forceinline__ void store_tile_global(uint16_t* orow, const f32x16& o, int hh, int ct)
{
    u16x8 o0, o1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o0[e] = f32_to_bf16_bits(o[e]);
        o1[e] = f32_to_bf16_bits(o[8 + e]);
    }
    u16x8* op = reinterpret_cast<u16x8*>(orow + 32 * ct + 16 * hh);
    __builtin_nontemporal_store(o0, op);
    __builtin_nontemporal_store(o1, op + 1);
}

// Workgroups per XCD group: the NKT query tiles of 8 consecutive units.
__host__ __device__ inline int step_grid(int units, int nkt) { return (units + 7) / 8 * 8 * nkt; }

template <int D, int NKT, bool kNorm, int M = 0>
__global__ __launch_bounds__(D / 32 * kWave) void step_bf16_mfma(StepArgs a)
{
    constexpr int NC = D / 32;              // value-column tiles = waves
    constexpr int NT = NC * kWave;          // threads
    constexpr int RK = NKT * 32;            // staged key / value rows
    constexpr int P = D + 8;                // LDS row pitch (bf16)
    // K and V row pitches at D = 128 (see the head-pair step kernel)
    constexpr int PK = D == 128 ? D + 24 : P, PV = D == 128 ? D + 32 : P;
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int CQ = 32 * CPR / NT;       // Q chunks per thread
    constexpr int CK = RK * CPR / NT;       // K (and V) chunks per thread
    static_assert(CQ * NT == 32 * CPR && CK * NT == RK * CPR, "even staging split");
    __shared__ __attribute__((aligned(16))) uint16_t sq[32 * P], skv[RK * PK + RK * PV];
    uint16_t* sk = skv;
    uint16_t* sv = skv + RK * PK;
    // after the softmax part, K and V are dead and each wave stages its S^T
    // tile there, a 32-feature quarter (32 rows x 128 bytes) at a time, at a
    // row pitch of SQP floats
    constexpr int SQP = 36, NQ = D / 32;
    static_assert(NC * 32 * SQP * 4 <= (RK * PK + RK * PV) * 2, "S^T quarters fit in the K/V staging");
    __shared__ __attribute__((aligned(16))) float sz[kNorm ? D : 4];   // normalised variant: the unit's z

    // workgroup -> (unit, query tile): the NKT tiles of a unit share b % 8
    const int b = blockIdx.x;
    const int qt = (b / 8) % NKT;
    const int unit = b / (8 * NKT) * 8 + b % 8;
    if (unit >= a.n_req * a.heads) return;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= qt * 32 || slot < 0 || slot >= a.n_slots) return;   // uniform per workgroup

    const int tid = threadIdx.x;
    const int lane = tid % kWave, ct = tid / kWave;
    const int l32 = lane % 32, hh = lane / 32;
    const int64_t rs = (int64_t)a.heads * D;                 // token row stride
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + base;
    uint16_t* out = static_cast<uint16_t*>(a.out) + base;
    const float* st = a.state + ((int64_t)slot * a.heads + h) * D * D;

    const int cA = 32 * ct + 16 * ((l32 / 4) % 2) + 4 * (l32 / 8) + l32 % 4;  // A row -> column
    const int last = Br - 1;
    const float sl2 = a.scale * 1.4426950408889634f;         // logits in log2 units

    // ---- global loads: this thread's Q/K/V chunks, then the wave's S^T tile,
    // non-temporal where this workgroup is their only reader (with two query
    // tiles the unit's other workgroup reads K, V and S again, on the same
    // XCD, from its L2); the S^T tile in 128-byte row pieces: load i of quarter qq
    // gives lane l features 32 qq + 4 (l % 8) .. + 3 of tile row 8 i + l / 8
    // (coalesced; the operand layout needs 32 bytes of each of 32 rows per
    // instruction, which the caches served poorly)
    u32x4 cq[CQ], ck[CK], cv[CK];
#pragma unroll
    for (int u = 0; u < CK; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        if (u < CQ) {
            const int rq = qt * 32 + row;
            cq[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + (int64_t)(rq < Br ? rq : last) * rs + c8));
        }
        const int64_t off = (int64_t)(row < Br ? row : last) * rs + c8;
        const u32x4* kp = reinterpret_cast<const u32x4*>(k + off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(v + off);
        ck[u] = NKT == 1 ? __builtin_nontemporal_load(kp) : *kp;
        cv[u] = NKT == 1 ? __builtin_nontemporal_load(vp) : *vp;
    }
    f32x4 sraw[NQ][4];
    const float* stile = st + (int64_t)(32 * ct + lane / 8) * D + 4 * (lane % 8);
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4* sp4 = reinterpret_cast<const f32x4*>(stile + (int64_t)8 * i * D + 32 * qq);
            sraw[qq][i] = NKT == 1 ? __builtin_nontemporal_load(sp4) : *sp4;
        }
    // keep the scheduler from sinking these loads next to their uses: the
    // whole wave's bytes must be in flight before the first wait
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CK; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        if (u < CQ) *reinterpret_cast<u32x4*>(sq + row * P + c8) = cq[u];
        *reinterpret_cast<u32x4*>(sk + row * PK + c8) = ck[u];
        *reinterpret_cast<u32x4*>(sv + row * PV + c8) = cv[u];
    }
    if constexpr (kNorm) stage_z<D>(sz, a.z + ((int64_t)slot * a.heads + h) * D, tid);
    __syncthreads();

    // ---- softmax part (overlaps the S stream)
    float qz = 0.f, beta = 1.f;
    if constexpr (kNorm) qz = query_dot_z<D, M>(sq + l32 * P, sz, hh);
    f32x16 o = softmax_tile<D, NKT, kNorm, PK, PV>(sq, sk, sv, Br, sl2, ct, lane, qz, &beta);
    f32x16 olin = {};                                   // normalised variant: the linear part apart
    // ---- linear part: O^T += S^T phi(Q)^T, S as hi + lo bf16.  Every wave is
    // done with K and V after this barrier; then each wave writes a quarter of
    // its S^T tile to its own part of their LDS and reads its A operands back
    // (row cA - 32 ct, features 16 s + 8 hh .. + 7): LDS accesses of one wave
    // complete in order, so no further barrier is needed
    __syncthreads();
    float* sbuf = reinterpret_cast<float*>(skv) + ct * 32 * SQP;
    const int arow = cA - 32 * ct;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(sbuf + (8 * i + lane / 8) * SQP + 4 * (lane % 8)) = sraw[qq][i];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int s = 2 * qq + s2;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(sbuf + arow * SQP + 16 * s2 + 8 * hh);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(sbuf + arow * SQP + 16 * s2 + 8 * hh + 4);
            const float sv8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            bf16x8 shi, slo;
            split_hi_lo(sv8, shi, slo);
            const u16x8 qv = *reinterpret_cast<const u16x8*>(sq + l32 * P + 16 * s + 8 * hh);
            if constexpr (kNorm) olin = linear_mfma<M>(olin, shi, slo, qv);
            else o = linear_mfma<M>(o, shi, slo, qv);
        }
    }
    if constexpr (kNorm) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[rr] = fmaf(beta, olin[rr], o[rr]);
    }
    // ---- store through LDS: lane holds query qt*32 + l32, columns
    // 32 ct + 16 hh + 0..15; the tile is written back row-major so that each
    // store instruction covers whole head rows
    __syncthreads();                                   // every wave is done with sq
    store_tile_lds<D>(sq, o, l32, hh, ct);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CQ; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        if (qt * 32 + row < Br)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(sq + row * P + c8),   // not read here again
                                        reinterpret_cast<u32x4*>(out + (int64_t)(qt * 32 + row) * rs + c8));
    }
}

// One 32 x 32 tile of the commit: acc holds the old state tile (value rows
// 32 ct + 16 hh + r, features 32 ft + l32 in register r of lane (l32, hh)) and
// gets phi(K)^T V of the block's first Br keys added by the matrix cores.  A is
// V^T and B is ReLU(K), both through the transposing LDS read of the staged
// rows (pitches PK and PV); keys past Br are zeroed in the V^T operand.
template <int D, int NKT, int PK = D + 8, int PV = D + 8, int M = 0>
__device__ __forceinline__ f32x16 commit_tile(f32x16 acc, const uint16_t* sk, const uint16_t* sv, int Br, int ct,
                                              int ft, int lane)
{
    const int hh = lane / 32, g = lane / 16, jl = lane % 16;
    const int vcol = 32 * ct + 16 * ((jl % 4) % 2) + 8 * (g % 2) + 4 * ((jl % 4) / 2);
    const int kcol = 32 * ft + 16 * (g % 2) + 4 * (jl % 4);
#pragma unroll
    for (int jt = 0; jt < NKT; ++jt) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            const int row0 = jt * 32 + 16 * gp + 4 * hh + jl / 4;
            const s16x4 v0 = lds_read_tr4(sv + row0 * PV + vcol);
            const s16x4 v1 = lds_read_tr4(sv + (row0 + 8) * PV + vcol);
            const s16x4 k0 = lds_read_tr4(sk + row0 * PK + kcol);
            const s16x4 k1 = lds_read_tr4(sk + (row0 + 8) * PK + kcol);
            const int key0 = jt * 32 + 16 * gp + 4 * hh;    // keys key0 + e, key0 + 8 + e
            u16x8 vop, kop;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vop[e] = key0 + e < Br ? static_cast<uint16_t>(v0[e]) : uint16_t(0);
                vop[4 + e] = key0 + 8 + e < Br ? static_cast<uint16_t>(v1[e]) : uint16_t(0);
                kop[e] = static_cast<uint16_t>(k0[e]);
                kop[4 + e] = static_cast<uint16_t>(k1[e]);
            }
            const PhiOp<M> kp = phi_op<M>(kop);
            acc = mfma32(as_bf16x8(vop), kp.hi, acc);
            if constexpr (!PhiOp<M>::kExact) acc = mfma32(as_bf16x8(vop), kp.lo, acc);
        }
    }
    return acc;
}

// ---------------------------------------------------------------------------
// Fused step + commit (the last denoising step of a block followed by its
// commit, worked example: block 2's output uses S_1, then
// S_{1,2} = S_1 + phi(K_2)^T V_2), bf16, blk <= 32 * NKT.
//
// One workgroup per (request, head) with NKT x D/32 waves: wave (qt, ct)
// computes the outputs of query tile qt, value columns [32 ct, 32 ct + 32),
// from the old S exactly as the step kernel does (its own S^T tile, split
// hi + lo).  After the outputs are staged and stored, every wave has consumed
// its S^T tile, and the commit adds phi(K)^T V into the state, reusing the
// staged K and V: wave (qt, ct) owns state rows [32 ct, 32 ct + 32) and the
// 32-feature tiles ft with ft % NKT == qt; per tile it reads the old values
// in the accumulator layout (an L2 hit: the rows were just streamed), runs
// the MFMA reduction over the block's keys (A = V^T through the transposing
// LDS read, keys past B_r zeroed; B = ReLU(K) through the same read) and
// writes the tile back.  Each state element is read for the step before the
// barrier and written once after it, by one wave; a unit's state is touched
// by one workgroup, so requests only need distinct slots.
// ---------------------------------------------------------------------------
template <int D, int NKT, bool kCommit, bool kNorm, int M = 0>
__global__ __launch_bounds__(NKT * D / 32 * kWave) void step_commit_bf16_mfma(StepArgs a)
{
    constexpr int KS = D / 16;
    constexpr int NC = D / 32;
    constexpr int NT = NKT * NC * kWave;
    constexpr int R = NKT * 32;             // staged rows of Q, K and V
    constexpr int P = D + 8;
    // K and V row pitches at D = 128 (see the head-pair step kernel)
    constexpr int PK = D == 128 ? D + 24 : P, PV = D == 128 ? D + 32 : P;
    constexpr int CPR = D / 8;
    constexpr int CPT = R * CPR / NT;
    // Two query tiles: S^T is staged in LDS (one workgroup per compute unit
    // fits).  One tile: each wave keeps its S^T operands in registers, as the
    // step kernel does, so that several workgroups share a compute unit, and
    // the commit re-reads the old tile from L2.
    constexpr bool kStageS = NKT > 1;
    constexpr int PS = D + 4;               // LDS row pitch of the state tile (fp32)
    constexpr int SPT = D * D / 4 / NT;     // 16-byte state chunks per thread
    static_assert(CPT * NT == R * CPR && SPT * NT * 4 == D * D, "even staging split");
    __shared__ __attribute__((aligned(16))) uint16_t sq[R * P], sk[R * PK], sv[R * PV];
    __shared__ __attribute__((aligned(16))) float ss[kStageS ? D * PS : 4];   // the unit's S^T
    __shared__ __attribute__((aligned(16))) float sz[kNorm ? D : 4];          // normalised variant: the unit's z

    const int unit = blockIdx.x;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;   // uniform per workgroup

    const int tid = threadIdx.x;
    const int lane = tid % kWave, w = tid / kWave;
    const int qt = w / NC, ct = w % NC;
    const int l32 = lane % 32, hh = lane / 32;
    const int64_t rs = (int64_t)a.heads * D;
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + base;
    uint16_t* out = static_cast<uint16_t*>(a.out) + base;
    const int64_t soff = ((int64_t)slot * a.heads + h) * D * D;
    const float* st = (kCommit ? a.state_rw : a.state) + soff;

    const int cA = 32 * ct + 16 * ((l32 / 4) % 2) + 4 * (l32 / 8) + l32 % 4;
    const int last = Br - 1;
    const float sl2 = a.scale * 1.4426950408889634f;

    u32x4 cq[CPT], ck[CPT], cv[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        const int64_t off = (int64_t)(row < Br ? row : last) * rs + c8;
        cq[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + off));   // read once
        ck[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
        cv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
    }
    // the unit's S^T (D x D fp32, contiguous) with whole-row coalesced loads,
    // or this wave's S^T operands
    f32x4 sc[kStageS ? SPT : 1];
    f32x4 sraw[KS][2];
    if constexpr (kStageS) {
#pragma unroll
        for (int u = 0; u < SPT; ++u) sc[u] = reinterpret_cast<const f32x4*>(st)[tid + u * NT];
    } else {
        const f32x4* srow = reinterpret_cast<const f32x4*>(st + (int64_t)cA * D + 8 * hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sraw[s][0] = srow[4 * s];
            sraw[s][1] = srow[4 * s + 1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        *reinterpret_cast<u32x4*>(sq + row * P + c8) = cq[u];
        *reinterpret_cast<u32x4*>(sk + row * PK + c8) = ck[u];
        *reinterpret_cast<u32x4*>(sv + row * PV + c8) = cv[u];
    }
    if constexpr (kStageS) {
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int c4 = tid + u * NT, row = c4 / (D / 4), col = (c4 % (D / 4)) * 4;
            *reinterpret_cast<f32x4*>(ss + row * PS + col) = sc[u];
        }
    }
    if constexpr (kNorm) stage_z<D>(sz, a.z + ((int64_t)slot * a.heads + h) * D, tid);
    __syncthreads();

    // ---- the step, from the old state
    float qz = 0.f, beta = 1.f;
    if constexpr (kNorm) qz = query_dot_z<D, M>(sq + (qt * 32 + l32) * P, sz, hh);
    f32x16 o = softmax_tile<D, NKT, kNorm, PK, PV>(sq + qt * 32 * P, sk, sv, Br, sl2, ct, lane, qz, &beta);
    f32x16 olin = {};                                   // normalised variant: the linear part apart
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        f32x4 s0, s1;
        if constexpr (kStageS) {
            s0 = *reinterpret_cast<const f32x4*>(ss + cA * PS + 16 * s + 8 * hh);
            s1 = *reinterpret_cast<const f32x4*>(ss + cA * PS + 16 * s + 8 * hh + 4);
        } else {
            s0 = sraw[s][0];
            s1 = sraw[s][1];
        }
        const float sv8[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        bf16x8 shi, slo;
        split_hi_lo(sv8, shi, slo);
        const u16x8 qv = *reinterpret_cast<const u16x8*>(sq + (qt * 32 + l32) * P + 16 * s + 8 * hh);
        if constexpr (kNorm) olin = linear_mfma<M>(olin, shi, slo, qv);
        else o = linear_mfma<M>(o, shi, slo, qv);
    }
    if constexpr (kNorm) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[rr] = fmaf(beta, olin[rr], o[rr]);
    }
    // outputs through LDS (sq is free now; the commit below still reads sk, sv)
    __syncthreads();
    store_tile_lds<D>(sq + qt * 32 * P, o, l32, hh, ct);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        if (row < Br)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(sq + row * P + c8),
                                        reinterpret_cast<u32x4*>(out + (int64_t)row * rs + c8));
    }

    if constexpr (!kCommit) return;
    // ---- the commit: S^T[c][f] += sum_j V[j][c] ReLU(K[j][f]) over j < Br
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int ft = qt; ft < NC; ft += NKT) {
        // accumulator register rr of lane (l32, hh): row 32 ct + 16 hh + rr, feature 32 ft + l32
        float* tile = a.state_rw + soff + (int64_t)(32 * ct + 16 * hh) * D + 32 * ft + l32;
        f32x16 acc;
        if constexpr (kStageS) {
            const float* old = ss + (32 * ct + 16 * hh) * PS + 32 * ft + l32;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) acc[rr] = old[rr * PS];
        } else {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) acc[rr] = tile[(int64_t)rr * D];
        }
        acc = commit_tile<D, NKT, PK, PV, M>(acc, sk, sv, Br, ct, ft, lane);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) tile[(int64_t)rr * D] = acc[rr];
    }
    // normalised variant: z += sum phi(k) over the block (z was staged before
    // the first barrier, so the step above used the old value)
    if constexpr (kNorm) commit_z<D, PK, M>(a.z + ((int64_t)slot * a.heads + h) * D, sk, Br, tid);
}

// ---------------------------------------------------------------------------
// Step for blocks of 33..64 rows with D in {64, 128}, optionally followed by
// the commit: one workgroup per (request, head) with 2 x D/32 waves; wave
// (qt, ct) produces the outputs of query tile qt, value columns
// [32 ct, 32 ct + 32).  Work that does not depend on ct is done once per
// workgroup instead of once per wave:
//  - S^T is read with whole-row coalesced loads and split into hi + lo bf16
//    once, into LDS, where each wave reads its A operands;
//  - each of the four 32 x 32 logit tiles (query tile qt, key tile jt) is
//    computed by one wave, which also takes the tile's row max and row sum and
//    writes the tile's probabilities relative to that max (hi + lo bf16, in
//    its lane order) to LDS.
// Without the commit the state loads are issued right after the Q/K/V loads,
// but only Q, K and V are staged before the first barrier: the logit waves run
// their softmax while the state is still in flight, and every wave stages its
// share of S^T after that.  With the commit S^T is staged before the first
// barrier and the waves without a logit tile do their linear part while the
// others run the softmax.
// After the second barrier every wave multiplies V^T by both probability tiles of its
// query tile into two accumulators and merges them with the two-tile softmax
// correction: with tile maxima m_j, sums l_j and M = max_j m_j, the weights are
// 2^(m_j - M) / sum_j l_j 2^(m_j - M).  With D = 128 the logit tiles go to
// waves (0, 0), (0, 1), (1, 2), (1, 3), one per SIMD (wave w runs on SIMD
// w % 4); with D = 64 every wave has one.
// With the commit, each wave also owns the state tiles (32 ct.., 32 ft..) with
// ft % 2 == qt: their old values are loaded in the accumulator layout right
// after the first barrier; once its outputs are stored, the wave adds
// phi(K)^T V to them and writes the tiles back.  The step's coalesced state
// reads complete before the second barrier and every state write follows it,
// each tile's second read precedes its write in the same wave, and every
// element is written once, by one wave.
// Each lane stores its outputs straight from the accumulator: it holds 16
// consecutive value columns of one query row.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D, bool kCommit, bool kNorm, int M = 0>
__global__ __launch_bounds__(2 * D / 32 * kWave) void step_pair_bf16_mfma(StepArgs a)
{
#pragma clang fp contract(off)
    constexpr int KS = D / 16, NC = D / 32, NT = 2 * NC * kWave;
    constexpr int R = 64, P = D + 8, CPR = D / 8;
    // row pitches (bf16) of the staged K and V at D = 128: the transposing
    // reads of V (and of K in the commit) are bank-conflict-free at D + 32 and
    // 2-way at D + 24, which keeps the 16-byte row reads of K conflict-free
    // (D + 8: 4-way for the transposing reads; measured on gfx950 with the LDS
    // bank-conflict counter)
    constexpr int PK = D == 128 ? D + 24 : P, PV = D == 128 ? D + 32 : P;
    constexpr int CPT = R * CPR / NT;            // 16-byte Q, K, V chunks per thread
    constexpr int SPT = D * D / 4 / NT;          // 16-byte S^T chunks per thread
    static_assert(NC >= 2 && CPT * NT == R * CPR && SPT * NT * 4 == D * D, "even staging split");
    // the step stages S^T after the softmax (the state loads are still in
    // flight meanwhile); with the commit, whose old-tile reads follow the
    // first barrier, staging it before that barrier measured faster
    constexpr bool kDeferS = !kCommit;
    // the step also loads V last and stages it after the linear part, so the
    // products with the state run while V arrives and only the products with
    // P follow the last byte
    constexpr bool kLateV = !kCommit;
    __shared__ __attribute__((aligned(16))) uint16_t sq[R * P], sk[R * PK], sv[R * PV];
    __shared__ __attribute__((aligned(16))) uint16_t shi[D * P], slo[D * P];   // S^T = hi + lo
    __shared__ __attribute__((aligned(16))) u16x8 sp[2][2][2][2][kWave];       // [qt][jt][gp][hi, lo][lane]
    __shared__ float smax[2][2][32], ssum[2][2][32];                            // [qt][jt][query]
    __shared__ __attribute__((aligned(16))) float sz[kNorm ? D : 4];           // normalised variant: z
    __shared__ float sqz[kNorm ? 2 : 1][32];                                    // and phi(q).z per query

    const int unit = blockIdx.x;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;   // uniform per workgroup

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int qt = w / NC, ct = w % NC;
    const int l32 = lane % 32, hh = lane / 32;
    const int g = lane / 16, jl = lane % 16;
    const bool has_l = NC == 2 || ct / 2 == qt;               // wave-uniform
    const int jt_l = ct % 2;                                  // its key tile
    const int64_t rs = (int64_t)a.heads * D;
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + base;
    uint16_t* out = static_cast<uint16_t*>(a.out) + base;
    const int64_t soff = ((int64_t)slot * a.heads + h) * D * D;
    const float* st = (kCommit ? a.state_rw : a.state) + soff;
    const int last = Br - 1;
    const float sl2 = a.scale * 1.4426950408889634f;

    // ---- loads: Q, K, V rows (rows past B_r repeat row B_r - 1; non-temporal,
    // read once: 9.6 % faster than ordinary loads), then S^T (and then V with
    // kLateV)
    u32x4 cq[CPT], ck[CPT], cv[CPT];
    auto v_off = [&](int u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        return (int64_t)(row < Br ? row : last) * rs + c8;
    };
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int64_t off = v_off(u);
        cq[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + off));
        ck[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
        if constexpr (!kLateV) cv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
    }
    // 16-byte chunk u of this thread's S^T share: the step reads whole rows
    // (chunk tid + u NT); with the commit, feature blocks (chunks 2b, 2b + 1
    // hold features [32 b, 32 b + 32) of rows (tid + (u % 2) NT) / 8, 8 lanes
    // per 128-byte row piece), which measured 1.5 % faster there and 1.8 %
    // slower in the step
    static_assert(SPT == 2 * (D / 32) && NT / 4 == D, "two chunks per thread and feature block");
    auto s_chunk = [&](int u) {
        return kDeferS ? tid + u * NT : ((tid + (u % 2) * NT) / 8) * (D / 4) + (u / 2) * 8 + tid % 8;
    };
    f32x4 sc[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        // the plain step reads the state once (non-temporal: 4 % faster); the
        // fused commit reads its tiles again for the update
        const f32x4* sp4 = reinterpret_cast<const f32x4*>(st) + s_chunk(u);
        if constexpr (kDeferS) sc[u] = __builtin_nontemporal_load(sp4);
        else sc[u] = *sp4;
    }
    if constexpr (kLateV) {
#pragma unroll
        for (int u = 0; u < CPT; ++u)
            cv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + v_off(u)));
    }
    __builtin_amdgcn_sched_barrier(0);
    auto stage_v = [&]() {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
            *reinterpret_cast<u32x4*>(sv + row * PV + c8) = cv[u];
        }
    };
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        *reinterpret_cast<u32x4*>(sq + row * P + c8) = cq[u];
        *reinterpret_cast<u32x4*>(sk + row * PK + c8) = ck[u];
    }
    if constexpr (!kLateV) stage_v();
    // this thread's S^T chunks into LDS as hi + lo bf16 (waits for their loads)
    auto stage_s = [&]() {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int c4 = s_chunk(u), row = c4 / (D / 4), col = (c4 % (D / 4)) * 4;
            uint32_t h0, h1, l0, l1;
            split_hi_lo2(f32x2{sc[u][0], sc[u][1]}, h0, l0);
            split_hi_lo2(f32x2{sc[u][2], sc[u][3]}, h1, l1);
            *reinterpret_cast<u32x2*>(shi + row * P + col) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(slo + row * P + col) = u32x2{l0, l1};
        }
    };
    if constexpr (!kDeferS) stage_s();
    if constexpr (kNorm) stage_z<D>(sz, a.z + ((int64_t)slot * a.heads + h) * D, tid);
    __syncthreads();

    // with the commit: this wave's old state tiles (value rows 32 ct + 16 hh + r,
    // features 32 ft + l32 in register r; ft = qt, qt + 2, ..) re-read in the
    // accumulator layout now (cache hits: the rows were just read), so that
    // they have arrived when the commit runs after the step
    constexpr int NFT = kCommit ? NC / 2 : 1;
    f32x16 old[NFT];
    if constexpr (kCommit) {
#pragma unroll
        for (int f = 0; f < NFT; ++f) {
            const float* tile = a.state_rw + soff + (int64_t)(32 * ct + 16 * hh) * D + 32 * (qt + 2 * f) + l32;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) old[f][rr] = tile[(int64_t)rr * D];
        }
    }

    const int cA = 32 * ct + 16 * ((l32 / 4) % 2) + 4 * (l32 / 8) + l32 % 4;   // A row -> value column
    const uint16_t* qrow = sq + (qt * 32 + l32) * P + 8 * hh;
    f32x16 o = {};
    // linear part O^T += S^T phi(Q)^T, S^T as hi + lo bf16 from LDS
    auto linear = [&]() {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u16x8 h8 = *reinterpret_cast<const u16x8*>(shi + cA * P + 16 * s + 8 * hh);
            const u16x8 l8 = *reinterpret_cast<const u16x8*>(slo + cA * P + 16 * s + 8 * hh);
            o = linear_mfma<M>(o, as_bf16x8(h8), as_bf16x8(l8), *reinterpret_cast<const u16x8*>(qrow + 16 * s));
        }
    };
    if (has_l) {
        // logit tile L^T = K Q^T (keys 32 jt.., queries 32 qt..): lane (l32, hh)
        // holds query l32 and keys 32 jt + 8 (rr / 4) + 4 hh + rr % 4
        const int jt = jt_l;
        f32x16 lt = {};
        const uint16_t* kr = sk + (jt * 32 + l32) * PK + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            lt = mfma32(as_bf16x8(*reinterpret_cast<const u16x8*>(kr + 16 * s)),
                        as_bf16x8(*reinterpret_cast<const u16x8*>(qrow + 16 * s)), lt);
        float m = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int j = jt * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
            const float x = j < Br ? lt[rr] * sl2 : -INFINITY;
            lt[rr] = x;
            m = fmaxf(m, x);
        }
        m = half_pair_max(m);
        const float mb = m == -INFINITY ? 0.f : m;   // key tile 1 has no valid key when B_r <= 32
        float sum = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float p = __builtin_amdgcn_exp2f(lt[rr] - mb);
            lt[rr] = p;
            sum += p;
        }
        sum = half_pair_sum(sum);
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            float pp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pp[e] = lt[8 * gp + e];
            bf16x8 phi, plo;
            split_hi_lo(pp, phi, plo);
            sp[qt][jt][gp][0][lane] = __builtin_bit_cast(u16x8, phi);
            sp[qt][jt][gp][1][lane] = __builtin_bit_cast(u16x8, plo);
        }
        if (hh == 0) {
            smax[qt][jt][l32] = m;
            ssum[qt][jt][l32] = sum;
        }
        if constexpr (kNorm) {
            if (jt == 0) {                                // one wave per query tile publishes phi(q).z
                const float qz = query_dot_z<D, M>(qrow - 8 * hh, sz, hh);
                if (hh == 0) sqz[qt][l32] = qz;
            }
        }
    } else if constexpr (!kDeferS) {
        linear();                                 // S^T is staged: waves without a logit tile start
    }
    if constexpr (kDeferS) stage_s();
    __syncthreads();

    // ---- O^T of each key tile = V^T P_j^T (V^T through the transposing read;
    // the column of lane i in 16-lane group g is 32 ct + 16 (q % 2) + 8 (g % 2)
    // + 4 (q / 2) + i % 4, q = i / 4, matching cA)
    const int vcol = 32 * ct + 16 * ((jl % 4) % 2) + 8 * (g % 2) + 4 * ((jl % 4) / 2);
    f32x16 opv[2] = {{}, {}};
    auto pv = [&]() {
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                const int row0 = jt * 32 + 16 * gp + 4 * hh + jl / 4;
                const s16x4 v0 = lds_read_tr4(sv + row0 * PV + vcol);
                const s16x4 v1 = lds_read_tr4(sv + (row0 + 8) * PV + vcol);
                u16x8 vop;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vop[e] = static_cast<uint16_t>(v0[e]);
                    vop[4 + e] = static_cast<uint16_t>(v1[e]);
                }
                opv[jt] = mfma32(as_bf16x8(vop), as_bf16x8(sp[qt][jt][gp][0][lane]), opv[jt]);
                opv[jt] = mfma32(as_bf16x8(vop), as_bf16x8(sp[qt][jt][gp][1][lane]), opv[jt]);
            }
        }
    };
    if constexpr (kLateV) {
        linear();
        stage_v();                                   // waits for V, the last loads
        __syncthreads();
        pv();
    } else {
        pv();
        if (kDeferS || has_l) linear();
    }
    // keep the softmax statistics' LDS reads (and their wait) between the
    // matrix-core work above and the first use of its results
    __builtin_amdgcn_sched_barrier(0);
    const float m0 = smax[qt][0][l32], m1 = smax[qt][1][l32];
    const float mx = fmaxf(m0, m1);                  // finite: key 0 is valid
    if constexpr (kNorm) {
        // one denominator for both key tiles and the prefix: divide by 2^c,
        // c = max(mx, log2(phi(q).z)) (as norm_weights does for one tile)
        const float qz = sqz[qt][l32];
        float c = mx;
        if (qz > 0.f) c = fmaxf(c, __builtin_amdgcn_logf(qz));
        c = fmaxf(c, -100.f);
        const float e0 = __builtin_amdgcn_exp2f(m0 - c), e1 = __builtin_amdgcn_exp2f(m1 - c);
        const float wl = __builtin_amdgcn_exp2f(-c);
        const float inv = __builtin_amdgcn_rcpf(ssum[qt][0][l32] * e0 + ssum[qt][1][l32] * e1 + wl * qz);
        const float c0 = e0 * inv, c1 = e1 * inv, beta = wl * inv;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[rr] = o[rr] * beta + (opv[0][rr] * c0 + opv[1][rr] * c1);
    } else {
        const float e0 = __builtin_amdgcn_exp2f(m0 - mx), e1 = __builtin_amdgcn_exp2f(m1 - mx);
        const float inv = __builtin_amdgcn_rcpf(ssum[qt][0][l32] * e0 + ssum[qt][1][l32] * e1);
        const float c0 = e0 * inv, c1 = e1 * inv;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[rr] = o[rr] + (opv[0][rr] * c0 + opv[1][rr] * c1);
    }

    // ---- outputs straight from the accumulator (rows past B_r are not written);
    // with the commit they drain while the state tiles are updated
    if (qt * 32 + l32 < Br) store_tile_global<D>(out + (int64_t)(qt * 32 + l32) * rs, o, hh, ct);

    // ---- the commit: wave (qt, ct) owns state rows [32 ct, 32 ct + 32) and the
    // feature tiles ft with ft % 2 == qt, starting from the old tiles loaded
    // above; it reads only the staged K and V
    if constexpr (kCommit) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < NFT; ++f) {
            const int ft = qt + 2 * f;
            float* tile = a.state_rw + soff + (int64_t)(32 * ct + 16 * hh) * D + 32 * ft + l32;
            const f32x16 acc = commit_tile<D, 2, PK, PV, M>(old[f], sk, sv, Br, ct, ft, lane);
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) __builtin_nontemporal_store(acc[rr], tile + (int64_t)rr * D);   // not read again here
        }
        // normalised variant: z += sum phi(k) over the block (the step used the
        // copy staged before the first barrier)
        if constexpr (kNorm) commit_z<D, PK, M>(a.z + ((int64_t)slot * a.heads + h) * D, sk, Br, tid);
    }
}

// ---------------------------------------------------------------------------
// Step for blocks of 33..64 rows at D = 128, optionally followed by the
// commit, with one wave per SIMD: one workgroup per (request, head) of four
// waves; wave ct produces the outputs of BOTH query tiles for value columns
// [32 ct, 32 ct + 32), so the S^T rows it needs (rows [32 ct, 32 ct + 32),
// 16 KB) are needed by no other wave.  It loads them in 128-byte row pieces
// behind its share of Q, K and V and consumes them a 32-feature quarter at a
// time as they arrive, through a private LDS buffer (fp32; no barrier), so
// that after the last byte only one quarter's multiplications and the stores
// remain.  Wave ct also computes the logit tile (query tile ct / 2, key tile
// ct % 2) and publishes its probabilities and row statistics in LDS, as the
// head-pair kernel does; the V^T operands of the products with P are read
// once for both query tiles.
// With the commit, the wave owns state rows [32 ct, 32 ct + 32) (every
// feature tile): the old tile of feature tile qq is taken from the quarter
// buffer in the accumulator layout, phi(K)^T V is added to it and the tile
// is written back as soon as the quarter's linear products are issued, so
// the state's writes overlap the later quarters' reads.
// ---------------------------------------------------------------------------
template <bool kCommit, bool kNorm, int M = 0>
__global__ __launch_bounds__(4 * kWave) void step_unit_bf16(StepArgs a)
{
#pragma clang fp contract(off)
    constexpr int D = 128, NC = D / 32, NT = NC * kWave;
    constexpr int R = 64, P = D + 8, CPR = D / 8;
    constexpr int PK = D + 24, PV = D + 32;        // as in the head-pair kernel
    constexpr int CPT = R * CPR / NT;              // 16-byte Q, K, V chunks per thread
    constexpr int SQP = 36;                        // fp32 row pitch of a quarter buffer
    static_assert(CPT * NT == R * CPR, "even staging split");
    __shared__ __attribute__((aligned(16))) uint16_t sq[R * P], sk[R * PK], sv[R * PV];
    __shared__ __attribute__((aligned(16))) u16x8 sp[2][2][2][2][kWave];       // [qt][jt][gp][hi, lo][lane]
    __shared__ float smax[2][2][32], ssum[2][2][32];                            // [qt][jt][query]
    __shared__ __attribute__((aligned(16))) float sz[kNorm ? D : 4];
    __shared__ float sqz[kNorm ? 2 : 1][32];
    __shared__ __attribute__((aligned(16))) float sbuf[NC][32 * SQP];          // each wave's quarter buffer

    const int unit = blockIdx.x;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;   // uniform per workgroup

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int ct = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l32 = lane % 32, hh = lane / 32;
    const int g = lane / 16, jl = lane % 16;
    const int64_t rs = (int64_t)a.heads * D;
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + base;
    uint16_t* out = static_cast<uint16_t*>(a.out) + base;
    const int64_t soff = ((int64_t)slot * a.heads + h) * D * D;
    const float* st = (kCommit ? a.state_rw : a.state) + soff;
    const int last = Br - 1;
    const float sl2 = a.scale * 1.4426950408889634f;

    // ---- loads: Q, K, V rows (rows past B_r repeat row B_r - 1), then the
    // wave's S^T rows: load i of quarter qq gives lane l features
    // 32 qq + 4 (l % 8) .. + 3 of row 32 ct + 8 i + l / 8.  All non-temporal:
    // each byte is read once (the commit takes its old values from LDS).
    u32x4 cq[CPT], ck[CPT], cv[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        const int64_t off = (int64_t)(row < Br ? row : last) * rs + c8;
        cq[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + off));
        ck[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
        cv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
    }
    f32x4 sraw[4][4];
    const float* stile = st + (int64_t)(32 * ct + lane / 8) * D + 4 * (lane % 8);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sraw[qq][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(stile + (int64_t)8 * i * D + 32 * qq));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
        *reinterpret_cast<u32x4*>(sq + row * P + c8) = cq[u];
        *reinterpret_cast<u32x4*>(sk + row * PK + c8) = ck[u];
        *reinterpret_cast<u32x4*>(sv + row * PV + c8) = cv[u];
    }
    if constexpr (kNorm) stage_z<D>(sz, a.z + ((int64_t)slot * a.heads + h) * D, tid);
    __syncthreads();

    // ---- logit tile (query tile ct / 2, key tile ct % 2): probabilities
    // relative to the tile's row max (hi + lo, lane order), max and sum
    {
        const int qt = ct / 2, jt = ct % 2;
        const uint16_t* qrow = sq + (qt * 32 + l32) * P + 8 * hh;
        f32x16 lt = {};
        const uint16_t* kr = sk + (jt * 32 + l32) * PK + 8 * hh;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            lt = mfma32(as_bf16x8(*reinterpret_cast<const u16x8*>(kr + 16 * s)),
                        as_bf16x8(*reinterpret_cast<const u16x8*>(qrow + 16 * s)), lt);
        float m = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int j = jt * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
            const float x = j < Br ? lt[rr] * sl2 : -INFINITY;
            lt[rr] = x;
            m = fmaxf(m, x);
        }
        m = half_pair_max(m);
        const float mb = m == -INFINITY ? 0.f : m;   // key tile 1 has no valid key when B_r <= 32
        float sum = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float p = __builtin_amdgcn_exp2f(lt[rr] - mb);
            lt[rr] = p;
            sum += p;
        }
        sum = half_pair_sum(sum);
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            float pp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pp[e] = lt[8 * gp + e];
            bf16x8 phi, plo;
            split_hi_lo(pp, phi, plo);
            sp[qt][jt][gp][0][lane] = __builtin_bit_cast(u16x8, phi);
            sp[qt][jt][gp][1][lane] = __builtin_bit_cast(u16x8, plo);
        }
        if (hh == 0) {
            smax[qt][jt][l32] = m;
            ssum[qt][jt][l32] = sum;
        }
        if constexpr (kNorm) {
            if (jt == 0) {
                const float qz = query_dot_z<D, M>(qrow - 8 * hh, sz, hh);
                if (hh == 0) sqz[qt][l32] = qz;
            }
        }
    }
    __syncthreads();

    // ---- O^T = V^T P^T for both query tiles (V^T through the transposing read,
    // once per key step for both), merged with the two-tile softmax weights
    const int vcol = 32 * ct + 16 * ((jl % 4) % 2) + 8 * (g % 2) + 4 * ((jl % 4) / 2);
    f32x16 opv[2][2] = {{{}, {}}, {{}, {}}};
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            const int row0 = jt * 32 + 16 * gp + 4 * hh + jl / 4;
            const s16x4 v0 = lds_read_tr4(sv + row0 * PV + vcol);
            const s16x4 v1 = lds_read_tr4(sv + (row0 + 8) * PV + vcol);
            u16x8 vop;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vop[e] = static_cast<uint16_t>(v0[e]);
                vop[4 + e] = static_cast<uint16_t>(v1[e]);
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                opv[qt][jt] = mfma32(as_bf16x8(vop), as_bf16x8(sp[qt][jt][gp][0][lane]), opv[qt][jt]);
                opv[qt][jt] = mfma32(as_bf16x8(vop), as_bf16x8(sp[qt][jt][gp][1][lane]), opv[qt][jt]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float beta[2] = {1.f, 1.f}, c0[2], c1[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const float m0 = smax[qt][0][l32], m1 = smax[qt][1][l32];
        const float mx = fmaxf(m0, m1);              // finite: key 0 is valid
        if constexpr (kNorm) {
            const float qz = sqz[qt][l32];
            float c = mx;
            if (qz > 0.f) c = fmaxf(c, __builtin_amdgcn_logf(qz));
            c = fmaxf(c, -100.f);
            const float e0 = __builtin_amdgcn_exp2f(m0 - c), e1 = __builtin_amdgcn_exp2f(m1 - c);
            const float wl = __builtin_amdgcn_exp2f(-c);
            const float inv = __builtin_amdgcn_rcpf(ssum[qt][0][l32] * e0 + ssum[qt][1][l32] * e1 + wl * qz);
            c0[qt] = e0 * inv;
            c1[qt] = e1 * inv;
            beta[qt] = wl * inv;
        } else {
            const float e0 = __builtin_amdgcn_exp2f(m0 - mx), e1 = __builtin_amdgcn_exp2f(m1 - mx);
            const float inv = __builtin_amdgcn_rcpf(ssum[qt][0][l32] * e0 + ssum[qt][1][l32] * e1);
            c0[qt] = e0 * inv;
            c1[qt] = e1 * inv;
        }
    }

    // ---- linear part O^T += S^T phi(Q)^T, a quarter (32 features) at a time
    // as it arrives: the raw rows go to the wave's buffer and come back as A
    // operands (row cA - 32 ct, features 16 s + 8 hh .. + 7); LDS accesses of
    // one wave complete in order, so no barrier is needed
    // With the commit, each quarter's state tile is updated and written back
    // as soon as its products are issued (only this wave reads or writes these
    // rows, and the old values are on chip), so the state's writes overlap the
    // later quarters' reads instead of following the outputs in one burst.
    const int arow = 16 * ((l32 / 4) % 2) + 4 * (l32 / 8) + l32 % 4;
    float* qb = sbuf[ct];
    f32x16 o[2] = {{}, {}};                          // the linear part first, as the head-pair kernel
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(qb + (8 * i + lane / 8) * SQP + 4 * (lane % 8)) = sraw[qq][i];
        f32x16 old;
        if constexpr (kCommit) {
            // the old tile of feature tile qq in the accumulator layout (rows
            // 32 ct + 16 hh + rr, features 32 qq + l32)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) old[rr] = qb[(16 * hh + rr) * SQP + l32];
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int s = 2 * qq + s2;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(qb + arow * SQP + 16 * s2 + 8 * hh);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(qb + arow * SQP + 16 * s2 + 8 * hh + 4);
            const float sv8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            bf16x8 shi, slo;
            split_hi_lo(sv8, shi, slo);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const u16x8 qv = *reinterpret_cast<const u16x8*>(sq + (qt * 32 + l32) * P + 16 * s + 8 * hh);
                o[qt] = linear_mfma<M>(o[qt], shi, slo, qv);
            }
        }
        if constexpr (kCommit) {
            // the commit of tile qq: S^T[c][f] += sum_j V[j][c] phi(K[j][f])
            const f32x16 acc = commit_tile<D, 2, PK, PV, M>(old, sk, sv, Br, ct, qq, lane);
            float* tile = a.state_rw + soff + (int64_t)(32 * ct + 16 * hh) * D + 32 * qq + l32;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) __builtin_nontemporal_store(acc[rr], tile + (int64_t)rr * D);
        }
    }
    // the sum of the two parts in the head-pair kernel's order, so the fused
    // call's outputs are bit-identical to the plain step's
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            if constexpr (kNorm) o[qt][rr] = o[qt][rr] * beta[qt] + (opv[qt][0][rr] * c0[qt] + opv[qt][1][rr] * c1[qt]);
            else o[qt][rr] = o[qt][rr] + (opv[qt][0][rr] * c0[qt] + opv[qt][1][rr] * c1[qt]);
        }
    }

    // ---- outputs straight from the accumulators (rows past B_r are not written)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
        if (qt * 32 + l32 < Br) store_tile_global<D>(out + (int64_t)(qt * 32 + l32) * rs, o[qt], hh, ct);

    if constexpr (kCommit && kNorm) commit_z<D, PK, M>(a.z + ((int64_t)slot * a.heads + h) * D, sk, Br, tid);
}

// ---------------------------------------------------------------------------
// bf16 matrix-core step for long blocks (65..256 rows): one workgroup per
// (request, head, 32-query tile) with D/32 waves (wave ct owns value columns
// [32 ct, 32 ct + 32)), numbered so that the tiles of a unit share an XCD.
// The keys and values stream through LDS in 32-row stages (double-buffered;
// the next stage's loads are issued before the current one is used), and
// each wave runs an online softmax over them (running max and sum per query,
// accumulator rescaled when the max grows), so nothing grows with the block.
// The wave's S^T operands are loaded straight from the state after the last
// key stage (32 contiguous bytes of row cA per lane and k-step) and added to
// the normalised softmax output.
// ---------------------------------------------------------------------------
template <int D, bool kNorm, int M = 0>
__global__ __launch_bounds__(D / 32 * kWave) void step_long_bf16(StepArgs a)
{
#pragma clang fp contract(off)
    constexpr int NC = D / 32, KS = D / 16, NT = NC * kWave;
    constexpr int P = D + 8;
    constexpr int PK = D == 128 ? D + 24 : P, PV = D == 128 ? D + 32 : P;
    constexpr int CPR = D / 8, C = 32 * CPR / NT;   // 16-byte chunks per thread of a 32-row tile
    static_assert(C * NT == 32 * CPR, "even staging split");
    __shared__ __attribute__((aligned(16))) uint16_t sq[32 * P], sk[2][32 * PK], sv[2][32 * PV];
    __shared__ __attribute__((aligned(16))) float sz[kNorm ? D : 4];

    const int b = blockIdx.x;
    const int nqt = (a.blk + 31) / 32;     // query tiles per unit in the grid
    const int qt = (b / 8) % nqt;
    const int unit = b / (8 * nqt) * 8 + b % 8;
    if (unit >= a.n_req * a.heads) return;
    const int r = unit / a.heads, h = unit % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= qt * 32 || slot < 0 || slot >= a.n_slots) return;   // uniform per workgroup

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int ct = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l32 = lane % 32, hh = lane / 32;
    const int g = lane / 16, jl = lane % 16;
    const int64_t rs = (int64_t)a.heads * D;
    const int64_t base = ((int64_t)r * a.blk * a.heads + h) * D;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + base;
    uint16_t* out = static_cast<uint16_t*>(a.out) + base;
    const float* st = a.state + ((int64_t)slot * a.heads + h) * D * D;
    const int last = Br - 1;
    const int nkt = (Br + 31) / 32;
    const float sl2 = a.scale * 1.4426950408889634f;

    auto load_tile = [&](const uint16_t* src, int row0, u32x4 (&x)[C]) {
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const int t = tid + u * NT, row = row0 + t / CPR, c8 = (t % CPR) * 8;
            x[u] = *reinterpret_cast<const u32x4*>(src + (int64_t)(row < Br ? row : last) * rs + c8);
        }
    };
    auto store_tile = [&](uint16_t* dst, int pitch, const u32x4 (&x)[C]) {
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const int t = tid + u * NT;
            *reinterpret_cast<u32x4*>(dst + (t / CPR) * pitch + (t % CPR) * 8) = x[u];
        }
    };

    u32x4 xq[C], xk[C], xv[C];
    load_tile(q, qt * 32, xq);
    load_tile(k, 0, xk);
    load_tile(v, 0, xv);
    store_tile(sq, P, xq);
    if constexpr (kNorm) stage_z<D>(sz, a.z + ((int64_t)slot * a.heads + h) * D, tid);

    const uint16_t* qrow = sq + l32 * P + 8 * hh;
    // V^T operand column of lane i in 16-lane group g (matching cA below)
    const int vcol = 32 * ct + 16 * ((jl % 4) % 2) + 8 * (g % 2) + 4 * ((jl % 4) / 2);
    float m = -INFINITY, l = 0.f;
    f32x16 o = {};
#pragma unroll 1
    for (int jt = 0; jt < nkt; ++jt) {
        const int buf = jt & 1;
        store_tile(sk[buf], PK, xk);
        store_tile(sv[buf], PV, xv);
        __syncthreads();     // also: every wave finished with this buffer two stages ago
        if (jt + 1 < nkt) {
            load_tile(k, (jt + 1) * 32, xk);
            load_tile(v, (jt + 1) * 32, xv);
        }
        f32x16 lt = {};
        const uint16_t* kr = sk[buf] + l32 * PK + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            lt = mfma32(as_bf16x8(*reinterpret_cast<const u16x8*>(kr + 16 * s)),
                        as_bf16x8(*reinterpret_cast<const u16x8*>(qrow + 16 * s)), lt);
        float mt = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int j = jt * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
            const float x = j < Br ? lt[rr] * sl2 : -INFINITY;
            lt[rr] = x;
            mt = fmaxf(mt, x);
        }
        mt = half_pair_max(mt);
        const float mn = fmaxf(m, mt);                        // finite: key jt*32 is valid
        const float corr = __builtin_amdgcn_exp2f(m - mn);    // 0 on the first tile
        float ls = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float p = __builtin_amdgcn_exp2f(lt[rr] - mn);
            lt[rr] = p;
            ls += p;
        }
        ls = half_pair_sum(ls);
        l = l * corr + ls;
        m = mn;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[rr] *= corr;
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            const int row0 = 16 * gp + 4 * hh + jl / 4;
            const s16x4 v0 = lds_read_tr4(sv[buf] + row0 * PV + vcol);
            const s16x4 v1 = lds_read_tr4(sv[buf] + (row0 + 8) * PV + vcol);
            u16x8 vop;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vop[e] = static_cast<uint16_t>(v0[e]);
                vop[4 + e] = static_cast<uint16_t>(v1[e]);
            }
            float pp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pp[e] = lt[8 * gp + e];
            bf16x8 phi, plo;
            split_hi_lo(pp, phi, plo);
            o = mfma32(as_bf16x8(vop), phi, o);
            o = mfma32(as_bf16x8(vop), plo, o);
        }
    }
    // the S^T operands (row cA, features 16 s + 8 hh .. + 7), then the
    // normalisation of the softmax part and the linear part
    const int cA = 32 * ct + 16 * ((l32 / 4) % 2) + 4 * (l32 / 8) + l32 % 4;
    const f32x4* srow = reinterpret_cast<const f32x4*>(st + (int64_t)cA * D + 8 * hh);
    f32x4 sr[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        sr[s][0] = srow[4 * s];
        sr[s][1] = srow[4 * s + 1];
    }
    float alpha, beta = 1.f;
    if constexpr (kNorm) norm_weights(m, l, query_dot_z<D, M>(sq + l32 * P, sz, hh), alpha, beta);
    else alpha = __builtin_amdgcn_rcpf(l);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) o[rr] *= alpha;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const float sv8[8] = {sr[s][0][0], sr[s][0][1], sr[s][0][2], sr[s][0][3],
                              sr[s][1][0], sr[s][1][1], sr[s][1][2], sr[s][1][3]};
        bf16x8 shi, slo;
        split_hi_lo(sv8, shi, slo);
        acc = linear_mfma<M>(acc, shi, slo, *reinterpret_cast<const u16x8*>(qrow + 16 * s));
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) o[rr] = kNorm ? fmaf(beta, acc[rr], o[rr]) : o[rr] + acc[rr];
    const int i = qt * 32 + l32;
    if (i < Br) store_tile_global<D>(out + (int64_t)i * rs, o, hh, ct);
}

// ---------------------------------------------------------------------------
// Plain fp32-arithmetic step for fp32 inputs (any supported d) and for bf16
// with d = 16.  One workgroup of 256 threads per (request, head); query rows
// are taken in groups of up to 32 whose softmax rows live in LDS, everything
// else is read from global memory.
// ---------------------------------------------------------------------------
constexpr int kGenericRows = 32;

template <typename T>
__global__ __launch_bounds__(256) void step_generic(StepArgs a)
{
    extern __shared__ float P[];                  // [rows][Br], then the linear term's weight per row
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
    const float* zg = a.z ? a.z + ((int64_t)slot * a.heads + h) * D : nullptr;
    const int rows = a.blk < kGenericRows ? a.blk : kGenericRows;   // as allocated: rows x (blk + 1) floats
    float* wlin = P + rows * Br;

    for (int i0 = 0; i0 < Br; i0 += rows) {
        const int nr = Br - i0 < rows ? Br - i0 : rows;
        __syncthreads();                          // the previous group's rows are consumed
        for (int idx = threadIdx.x; idx < nr * Br; idx += blockDim.x) {
            const int i = i0 + idx / Br, j = idx % Br;
            float dot = 0.f;
            for (int c = 0; c < D; ++c) dot = fmaf(Elem<T>::load(q, i * rs + c), Elem<T>::load(k, j * rs + c), dot);
            P[idx] = a.scale * dot;
        }
        __syncthreads();
        for (int ii = threadIdx.x; ii < nr; ii += blockDim.x) {
            const int i = i0 + ii;
            float* row = P + ii * Br;
            float m = -INFINITY;
            for (int j = 0; j < Br; ++j) m = fmaxf(m, row[j]);
            float sum = 0.f;
            for (int j = 0; j < Br; ++j) {
                const float p = expf(row[j] - m);
                row[j] = p;
                sum += p;
            }
            float inv = 1.f / sum, beta = 1.f;
            if (zg) {
                // normalised variant: one denominator, both sides divided by e^c,
                // c = max(m, ln(phi(q).z)) (kept above -69, where e^-c stays finite)
                float qz = 0.f;
                for (int f = 0; f < D; ++f) qz = fmaf(phi_rt(a.phi, Elem<T>::load(q, i * rs + f)), zg[f], qz);
                float c = m;
                if (qz > 0.f) c = fmaxf(c, logf(qz));
                c = fmaxf(c, -69.f);
                const float ws = expf(m - c), wl = expf(-c);
                const float den = fmaf(ws, sum, wl * qz);
                inv = ws / den;
                beta = wl / den;
            }
            for (int j = 0; j < Br; ++j) row[j] *= inv;
            wlin[ii] = beta;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nr * D; idx += blockDim.x) {
            const int ii = idx / D, i = i0 + ii, c = idx % D;
            float acc = 0.f;
            for (int j = 0; j < Br; ++j) acc = fmaf(P[ii * Br + j], Elem<T>::load(v, j * rs + c), acc);
            if (zg) {
                float lin = 0.f;
                for (int f = 0; f < D; ++f)
                    lin = fmaf(phi_rt(a.phi, Elem<T>::load(q, i * rs + f)), st[(int64_t)c * D + f], lin);
                acc = fmaf(wlin[ii], lin, acc);
            } else {
                for (int f = 0; f < D; ++f)
                    acc = fmaf(phi_rt(a.phi, Elem<T>::load(q, i * rs + f)), st[(int64_t)c * D + f], acc);
            }
            Elem<T>::store(out, i * rs + c, acc);
        }
    }
}

// ---------------------------------------------------------------------------
// The step on the matrix cores for map M; returns false for the shapes that
// take the fp32 kernel (and, for ELU + 1, blocks of more than 64 rows).
template <int D, int M>
static bool launch_step_d(const StepArgs& a, int units, hipStream_t stream)
{
    constexpr int NT = D / 32 * kWave;
    const bool norm = a.z != nullptr;
    if (a.blk <= 32) {
        if (norm) step_bf16_mfma<D, 1, true, M><<<step_grid(units, 1), NT, 0, stream>>>(a);
        else step_bf16_mfma<D, 1, false, M><<<step_grid(units, 1), NT, 0, stream>>>(a);
        return true;
    }
    if (a.blk <= 64) {
        if constexpr (D >= 64) {
            if (norm) step_pair_bf16_mfma<D, false, true, M><<<units, 2 * NT, 0, stream>>>(a);
            else step_pair_bf16_mfma<D, false, false, M><<<units, 2 * NT, 0, stream>>>(a);
            return true;
        } else {
            if (norm) return false;
            step_bf16_mfma<D, 2, false, M><<<step_grid(units, 2), NT, 0, stream>>>(a);
            return true;
        }
    }
    const int grid = step_grid(units, (a.blk + 31) / 32);
    if (norm) step_long_bf16<D, true, M><<<grid, NT, 0, stream>>>(a);
    else step_long_bf16<D, false, M><<<grid, NT, 0, stream>>>(a);
    return true;
}

// The fused step + commit on the matrix cores for map M (blocks of up to 64
// rows); returns false for the shapes that run the step and then the commit.
template <int D, int M>
static bool launch_step_commit_d(const StepArgs& a, int units, hipStream_t stream)
{
    constexpr int NT = D / 32 * kWave;
    const bool norm = a.z != nullptr;
    if (a.blk > 64) return false;
    if (a.blk <= 32) {
        if (norm) step_commit_bf16_mfma<D, 1, true, true, M><<<units, NT, 0, stream>>>(a);
        else step_commit_bf16_mfma<D, 1, true, false, M><<<units, NT, 0, stream>>>(a);
        return true;
    }
    if constexpr (D == 32) {
        if (norm) return false;
        step_commit_bf16_mfma<D, 2, true, false, M><<<units, 2 * NT, 0, stream>>>(a);
    } else if constexpr (D == 64) {
        if (norm) step_pair_bf16_mfma<D, true, true, M><<<units, 2 * NT, 0, stream>>>(a);
        else step_pair_bf16_mfma<D, true, false, M><<<units, 2 * NT, 0, stream>>>(a);
    } else {
        if (norm) step_unit_bf16<true, true, M><<<units, 4 * kWave, 0, stream>>>(a);
        else step_unit_bf16<true, false, M><<<units, 4 * kWave, 0, stream>>>(a);
    }
    return true;
}

template <int M>
static bool launch_step_m(const StepArgs& a, int units, hipStream_t stream)
{
    switch (a.d) {
    case 32: return launch_step_d<32, M>(a, units, stream);
    case 64: return launch_step_d<64, M>(a, units, stream);
    default: return launch_step_d<128, M>(a, units, stream);
    }
}

template <int M>
static bool launch_step_commit_m(const StepArgs& a, int units, hipStream_t stream)
{
    switch (a.d) {
    case 32: return launch_step_commit_d<32, M>(a, units, stream);
    case 64: return launch_step_commit_d<64, M>(a, units, stream);
    default: return launch_step_commit_d<128, M>(a, units, stream);
    }
}

// z += sum over the block's first B_r rows of phi(k), one workgroup per
// (request, head), thread f < d owning feature f (the normaliser state of the
// normalised variant; the commit of S runs separately).
template <typename T>
__global__ __launch_bounds__(128) void znorm_commit(StepArgs a)
{
    const int D = a.d;
    const int r = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    const int f = threadIdx.x;
    if (Br <= 0 || slot < 0 || slot >= a.n_slots || f >= D) return;
    const int64_t rs = (int64_t)a.heads * D;
    const T* kb = static_cast<const T*>(a.k) + ((int64_t)r * a.blk * a.heads + h) * D + f;
    float acc = 0.f;
    for (int j = 0; j < Br; ++j) acc += phi_rt(a.phi, Elem<T>::load(kb, j * rs));
    a.z[((int64_t)slot * a.heads + h) * D + f] += acc;
}

hipError_t launch_znorm_commit(const StepArgs& a, hipStream_t stream)
{
    const int units = a.n_req * a.heads;
    if (a.dtype_bf16) znorm_commit<uint16_t><<<units, 128, 0, stream>>>(a);
    else znorm_commit<float><<<units, 128, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_step_commit(const StepArgs& a, hipStream_t stream)
{
    const int units = a.n_req * a.heads;
    if (a.dtype_bf16 && a.d >= 32) {
        const bool done = a.phi == 1 ? launch_step_commit_m<1>(a, units, stream)
                                     : launch_step_commit_m<0>(a, units, stream);
        if (done) return hipGetLastError();
    }
    // other shapes: the step, then the commit (and the normaliser's), on the
    // same stream
    hipError_t e = launch_step(a, stream);
    if (e != hipSuccess) return e;
    PhiKVArgs c{};
    c.k = a.k;
    c.v = a.v;
    c.state = a.state_rw;
    c.slots = a.slots;
    c.blk_lens = a.blk_lens;
    c.n_req = a.n_req;
    c.n_slots = a.n_slots;
    c.heads = a.heads;
    c.blk = a.blk;
    c.d = a.d;
    c.dtype_bf16 = a.dtype_bf16;
    c.phi = a.phi;
    e = launch_commit(c, stream);
    if (e != hipSuccess || !a.z) return e;
    return launch_znorm_commit(a, stream);
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream)
{
    const int units = a.n_req * a.heads;
    bool done = false;
    if (a.dtype_bf16 && a.d >= 32)
        done = a.phi == 1 ? launch_step_m<1>(a, units, stream) : launch_step_m<0>(a, units, stream);
    if (!done) {
        const int rows = a.blk < kGenericRows ? a.blk : kGenericRows;
        const size_t lds = sizeof(float) * ((size_t)rows * a.blk + rows);
        if (a.dtype_bf16) step_generic<uint16_t><<<units, 256, lds, stream>>>(a);
        else step_generic<float><<<units, 256, lds, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace ha
