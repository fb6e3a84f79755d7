// Exact full-prefix step: the attention block-hybrid attention replaces.
// Without linearisation every denoising step of the active block attends to
// all previous blocks through the KV cache ("Retrofitting Linear Attention
// into Diffusion Language Models", abstract):
//
//   O = Softmax(scale Q_a [K_p; K_a]^T) [V_p; V_a]
//
// per (request, head), one softmax over the P prefix keys followed by the B_r
// active keys.  It is the comparator of the hybrid step at the same shapes.
#include "device_common.h"
#include "kernels.h"

namespace ha {

typedef short s16x4e __attribute__((ext_vector_type(4)));
typedef s16x4e __attribute__((address_space(3))) lds_s16x4e;

// Four consecutive rows of one column per lane (gfx950 transposing LDS read):
// within each 16-lane group, lane j' supplies the address of 4 bf16 at
// (row0 + j'/4, col(j'%4)) and lane i receives element i%4 of the rows
// supplied by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ s16x4e lds_read_tr4e(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4e*)(p));
}

// ---------------------------------------------------------------------------
// Plan (one workgroup): request r has N_r = P_r + B_r keys in chunks of
// `chunk`; plan[r] = heads * sum_{r' < r} ceil(N_r' / chunk), plan[n_req] = C,
// plan[n_req + 1] = chunks per slice.  A request with no valid query rows
// (B_r <= 0) has no chunks (and no output); malformed prefix offsets (outside
// [0, total_prefix] or running backwards) count as an empty prefix.
// ---------------------------------------------------------------------------

// Valid rows, prefix length and key chunks of request r; Load is uniform_load
// where r is the same in every lane, lane_load otherwise.
template <bool Uniform>
__device__ __forceinline__ int exact_rows(const ExactArgs& a, int r)
{
    const int Br = a.blk_lens ? (Uniform ? uniform_load(a.blk_lens, r) : lane_load(a.blk_lens, r)) : a.blk;
    return Br > a.blk ? a.blk : (Br < 0 ? 0 : Br);
}

template <bool Uniform>
__device__ __forceinline__ int64_t exact_prefix(const ExactArgs& a, int r)
{
    const int64_t s0 = Uniform ? uniform_load(a.cu, r) : lane_load(a.cu, r);
    const int64_t s1 = Uniform ? uniform_load(a.cu, r + 1) : lane_load(a.cu, r + 1);
    return (s0 < 0 || s1 > a.total_prefix || s1 < s0) ? 0 : s1 - s0;
}

__device__ __forceinline__ int64_t exact_chunks(const ExactArgs& a, int r)
{
    const int Br = exact_rows<false>(a, r);
    if (Br <= 0) return 0;
    return (exact_prefix<false>(a, r) + Br + a.chunk - 1) / a.chunk;
}

__global__ __launch_bounds__(256) void exact_plan(ExactArgs a)
{
    __shared__ int64_t part[257];
    const int n = a.n_req, tid = threadIdx.x;
    const int per = (n + 255) / 256;
    const int r0 = tid * per < n ? tid * per : n;
    const int r1 = (r0 + per < n) ? r0 + per : n;
    int64_t s = 0;
    for (int r = r0; r < r1; ++r) s += exact_chunks(a, r);
    part[tid + 1] = s;
    scan256(part, tid);
    int64_t run = part[tid];
    for (int r = r0; r < r1; ++r) {
        a.plan[r] = run * a.heads;
        run += exact_chunks(a, r);
    }
    if (tid == 0) {
        const int64_t C = part[256] * a.heads;
        a.plan[n] = C;
        const int64_t S = (C + a.slices - 1) / a.slices;
        a.plan[n + 1] = S > 0 ? S : 1;
    }
}

// Cursor over one slice's chunk range [c0, c1): pieces are (unit, key range).
// Key j of unit (r, h) is prefix cache row cu[r] + j for j < P, else active
// row j - P; its element offset is (j < P ? cbase : abase) + j * heads * d in
// the cache or the active block respectively.
struct ExactCursor {
    int r, h, Br;
    int64_t c0, c1;     // remaining chunks of the slice
    int64_t j, j1;      // current key stage start and the piece's end (key index within the unit)
    int64_t P;          // prefix length of the unit
    int64_t cbase, abase;
    bool live;
};

__device__ __forceinline__ void exact_next_piece(const ExactArgs& a, ExactCursor& c)
{
    c.live = c.c0 < c.c1;
    if (!c.live) return;
    while (uniform_load(a.plan, c.r + 1) <= c.c0) ++c.r;     // skip finished and empty requests
    const int64_t pr = uniform_load(a.plan, c.r);
    const int64_t nch = (uniform_load(a.plan, c.r + 1) - pr) / a.heads;
    const int64_t local = c.c0 - pr;
    c.h = (int)(local / nch);
    const int64_t k0 = local % nch;
    const int64_t k1 = (k0 + (c.c1 - c.c0) < nch) ? k0 + (c.c1 - c.c0) : nch;
    const int64_t rs = (int64_t)a.heads * a.d;
    c.P = exact_prefix<true>(a, c.r);
    c.Br = exact_rows<true>(a, c.r);
    c.cbase = (c.P > 0 ? uniform_load(a.cu, c.r) : 0) * rs + (int64_t)c.h * a.d;
    c.abase = ((int64_t)c.r * a.blk * a.heads + c.h) * a.d - c.P * rs;
    const int64_t N = c.P + c.Br;
    c.j = k0 * a.chunk;
    c.j1 = k1 * a.chunk < N ? k1 * a.chunk : N;
    c.c0 += k1 - k0;
}

__device__ __forceinline__ bool exact_begin(const ExactArgs& a, ExactCursor& c)
{
    const int64_t C = uniform_load(a.plan, a.n_req), S = uniform_load(a.plan, a.n_req + 1);
    c.c0 = (int64_t)blockIdx.x * S;
    c.c1 = c.c0 + S < C ? c.c0 + S : C;
    if (c.c0 >= c.c1) return false;
    int lo = 0, hi = a.n_req;
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (uniform_load(a.plan, mid) <= c.c0) lo = mid;
        else hi = mid;
    }
    c.r = lo;
    exact_next_piece(a, c);
    return true;
}

// ---------------------------------------------------------------------------
// bf16 matrix-core slice workgroup, head dim D, NQ query tiles of 32 rows.
// D/32 waves; wave ct owns value columns [32 ct, 32 ct + 32) of every query
// row and recomputes the (cheap) logits of each key tile.  Per piece, the
// unit's query block is staged in LDS; key/value rows are staged in 32-key
// stages (row-major, double-buffered, three stages of loads in flight).  The
// online softmax keeps, per query row, the running max m and sum l (lane pair
// l, l ^ 32 hold one query) and rescales the output accumulator when m grows;
// logits are kept in base-2 units (scale * log2 e folded in).  At the end of
// a piece the unnormalised output and (m, l) are written to partial slot
// (slice + unit).
// ---------------------------------------------------------------------------
template <int D, int NQ>
__global__ __launch_bounds__(D / 32 * kWave) __attribute__((amdgpu_waves_per_eu(NQ == 1 ? 3 : (NQ == 2 ? 2 : 1)))) void exact_slices_bf16_mfma(ExactArgs a)
{
    constexpr int KS = D / 16, NC = D / 32, NT = NC * kWave;
    constexpr int TK = 32;                         // keys per stage
    constexpr int RB = 32 * NQ;                    // query rows per unit (padded)
    constexpr int P = D + 8;                       // LDS row pitch (bf16)
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int KCPT = TK * CPR / NT;            // K (and V) chunks per thread per stage
    constexpr int QCPT = RB * CPR / NT;            // Q chunks per thread
    static_assert(KCPT * NT == TK * CPR && QCPT * NT == RB * CPR, "even staging split");
    __shared__ __attribute__((aligned(16))) uint16_t sq[RB * P];
    __shared__ __attribute__((aligned(16))) uint16_t skv[2][2][TK * P];   // [buf][K, V]

    ExactCursor cp;
    if (!exact_begin(a, cp)) return;
    ExactCursor ld = cp;

    const int tid = threadIdx.x, lane = tid % kWave, ct = tid / kWave;
    const int l32 = lane % 32, hh = lane / 32;
    const int64_t rs = (int64_t)a.heads * D;
    const uint16_t* qa = static_cast<const uint16_t*>(a.q);
    const uint16_t* ka = static_cast<const uint16_t*>(a.k);
    const uint16_t* va = static_cast<const uint16_t*>(a.v);
    const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
    const uint16_t* vc = static_cast<const uint16_t*>(a.vc);
    const float sl2 = a.scale * 1.4426950408889634f;
    static_assert(RB == 32 * NQ, "one 32-row query tile per NQ");
    const int slot_floats = RB * (D + 2);       // exact_slot_rows(blk) == RB for the blk this runs with

    auto key_row = [&](const ExactCursor& c, int64_t j, const uint16_t* cache, const uint16_t* act) {
        const int64_t jc = j < c.j1 ? j : c.j1 - 1;             // clamp past the piece
        const bool pre = jc < c.P;
        return (pre ? cache : act) + ((pre ? c.cbase : c.abase) + jc * rs);
    };
    auto load_stage = [&](u32x4 (&x)[2 * KCPT]) {
#pragma unroll
        for (int u = 0; u < KCPT; ++u) {
            const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
            // the cache is streamed once: non-temporal loads (6 % faster)
            x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(key_row(ld, ld.j + row, kc, ka) + c8));
            x[KCPT + u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(key_row(ld, ld.j + row, vc, va) + c8));
        }
        if (ld.live) {
            ld.j += TK;
            if (ld.j >= ld.j1) exact_next_piece(a, ld);
        }
    };
    auto store_stage = [&](int buf, const u32x4 (&x)[2 * KCPT]) {
#pragma unroll
        for (int u = 0; u < KCPT; ++u) {
            const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
            *reinterpret_cast<u32x4*>(&skv[buf][0][row * P + c8]) = x[u];
            *reinterpret_cast<u32x4*>(&skv[buf][1][row * P + c8]) = x[KCPT + u];
        }
    };
    // stage the current piece's query block (rows past B_r repeat row B_r - 1)
    auto load_q = [&]() {
        const int Br = cp.Br;
        const uint16_t* q0 = qa + ((int64_t)cp.r * a.blk * a.heads + cp.h) * D;
#pragma unroll
        for (int u = 0; u < QCPT; ++u) {
            const int t = tid + u * NT, row = t / CPR, c8 = (t % CPR) * 8;
            *reinterpret_cast<u32x4*>(&sq[row * P + c8]) =
                *reinterpret_cast<const u32x4*>(q0 + (int64_t)(row < Br ? row : Br - 1) * rs + c8);
        }
    };

    // Per stage and query tile, one wave (rotating with the stage, so the work
    // spreads over the SIMDs) computes the logits and the online-softmax
    // update and publishes, in LDS, the probabilities as the PV operand of
    // every lane (hi + lo bf16, in lane order), the rescale factor of each
    // query, and the running max and sum.  Every wave then rescales its
    // accumulator and adds V^T P^T for its value columns.
    __shared__ __attribute__((aligned(16))) u16x8 sp[NQ][2][2][kWave];   // [qt][key half gp][hi, lo][lane]
    __shared__ float scorr[NQ][32], sm[NQ][32], sl[NQ][32];
    const int g = lane / 16, jl = lane % 16;
    const int vcol = 32 * ct + 16 * ((jl % 4) % 2) + 8 * (g % 2) + 4 * ((jl % 4) / 2);
    f32x16 o[NQ];
    auto reset = [&]() {                        // a new piece: accumulators and running max / sum
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) o[qt] = f32x16{};
        if (tid < 32 * NQ) {
            sm[tid / 32][tid % 32] = -INFINITY;
            sl[tid / 32][tid % 32] = 0.f;
        }
    };
    reset();
    load_q();
    u32x4 x0[2 * KCPT], x1[2 * KCPT], x2[2 * KCPT];
    load_stage(x0);
    load_stage(x1);
    load_stage(x2);
    int sg = 0;
    // One stage.  Staging and the next loads happen on every path (once the
    // slice is exhausted they repeat the last valid rows), so every path
    // around the loop issues the three register sets' loads in the same order
    // and each stage waits only for its own set; only the arithmetic is
    // skipped past the end.
    auto run_stage = [&](u32x4 (&x)[2 * KCPT]) {
        const int buf = sg & 1;
        store_stage(buf, x);
        __syncthreads();
        load_stage(x);
        if (!cp.live) return;                                   // uniform
        const uint16_t* sk = skv[buf][0];
        const uint16_t* sv = skv[buf][1];
        const int nq = (cp.Br + 31) / 32;
        const int kvalid = (int)(cp.j1 - cp.j < TK ? cp.j1 - cp.j : TK);
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) {
            if (qt >= nq || ct != (sg + qt) % NC) continue;     // uniform per wave
            // L^T = K Q^T for this stage's 32 keys (lane: query qt*32 + l32)
            f32x16 lt = {};
            const uint16_t* qr = sq + (qt * 32 + l32) * P + 8 * hh;
            const uint16_t* kr = sk + l32 * P + 8 * hh;
            // four k-steps of operands at a time keep the register footprint
            // (and so the occupancy) down
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                lt = mfma32(as_bf16x8(*reinterpret_cast<const u16x8*>(kr + 16 * s)),
                            as_bf16x8(*reinterpret_cast<const u16x8*>(qr + 16 * s)), lt);
                if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
            float mt = -INFINITY;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int j = 8 * (rr / 4) + 4 * hh + rr % 4;
                const float xv = j < kvalid ? lt[rr] * sl2 : -INFINITY;
                lt[rr] = xv;
                mt = fmaxf(mt, xv);
            }
            mt = half_pair_max(mt);
            const float mo = sm[qt][l32];
            const float mn = fmaxf(mo, mt);
            const float corr = __builtin_amdgcn_exp2f(mo - mn);     // 0 on the piece's first stage
            float ls = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const float p = __builtin_amdgcn_exp2f(lt[rr] - mn);
                lt[rr] = p;
                ls += p;
            }
            ls = half_pair_sum(ls);
            const float ln = sl[qt][l32] * corr + ls;
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                float pp[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pp[e] = lt[8 * gp + e];
                bf16x8 phi, plo;
                split_hi_lo(pp, phi, plo);
                sp[qt][gp][0][lane] = __builtin_bit_cast(u16x8, phi);
                sp[qt][gp][1][lane] = __builtin_bit_cast(u16x8, plo);
            }
            if (hh == 0) {
                sm[qt][l32] = mn;
                sl[qt][l32] = ln;
                scorr[qt][l32] = corr;
            }
        }
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) {
            if (qt >= nq) continue;
            const float corr = scorr[qt][l32];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) o[qt][rr] *= corr;
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                const int row0 = 16 * gp + 4 * hh + jl / 4;
                const s16x4e v0 = lds_read_tr4e(sv + row0 * P + vcol);
                const s16x4e v1 = lds_read_tr4e(sv + (row0 + 8) * P + vcol);
                u16x8 vop;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vop[e] = static_cast<uint16_t>(v0[e]);
                    vop[4 + e] = static_cast<uint16_t>(v1[e]);
                }
                o[qt] = mfma32(as_bf16x8(vop), as_bf16x8(sp[qt][gp][0][lane]), o[qt]);
                o[qt] = mfma32(as_bf16x8(vop), as_bf16x8(sp[qt][gp][1][lane]), o[qt]);
            }
        }
        ++sg;
        if (cp.j + TK >= cp.j1) {
            // end of the piece: write O (unnormalised, transposed rows of this
            // wave's columns), m and l into slot (slice + unit), then move on
            const int64_t unit = (int64_t)cp.r * a.heads + cp.h;
            float* slotp = a.partial + ((int64_t)blockIdx.x + unit) * slot_floats;
#pragma unroll
            for (int qt = 0; qt < NQ; ++qt) {
                const int i = qt * 32 + l32;
#pragma unroll
                for (int e = 0; e < 16; ++e) slotp[(int64_t)i * D + 32 * ct + 16 * hh + e] = o[qt][e];
                if (ct == 0 && hh == 0) {
                    slotp[RB * D + i] = sm[qt][l32];
                    slotp[RB * D + RB + i] = sl[qt][l32];
                }
            }
            __syncthreads();                       // the running max / sum are read before they are reset
            reset();
            cp.j = cp.j1;
            exact_next_piece(a, cp);
            if (cp.live) load_q();                 // every wave passed the barrier: the old block is done
        } else {
            cp.j += TK;
        }
    };
    while (cp.live) {
        run_stage(x0);
        run_stage(x1);
        run_stage(x2);
    }
}

// ---------------------------------------------------------------------------
// Plain fp32-arithmetic slice workgroup (fp32 inputs, and bf16 with d = 16):
// one thread per (query row, value column) with its own online softmax, in
// the same base-2 units as the matrix-core kernel.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void exact_slices_generic(ExactArgs a)
{
    ExactCursor c;
    if (!exact_begin(a, c)) return;
    const int D = a.d;
    const int RB = exact_slot_rows(a.blk);
    const int slot_floats = RB * (D + 2);
    const int64_t rs = (int64_t)a.heads * D;
    const T* qa = static_cast<const T*>(a.q);
    const T* ka = static_cast<const T*>(a.k);
    const T* va = static_cast<const T*>(a.v);
    const T* kc = static_cast<const T*>(a.kc);
    const T* vc = static_cast<const T*>(a.vc);
    const float sl2 = a.scale * 1.4426950408889634f;
    while (c.live) {
        const int64_t Pr = c.P;
        const int Br = c.Br;
        const int64_t unit = (int64_t)c.r * a.heads + c.h;
        float* slotp = a.partial + ((int64_t)blockIdx.x + unit) * slot_floats;
        for (int e = threadIdx.x; e < Br * D; e += blockDim.x) {
            const int i = e / D, col = e % D;
            const T* qi = qa + (((int64_t)c.r * a.blk + i) * a.heads + c.h) * D;
            float m = -INFINITY, l = 0.f, acc = 0.f;
            for (int64_t j = c.j; j < c.j1; ++j) {
                const int64_t off = (j < Pr ? c.cbase : c.abase) + j * rs;
                const T* kj = (j < Pr ? kc : ka) + off;
                const T* vj = (j < Pr ? vc : va) + off;
                float dot = 0.f;
                for (int f = 0; f < D; ++f) dot = fmaf(Elem<T>::load(qi, f), Elem<T>::load(kj, f), dot);
                const float x = sl2 * dot;
                const float mn = fmaxf(m, x);
                const float corr = exp2f(m - mn), p = exp2f(x - mn);
                l = l * corr + p;
                acc = acc * corr + p * Elem<T>::load(vj, col);
                m = mn;
            }
            slotp[(int64_t)i * D + col] = acc;
            if (col == 0) {
                slotp[RB * D + i] = m;
                slotp[RB * D + RB + i] = l;
            }
        }
        c.j = c.j1;
        exact_next_piece(a, c);
    }
}

// ---------------------------------------------------------------------------
// Combine: out[i][c] = sum_w 2^(m_w - M) O_w[i][c] / sum_w 2^(m_w - M) l_w
// over the unit's slices w in ascending order, M = max_w m_w.  One workgroup
// per unit: the row maxima and normalisers first (one thread per row, into
// LDS), then four adjacent columns per thread.  Rows past B_r are not
// written.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void exact_combine(ExactArgs a)
{
    __shared__ float rowM[kMaxBlk], rowInv[kMaxBlk];
    const int r = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
    const int64_t nch = (a.plan[r + 1] - a.plan[r]) / a.heads;
    if (nch <= 0) return;                       // uniform: no valid rows
    const int D = a.d, Br = exact_rows<true>(a, r);
    const int RB = exact_slot_rows(a.blk);
    const int64_t slot_floats = (int64_t)RB * (D + 2);
    const int64_t S = a.plan[a.n_req + 1];
    const int64_t cfirst = a.plan[r] + h * nch, clast = cfirst + nch - 1;
    const int64_t w0 = cfirst / S, w1 = clast / S;
    const int64_t unit = (int64_t)r * a.heads + h;
    const float* p0 = a.partial + (w0 + unit) * slot_floats;
    for (int i = threadIdx.x; i < Br; i += blockDim.x) {
        float M = -INFINITY;
        for (int64_t w = 0; w <= w1 - w0; ++w) M = fmaxf(M, p0[w * slot_floats + RB * D + i]);
        float den = 0.f;
        for (int64_t w = 0; w <= w1 - w0; ++w)
            den += exp2f(p0[w * slot_floats + RB * D + i] - M) * p0[w * slot_floats + RB * D + RB + i];
        rowM[i] = M;
        rowInv[i] = 1.f / den;
    }
    __syncthreads();
    T* out = static_cast<T*>(a.out);
    const int D4 = D / 4;
    for (int e = threadIdx.x; e < Br * D4; e += blockDim.x) {
        const int i = e / D4, c = 4 * (e % D4);
        const float M = rowM[i];
        f32x4 num = {};
        for (int64_t w = 0; w <= w1 - w0; ++w) {
            const float* sp = p0 + w * slot_floats;
            const float f = exp2f(sp[RB * D + i] - M);
            const f32x4 o = *reinterpret_cast<const f32x4*>(sp + (int64_t)i * D + c);
            num += f * o;
        }
        const int64_t o0 = (((int64_t)r * a.blk + i) * a.heads + h) * D + c;
#pragma unroll
        for (int u = 0; u < 4; ++u) Elem<T>::store(out, o0 + u, num[u] * rowInv[i]);
    }
}

// ---------------------------------------------------------------------------

template <int D>
static void launch_exact_mfma(const ExactArgs& a, hipStream_t stream)
{
    const dim3 grid(a.slices), block(D / 32 * kWave);
    if (a.blk <= 32) exact_slices_bf16_mfma<D, 1><<<grid, block, 0, stream>>>(a);
    else if (a.blk <= 64) exact_slices_bf16_mfma<D, 2><<<grid, block, 0, stream>>>(a);
    else exact_slices_bf16_mfma<D, 4><<<grid, block, 0, stream>>>(a);
}

hipError_t launch_exact(const ExactArgs& a, hipStream_t stream)
{
    exact_plan<<<1, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dtype_bf16 && a.d == 128) launch_exact_mfma<128>(a, stream);
    else if (a.dtype_bf16 && a.d == 64) launch_exact_mfma<64>(a, stream);
    else if (a.dtype_bf16 && a.d == 32) launch_exact_mfma<32>(a, stream);
    else if (a.dtype_bf16) exact_slices_generic<uint16_t><<<a.slices, 256, 0, stream>>>(a);
    else exact_slices_generic<float><<<a.slices, 256, 0, stream>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dtype_bf16) exact_combine<uint16_t><<<a.n_req * a.heads, 256, 0, stream>>>(a);
    else exact_combine<float><<<a.n_req * a.heads, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace ha
