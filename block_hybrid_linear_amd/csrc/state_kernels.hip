// Prefix-state kernels: block commit S += ReLU(K)^T V and prompt prefill
// S = sum_t ReLU(k_t)^T v_t ("Retrofitting Linear Attention into Diffusion
// Language Models", paper-daily summary page, section "technical details in
// action": S_1 = phi(K_1)^T V_1, S_{1,2} = phi(K_1)^T V_1 + phi(K_2)^T V_2).
// The state is stored transposed: state[c][f] = S[f][c].
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace ha {

// ---------------------------------------------------------------------------
// bf16 matrix-core reduction of ReLU(K)^T V over a range of token rows.
//
//   dS^T[c][f] = sum_j V[j][c] * ReLU(K[j][f])      (A = V^T, B = ReLU(K), k = token)
//
// The reduction runs over tokens, which are the strided dimension of the
// token-major inputs, so K and V go through LDS transposed: each thread loads
// an 8-token x 8-column block with eight 16-byte loads, transposes it in
// registers and writes eight 16-byte rows of K^T / V^T.  Matrix-core operands
// are then one 16-byte LDS read each.
//
// Lane mapping and LDS layout (d = 128): the column group varies fastest
// across lanes, so a wave's load instruction reads four whole 256-byte head
// rows -- measurably faster from HBM than 128-byte pieces.  The 16 lanes of
// one transposed write then target rows 8 apart, which with the 16-byte row
// padding would share two bank groups; LDS rows are therefore permuted
// within each 16-row block, row c -> (c & ~15) | ((c + c / 16) & 15), which
// spreads those 16 rows over all banks and keeps the 16 consecutive rows of
// an operand read distinct too.  Operand addresses stay affine in the
// k-step, so they fold into instruction offsets.  (d = 64, 32: the token
// group varies fastest, which is conflict-free without a permutation.)
//
// Stages of T tokens are double-buffered in LDS; PF stages of global loads
// are in flight while a stage is multiplied (prefill: 3, commit: 1), one
// barrier per stage.  In the prefill loop every stage issues its loads
// unconditionally (a stage past the end re-reads the last valid rows, which
// hit in L2, and is zeroed when stored), so the number of loads in flight is
// the same on every path.
//
// Output tiles are 32 x 32; wave w owns value-row tile ct = (w*TPW)/NT and
// TPW feature tiles.  Accumulator register r of lane l holds
// c = 32 ct + 8 (r/4) + 4 (l/32) + r%4 and f = 32 ft + l%32, so every register
// of a wave is two 128-byte runs of one state row: coalesced read-modify-write.
// ---------------------------------------------------------------------------
template <int D> struct PhiKVShape;
template <> struct PhiKVShape<128> { static constexpr int NW = 4, T = 64; };
template <> struct PhiKVShape<64> { static constexpr int NW = 4, T = 128; };
template <> struct PhiKVShape<32> { static constexpr int NW = 1, T = 64; };

// HP adjacent heads per workgroup (prefill with d = 128 takes two: their
// columns are contiguous in a token row, so every load instruction reads two
// whole 512-byte row segments, which HBM serves measurably faster than
// 256-byte ones), NW_ waves and T_-token stages.  The LDS tiles then hold
// HP * D rows; wave w works on head w / (NW / HP) of the group.
template <int D, int HP = 1, int NW_ = PhiKVShape<D>::NW * HP, int T_ = PhiKVShape<D>::T>
struct PhiKVTile {
    static constexpr int NW = NW_, T = T_;
    static constexpr int NT = D / 32;                   // tiles per dimension (per head)
    static constexpr int TPW = NT * NT * HP / NW;       // tiles per wave
    static constexpr int PITCH = T + 8;                 // LDS row pitch in bf16 (16 B pad)
    static constexpr int CG = HP * D / 8;               // 8-column groups per token row segment
    static constexpr int NLT = 2 * (T / 8) * CG;        // threads that load a stage, one 8x8 block each
    static_assert(NLT % kWave == 0 && NLT <= NW * kWave, "whole loader waves");
    static constexpr bool kColsFast = D == 128;         // lane mapping, see above
    // 32-token stages (four 16-byte token groups per row): rows c and c ^ 4
    // share a 128-byte line, each in the half that bit 2 of
    // h = ((c >> 3) ^ c) & 7 selects, with the token group at chunk g ^ h.
    // Measured with the LDS bank-conflict counter on gfx950, that is
    // conflict-free both for the staging writes (8 consecutive lanes write
    // rows 8 apart) and for the operand reads (32 consecutive rows, two token
    // groups), where the padded, rotated layout below is 2-way conflicted for
    // each; it also needs no padding.
    static constexpr bool kPacked = T == 32;
    typedef uint16_t Lds[2][2][kPacked ? HP * D * T : HP * D * PITCH];   // [buf][K^T, V^T]
    __device__ __forceinline__ static int row(int c) { return kColsFast ? (c & ~15) | ((c + (c >> 4)) & 15) : c; }
    // element offset of token group g (8 tokens) of logical LDS row c
    __device__ __forceinline__ static int slot(int c, int g)
    {
        if constexpr (kPacked) return (((c >> 3) << 2) | (c & 3)) * 64 + 8 * (g ^ (((c >> 3) ^ c) & 7));
        else return row(c) * PITCH + 8 * g;
    }
};

// Adds ReLU(K)^T V over rows [0, nrows) of (kb, vb) (rows rs elements apart)
// into acc.  nrows >= 1.  Every thread of the workgroup must call it.
template <int D, int PF>
__device__ __forceinline__ void phikv_accumulate(const uint16_t* kb, const uint16_t* vb, int64_t rs,
                                                 int64_t nrows, typename PhiKVTile<D>::Lds& lds,
                                                 f32x16 (&acc)[PhiKVTile<D>::TPW])
{
    using P = PhiKVTile<D>;
    constexpr int T = P::T, NT = P::NT, TPW = P::TPW, CG = P::CG;
    static_assert(P::NLT == P::NW * kWave, "every thread stages one block");
    const int tid = threadIdx.x;
    const int lane = tid % kWave, w = tid / kWave;
    const int l32 = lane % 32, hh = lane / 32;

    // this thread's 8x8 staging block: tensor (K or V), token group, column group
    const int blocks_per_tensor = (T / 8) * CG;
    const int tensor = tid / blocks_per_tensor;          // 0 = K, 1 = V
    const int bidx = tid % blocks_per_tensor;
    const int tg = P::kColsFast ? bidx / CG : bidx % (T / 8);
    const int cg = P::kColsFast ? bidx % CG : bidx / (T / 8);
    const uint16_t* src = (tensor == 0 ? kb : vb) + cg * 8;

    auto load_stage = [&](int64_t t0, u32x4 (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t t = t0 + tg * 8 + e;
            const int64_t tc = t < nrows ? t : nrows - 1;   // unconditional load; zeroed at store
            x[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + tc * rs));   // read once
        }
    };
    // zero rows past the range, transpose the 8x8 bf16 block, write 8 rows
    auto store_stage = [&](int buf, int64_t t0, const u32x4 (&xin)[8]) {
        u32x4 x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (t0 + tg * 8 + e < nrows) ? xin[e] : u32x4{0, 0, 0, 0};
        uint16_t* dst = lds[buf][tensor];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 y;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = x[2 * p][c / 2], hi = x[2 * p + 1][c / 2];
                y[p] = (c % 2 == 0) ? ((lo & 0xffffu) | (hi << 16)) : ((lo >> 16) | (hi & 0xffff0000u));
            }
            *reinterpret_cast<u32x4*>(dst + P::slot(cg * 8 + c, tg)) = y;
        }
    };
    auto mma_stage = [&](int buf) {
        const uint16_t* kt = lds[buf][0];
        const uint16_t* vt = lds[buf][1];
#pragma unroll
        for (int s = 0; s < T / 16; ++s) {
            const int g = 2 * s + hh;                       // token group of this lane's 8 tokens
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int t = w * TPW + u, ct = t / NT, ft = t % NT;
                const u16x8 av = *reinterpret_cast<const u16x8*>(vt + P::slot(ct * 32 + l32, g));
                const u16x8 bk = *reinterpret_cast<const u16x8*>(kt + P::slot(ft * 32 + l32, g));
                acc[u] = mfma32(as_bf16x8(av), as_bf16x8(relu_bf16x8(bk)), acc[u]);
            }
        }
    };

    const int nstages = (int)((nrows + T - 1) / T);
    u32x4 x0[8], x1[8], x2[8];
    load_stage(0, x0);
    if (PF > 1) load_stage((int64_t)T, x1);
    if (PF > 2) load_stage((int64_t)2 * T, x2);
    auto run_stage = [&](int sg, u32x4 (&x)[8], bool more) {
        const int buf = sg & 1;
        // The barrier also guarantees every wave finished reading this buffer
        // two stages ago, before it is overwritten.
        store_stage(buf, (int64_t)sg * T, x);
        __syncthreads();
        if (more) load_stage((int64_t)(sg + PF) * T, x);
        mma_stage(buf);
    };
    if (PF == 1) {
        for (int sg = 0; sg < nstages; ++sg) run_stage(sg, x0, sg + 1 < nstages);
    } else {
        for (int sg = 0; sg < nstages; sg += 3) {
            run_stage(sg, x0, true);
            run_stage(sg + 1, x1, true);
            run_stage(sg + 2, x2, true);
        }
    }
    __syncthreads();   // LDS is reused by the caller's next range
}

// Writes (store = true) or reads (store = false) the tiles of a d x d state
// that wave w of the WPH waves working on it holds.  The writes are
// non-temporal (the kernel never reads them back; for the prefill's partial
// states that measured 2.9 % faster, with the reduce's non-temporal reads).
template <int D, int WPH = PhiKVShape<D>::NW>
__device__ __forceinline__ void tiles_io(float* base, f32x16 (&acc)[(D / 32) * (D / 32) / WPH], bool store, int w)
{
    constexpr int NT = D / 32, TPW = NT * NT / WPH;
    const int lane = threadIdx.x % kWave;
    const int l32 = lane % 32, hh = lane / 32;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = w * TPW + u, ct = t / NT, ft = t % NT;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int c = ct * 32 + 8 * (rr / 4) + 4 * hh + rr % 4;
            float* p = base + (int64_t)c * D + ft * 32 + l32;
            if (store) __builtin_nontemporal_store(acc[u][rr], p);
            else acc[u][rr] = *p;
        }
    }
}

// ---------------------------------------------------------------------------
// Commit: one workgroup per (request, head); the accumulators start from the
// old state tiles, so the matrix cores add ReLU(K)^T V onto S in fp32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(PhiKVShape<D>::NW * kWave) void commit_bf16_mfma(PhiKVArgs a)
{
    using P = PhiKVTile<D>;
    __shared__ __attribute__((aligned(16))) typename P::Lds lds;
    const int r = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;
    const int64_t rs = (int64_t)a.heads * D;
    const int64_t off = (int64_t)r * a.blk * rs + (int64_t)h * D;
    float* st = a.state + ((int64_t)slot * a.heads + h) * D * D;
    f32x16 acc[P::TPW];
    tiles_io<D>(st, acc, false, threadIdx.x / kWave);
    phikv_accumulate<D, 1>(static_cast<const uint16_t*>(a.k) + off, static_cast<const uint16_t*>(a.v) + off, rs,
                           Br, lds, acc);
    tiles_io<D>(st, acc, true, threadIdx.x / kWave);
}

// ---------------------------------------------------------------------------
// Prefill, step 1 (one workgroup): the plan.  A unit is a group of hp
// adjacent heads (hp = 1 or 2, upr = heads / hp units per request).  Prompt r
// is cut into nch_r = ceil(L_r / chunk) chunks.  The work list is laid out
// unit by unit, and within a unit prompt by prompt: unit u's part is the
// N = sum_r nch_r chunks of all prompts in order, the same for every unit.
// plan[r] = sum over r' < r of nch_r' (exclusive prefix), plan[n_req] = N and
// plan[n_req + 1] = chunks per slice ceil(N / spu) (spu slices per unit).
// Malformed offsets (outside [0, total_tokens] or decreasing) count as empty
// prompts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t chunks_of(const PhiKVArgs& a, int r)
{
    const int64_t s0 = a.cu[r], s1 = a.cu[r + 1];
    if (s0 < 0 || s1 > a.total_tokens || s1 < s0) return 0;
    return (s1 - s0 + a.chunk - 1) / a.chunk;
}

__global__ __launch_bounds__(256) void prefill_plan(PhiKVArgs a)
{
    __shared__ int64_t part[257];
    const int n = a.n_req, tid = threadIdx.x;
    const int per = (n + 255) / 256;
    const int r0 = tid * per < n ? tid * per : n;
    const int r1 = (r0 + per < n) ? r0 + per : n;
    int64_t s = 0;
    for (int r = r0; r < r1; ++r) s += chunks_of(a, r);
    part[tid + 1] = s;
    scan256(part, tid);
    int64_t run = part[tid];
    for (int r = r0; r < r1; ++r) {
        a.plan[r] = run;
        run += chunks_of(a, r);
    }
    if (tid == 0) {
        const int64_t N = part[256];
        a.plan[n] = N;
        const int64_t S = (N + a.spu - 1) / a.spu;
        a.plan[n + 1] = S > 0 ? S : 1;
    }
}

// ---------------------------------------------------------------------------
// Prefill, step 2: slice workgroups.  Slice w = u spu + i owns chunks
// [i S, (i+1) S) of unit u's part of the list -- the same number of chunks for
// every workgroup, whatever the prompt lengths, and cut at the same token
// positions for every unit, so the workgroups of the units of one prompt
// stream the same token rows (the same DRAM pages) at the same time.  It
// writes one fp32 partial state per head of each (unit, prompt) it touches,
// into slot w + u n_req + r (hp states per slot).  (The slot is unique:
// slices and (unit, prompt) pieces are both consecutive intervals of the one
// list, so a later slice never overlaps an earlier piece.)
// ---------------------------------------------------------------------------
struct SliceCursor {
    int r;              // request
    int u;              // unit (head group) of the slice
    int w;              // slice index in list order, u spu + i
    int64_t c0, c1;     // remaining chunk range of this slice within the unit's part
};

__device__ __forceinline__ bool slice_begin(const PhiKVArgs& a, SliceCursor& cur)
{
    const int64_t N = uniform_load(a.plan, a.n_req), S = uniform_load(a.plan, a.n_req + 1);
    // workgroups are numbered unit-fast (consecutive workgroups, which the
    // dispatcher deals to different XCDs, take different units of the same
    // token range)
    const int upr = a.heads / a.hp;
    cur.u = (int)blockIdx.x % upr;
    const int i = (int)blockIdx.x / upr;
    cur.w = cur.u * a.spu + i;
    cur.c0 = (int64_t)i * S;
    cur.c1 = cur.c0 + S < N ? cur.c0 + S : N;
    if (cur.c0 >= cur.c1) return false;
    int lo = 0, hi = a.n_req;                 // last r with plan[r] <= c0
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (uniform_load(a.plan, mid) <= cur.c0) lo = mid;
        else hi = mid;
    }
    cur.r = lo;
    return true;
}

// Next piece of the slice: unit h = cur.u of prompt r (heads hp h ..
// hp h + hp - 1), token rows [t0, t1) of prompt r, whose first row starts at
// element p0 of k and v.
__device__ __forceinline__ void slice_piece(const PhiKVArgs& a, SliceCursor& cur, int& h, int64_t& t0, int64_t& t1,
                                            int64_t& p0)
{
    while (uniform_load(a.plan, cur.r + 1) <= cur.c0) ++cur.r;   // skip finished and empty prompts
    const int64_t pr = uniform_load(a.plan, cur.r), pe = uniform_load(a.plan, cur.r + 1);
    const int64_t k0 = cur.c0 - pr;
    const int64_t k1 = (cur.c1 < pe ? cur.c1 : pe) - pr;
    const int64_t s0 = uniform_load(a.cu, cur.r);
    const int64_t L = uniform_load(a.cu, cur.r + 1) - s0;
    h = cur.u;
    p0 = s0 * a.heads * a.d + (int64_t)h * a.hp * a.d;
    t0 = k0 * a.chunk;
    t1 = k1 * a.chunk < L ? k1 * a.chunk : L;
    cur.c0 += k1 - k0;
}

// A slice is processed as one stream of T-token stages; a stage never spans
// two (request, head) units.  Cursor state is uniform across the workgroup.
struct StageCursor {
    SliceCursor sl;     // chunk position of the next piece
    int r, h;           // unit of the current piece
    int64_t t, t1;      // current stage's first row and the piece's end (rows of prompt r)
    int64_t p0;         // element offset of the piece's prompt row 0, head h
    bool live;
};

__device__ __forceinline__ void stage_next_piece(const PhiKVArgs& a, StageCursor& s)
{
    s.live = s.sl.c0 < s.sl.c1;
    if (!s.live) return;
    slice_piece(a, s.sl, s.h, s.t, s.t1, s.p0);
    s.r = s.sl.r;
}

__device__ __forceinline__ void stage_advance(const PhiKVArgs& a, StageCursor& s, int T)
{
    if (!s.live) return;
    s.t += T;
    if (s.t >= s.t1) stage_next_piece(a, s);
}

// Prefill tile shapes: one head per workgroup as in the commit (4-wave
// workgroups, two per compute unit, every wave loading its block of a stage
// and multiplying its tiles), or a head pair with 32-token stages (64 KB of
// LDS, one workgroup per compute unit) and the roles split: four loader waves
// load, transpose and stage K and V, four compute waves own eight 32 x 32
// tiles each.  Four waves issuing a compute unit's loads stream faster than
// eight with the same bytes in flight (6.7 vs 6.4 TB/s in a load-only probe),
// and the loaders issue each stage's loads right after the barrier instead
// of after their share of the multiplications.
template <int D, int HP> struct PrefillTile {
    typedef PhiKVTile<D> type;
    static constexpr int kLoaders = 0;         // 0: every wave loads and computes
};
template <> struct PrefillTile<128, 2> {
    typedef PhiKVTile<128, 2, 4, 32> type;
    static constexpr int kLoaders = 4;
};
template <int D, int HP>
constexpr int prefill_threads() { return (PrefillTile<D, HP>::type::NW + PrefillTile<D, HP>::kLoaders) * kWave; }

// In the prefill the thread owning token group tg holds tokens tg + (T/8) e,
// e = 0..7 (not 8 tg + e): the lanes of one load instruction then read
// consecutive token rows, which HBM serves faster than rows 8 apart.  LDS
// group g holds that permutation of the stage's tokens for K and V alike, so
// the token reduction is unchanged.
template <int D, int HP, bool kNorm>
__global__ __launch_bounds__((prefill_threads<D, HP>()), 2 / HP) void prefill_slices_bf16_mfma(PhiKVArgs a)
{
    using P = typename PrefillTile<D, HP>::type;
    constexpr int NLD = PrefillTile<D, HP>::kLoaders;
    constexpr int T = P::T, NT = P::NT, TPW = P::TPW, CG = P::CG;
    constexpr int TG = T / 8;                  // token groups per stage
    constexpr int WPH = P::NW / HP;            // compute waves per head
    static_assert(NLD == 0 ? P::NLT == P::NW * kWave : P::NLT == NLD * kWave, "one staging block per loader thread");
    __shared__ __attribute__((aligned(16))) typename P::Lds lds;
    StageCursor cp, ld;                        // compute and load cursors
    if (!slice_begin(a, cp.sl)) return;
    stage_next_piece(a, cp);
    ld = cp;

    const int64_t rs = (int64_t)a.heads * D;
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k);
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v);
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wc = NLD == 0 ? w : w - NLD;               // compute wave index
    const int l32 = lane % 32, hh = lane / 32;
    const int hw = wc / WPH, w4 = wc % WPH;              // the compute wave's head in the group, its index there
    // loader threads (tid < NLT): tensor, token group and column group
    constexpr int blocks_per_tensor = TG * CG;
    const int tensor = tid / blocks_per_tensor;          // 0 = K, 1 = V
    const int bidx = tid % blocks_per_tensor;
    const int tg = P::kColsFast ? bidx / CG : bidx % TG;
    const int cg = P::kColsFast ? bidx % CG : bidx / TG;
    const uint16_t* tbase = (tensor == 0 ? kbase : vbase) + cg * 8;

    // loads of the stage under the load cursor (rows past the piece re-read its
    // last row; a finished cursor re-reads the last row it had).  Non-temporal:
    // every key/value byte is read once, and the stream measured 6 % faster
    // with the non-temporal hint than with ordinary loads.
    auto load_stage = [&](u32x4 (&x)[8]) {
        const uint16_t* src = tbase + ld.p0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t t = ld.t + tg + TG * e;
            const int64_t tc = t < ld.t1 ? t : ld.t1 - 1;
            x[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + tc * rs));
        }
        stage_advance(a, ld, T);
    };
    // The stage buffer is reloaded right after it is stored, so rows past the
    // piece are zeroed in place (no second copy of the stage in registers).
    auto store_stage = [&](int buf, int64_t valid, u32x4 (&x)[8]) {
        if (valid < T) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (tg + TG * e >= valid) x[e] = u32x4{0, 0, 0, 0};
        }
        uint16_t* dst = lds[buf][tensor];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 y;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = x[2 * p][c / 2], hi = x[2 * p + 1][c / 2];
                y[p] = (c % 2 == 0) ? ((lo & 0xffffu) | (hi << 16)) : ((lo >> 16) | (hi & 0xffff0000u));
            }
            *reinterpret_cast<u32x4*>(dst + P::slot(cg * 8 + c, tg)) = y;
        }
    };
    f32x16 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
    // normalised variant: z = sum phi(k) per feature, from the ReLU(K) operands
    // the wave already reads.  The wave's first NZ tiles share one value-row
    // tile and cover NZ distinct feature tiles; in the waves whose first tile
    // is in value row 0 (the ones that write z), lane (l32, hh) sums in fp32
    // its half of each k-step's tokens of feature 32 ft + l32.
    constexpr int NZ = TPW < NT ? TPW : NT;
    const bool zwriter = (w4 * TPW) / NT == 0;           // wave-uniform
    float zacc[kNorm ? NZ : 1];
#pragma unroll
    for (int u = 0; u < (kNorm ? NZ : 1); ++u) zacc[u] = 0.f;
    auto mma_stage = [&](int buf) {
        const uint16_t* kt = lds[buf][0];
        const uint16_t* vt = lds[buf][1];
#pragma unroll
        for (int s = 0; s < T / 16; ++s) {
            const int g = 2 * s + hh;
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int t = w4 * TPW + u, ct = t / NT, ft = t % NT;
                const u16x8 av = *reinterpret_cast<const u16x8*>(vt + P::slot(hw * D + ct * 32 + l32, g));
                const u16x8 bk = relu_bf16x8(*reinterpret_cast<const u16x8*>(kt + P::slot(hw * D + ft * 32 + l32, g)));
                acc[u] = mfma32(as_bf16x8(av), as_bf16x8(bk), acc[u]);
                if constexpr (kNorm && HP == 2) {
                    // head pairs: the z sums from the operand in hand (a second
                    // read as below does not fit in the registers); every wave
                    // sums, only the writer waves' sums are stored
                    if (u < NZ) {
                        const u32x4 w = __builtin_bit_cast(u32x4, bk);
                        float s8 = 0.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            s8 += __uint_as_float(w[e] << 16) + __uint_as_float(w[e] & 0xffff0000u);
                        zacc[u] += s8;
                    }
                }
            }
        }
    };
    // normalised variant, writer waves: the stage's sums of phi(k), re-reading
    // the K^T operands of the first NZ tiles after the multiplications
    auto z_stage = [&](int buf) {
        const uint16_t* kt = lds[buf][0];
#pragma unroll
        for (int s = 0; s < T / 16; ++s) {
            const int g = 2 * s + hh;
#pragma unroll
            for (int u = 0; u < NZ; ++u) {
                const int ft = (w4 * TPW + u) % NT;
                const u32x4 w = __builtin_bit_cast(
                    u32x4, relu_bf16x8(*reinterpret_cast<const u16x8*>(kt + P::slot(hw * D + ft * 32 + l32, g))));
                float s8 = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) s8 += __uint_as_float(w[e] << 16) + __uint_as_float(w[e] & 0xffff0000u);
                zacc[u] += s8;
            }
        }
    };

    // One stage: the loading waves store the compute cursor's stage and issue
    // the loads three stages ahead; the computing waves multiply and flush the
    // unit's partial state when its piece ends.  Staging and loads run on
    // every path (past the end they repeat the last rows), so every path
    // around a loading wave's loop issues the three register sets' loads in
    // the same order and each stage waits only for its own set; only the
    // arithmetic is skipped past the end.  With split roles, loader and
    // compute waves run separate copies of the loop with the same barriers
    // (the cursors are workgroup-uniform), so the compute copy has no loads
    // for the wait counters to track.
    int sg = 0;
    auto run_all = [&](auto load_tag, auto mma_tag) {
        constexpr bool kLoad = decltype(load_tag)::value, kMma = decltype(mma_tag)::value;
        u32x4 x0[8], x1[8], x2[8];
        if constexpr (kLoad) {
            load_stage(x0);
            load_stage(x1);
            load_stage(x2);
        }
        auto run_stage = [&](u32x4 (&x)[8]) {
            const int buf = sg & 1;
            if constexpr (kLoad) store_stage(buf, cp.t1 - cp.t, x);
            __syncthreads();
            if constexpr (kLoad) load_stage(x);
            if (!cp.live) return;              // uniform
            if constexpr (kMma) {
                mma_stage(buf);
                if constexpr (kNorm && HP == 1) {
                    if (zwriter) z_stage(buf);
                }
                if (cp.t + T >= cp.t1) {
                    const int64_t piece = (int64_t)cp.h * a.n_req + cp.r;    // (unit, prompt) of the piece
                    tiles_io<D, WPH>(a.partial + (((int64_t)cp.sl.w + piece) * HP + hw) * D * D, acc, true, w4);
#pragma unroll
                    for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
                    if constexpr (kNorm) {
                        float* zp = a.zpartial + (((int64_t)cp.sl.w + piece) * HP + hw) * D;
#pragma unroll
                        for (int u = 0; u < NZ; ++u) {
                            const float zs = half_pair_sum(zacc[u]);
                            if (zwriter && hh == 0) zp[((w4 * TPW + u) % NT) * 32 + l32] = zs;
                            zacc[u] = 0.f;
                        }
                    }
                }
            }
            ++sg;
            stage_advance(a, cp, T);
        };
        while (cp.live) {
            run_stage(x0);
            run_stage(x1);
            run_stage(x2);
        }
    };
    if constexpr (NLD == 0) run_all(std::true_type{}, std::true_type{});
    else if (w < NLD) run_all(std::true_type{}, std::false_type{});
    else run_all(std::false_type{}, std::true_type{});
}

// Plain fp32-arithmetic version of the slice workgroup (fp32 inputs, and bf16
// with d = 16; one head per unit): one thread per state element, looping over
// the piece's rows.
template <typename T>
__global__ __launch_bounds__(256) void prefill_slices_generic(PhiKVArgs a)
{
    SliceCursor cur;
    if (!slice_begin(a, cur)) return;
    const int D = a.d;
    const int64_t rs = (int64_t)a.heads * D;
    while (cur.c0 < cur.c1) {
        int h;
        int64_t t0, t1, p0;
        slice_piece(a, cur, h, t0, t1, p0);
        const T* kb = static_cast<const T*>(a.k) + p0 + t0 * rs;
        const T* vb = static_cast<const T*>(a.v) + p0 + t0 * rs;
        const int64_t piece = (int64_t)cur.w + (int64_t)h * a.n_req + cur.r;
        float* dst = a.partial + piece * D * D;
        for (int e = threadIdx.x; e < D * D; e += blockDim.x) {
            const int c = e / D, f = e % D;
            float acc = 0.f;
            for (int64_t t = 0; t < t1 - t0; ++t)
                acc = fmaf(Elem<T>::load(vb, t * rs + c), relu(Elem<T>::load(kb, t * rs + f)), acc);
            dst[e] = acc;
        }
        if (a.z) {                                       // normalised variant: sum phi(k) of the piece
            for (int f = threadIdx.x; f < D; f += blockDim.x) {
                float acc = 0.f;
                for (int64_t t = 0; t < t1 - t0; ++t) acc += relu(Elem<T>::load(kb, t * rs + f));
                a.zpartial[piece * D + f] = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill, step 3: S[slot] = sum of the head's partials in ascending slice
// order (deterministic), 0 for an empty prompt.  Each thread owns four
// consecutive floats of one (request, head) state.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_reduce(PhiKVArgs a)
{
    const int h = blockIdx.y, r = blockIdx.z;
    const int slot = a.slots[r];
    if (slot < 0 || slot >= a.n_slots) return;
    const int64_t dd = (int64_t)a.d * a.d;
    const int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e4 >= dd / 4) return;
    const int hu = h / a.hp, sub = h % a.hp;
    const int64_t S = a.plan[a.n_req + 1];
    const int64_t cfirst = a.plan[r], cend = a.plan[r + 1];
    const int64_t piece = (int64_t)hu * a.n_req + r, w0 = (int64_t)hu * a.spu;
    // slices w0 + cfirst / S .. w0 + (cend - 1) / S hold the head's partials
    const int64_t wfirst = w0 + (cend > cfirst ? cfirst / S : 0);
    const int64_t nw = cend > cfirst ? (cend - 1) / S - cfirst / S + 1 : 0;
    // sum of the n partials at base + (wfirst + i + piece) hp stride, i < n, in
    // ascending order; loaded four at a time (indices clamped to the last one,
    // so every load is valid) so that their latencies overlap, non-temporal
    // (each partial is read once)
    auto sum_partials = [&](const float* base, int64_t stride) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int64_t i0 = 0; i0 < nw; i0 += 4) {
            f32x4 p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t w = wfirst + (i0 + j < nw ? i0 + j : nw - 1);
                p[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + ((w + piece) * a.hp + sub) * stride) + e4);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i0 + j < nw) acc += p[j];
        }
        return acc;
    };
    reinterpret_cast<f32x4*>(a.state + ((int64_t)slot * a.heads + h) * dd)[e4] = sum_partials(a.partial, dd);
    if (a.z && e4 < a.d / 4)                             // normalised variant: z, the same way
        reinterpret_cast<f32x4*>(a.z + ((int64_t)slot * a.heads + h) * a.d)[e4] = sum_partials(a.zpartial, a.d);
}

// ---------------------------------------------------------------------------
// Plain fp32-arithmetic commit (fp32 inputs, and bf16 with d = 16): one
// thread per state element, looping over the block's rows.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void commit_generic(PhiKVArgs a)
{
    const int D = a.d;
    const int r = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
    int Br = a.blk_lens ? a.blk_lens[r] : a.blk;
    Br = Br > a.blk ? a.blk : Br;
    const int slot = a.slots[r];
    if (Br <= 0 || slot < 0 || slot >= a.n_slots) return;
    const int64_t rs = (int64_t)a.heads * D;
    const T* kb = static_cast<const T*>(a.k) + (int64_t)r * a.blk * rs + (int64_t)h * D;
    const T* vb = static_cast<const T*>(a.v) + (int64_t)r * a.blk * rs + (int64_t)h * D;
    float* st = a.state + ((int64_t)slot * a.heads + h) * D * D;
    for (int e = threadIdx.x; e < D * D; e += blockDim.x) {
        const int c = e / D, f = e % D;
        float acc = 0.f;
        for (int j = 0; j < Br; ++j)
            acc = fmaf(Elem<T>::load(vb, j * rs + c), relu(Elem<T>::load(kb, j * rs + f)), acc);
        st[e] += acc;
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_commit(const PhiKVArgs& a, hipStream_t stream)
{
    const dim3 grid(a.n_req * a.heads);
    if (a.dtype_bf16 && a.d >= 32) {
        switch (a.d) {
        case 32: commit_bf16_mfma<32><<<grid, PhiKVShape<32>::NW * kWave, 0, stream>>>(a); break;
        case 64: commit_bf16_mfma<64><<<grid, PhiKVShape<64>::NW * kWave, 0, stream>>>(a); break;
        default: commit_bf16_mfma<128><<<grid, PhiKVShape<128>::NW * kWave, 0, stream>>>(a); break;
        }
    } else if (a.dtype_bf16) {
        commit_generic<uint16_t><<<grid, 256, 0, stream>>>(a);
    } else {
        commit_generic<float><<<grid, 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

template <bool kNorm>
static void launch_prefill_slices(const PhiKVArgs& a, dim3 grid, hipStream_t stream)
{
    switch (a.d) {
    case 32: prefill_slices_bf16_mfma<32, 1, kNorm><<<grid, prefill_threads<32, 1>(), 0, stream>>>(a); break;
    case 64: prefill_slices_bf16_mfma<64, 1, kNorm><<<grid, prefill_threads<64, 1>(), 0, stream>>>(a); break;
    default:
        if (a.hp == 2) {
            prefill_slices_bf16_mfma<128, 2, kNorm><<<grid, prefill_threads<128, 2>(), 0, stream>>>(a);
            break;
        }
        prefill_slices_bf16_mfma<128, 1, kNorm><<<grid, prefill_threads<128, 1>(), 0, stream>>>(a);
        break;
    }
}

hipError_t launch_prefill(const PhiKVArgs& a, hipStream_t stream)
{
    prefill_plan<<<1, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.total_tokens > 0) {
        const dim3 grid(a.slices);
        if (a.dtype_bf16 && a.d >= 32) {
            if (a.z) launch_prefill_slices<true>(a, grid, stream);
            else launch_prefill_slices<false>(a, grid, stream);
        } else if (a.dtype_bf16) {
            prefill_slices_generic<uint16_t><<<grid, 256, 0, stream>>>(a);
        } else {
            prefill_slices_generic<float><<<grid, 256, 0, stream>>>(a);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n4 = (int64_t)a.d * a.d / 4;
    prefill_reduce<<<dim3((unsigned)((n4 + 255) / 256), a.heads, a.n_req), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace ha
