// Prefix-state kernels: block commit S += phi(K)^T V and prompt prefill
// S = sum_t phi(k_t)^T v_t ("Retrofitting Linear Attention into Diffusion
// Language Models", paper-daily summary page, section "technical details in
// action": S_1 = phi(K_1)^T V_1, S_{1,2} = phi(K_1)^T V_1 + phi(K_2)^T V_2,
// with phi = ReLU; ELU + 1 as the second fixed map, template argument M).
// The state is stored transposed: state[c][f] = S[f][c].
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace ha {

// ---------------------------------------------------------------------------
// bf16 matrix-core reduction of phi(K)^T V over a range of token rows.
//
//   dS^T[c][f] = sum_j V[j][c] * phi(K[j][f])      (A = V^T, B = phi(K), k = token)
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
// Stages of T tokens are double-buffered in LDS, one barrier per stage.  In
// the commit the next stage's loads are in flight while a stage is
// multiplied; the prefill's own loop keeps three stages of loads in flight,
// issued unconditionally on every path (a stage past the end re-reads the
// last valid rows, which hit in L2, and is padded when stored).
//
// Output tiles are 32 x 32; wave w owns value-row tile ct = (w*TPW)/NT and
// TPW feature tiles.  Accumulator register r of lane l holds
// c = 32 ct + 8 (r/4) + 4 (l/32) + r%4 and f = 32 ft + l%32, so every register
// of a wave is two 128-byte runs of one state row: coalesced read-modify-write.
// ---------------------------------------------------------------------------
// Two bf16 -inf: the key rows that pad a stage (phi(-inf) = 0 for ReLU and
// for ELU + 1, where a zero key would give phi = 1).
constexpr uint32_t kPadKeys = 0xFF80FF80u;

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

// The tiles wave w4 of the waves on one head owns, t = w4 TPW + u, share
// their operands: tile u is value-row tile ct0 + u / NFT and feature tile
// ft0 + u % NFT, so each k-step reads NCT V^T and NFT K^T operands once
// (and applies phi once per K^T operand) for its TPW products.  Written out
// rather than left to the compiler to merge the repeated reads, which it
// does or not depending on the code around.
template <int NT, int TPW> struct TileOperands {
    static constexpr int NFT = TPW < NT ? TPW : NT;      // distinct feature tiles
    static constexpr int NCT = TPW / NFT;                // distinct value-row tiles
    static_assert(NCT * NFT == TPW, "tiles form a ct x ft block");
    __device__ __forceinline__ static int ct0(int w4) { return (w4 * TPW) / NT; }
    __device__ __forceinline__ static int ft0(int w4) { return (w4 * TPW) % NT; }
};

// Adds phi(K)^T V over rows [0, nrows) of (kb, vb) (rows rs elements apart)
// into acc, in stages of tile P.  nrows >= 1.  Every thread of the workgroup
// must call it.  The first P::NLT threads (whole waves) stage K and V; with
// 32-token stages that is fewer than the workgroup, and the other waves only
// multiply.
template <class P, int M = 0>
__device__ __forceinline__ void phikv_accumulate(const uint16_t* kb, const uint16_t* vb, int64_t rs,
                                                 int64_t nrows, typename P::Lds& lds, f32x16 (&acc)[P::TPW])
{
    constexpr int T = P::T, NT = P::NT, TPW = P::TPW, CG = P::CG;
    static_assert(P::NLT <= P::NW * kWave, "at most one staging block per thread");
    const int tid = threadIdx.x;
    const int lane = tid % kWave, w = tid / kWave;
    const int l32 = lane % 32, hh = lane / 32;
    const bool loader = tid < P::NLT;                    // wave-uniform

    // this thread's 8x8 staging block: tensor (K or V), token group, column group
    const int blocks_per_tensor = (T / 8) * CG;
    const int tensor = loader ? tid / blocks_per_tensor : 0;   // 0 = K, 1 = V
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
    // rows past the range: values 0 and keys -inf (phi(-inf) = 0 for every
    // map, so they add nothing to S or to sums of phi(k)); transpose the 8x8
    // bf16 block, write 8 rows
    const uint32_t pad = tensor == 0 ? kPadKeys : 0u;
    auto store_stage = [&](int buf, int64_t t0, const u32x4 (&xin)[8]) {
        u32x4 x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (t0 + tg * 8 + e < nrows) ? xin[e] : u32x4{pad, pad, pad, pad};
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
    using O = TileOperands<NT, TPW>;
    const int ct0 = O::ct0(w), ft0 = O::ft0(w);
    auto mma_stage = [&](int buf) {
        const uint16_t* kt = lds[buf][0];
        const uint16_t* vt = lds[buf][1];
#pragma unroll
        for (int s = 0; s < T / 16; ++s) {
            const int g = 2 * s + hh;                       // token group of this lane's 8 tokens
            u16x8 av[O::NCT];
#pragma unroll
            for (int c = 0; c < O::NCT; ++c)
                av[c] = *reinterpret_cast<const u16x8*>(vt + P::slot((ct0 + c) * 32 + l32, g));
#pragma unroll
            for (int f = 0; f < O::NFT; ++f) {
                const PhiOp<M> kp = phi_op<M>(*reinterpret_cast<const u16x8*>(kt + P::slot((ft0 + f) * 32 + l32, g)));
#pragma unroll
                for (int c = 0; c < O::NCT; ++c) {                // tile u = c NFT + f
                    f32x16& d = acc[c * O::NFT + f];
                    d = mfma32(as_bf16x8(av[c]), kp.hi, d);
                    if constexpr (!PhiOp<M>::kExact) d = mfma32(as_bf16x8(av[c]), kp.lo, d);   // ELU + 1
                }
            }
        }
    };

    const int nstages = (int)((nrows + T - 1) / T);
    u32x4 x[8];
    if (loader) load_stage(0, x);
    for (int sg = 0; sg < nstages; ++sg) {
        const int buf = sg & 1;
        // The barrier also guarantees every wave finished reading this buffer
        // two stages ago, before it is overwritten.
        if (loader) store_stage(buf, (int64_t)sg * T, x);
        __syncthreads();
        if (loader && sg + 1 < nstages) load_stage((int64_t)(sg + 1) * T, x);
        mma_stage(buf);
    }
    __syncthreads();   // LDS is reused by the caller's next range
}

// Writes (store = true) or reads (store = false) the tiles of a d x d state
// that wave w of the WPH waves working on it holds.  The writes are
// non-temporal (the kernel never reads them back; for the prefill's partial
// states that measured 2.9 % faster, with the reduce's non-temporal reads).
//
// Addressing: register r of tile (ct, ft) is row c = 32 ct + 8 (r/4) + 4 hh +
// r%4, column 32 ft + l32.  The wave-uniform part (tile and r/4) goes into a
// scalar base pointer, the lane's part is one offset (4 hh) D + l32, and r%4
// is an immediate.  The offset is made opaque to the optimiser, which would
// otherwise precompute and hold one 64-bit address per register (128 of them
// for eight tiles).
template <int D>
__device__ __forceinline__ uint32_t tile_lane_offset()
{
    const int lane = threadIdx.x % kWave;
    uint32_t lo = (uint32_t)((4 * (lane / 32)) * D + lane % 32);
    asm volatile("" : "+v"(lo));
    return lo;
}

// rot (wave-uniform): accumulator u holds feature tile (t + rot) mod NT of
// its value-row tile instead of t mod NT (a wave whose TPW tiles cover every
// feature tile of one value-row tile may take them in a rotated order).
template <int D, int WPH = PhiKVShape<D>::NW>
__device__ __forceinline__ void tiles_io(float* base, f32x16 (&acc)[(D / 32) * (D / 32) / WPH], bool store, int w,
                                         int rot = 0)
{
    constexpr int NT = D / 32, TPW = NT * NT / WPH;
    const uint32_t lo = tile_lane_offset<D>();
    w = __builtin_amdgcn_readfirstlane(w);
    asm volatile("" : "+s"(base), "+s"(w));  // the tile bases, computed here, not hoisted and held
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = w * TPW + u, ct = t / NT, ft = (t + rot) % NT;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float* b = base + (int64_t)(ct * 32 + 8 * q) * D + ft * 32;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float* p = b + lo + e * D;
                if (store) __builtin_nontemporal_store(acc[u][4 * q + e], p);
                else acc[u][4 * q + e] = *p;
            }
        }
    }
}

// Adds to acc the tiles that tiles_io would read for wave w, with
// non-temporal loads (each partial state is read once).
template <int D, int WPH = PhiKVShape<D>::NW>
__device__ __forceinline__ void tiles_add(const float* base, f32x16 (&acc)[(D / 32) * (D / 32) / WPH], int w)
{
    constexpr int NT = D / 32, TPW = NT * NT / WPH;
    const uint32_t lo = tile_lane_offset<D>();
    w = __builtin_amdgcn_readfirstlane(w);
    asm volatile("" : "+s"(base), "+s"(w));
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = w * TPW + u, ct = t / NT, ft = t % NT;
        f32x16 p;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float* b = base + (int64_t)(ct * 32 + 8 * q) * D + ft * 32;
#pragma unroll
            for (int e = 0; e < 4; ++e) p[4 * q + e] = __builtin_nontemporal_load(b + lo + e * D);
        }
        acc[u] += p;
    }
}

// ---------------------------------------------------------------------------
// Commit: one workgroup per (request, head); the accumulators start from the
// old state tiles, so the matrix cores add phi(K)^T V onto S in fp32.
// ---------------------------------------------------------------------------
// Blocks of at most 32 rows take 32-token stages (T32): a 64- or 128-token
// stage would multiply that many padding rows as well.  The 32-token tile
// has fewer staging blocks than threads, so only the first waves load.
template <int D, int M = 0, bool T32 = false>
__global__ __launch_bounds__(PhiKVShape<D>::NW * kWave) void commit_bf16_mfma(PhiKVArgs a)
{
    using P = PhiKVTile<D, 1, PhiKVShape<D>::NW, T32 ? 32 : PhiKVShape<D>::T>;
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
    phikv_accumulate<P, M>(static_cast<const uint16_t*>(a.k) + off, static_cast<const uint16_t*>(a.v) + off, rs,
                              Br, lds, acc);
    tiles_io<D>(st, acc, true, threadIdx.x / kWave);
}

// ---------------------------------------------------------------------------
// Prefill: two launches, the slice workgroups and the reduce.  A unit is a
// group of hp adjacent heads (hp = 1 or 2, upr = heads / hp units per
// request).  Prompt r is cut into nch_r = ceil(L_r / chunk) chunks.  The work
// list is laid out unit by unit, and within a unit prompt by prompt: unit u's
// part is the N = sum_r nch_r chunks of all prompts in order, the same for
// every unit.  Malformed offsets (outside [0, total_tokens] or decreasing)
// count as empty prompts.  Slice w = u spu + i owns chunks [i S, (i+1) S) of
// unit u's part, S = ceil(N / spu) -- the same number of chunks for every
// workgroup, whatever the prompt lengths, and cut at the same token positions
// for every unit, so the workgroups of the units of one prompt stream the
// same token rows (the same DRAM pages) at the same time.
//
// Each workgroup works out N, S and the prompt holding its first chunk from
// cu_seqlens itself: thread t sums the chunk counts of a run of
// ceil(n_req / 256) prompts, one scan over the 256 run sums gives N and every
// run's first chunk, and the thread whose run holds chunk i S walks its run
// to the prompt.  Workgroup 0 also records the plan for the reduce:
// plan[r] = chunks of the prompts before r (exclusive prefix), plan[n_req] =
// N and plan[n_req + 1] = S.
//
// The (unit, prompt) pieces of a slice each end in one fp32 state per head.
// A piece whose prompt lies inside this slice is written to the state
// directly; a piece of a prompt that spans slices i_first .. i_last becomes a
// partial state in workspace slot w + u n_req + r (hp states per slot;
// unique, because slices and pieces are both consecutive intervals of the
// one list), which the reduce adds up.  (Summing them in the slice kernel,
// by whichever workgroup finishes a prompt last, measured slower: the
// cross-workgroup hand-off needs an agent-scope release, a write-back of the
// whole L2, per arrival, and the sums bunch up at the kernel's end in a few
// waves, where the reduce spreads them over the whole GPU.)
// ---------------------------------------------------------------------------
// A value that is the same in every lane, as such (kept in scalar registers).
__device__ __forceinline__ int64_t first_lane64(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// floor(n / d) for 0 <= n < 2^53 and 1 <= d < 2^53: the correctly rounded
// fp64 quotient truncates to the true quotient or to one more or less, which
// one integer comparison corrects.  A handful of instructions where a 64-bit
// integer division expands to a long sequence (and these are inlined into
// every copy of the cursor code).
__device__ __forceinline__ int64_t div_floor(int64_t n, int64_t d)
{
    int64_t q = (int64_t)((double)n / (double)d);
    if (q * d > n) --q;
    else if ((q + 1) * d <= n) ++q;
    return q;
}

__device__ __forceinline__ int64_t chunks_of(const PhiKVArgs& a, int r)
{
    const int64_t s0 = a.cu[r], s1 = a.cu[r + 1];
    if (s0 < 0 || s1 > a.total_tokens || s1 < s0) return 0;
    return div_floor(s1 - s0 + a.chunk - 1, a.chunk);
}

// The same where r is the same in every lane (the cursor's prompt).
__device__ __forceinline__ int64_t chunks_of_uniform(const PhiKVArgs& a, int r)
{
    const int64_t s0 = uniform_load(a.cu, r), s1 = uniform_load(a.cu, r + 1);
    if (s0 < 0 || s1 > a.total_tokens || s1 < s0) return 0;
    return first_lane64(div_floor(s1 - s0 + a.chunk - 1, a.chunk));
}

struct SliceCursor {
    int r;              // request
    int u;              // unit (head group) of the slice
    int w;              // slice index in list order, u spu + i
    int64_t c0, c1;     // remaining chunk range of this slice within the unit's part
    int64_t pr;         // chunks of the prompts before r in the unit's part
    int64_t lo, hi;     // the slice's whole chunk range
};

// Plans the workgroup's slice (see above); workgroup 0 also writes the plan
// for the reduce.  part: 259 int64 of LDS, free again on return.  Every
// thread of the workgroup calls it; returns false when the slice has no
// chunks.
__device__ __forceinline__ bool slice_begin(const PhiKVArgs& a, SliceCursor& cur, int64_t* part)
{
    // 256 runs whatever the workgroup size (64, 256 or 512 threads): thread
    // tid handles runs tid, tid + blockDim.x, ...
    constexpr int kRuns = 256, kMaxRunsPerThread = 4;
    const int tid = threadIdx.x, nt = blockDim.x, n = a.n_req;
    const int per = (n + kRuns - 1) / kRuns;
    auto run_first = [&](int v) { return v * per < n ? v * per : n; };
    auto run_end = [&](int v) { return run_first(v) + per < n ? run_first(v) + per : n; };
    for (int v = tid; v < kRuns; v += nt) {
        int64_t s = 0;
        for (int r = run_first(v); r < run_end(v); ++r) s += chunks_of(a, r);
        part[v + 1] = s;
    }
    if (tid == 0) part[0] = 0;
    for (int off = 1; off < kRuns; off <<= 1) {          // inclusive scan of part[1..256]
        __syncthreads();
        int64_t add[kMaxRunsPerThread];
#pragma unroll
        for (int j = 0; j < kMaxRunsPerThread; ++j) {
            const int v = tid + j * nt;
            add[j] = (v < kRuns && v >= off) ? part[v + 1 - off] : 0;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxRunsPerThread; ++j) {
            const int v = tid + j * nt;
            if (v < kRuns) part[v + 1] += add[j];
        }
    }
    __syncthreads();
    const int64_t N = first_lane64(part[256]);
    const int64_t S = N > 0 ? first_lane64(div_floor(N + a.spu - 1, a.spu)) : 1;
    if (blockIdx.x == 0) {
        for (int v = tid; v < kRuns; v += nt) {
            int64_t pr = part[v];
            for (int r = run_first(v); r < run_end(v); ++r) {
                a.plan[r] = pr;
                pr += chunks_of(a, r);
            }
        }
        if (tid == 0) {
            a.plan[n] = N;
            a.plan[n + 1] = S;
        }
    }
    // workgroups are numbered unit-fast (consecutive workgroups, which the
    // dispatcher deals to different XCDs, take different units of the same
    // token range)
    const int upr = a.heads / a.hp;
    cur.u = (int)blockIdx.x % upr;
    const int i = (int)blockIdx.x / upr;
    cur.w = cur.u * a.spu + i;
    cur.c0 = (int64_t)i * S;
    cur.c1 = cur.c0 + S < N ? cur.c0 + S : N;
    cur.lo = cur.c0;
    cur.hi = cur.c1;
    for (int v = tid; v < kRuns; v += nt) {              // the one run holding chunk c0
        if (cur.c0 < cur.c1 && part[v] <= cur.c0 && cur.c0 < part[v + 1]) {
            int64_t pr = part[v];
            int r = run_first(v);
            for (int64_t ch = chunks_of(a, r); pr + ch <= cur.c0; ch = chunks_of(a, r)) {
                pr += ch;
                ++r;
            }
            part[257] = r;
            part[258] = pr;
        }
    }
    __syncthreads();
    cur.r = cur.c0 < cur.c1 ? (int)first_lane64(part[257]) : 0;
    cur.pr = cur.c0 < cur.c1 ? first_lane64(part[258]) : 0;
    __syncthreads();                                     // part is free again
    return cur.c0 < cur.c1;
}

// Next piece of the slice: unit h = cur.u of prompt r (heads hp h ..
// hp h + hp - 1), token rows [t0, t1) of prompt r, whose first row starts at
// element p0 of k and v; [pr, pe) is the prompt's chunk range in the unit's
// part.
__device__ __forceinline__ void slice_piece(const PhiKVArgs& a, SliceCursor& cur, int& h, int64_t& t0, int64_t& t1,
                                            int64_t& p0, int64_t& pr, int64_t& pe)
{
    int64_t ch = chunks_of_uniform(a, cur.r);
    while (cur.pr + ch <= cur.c0) {                      // skip finished and empty prompts
        cur.pr += ch;
        ++cur.r;
        ch = chunks_of_uniform(a, cur.r);
    }
    pr = cur.pr;
    pe = pr + ch;
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
    int64_t pr, pe;     // the prompt's chunk range in the unit's part
    bool live;
};

__device__ __forceinline__ void stage_next_piece(const PhiKVArgs& a, StageCursor& s)
{
    s.live = s.sl.c0 < s.sl.c1;
    if (!s.live) return;
    slice_piece(a, s.sl, s.h, s.t, s.t1, s.p0, s.pr, s.pe);
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
template <int D, int HP, bool kNorm, int M = 0>
__global__ __launch_bounds__((prefill_threads<D, HP>()), 2 / HP) void prefill_slices_bf16_mfma(PhiKVArgs a)
{
    using P = typename PrefillTile<D, HP>::type;
    constexpr int NLD = PrefillTile<D, HP>::kLoaders;
    constexpr int T = P::T, NT = P::NT, TPW = P::TPW, CG = P::CG;
    constexpr int TG = T / 8;                  // token groups per stage
    constexpr int WPH = P::NW / HP;            // compute waves per head
    static_assert(NLD == 0 ? P::NLT == P::NW * kWave : P::NLT == NLD * kWave, "one staging block per loader thread");
    __shared__ __attribute__((aligned(16))) typename P::Lds lds;
    static_assert(sizeof(lds) >= 259 * sizeof(int64_t), "the plan scan borrows the stage buffers");
    StageCursor cp, ld;                        // compute and load cursors
    if (!slice_begin(a, cp.sl, reinterpret_cast<int64_t*>(&lds))) return;
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
    // `valid` records the stage's rows in its piece (0 past the slice's end),
    // for the store three stages later.
    auto load_stage = [&](u32x4 (&x)[8], int64_t& valid) {
        valid = ld.live ? ld.t1 - ld.t : 0;
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
    // piece are padded in place (no second copy of the stage in registers):
    // values 0, keys -inf, whose phi is 0 for every map.
    const uint32_t pad = tensor == 0 ? kPadKeys : 0u;
    auto store_stage = [&](int buf, int64_t valid, u32x4 (&x)[8]) {
        if (valid < T) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (tg + TG * e >= valid) x[e] = u32x4{pad, pad, pad, pad};
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
    // normalised variant: z = sum phi(k) per feature, from the phi(K) operands
    // the wave holds for its products; lane (l32, hh) sums in fp32 its half of
    // each k-step's tokens of feature 32 ft + l32.  Head pairs: every compute
    // wave sums its NZ distinct feature tiles and the waves whose first tile
    // is in value row 0 write them.  One head per workgroup: feature tile ft
    // is summed and written by wave ft alone, so the work is spread over the
    // waves (one writer summing every tile made it the straggler at each
    // stage's barrier).  Where a wave's tiles are every feature tile of one
    // value row (d = 128), wave w4 takes them in the order w4, w4 + 1, .. (mod
    // NT), so its own tile is always the first and the sum needs no branch.
    constexpr int NZ = TPW < NT ? TPW : NT;
    constexpr int NZA = HP == 2 ? NZ : 1;                // z accumulators per lane
    static_assert(HP == 2 || (NT <= WPH && (TPW == 1 || TPW >= NT)),
                  "one head per workgroup: wave ft < NT holds feature tile ft among its operands");
    const bool zwriter = HP == 2 ? (w4 * TPW) / NT == 0 : w4 < NT;   // wave-uniform
    float zacc[kNorm ? NZA : 1];
    using O0 = TileOperands<NT, TPW>;
    constexpr bool kRot = kNorm && HP == 1 && O0::NFT == NT && O0::NCT == 1;
    const int rot = kRot ? w4 : 0;                       // wave-uniform
#pragma unroll
    for (int u = 0; u < (kNorm ? NZA : 1); ++u) zacc[u] = 0.f;
    auto zsum8 = [&](const PhiOp<M>& kp) {               // phi of the operand's 8 tokens, summed
        float s8 = 0.f;
        if constexpr (M == 0) {
            const u32x4 b = __builtin_bit_cast(u32x4, kp.hi);
#pragma unroll
            for (int e = 0; e < 4; ++e) s8 += __uint_as_float(b[e] << 16) + __uint_as_float(b[e] & 0xffff0000u);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) s8 += kp.f[2 * e] + kp.f[2 * e + 1];
        }
        return s8;
    };
    using O = TileOperands<NT, TPW>;
    static_assert(O::NFT == NZ, "the z sums cover the distinct feature tiles");
    const int ct0 = O::ct0(w4), ft0 = O::ft0(w4);
    auto mma_stage = [&](int buf) {
        const uint16_t* kt = lds[buf][0];
        const uint16_t* vt = lds[buf][1];
#pragma unroll
        for (int s = 0; s < T / 16; ++s) {
            const int g = 2 * s + hh;
            u16x8 av[O::NCT];
#pragma unroll
            for (int c = 0; c < O::NCT; ++c)
                av[c] = *reinterpret_cast<const u16x8*>(vt + P::slot(hw * D + (ct0 + c) * 32 + l32, g));
#pragma unroll
            for (int f = 0; f < O::NFT; ++f) {
                const int ft = kRot ? (f + rot) % NT : ft0 + f;
                const PhiOp<M> kp = phi_op<M>(*reinterpret_cast<const u16x8*>(kt + P::slot(hw * D + ft * 32 + l32, g)));
#pragma unroll
                for (int c = 0; c < O::NCT; ++c) {                // tile u = c NFT + f
                    f32x16& d = acc[c * O::NFT + f];
                    d = mfma32(as_bf16x8(av[c]), kp.hi, d);
                    if constexpr (!PhiOp<M>::kExact) d = mfma32(as_bf16x8(av[c]), kp.lo, d);   // ELU + 1
                }
                if constexpr (kNorm && HP == 2) zacc[f] += zsum8(kp);
                if constexpr (kNorm && HP == 1) {
                    if constexpr (kRot) {
                        if (f == 0) zacc[0] += zsum8(kp);            // the wave's own tile, rot = w4
                    } else if (ft0 + f == w4) {
                        zacc[0] += zsum8(kp);                         // wave-uniform: wave ft owns tile ft
                    }
                }
                // ELU + 1, and the normalised one-head shapes: keep the
                // scheduler from preparing several K^T operands at once (their
                // temporaries exhausted the registers of the one-head d = 128
                // kernels, which also hold three stages of loads)
                if constexpr (M != 0 || (kNorm && HP == 1)) __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // End of a piece in a computing wave: the wave's tiles of the (unit,
    // prompt) go to the state directly when the prompt lies inside this
    // slice, else to the piece's partial slot for the reduce (see above).
    // z: lanes hh = 0 of the writer waves hold feature 32 ft + l32 of their
    // tiles.
    auto finish_piece = [&]() {
        const int64_t piece = (int64_t)cp.h * a.n_req + cp.r;       // (unit, prompt)
        const bool inside = cp.pr >= cp.sl.lo && cp.pe <= cp.sl.hi;    // the whole prompt is in this slice
        const int slot = uniform_load(a.slots, cp.r);
        if (inside && (slot < 0 || slot >= a.n_slots)) {
#pragma unroll
            for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
            if constexpr (kNorm) {
#pragma unroll
                for (int u = 0; u < NZA; ++u) zacc[u] = 0.f;
            }
            return;
        }
        const int64_t dst = inside ? (int64_t)slot * a.heads + (int64_t)cp.h * HP + hw
                                   : ((int64_t)cp.sl.w + piece) * HP + hw;
        tiles_io<D, WPH>((inside ? a.state : a.partial) + dst * D * D, acc, true, w4, rot);
#pragma unroll
        for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
        if constexpr (kNorm) {
            float* zd = (inside ? a.z : a.zpartial) + dst * D;
#pragma unroll
            for (int u = 0; u < NZA; ++u) {
                const float zs = half_pair_sum(zacc[u]);
                const int ft = HP == 2 ? (w4 * TPW + u) % NT : w4;
                if (zwriter && hh == 0) zd[ft * 32 + l32] = zs;
                zacc[u] = 0.f;
            }
        }
    };

    // One stage: the loading waves store the stage and issue the loads three
    // stages ahead; the computing waves multiply and finish the piece when it
    // ends.  Staging and loads run on every path (past the end they repeat
    // the last rows), so every path around a loading wave's loop issues the
    // three register sets' loads in the same order and each stage waits only
    // for its own set; only the arithmetic is skipped past the end.  With
    // split roles, loader and compute waves run separate loops with the same
    // barriers (the cursors are workgroup-uniform), so the compute loop has
    // no loads for the wait counters to track.
    int sg = 0;
    auto run_all = [&](auto load_tag, auto mma_tag) {
        constexpr bool kLoad = decltype(load_tag)::value, kMma = decltype(mma_tag)::value;
        u32x4 x0[8], x1[8], x2[8];
        int64_t v0 = 0, v1 = 0, v2 = 0;                // rows of the stage each register set holds
        if constexpr (kLoad) {
            load_stage(x0, v0);
            load_stage(x1, v1);
            load_stage(x2, v2);
        }
        // One stage; returns whether it was live.  The loading waves of a
        // split workgroup keep no compute cursor: the stage they store is
        // the one their register set was loaded with three stages earlier.
        auto run_stage = [&](u32x4 (&x)[8], int64_t& valid) {
            const int buf = sg & 1;
            if constexpr (kLoad) store_stage(buf, kMma ? cp.t1 - cp.t : valid, x);
            __syncthreads();
            if constexpr (kLoad) load_stage(x, valid);
            if constexpr (kMma) {
                if (!cp.live) return;          // uniform
                mma_stage(buf);
                if (cp.t + T >= cp.t1) finish_piece();
                stage_advance(a, cp, T);
            }
            ++sg;
        };
        if constexpr (kMma && kLoad) {
            while (cp.live) {
                run_stage(x0, v0);
                run_stage(x1, v1);
                run_stage(x2, v2);
            }
        } else if constexpr (kLoad) {
            while (v0 > 0) {                   // the stage about to be stored is live
                run_stage(x0, v0);
                run_stage(x1, v1);
                run_stage(x2, v2);
            }
        } else {
            // computing waves of a split workgroup: no register sets to
            // rotate, so one stage per turn, then the loaders' barrier count
            // (the stages rounded up to a multiple of three)
            int n = 0;
            for (; cp.live; ++n) run_stage(x0, v0);
            for (; n % 3 != 0; ++n) __syncthreads();
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
    __shared__ int64_t part[259];
    SliceCursor cur;
    if (!slice_begin(a, cur, part)) return;
    const int D = a.d;
    const int64_t rs = (int64_t)a.heads * D, dd = (int64_t)D * D;
    while (cur.c0 < cur.c1) {
        int h;
        int64_t t0, t1, p0, pr, pe;
        slice_piece(a, cur, h, t0, t1, p0, pr, pe);
        const T* kb = static_cast<const T*>(a.k) + p0 + t0 * rs;
        const T* vb = static_cast<const T*>(a.v) + p0 + t0 * rs;
        const bool inside = pr >= cur.lo && pe <= cur.hi;           // the whole prompt is in this slice
        const int slot = a.slots[cur.r];
        if (inside && (slot < 0 || slot >= a.n_slots)) continue;
        const int64_t dst = inside ? (int64_t)slot * a.heads + h : (int64_t)cur.w + (int64_t)h * a.n_req + cur.r;
        float* sd = (inside ? a.state : a.partial) + dst * dd;
        for (int e = threadIdx.x; e < D * D; e += blockDim.x) {
            const int c = e / D, f = e % D;
            float acc = 0.f;
            for (int64_t t = 0; t < t1 - t0; ++t)
                acc = fmaf(Elem<T>::load(vb, t * rs + c), phi_rt(a.phi, Elem<T>::load(kb, t * rs + f)), acc);
            sd[e] = acc;
        }
        if (a.z) {                                       // normalised variant: sum phi(k) of the piece
            float* zd = (inside ? a.z : a.zpartial) + dst * D;
            for (int f = threadIdx.x; f < D; f += blockDim.x) {
                float acc = 0.f;
                for (int64_t t = 0; t < t1 - t0; ++t) acc += phi_rt(a.phi, Elem<T>::load(kb, t * rs + f));
                zd[f] = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill, the reduce: S[slot] = sum of the head's partials in ascending
// slice order (deterministic), 0 for an empty prompt; a prompt that lay in
// one slice was written by it.  Each thread owns four consecutive floats of
// one (request, head) state.
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
    const int64_t wfirst = w0 + (cend > cfirst ? div_floor(cfirst, S) : 0);
    const int64_t nw = cend > cfirst ? div_floor(cend - 1, S) - div_floor(cfirst, S) + 1 : 0;
    if (nw == 1) return;                                 // written by its slice
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
            acc = fmaf(Elem<T>::load(vb, j * rs + c), phi_rt(a.phi, Elem<T>::load(kb, j * rs + f)), acc);
        st[e] += acc;
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_commit(const PhiKVArgs& a, hipStream_t stream)
{
    const dim3 grid(a.n_req * a.heads);
    if (a.dtype_bf16 && a.d >= 32) {
        const bool elu = a.phi == 1;
        const bool t32 = a.blk <= 32;          // one 32-token stage holds the block
        switch (a.d) {
        case 32:
            if (elu) commit_bf16_mfma<32, 1><<<grid, PhiKVShape<32>::NW * kWave, 0, stream>>>(a);
            else commit_bf16_mfma<32, 0><<<grid, PhiKVShape<32>::NW * kWave, 0, stream>>>(a);
            break;
        case 64:
            if (elu && t32) commit_bf16_mfma<64, 1, true><<<grid, PhiKVShape<64>::NW * kWave, 0, stream>>>(a);
            else if (elu) commit_bf16_mfma<64, 1><<<grid, PhiKVShape<64>::NW * kWave, 0, stream>>>(a);
            else if (t32) commit_bf16_mfma<64, 0, true><<<grid, PhiKVShape<64>::NW * kWave, 0, stream>>>(a);
            else commit_bf16_mfma<64, 0><<<grid, PhiKVShape<64>::NW * kWave, 0, stream>>>(a);
            break;
        default:
            if (elu && t32) commit_bf16_mfma<128, 1, true><<<grid, PhiKVShape<128>::NW * kWave, 0, stream>>>(a);
            else if (elu) commit_bf16_mfma<128, 1><<<grid, PhiKVShape<128>::NW * kWave, 0, stream>>>(a);
            else if (t32) commit_bf16_mfma<128, 0, true><<<grid, PhiKVShape<128>::NW * kWave, 0, stream>>>(a);
            else commit_bf16_mfma<128, 0><<<grid, PhiKVShape<128>::NW * kWave, 0, stream>>>(a);
            break;
        }
    } else if (a.dtype_bf16) {
        commit_generic<uint16_t><<<grid, 256, 0, stream>>>(a);
    } else {
        commit_generic<float><<<grid, 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

template <bool kNorm, int M>
static void launch_prefill_slices(const PhiKVArgs& a, dim3 grid, hipStream_t stream)
{
    switch (a.d) {
    case 32: prefill_slices_bf16_mfma<32, 1, kNorm, M><<<grid, prefill_threads<32, 1>(), 0, stream>>>(a); break;
    case 64: prefill_slices_bf16_mfma<64, 1, kNorm, M><<<grid, prefill_threads<64, 1>(), 0, stream>>>(a); break;
    default:
        if (a.hp == 2) {
            prefill_slices_bf16_mfma<128, 2, kNorm, M><<<grid, prefill_threads<128, 2>(), 0, stream>>>(a);
            break;
        }
        prefill_slices_bf16_mfma<128, 1, kNorm, M><<<grid, prefill_threads<128, 1>(), 0, stream>>>(a);
        break;
    }
}

hipError_t launch_prefill(const PhiKVArgs& a, hipStream_t stream)
{
    const dim3 grid(a.slices);
    if (a.dtype_bf16 && a.d >= 32) {
        if (a.phi == 1) {
            if (a.z) launch_prefill_slices<true, 1>(a, grid, stream);
            else launch_prefill_slices<false, 1>(a, grid, stream);
        } else {
            if (a.z) launch_prefill_slices<true, 0>(a, grid, stream);
            else launch_prefill_slices<false, 0>(a, grid, stream);
        }
    } else if (a.dtype_bf16) {
        prefill_slices_generic<uint16_t><<<grid, 256, 0, stream>>>(a);
    } else {
        prefill_slices_generic<float><<<grid, 256, 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = (int64_t)a.d * a.d / 4;
    prefill_reduce<<<dim3((unsigned)((n4 + 255) / 256), a.heads, a.n_req), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace ha
