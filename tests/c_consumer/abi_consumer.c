/*
 * A plain C consumer of libhybrid_attn.so: device memory from hipMalloc, the
 * calls through include/hybrid_attn.h only (no Python, no torch), results
 * checked against the fp64 C oracle (oracle/hybrid_oracle.c, linked as
 * liboracle.so; test code only).
 *
 * Sequence (the worked example's order on one layer: a prompt folded into S,
 * a denoising step of the active block against S, the block's commit):
 *   hybrid_state_prefill  prompts of 700, 0 and 333 tokens into slots 2, 0, 3
 *   hybrid_attn_step      blocks of 48 rows, valid lengths 48, 30 and 1
 *   hybrid_state_commit   the same blocks' K and V
 *   an unsupported head dim, which must fail before anything is enqueued.
 * Slot 1 is named by no request and must keep its bytes.  Each check uses
 * the bf16 rule (max abs error <= 2e-2 x max |reference|); the oracle gets
 * the same state the GPU started from, so each call is checked on its own.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "../../include/hybrid_attn.h"

/* the last argument selects the feature map; 0 is ReLU */
void oracle_step(const double* q, const double* k, const double* v, const double* S, const int32_t* slots,
                 const int32_t* blk_lens, double* out, int n_req, int n_slots, int H, int blk, int d,
                 double scale, int map);
void oracle_commit(const double* k, const double* v, double* S, const int32_t* slots, const int32_t* blk_lens,
                   int n_req, int n_slots, int H, int blk, int d, int map);
void oracle_prefill(const double* k, const double* v, const int64_t* cu, double* S, const int32_t* slots,
                    int n_req, int n_slots, int H, int d, int map);

enum { N_REQ = 3, N_SLOTS = 4, H = 2, D = 128, BLK = 48, CHUNK = 256 };
static const int32_t kSlots[N_REQ] = {2, 0, 3};
static const int32_t kLens[N_REQ] = {48, 30, 1};
static const int64_t kPrompt[N_REQ] = {700, 0, 333};
static const uint16_t kSentinel = 0xC480;        /* -1024 in bf16 */
static const double kRel = 2e-2;

static int failures = 0;

#define HIP_CHECK(x)                                                                    \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                    \
        }                                                                               \
    } while (0)

#define HA_CHECK(x)                                                                     \
    do {                                                                                \
        ha_status s_ = (x);                                                             \
        if (s_ != HA_OK) {                                                              \
            fprintf(stderr, "%s failed (%d): %s\n", #x, (int)s_, hybrid_last_error()); \
            exit(2);                                                                    \
        }                                                                               \
    } while (0)

/* Seeded inputs: splitmix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014) feeding the Box-Muller transform. */
static uint64_t rng_state;
static uint64_t splitmix64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform01(void) { return ((double)(splitmix64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
static double normal01(void)
{
    const double u1 = uniform01(), u2 = uniform01();
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static uint16_t to_bf16(float f)                  /* round to nearest even (finite inputs) */
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}
static double from_bf16(uint16_t h)
{
    const uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* n seeded bf16 values, with their exact fp64 values for the oracle */
static void seeded_bf16(uint64_t seed, size_t n, uint16_t* bits, double* exact)
{
    rng_state = seed;
    for (size_t i = 0; i < n; ++i) {
        bits[i] = to_bf16((float)normal01());
        exact[i] = from_bf16(bits[i]);
    }
}

/* library layout state[s][h][c][f] <-> oracle layout S[s][h][f][c] */
static void state_to_oracle(const float* st, double* S)
{
    for (size_t u = 0; u < (size_t)N_SLOTS * H; ++u)
        for (int c = 0; c < D; ++c)
            for (int f = 0; f < D; ++f) S[(u * D + f) * D + c] = st[(u * D + c) * D + f];
}

static void check(const char* what, const double* got, const double* ref, size_t n)
{
    double err = 0.0, mag = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double e = fabs(got[i] - ref[i]);
        if (!(e <= err)) err = e;                  /* NaN propagates into err */
        if (fabs(ref[i]) > mag) mag = fabs(ref[i]);
    }
    const int ok = err <= kRel * mag;
    printf("[c-abi] %-34s max abs err %.3e, max |ref| %.3e: %s\n", what, err, mag, ok ? "ok" : "FAIL");
    if (!ok) ++failures;
}

int main(void)
{
    const size_t blk_elems = (size_t)N_REQ * BLK * H * D;
    const size_t st_elems = (size_t)N_SLOTS * H * D * D;
    int64_t cu[N_REQ + 1] = {0};
    for (int r = 0; r < N_REQ; ++r) cu[r + 1] = cu[r] + kPrompt[r];
    const int64_t total = cu[N_REQ];
    const size_t p_elems = (size_t)total * H * D;

    uint16_t *hq = malloc(blk_elems * 2), *hk = malloc(blk_elems * 2), *hv = malloc(blk_elems * 2);
    uint16_t *hout = malloc(blk_elems * 2), *hpk = malloc(p_elems * 2), *hpv = malloc(p_elems * 2);
    double *q = malloc(blk_elems * 8), *k = malloc(blk_elems * 8), *v = malloc(blk_elems * 8);
    double *pk = malloc(p_elems * 8), *pv = malloc(p_elems * 8), *o64 = malloc(blk_elems * 8);
    double *ref = calloc(blk_elems, 8), *S = malloc(st_elems * 8), *Sref = malloc(st_elems * 8);
    float *st0 = malloc(st_elems * 4), *st = malloc(st_elems * 4);
    seeded_bf16(11, blk_elems, hq, q);
    seeded_bf16(12, blk_elems, hk, k);
    seeded_bf16(13, blk_elems, hv, v);
    seeded_bf16(14, p_elems, hpk, pk);
    seeded_bf16(15, p_elems, hpv, pv);
    rng_state = 16;
    for (size_t i = 0; i < st_elems; ++i) st0[i] = (float)normal01();

    void *dq, *dk, *dv, *dout, *dpk, *dpv, *dws;
    float* dst;
    int32_t *dslots, *dlens;
    int64_t* dcu;
    const size_t ws_bytes = hybrid_state_prefill_workspace_bytes(N_REQ, H, D, total, 700, CHUNK);
    HIP_CHECK(hipMalloc(&dq, blk_elems * 2));
    HIP_CHECK(hipMalloc(&dk, blk_elems * 2));
    HIP_CHECK(hipMalloc(&dv, blk_elems * 2));
    HIP_CHECK(hipMalloc(&dout, blk_elems * 2));
    HIP_CHECK(hipMalloc(&dpk, p_elems * 2));
    HIP_CHECK(hipMalloc(&dpv, p_elems * 2));
    HIP_CHECK(hipMalloc(&dws, ws_bytes));
    HIP_CHECK(hipMalloc((void**)&dst, st_elems * 4));
    HIP_CHECK(hipMalloc((void**)&dslots, sizeof kSlots));
    HIP_CHECK(hipMalloc((void**)&dlens, sizeof kLens));
    HIP_CHECK(hipMalloc((void**)&dcu, sizeof cu));
    HIP_CHECK(hipMemcpy(dq, hq, blk_elems * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dk, hk, blk_elems * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dv, hv, blk_elems * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dpk, hpk, p_elems * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dpv, hpv, p_elems * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dst, st0, st_elems * 4, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dslots, kSlots, sizeof kSlots, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dlens, kLens, sizeof kLens, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dcu, cu, sizeof cu, hipMemcpyHostToDevice));
    printf("[c-abi] ABI version %d, prefill workspace %zu bytes\n", (int)hybrid_abi_version(), ws_bytes);

    /* prefill: named slots overwritten (slot 0 by the empty prompt: zero) */
    HA_CHECK(hybrid_state_prefill(dpk, dpv, dcu, total, 700, dst, dslots, N_REQ, N_SLOTS, H, D, CHUNK, dws,
                                  ws_bytes, HA_BF16, NULL));
    HIP_CHECK(hipDeviceSynchronize());
    HIP_CHECK(hipMemcpy(st, dst, st_elems * 4, hipMemcpyDeviceToHost));
    state_to_oracle(st0, Sref);
    oracle_prefill(pk, pv, cu, Sref, kSlots, N_REQ, N_SLOTS, H, D, 0);
    state_to_oracle(st, S);
    check("prefill: state", S, Sref, st_elems);
    if (memcmp(st + (size_t)1 * H * D * D, st0 + (size_t)1 * H * D * D, (size_t)H * D * D * 4) != 0) {
        printf("[c-abi] prefill wrote slot 1, which no request names: FAIL\n");
        ++failures;
    }

    /* step against the state the prefill left */
    for (size_t i = 0; i < blk_elems; ++i) hout[i] = kSentinel;
    HIP_CHECK(hipMemcpy(dout, hout, blk_elems * 2, hipMemcpyHostToDevice));
    const float scale = 1.0f / sqrtf((float)D);
    HA_CHECK(hybrid_attn_step(dq, dk, dv, dst, dslots, dout, dlens, N_REQ, N_SLOTS, H, BLK, D, scale, HA_BF16,
                              NULL));
    HIP_CHECK(hipDeviceSynchronize());
    HIP_CHECK(hipMemcpy(hout, dout, blk_elems * 2, hipMemcpyDeviceToHost));
    oracle_step(q, k, v, S, kSlots, kLens, ref, N_REQ, N_SLOTS, H, BLK, D, (double)scale, 0);
    int untouched = 1;
    for (int r = 0; r < N_REQ; ++r)
        for (int i = 0; i < BLK; ++i)
            for (size_t e = 0; e < (size_t)H * D; ++e) {
                const size_t idx = ((size_t)r * BLK + i) * H * D + e;
                if (i < kLens[r]) o64[idx] = from_bf16(hout[idx]);
                else {
                    untouched &= hout[idx] == kSentinel;
                    o64[idx] = ref[idx] = 0.0;     /* rows past B_r: not compared */
                }
            }
    check("step: outputs", o64, ref, blk_elems);
    if (!untouched) {
        printf("[c-abi] step wrote rows past B_r: FAIL\n");
        ++failures;
    }

    /* commit of the same block's K and V into that state */
    HA_CHECK(hybrid_state_commit(dk, dv, dst, dslots, dlens, N_REQ, N_SLOTS, H, BLK, D, HA_BF16, NULL));
    HIP_CHECK(hipDeviceSynchronize());
    memcpy(Sref, S, st_elems * 8);
    oracle_commit(k, v, Sref, kSlots, kLens, N_REQ, N_SLOTS, H, BLK, D, 0);
    HIP_CHECK(hipMemcpy(st, dst, st_elems * 4, hipMemcpyDeviceToHost));
    state_to_oracle(st, S);
    check("commit: state", S, Sref, st_elems);

    /* a rejected call: reported before anything is enqueued */
    const ha_status bad = hybrid_attn_step(dq, dk, dv, dst, dslots, dout, dlens, N_REQ, N_SLOTS, H, BLK, 100,
                                           scale, HA_BF16, NULL);
    const int bad_ok = bad == HA_ERR_UNSUPPORTED && hybrid_last_error()[0] != '\0';
    printf("[c-abi] head dim 100 rejected (%d): \"%s\": %s\n", (int)bad, hybrid_last_error(),
           bad_ok ? "ok" : "FAIL");
    if (!bad_ok) ++failures;

    hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dout); hipFree(dpk); hipFree(dpv); hipFree(dws);
    hipFree(dst); hipFree(dslots); hipFree(dlens); hipFree(dcu);
    free(hq); free(hk); free(hv); free(hout); free(hpk); free(hpv); free(q); free(k); free(v);
    free(pk); free(pv); free(o64); free(ref); free(S); free(Sref); free(st0); free(st);
    printf("[c-abi] %s\n", failures ? "FAILED" : "all checks passed");
    return failures ? 1 : 0;
}
