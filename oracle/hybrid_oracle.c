/*
 * Plain CPU oracle for block-hybrid attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke entry and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and the two share
 * no code.
 *
 * Everything is fp64 with straight loops and no blocking, fusion or
 * reordering: each function is the definition written out so a reader can
 * check it against the pages by eye.  Independent (request, head) units are
 * spread over OpenMP threads; that changes nothing inside a unit.
 *
 * Sources (the pages):
 *   [F]  "Retrofitting Linear Attention into Diffusion Language Models",
 *        paper-daily summary page, section "core formula": the hybrid output
 *        is Softmax(Q_a K_a^T) V_a + phi(Q) phi(K_p)^T V_p, with a = active
 *        block and p = previous blocks.
 *   [W]  same page, section "technical details in action" (worked example):
 *        L = 10, B = 4, blocks of 4/4/2 tokens; phi(x) = ReLU(x); the prefix
 *        summary S_1 = phi(K_1)^T V_1; the active block's linear term is
 *        phi(Q_2) S_1; the block output is the SUM of the softmax result and
 *        the linear result; after block 2, S_{1,2} = phi(K_1)^T V_1 +
 *        phi(K_2)^T V_2.
 *   [A]  same paper, abstract (fugumt.com page): exact softmax attention
 *        inside the active denoising block, linear attention over previous
 *        blocks; blocks generated autoregressively, tokens in a block
 *        denoised in parallel.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the linear term uses phi of the ACTIVE block's queries (the worked
 *     example's phi(Q_2) S_1), not of prefix queries;
 *   - an explicit softmax scale multiplies the logits only;
 *   - no mask inside the active block; rows >= the valid length B_r are
 *     neither read as keys nor written as outputs;
 *   - the two terms are added with no normaliser or mixing weight.
 *
 * A second, normalised variant ([N] below): the pages say the retrofit
 * largely follows LoLCATs (summary page, sections "problem solving" and
 * "method"; abstract page) but print no formula for it.  The reading taken
 * is that method's hybrid of exact and linear attention with ONE shared
 * denominator: the block's softmax scores exp(l_ij) and the prefix tokens'
 * linear scores phi(q_i).phi(k_p) are normalised together, which needs a
 * second state z = sum over prefix tokens of phi(k_p) next to S.
 *
 * Layouts (logical, row-major, all fp64):
 *   q, k, v, out  [n_req][blk][H][d]      token-major active block
 *   S             [n_slots][H][d][d]      S[slot][h][f][c]: f = feature of
 *                                         phi(k), c = value dimension
 *   packed        [total][H][d] + cu[n_req+1] for prompts / prefixes
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * The feature map phi, chosen by `map` in every function that applies it:
 *   0  ReLU: phi(x) = max(x, 0), the worked example's map [W];
 *   1  ELU + 1: phi(x) = x + 1 for x > 0 and e^x otherwise, another fixed
 *      map.  [F] calls phi only "a kernel-function map"; ELU + 1 is the
 *      common fixed choice of linear attention, positive everywhere (so the
 *      normalised variant's denominator never vanishes) and continuous with
 *      a continuous slope at 0.
 */
static double feature(int map, double x)
{
    if (map == 1) return x > 0.0 ? x + 1.0 : exp(x);
    return x > 0.0 ? x : 0.0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n >= 1); changes nothing inside a unit. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Index helpers for the token-major [n][T][H][d] layout. */
static size_t tok(int64_t r, int64_t t, int64_t h, int64_t T, int64_t H, int64_t d)
{
    return (size_t)(((r * T + t) * H + h) * d);
}

/*
 * Softmax attention of the active block against itself [F], [A]:
 * O_s[i] = sum_j p_ij v_j, p_ij = exp(l_ij - m_i) / sum_j' exp(l_ij' - m_i),
 * l_ij = scale * <q_i, k_j>, over the Br valid rows.  Subtracting the row
 * maximum m_i changes nothing mathematically; it only keeps exp finite.
 * qi: one query row; kb, vb: first key/value row of the block, rows `stride`
 * apart; adds the result into acc[d].
 */
static void softmax_block_row(const double* qi, const double* kb, const double* vb,
                              size_t stride, int Br, int d, double scale,
                              double* logit /* scratch [Br] */, double* acc)
{
    double m = -INFINITY;
    for (int j = 0; j < Br; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qi[c] * kb[j * stride + c];
        logit[j] = scale * dot;
        if (logit[j] > m) m = logit[j];
    }
    double l = 0.0;
    for (int j = 0; j < Br; ++j) {
        logit[j] = exp(logit[j] - m);
        l += logit[j];
    }
    for (int j = 0; j < Br; ++j) {
        double p = logit[j] / l;
        for (int c = 0; c < d; ++c) acc[c] += p * vb[j * stride + c];
    }
}

/*
 * Hybrid step, state form [F] with [W]:
 *   O = Softmax(scale Q_a K_a^T) V_a + phi(Q_a) S
 * for every request r (state slot slots[r]) and head h.  Only the first
 * Br = blk_lens[r] rows (all blk if blk_lens is NULL) are read and written.
 */
void oracle_step(const double* q, const double* k, const double* v, const double* S,
                 const int32_t* slots, const int32_t* blk_lens, double* out,
                 int n_req, int n_slots, int H, int blk, int d, double scale, int map)
{
    (void)n_slots;
    const size_t stride = (size_t)H * d;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            const double* Su = S + ((size_t)slots[r] * H + h) * d * d;
            double* logit = (double*)malloc(sizeof(double) * (Br > 0 ? Br : 1));
            double* acc = (double*)malloc(sizeof(double) * d);
            for (int i = 0; i < Br; ++i) {
                const double* qi = q + tok(r, i, h, blk, H, d);
                for (int c = 0; c < d; ++c) acc[c] = 0.0;
                /* softmax part: exact attention inside the active block */
                softmax_block_row(qi, k + tok(r, 0, h, blk, H, d), v + tok(r, 0, h, blk, H, d),
                                  stride, Br, d, scale, logit, acc);
                /* linear part: phi(q_i) S, S summarising the previous blocks */
                for (int c = 0; c < d; ++c) {
                    double lin = 0.0;
                    for (int f = 0; f < d; ++f) lin += feature(map, qi[f]) * Su[(size_t)f * d + c];
                    acc[c] += lin;
                }
                double* oi = out + tok(r, i, h, blk, H, d);
                for (int c = 0; c < d; ++c) oi[c] = acc[c];
            }
            free(logit);
            free(acc);
        }
    }
}

/*
 * Block commit [W]: S_{1..b} = S_{1..b-1} + phi(K_b)^T V_b, i.e.
 * S[f][c] += sum_{j < Br} phi(K[j][f]) V[j][c], in place.
 */
void oracle_commit(const double* k, const double* v, double* S, const int32_t* slots,
                   const int32_t* blk_lens, int n_req, int n_slots, int H, int blk, int d, int map)
{
    (void)n_slots;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            double* Su = S + ((size_t)slots[r] * H + h) * d * d;
            for (int f = 0; f < d; ++f) {
                for (int c = 0; c < d; ++c) {
                    double sum = 0.0;
                    for (int j = 0; j < Br; ++j)
                        sum += feature(map, k[tok(r, j, h, blk, H, d) + f]) * v[tok(r, j, h, blk, H, d) + c];
                    Su[(size_t)f * d + c] += sum;
                }
            }
        }
    }
}

/*
 * Prefill: a prompt folds into the state exactly as committed blocks do
 * ([W]'s S as a sum over previous tokens), overwriting the slot:
 * S[f][c] = sum_{t < L_r} phi(K[t][f]) V[t][c].  No chunking here: the
 * chunk size of the GPU path must not change this value.  k, v packed
 * [total][H][d] with request r's tokens at rows cu[r] .. cu[r+1]-1.
 */
void oracle_prefill(const double* k, const double* v, const int64_t* cu, double* S,
                    const int32_t* slots, int n_req, int n_slots, int H, int d, int map)
{
    (void)n_slots;
    const size_t stride = (size_t)H * d;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            double* Su = S + ((size_t)slots[r] * H + h) * d * d;
            for (size_t e = 0; e < (size_t)d * d; ++e) Su[e] = 0.0;
            /* one outer product phi(k_t)^T v_t per prompt token, summed */
            for (int64_t t = cu[r]; t < cu[r + 1]; ++t) {
                const double* kt = k + t * stride + (size_t)h * d;
                const double* vt = v + t * stride + (size_t)h * d;
                for (int f = 0; f < d; ++f) {
                    const double pk = feature(map, kt[f]);
                    for (int c = 0; c < d; ++c) Su[(size_t)f * d + c] += pk * vt[c];
                }
            }
        }
    }
}

/*
 * The formula's own form [F], recomputing the linear term from the retained
 * prefix keys and values instead of the state (the worked example keeps the
 * previous blocks' keys and values in the KV cache, [W]):
 *   O = Softmax(scale Q_a K_a^T) V_a + (phi(Q_a) phi(K_p)^T) V_p
 * The (B_r x P) matrix phi(Q_a) phi(K_p)^T is formed first, then multiplied
 * by V_p.  By associativity this equals oracle_step with S = phi(K_p)^T V_p.
 * kp, vp packed [total][H][d] with cu[r] .. cu[r+1]-1 the prefix of request r.
 */
void oracle_step_recompute(const double* q, const double* k, const double* v,
                           const double* kp, const double* vp, const int64_t* cu,
                           const int32_t* blk_lens, double* out,
                           int n_req, int H, int blk, int d, double scale, int map)
{
    const size_t stride = (size_t)H * d;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            const int64_t P = cu[r + 1] - cu[r];
            double* logit = (double*)malloc(sizeof(double) * (Br > 0 ? Br : 1));
            double* acc = (double*)malloc(sizeof(double) * d);
            double* a = (double*)malloc(sizeof(double) * (P > 0 ? P : 1));
            for (int i = 0; i < Br; ++i) {
                const double* qi = q + tok(r, i, h, blk, H, d);
                for (int c = 0; c < d; ++c) acc[c] = 0.0;
                softmax_block_row(qi, k + tok(r, 0, h, blk, H, d), v + tok(r, 0, h, blk, H, d),
                                  stride, Br, d, scale, logit, acc);
                /* row i of phi(Q_a) phi(K_p)^T */
                for (int64_t t = 0; t < P; ++t) {
                    const double* kt = kp + (cu[r] + t) * stride + h * d;
                    double dot = 0.0;
                    for (int f = 0; f < d; ++f) dot += feature(map, qi[f]) * feature(map, kt[f]);
                    a[t] = dot;
                }
                /* times V_p */
                for (int64_t t = 0; t < P; ++t) {
                    const double* vt = vp + (cu[r] + t) * stride + h * d;
                    for (int c = 0; c < d; ++c) acc[c] += a[t] * vt[c];
                }
                double* oi = out + tok(r, i, h, blk, H, d);
                for (int c = 0; c < d; ++c) oi[c] = acc[c];
            }
            free(a);
            free(logit);
            free(acc);
        }
    }
}

/*
 * Exact full-prefix step: the baseline this method replaces (abstract [A]:
 * without linearisation every denoising step attends to all previous blocks
 * through the KV cache).  One softmax over the P prefix keys followed by the
 * Br active keys:
 *   O = Softmax(scale Q_a [K_p; K_a]^T) [V_p; V_a]
 */
void oracle_exact_step(const double* q, const double* k, const double* v,
                       const double* kp, const double* vp, const int64_t* cu,
                       const int32_t* blk_lens, double* out,
                       int n_req, int H, int blk, int d, double scale)
{
    const size_t stride = (size_t)H * d;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            const int64_t P = cu[r + 1] - cu[r];
            const int64_t n = P + Br;
            double* logit = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
            for (int i = 0; i < Br; ++i) {
                const double* qi = q + tok(r, i, h, blk, H, d);
                double m = -INFINITY;
                for (int64_t j = 0; j < n; ++j) {
                    const double* kj = j < P ? kp + (cu[r] + j) * stride + h * d
                                             : k + tok(r, (int)(j - P), h, blk, H, d);
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
                    logit[j] = scale * dot;
                    if (logit[j] > m) m = logit[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    logit[j] = exp(logit[j] - m);
                    l += logit[j];
                }
                double* oi = out + tok(r, i, h, blk, H, d);
                for (int c = 0; c < d; ++c) oi[c] = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    const double* vj = j < P ? vp + (cu[r] + j) * stride + h * d
                                             : v + tok(r, (int)(j - P), h, blk, H, d);
                    const double p = logit[j] / l;
                    for (int c = 0; c < d; ++c) oi[c] += p * vj[c];
                }
            }
            free(logit);
        }
    }
}

/*
 * [N] Normalised step, state form:
 *   O_i = (sum_j exp(l_ij) v_j + phi(q_i) S) / (sum_j exp(l_ij) + phi(q_i) . z)
 * over the Br valid block keys j, l_ij = scale * <q_i, k_j>; S as in
 * oracle_step, z[f] = sum over prefix tokens of phi(k_p[f]).  The block
 * maximum m_i is factored out of numerator and denominator (exp(l_ij - m_i)
 * and exp(-m_i) in place of exp(l_ij) and 1), which changes nothing
 * mathematically.  z is [n_slots][H][d].
 */
void oracle_step_norm(const double* q, const double* k, const double* v, const double* S, const double* z,
                      const int32_t* slots, const int32_t* blk_lens, double* out,
                      int n_req, int n_slots, int H, int blk, int d, double scale, int map)
{
    (void)n_slots;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            const double* Su = S + ((size_t)slots[r] * H + h) * d * d;
            const double* zu = z + ((size_t)slots[r] * H + h) * d;
            double* w = (double*)malloc(sizeof(double) * (Br > 0 ? Br : 1));
            for (int i = 0; i < Br; ++i) {
                const double* qi = q + tok(r, i, h, blk, H, d);
                double* oi = out + tok(r, i, h, blk, H, d);
                /* block scores */
                double m = -INFINITY;
                for (int j = 0; j < Br; ++j) {
                    const double* kj = k + tok(r, j, h, blk, H, d);
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
                    w[j] = scale * dot;
                    if (w[j] > m) m = w[j];
                }
                double den = 0.0;
                for (int c = 0; c < d; ++c) oi[c] = 0.0;
                for (int j = 0; j < Br; ++j) {
                    const double e = exp(w[j] - m);
                    const double* vj = v + tok(r, j, h, blk, H, d);
                    for (int c = 0; c < d; ++c) oi[c] += e * vj[c];
                    den += e;
                }
                /* prefix: phi(q_i) S over the numerator, phi(q_i) . z over the denominator */
                const double em = exp(-m);
                double qz = 0.0;
                for (int f = 0; f < d; ++f) qz += feature(map, qi[f]) * zu[f];
                den += em * qz;
                for (int c = 0; c < d; ++c) {
                    double lin = 0.0;
                    for (int f = 0; f < d; ++f) lin += feature(map, qi[f]) * Su[(size_t)f * d + c];
                    oi[c] = (oi[c] + em * lin) / den;
                }
            }
            free(w);
        }
    }
}

/* [N] Commit of the normaliser state: z[f] += sum_{j < Br} phi(K[j][f]). */
void oracle_znorm_commit(const double* k, double* z, const int32_t* slots, const int32_t* blk_lens,
                         int n_req, int n_slots, int H, int blk, int d, int map)
{
    (void)n_slots;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            double* zu = z + ((size_t)slots[r] * H + h) * d;
            for (int f = 0; f < d; ++f) {
                double sum = 0.0;
                for (int j = 0; j < Br; ++j) sum += feature(map, k[tok(r, j, h, blk, H, d) + f]);
                zu[f] += sum;
            }
        }
    }
}

/* [N] Prefill of the normaliser state: z[f] = sum_{t < L_r} phi(K[t][f]). */
void oracle_znorm_prefill(const double* k, const int64_t* cu, double* z, const int32_t* slots,
                          int n_req, int n_slots, int H, int d, int map)
{
    (void)n_slots;
    const size_t stride = (size_t)H * d;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            double* zu = z + ((size_t)slots[r] * H + h) * d;
            for (int f = 0; f < d; ++f) zu[f] = 0.0;
            for (int64_t t = cu[r]; t < cu[r + 1]; ++t) {
                const double* kt = k + t * stride + (size_t)h * d;
                for (int f = 0; f < d; ++f) zu[f] += feature(map, kt[f]);
            }
        }
    }
}

/*
 * [N] The normalised output from the retained prefix tokens: one weight per
 * key, exp(l_ij) for the block keys and phi(q_i) . phi(k_t) for each prefix
 * token, and O_i = sum of weight x value / sum of weights (the block maximum
 * factored out as in oracle_step_norm).  By associativity this equals
 * oracle_step_norm with S = sum phi(k_t)^T v_t and z = sum phi(k_t).
 */
void oracle_step_norm_recompute(const double* q, const double* k, const double* v,
                                const double* kp, const double* vp, const int64_t* cu,
                                const int32_t* blk_lens, double* out,
                                int n_req, int H, int blk, int d, double scale, int map)
{
    const size_t stride = (size_t)H * d;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < n_req; ++r) {
        for (int h = 0; h < H; ++h) {
            const int Br = blk_lens ? blk_lens[r] : blk;
            const int64_t P = cu[r + 1] - cu[r];
            double* w = (double*)malloc(sizeof(double) * (Br + P > 0 ? Br + P : 1));
            for (int i = 0; i < Br; ++i) {
                const double* qi = q + tok(r, i, h, blk, H, d);
                double m = -INFINITY;
                for (int j = 0; j < Br; ++j) {
                    const double* kj = k + tok(r, j, h, blk, H, d);
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
                    w[j] = scale * dot;
                    if (w[j] > m) m = w[j];
                }
                for (int j = 0; j < Br; ++j) w[j] = exp(w[j] - m);
                for (int64_t t = 0; t < P; ++t) {
                    const double* kt = kp + (cu[r] + t) * stride + h * d;
                    double dot = 0.0;
                    for (int f = 0; f < d; ++f) dot += feature(map, qi[f]) * feature(map, kt[f]);
                    w[Br + t] = exp(-m) * dot;
                }
                double den = 0.0;
                for (int64_t j = 0; j < Br + P; ++j) den += w[j];
                double* oi = out + tok(r, i, h, blk, H, d);
                for (int c = 0; c < d; ++c) {
                    double num = 0.0;
                    for (int j = 0; j < Br; ++j) num += w[j] * v[tok(r, j, h, blk, H, d) + c];
                    for (int64_t t = 0; t < P; ++t) num += w[Br + t] * vp[(cu[r] + t) * stride + h * d + c];
                    oi[c] = num / den;
                }
            }
            free(w);
        }
    }
}
