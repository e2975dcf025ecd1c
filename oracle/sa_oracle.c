/*
 * Oracle for masked sparse attention (forward).  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously correct CPU definition that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the bench's CPU-baseline leg may load it.  It shares no code, header or
 * constant with the product library; the two are compiled separately and
 * neither includes or links the other.
 *
 * Arithmetic is fp64 throughout.  Inputs arrive as fp32 arrays (bf16 inputs
 * are widened to fp32 exactly before they get here) and are widened to fp64
 * exactly.  The result is never rounded.
 *
 * Sources (cited by page title and section):
 *   - "Sparse attention" (glossary.selfmadequant.com), section "Choose the
 *     available reads": y_i = sum_{j in S_i} a_ij v_j with a_ij the softmax of
 *     q_i.k_j / sqrt(d_k) renormalised over S_i only.
 *   - "Attention variants" (sreshtalluri.github.io), section 1 "Intuition" and
 *     section 4 "Build it from scratch": causal rule j <= i, window i-j < w
 *     counting the query, strided columns, global rows and columns, and the
 *     union-of-rules composition.
 *   - "Sparse attention" (octlm.ramaa.tech lab note), section "One mask
 *     function for every pattern": window 0 means the full causal triangle;
 *     strided columns at multiples of s (phase 0).
 *   - "Sparse Attention" (ai360xpert.com), "How It Actually Works": a
 *     non-causal local neighbourhood on either side, read as a radius r.
 *   - "Attention variants", section 6 "Knowledge check" (the dilated-mask
 *     exercise): a dilated window of w keys with dilation g reads the keys
 *     at distances 0, g, 2g, ..., (w-1)g behind the query.  ("Sparse and
 *     sliding-window attention", section "Dilated sliding window", describes
 *     a different, symmetric variant; it is not the one used.)
 *
 * Mask rule used here (the plainest reading that covers every page):
 *   allowed(i,j) = C(i,j) and ( L(i,j) or St(j) or Gl(i,j) )
 *   C  : causal -> j <= i ; bidirectional -> always
 *   L  : with dilation g (default 1) and gap = i - j:
 *        causal -> gap mod g == 0 and (window == 0 or gap < window * g)
 *        bidirectional -> |gap| mod g == 0 and (no radius or |gap| <= radius * g)
 *   St : stride > 0 and j mod stride == phase
 *   Gl : i in G or j in G     (G = union of half-open index ranges)
 * In causal mode C is applied to the global term too, so a global token
 * never reads or is read from the future ("Attention variants", section 4:
 * global tokens in a decoder must stay causal).
 *
 * Block mode (BigBird, "Sparse and sliding-window attention", section
 * "Block-sparse attention: BigBird": a local window of 3 blocks, R random
 * blocks and G global blocks, block size 64): with block size S, query block
 * qb = i / S and key block kb = j / S,
 *   allowed(i,j) = |qb - kb| <= radius  or  kb in Rand(qb)  or St(j)  or Gl(i,j)
 * with no causal cut (the pattern is bidirectional).  Rand(qb) holds R
 * distinct key blocks drawn uniformly from all ceil(T/S) blocks, local and
 * global ones included ("from anywhere"): the draws are the SplitMix64
 * stream (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) started from state (seed << 32) | qb, each draw
 * x giving block (x >> 32) mod nkb; repeats are skipped, at most 64*R draws
 * are made, and with nkb <= R every block is taken.
 *
 * Parity pins: see the module docstring of oracle/__init__.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t causal;      /* 1: causal, 0: bidirectional */
    int32_t has_radius;  /* bidirectional only: 1 if a radius was given */
    int64_t window;      /* causal only: 0 means unlimited */
    int64_t radius;      /* bidirectional only */
    int64_t stride;      /* 0 means no strided columns */
    int64_t phase;       /* 0 <= phase < stride */
    int32_t n_global;    /* number of half-open ranges in lo/hi */
    int32_t dilation;    /* >= 1; 1 = contiguous window */
    const int64_t* global_lo;
    const int64_t* global_hi;
    int64_t block;       /* > 0: block mode with this block size */
    int64_t n_random;    /* block mode: random key blocks per query block */
    uint64_t seed;       /* block mode: random stream seed */
} oracle_mask;

/* One SplitMix64 step: advance the state by the golden gamma, then mix. */
uint64_t oracle_splitmix64(uint64_t* state) {
    uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Rand(qb) for T keys: writes up to n_random distinct key blocks (in draw
 * order) to out, returns how many. */
int64_t oracle_random_blocks(const oracle_mask* m, int64_t T, int64_t qb, int64_t* out) {
    const int64_t nkb = (T + m->block - 1) / m->block;
    int64_t n = 0;
    if (nkb <= m->n_random) {
        for (int64_t kb = 0; kb < nkb; ++kb) out[n++] = kb;
        return n;
    }
    uint64_t state = (m->seed << 32) | (uint64_t)qb;
    for (int64_t draw = 0; draw < 64 * m->n_random && n < m->n_random; ++draw) {
        const int64_t kb = (int64_t)((oracle_splitmix64(&state) >> 32) % (uint64_t)nkb);
        int seen = 0;
        for (int64_t t = 0; t < n; ++t) seen |= (out[t] == kb);
        if (!seen) out[n++] = kb;
    }
    return n;
}

static int in_global(const oracle_mask* m, int64_t x) {
    for (int32_t r = 0; r < m->n_global; ++r)
        if (x >= m->global_lo[r] && x < m->global_hi[r]) return 1;
    return 0;
}

/* St(j) and Gl(i,j), shared by the token and block rules. */
static int strided_col(const oracle_mask* m, int64_t j) {
    return (m->stride > 0) && (j % m->stride == m->phase);
}

static int global_pair(const oracle_mask* m, int64_t i, int64_t j) {
    int global = in_global(m, i) || in_global(m, j);
    return global;
}

static int oracle_allowed_blocks(const oracle_mask* m, int64_t T, int64_t i, int64_t j) {
    const int64_t qb = i / m->block, kb = j / m->block;
    const int64_t dist = qb > kb ? qb - kb : kb - qb;
    int local = dist <= m->radius;
    int rnd = 0;
    if (m->n_random > 0) {
        int64_t blocks[4096];
        const int64_t n = oracle_random_blocks(m, T, qb, blocks);
        for (int64_t t = 0; t < n; ++t) rnd |= (blocks[t] == kb);
    }
    return local || rnd || strided_col(m, j) || global_pair(m, i, j);
}

/* The rule of "allowed", one (query, key) pair at a time (T matters only
 * in block mode, where it fixes the number of key blocks). */
int oracle_allowed_T(const oracle_mask* m, int64_t T, int64_t i, int64_t j) {
    if (m->block > 0) return oracle_allowed_blocks(m, T, i, j);
    int causal_ok = m->causal ? (j <= i) : 1;
    if (!causal_ok) return 0;
    int local;
    if (m->causal) {
        int64_t gap = i - j;
        local = (gap % m->dilation == 0) && (m->window == 0 || gap < m->window * m->dilation);
    } else {
        int64_t dist = i > j ? i - j : j - i;
        local = (dist % m->dilation == 0) && (!m->has_radius || dist <= m->radius * m->dilation);
    }
    int strided = strided_col(m, j);
    int global = global_pair(m, i, j);
    return local || strided || global;
}

/* Token-level masks do not depend on T; block masks take T = 2^62. */
int oracle_allowed(const oracle_mask* m, int64_t i, int64_t j) {
    return oracle_allowed_T(m, (int64_t)1 << 62, i, j);
}

/* S_i written out as a sorted list by scanning every key; returns |S_i|. */
int64_t oracle_row_set(const oracle_mask* m, int64_t T, int64_t i, int64_t* out) {
    int64_t n = 0;
    for (int64_t j = 0; j < T; ++j)
        if (oracle_allowed_T(m, T, i, j)) {
            if (out) out[n] = j;
            ++n;
        }
    return n;
}

/* E = sum_i |S_i| by scanning all T*T pairs; optional per-row counts. */
int64_t oracle_count(const oracle_mask* m, int64_t T, int64_t* row_counts) {
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : total)
    for (int64_t i = 0; i < T; ++i) {
        int64_t c = oracle_row_set(m, T, i, NULL);
        if (row_counts) row_counts[i] = c;
        total += c;
    }
    return total;
}

/* Tile classes, decided by counting allowed pairs among a tile's in-range
 * cells (rows i < T and keys j < T): 0 = no allowed pair, 1 = every in-range
 * pair allowed, 2 = some but not all. */
void oracle_tile_map(const oracle_mask* m, int64_t T, int64_t bq, int64_t bk,
                     uint8_t* map) {
    int64_t nqb = (T + bq - 1) / bq, nkb = (T + bk - 1) / bk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t qb = 0; qb < nqb; ++qb) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int64_t cells = 0, allowed = 0;
            for (int64_t i = qb * bq; i < (qb + 1) * bq && i < T; ++i)
                for (int64_t j = kb * bk; j < (kb + 1) * bk && j < T; ++j) {
                    ++cells;
                    allowed += oracle_allowed_T(m, T, i, j);
                }
            map[qb * nkb + kb] = allowed == 0 ? 0 : (allowed == cells ? 1 : 2);
        }
    }
}

/*
 * Forward pass for a list of rows.  Tensors are [BH][T][d] fp32, row-major.
 * rows[r] = bh * T + i selects query i of head bh.  For each selected row:
 *   1. S_i by scanning every key,
 *   2. s_j = (q_i . k_j) / sqrt(d),
 *   3. mx = max_j s_j,
 *   4. l = sum_j exp(s_j - mx),
 *   5. o = (sum_j exp(s_j - mx) v_j) / l,   lse = mx + log(l).
 * Outputs: O[r][d] and lse[r] in fp64, nset[r] = |S_i| (any may be NULL
 * except O).  Returns 0, or -1 if a row is out of range or memory runs out.
 * An empty S_i (not reachable through the mask grammar, whose window or
 * radius always keeps the query itself) gives o = 0 and lse = -inf.
 */
int oracle_forward_rows(const oracle_mask* m, const float* Q, const float* K,
                        const float* V, int64_t BH, int64_t T, int64_t d,
                        const int64_t* rows, int64_t n_rows, double* O,
                        double* lse, int64_t* nset) {
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= BH * T) return -1;
    int failed = 0;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
#pragma omp parallel reduction(| : failed)
    {
        int64_t* set = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        if (!set || !s || !acc) failed = 1;
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (failed) continue;
            int64_t bh = rows[r] / T, i = rows[r] % T;
            const float* q = Q + (bh * T + i) * d;
            int64_t n = oracle_row_set(m, T, i, set);
            if (nset) nset[r] = n;
            double* o = O + r * d;
            if (n == 0) {
                for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
                if (lse) lse[r] = -INFINITY;
                continue;
            }
            double mx = -INFINITY;
            for (int64_t t = 0; t < n; ++t) {
                const float* k = K + (bh * T + set[t]) * d;
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c) dot += (double)q[c] * (double)k[c];
                s[t] = dot * inv_sqrt_d;
                if (s[t] > mx) mx = s[t];
            }
            double l = 0.0;
            for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                double p = exp(s[t] - mx);
                l += p;
                const float* v = V + (bh * T + set[t]) * d;
                for (int64_t c = 0; c < d; ++c) acc[c] += p * (double)v[c];
            }
            for (int64_t c = 0; c < d; ++c) o[c] = acc[c] / l;
            if (lse) lse[r] = mx + log(l);
        }
        free(set);
        free(s);
        free(acc);
    }
    return failed ? -1 : 0;
}

/*
 * Backward pass of the same attention (the pages define only the forward;
 * this is the gradient of its definition, "Choose the available reads",
 * by the chain rule through the softmax over S_i).  With s_ij = q_i.k_j /
 * sqrt(d) for j in S_i, p_ij = exp(s_ij - lse_i) and an upstream gradient
 * dO (the gradient of the loss with respect to O):
 *   dV_j  = sum_i p_ij dO_i
 *   dp_ij = dO_i . v_j
 *   D_i   = sum_j p_ij dp_ij            (= dO_i . o_i)
 *   ds_ij = p_ij (dp_ij - D_i)
 *   dQ_i  = sum_j ds_ij k_j / sqrt(d)
 *   dK_j  = sum_i ds_ij q_i / sqrt(d)
 * Written as two passes so that each output is owned by one loop iteration:
 * a pass over rows i (the weights of S_i, D_i and dQ_i), then a pass over
 * keys j that visits every row i whose S_i holds j, in increasing i (dK_j,
 * dV_j).  Tensors [BH][T][d] fp32 in, fp64 out (dQ, dK, dV written in full).
 * Returns 0, or -1 if memory runs out.
 */
int oracle_backward(const oracle_mask* m, const float* Q, const float* K, const float* V,
                    const float* dO, int64_t BH, int64_t T, int64_t d, double* dQ, double* dK,
                    double* dV) {
    int failed = 0;
    const double rscale = sqrt(1.0 / (double)d);
    for (int64_t x = 0; x < BH * T * d; ++x) dQ[x] = dK[x] = dV[x] = 0.0;
    /* per row: the max and the sum of the softmax, and D */
    double* rmx = (double*)malloc(sizeof(double) * (size_t)(BH * T > 0 ? BH * T : 1));
    double* rl = (double*)malloc(sizeof(double) * (size_t)(BH * T > 0 ? BH * T : 1));
    double* rD = (double*)malloc(sizeof(double) * (size_t)(BH * T > 0 ? BH * T : 1));
    if (!rmx || !rl || !rD) {
        free(rmx);
        free(rl);
        free(rD);
        return -1;
    }
    /* pass 1: rows */
#pragma omp parallel reduction(| : failed)
    {
        int64_t* set = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        if (!set || !p || !dp) failed = 1;
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < BH * T; ++r) {
            if (failed) continue;
            const int64_t bh = r / T, i = r % T;
            const float* q = Q + (bh * T + i) * d;
            const float* g = dO + (bh * T + i) * d;
            const int64_t n = oracle_row_set(m, T, i, set);
            rmx[r] = 0.0;
            rl[r] = 0.0;
            rD[r] = 0.0;
            if (n == 0) continue;
            /* softmax weights over S_i */
            double mx = -INFINITY;
            for (int64_t t = 0; t < n; ++t) {
                const float* kr = K + d * (bh * T + set[t]);
                double qk = 0.0;
                for (int64_t c = 0; c < d; ++c) qk += (double)q[c] * (double)kr[c];
                p[t] = qk * rscale;
                if (p[t] > mx) mx = p[t];
            }
            double l = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                p[t] = exp(p[t] - mx);
                l += p[t];
            }
            for (int64_t t = 0; t < n; ++t) p[t] /= l;
            /* dp and D */
            double D = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                const float* vr = V + d * (bh * T + set[t]);
                double gv = 0.0;
                for (int64_t c = 0; c < d; ++c) gv += (double)g[c] * (double)vr[c];
                dp[t] = gv;
                D += p[t] * gv;
            }
            rmx[r] = mx;
            rl[r] = l;
            rD[r] = D;
            /* dQ_i */
            double* dq = dQ + (bh * T + i) * d;
            for (int64_t t = 0; t < n; ++t) {
                const double ds = p[t] * (dp[t] - D);
                const float* kr = K + d * (bh * T + set[t]);
                for (int64_t c = 0; c < d; ++c) dq[c] += ds * (double)kr[c] * rscale;
            }
        }
        free(set);
        free(p);
        free(dp);
    }
    /* pass 2: keys, each over the rows that read it */
    if (!failed) {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t col = 0; col < BH * T; ++col) {
            const int64_t bh = col / T, j = col % T;
            const float* kr = K + d * (bh * T + j);
            const float* vr = V + d * (bh * T + j);
            double* dk = dK + d * (bh * T + j);
            double* dv = dV + d * (bh * T + j);
            for (int64_t i = 0; i < T; ++i) {
                if (!oracle_allowed_T(m, T, i, j)) continue;
                const int64_t r = bh * T + i;
                const float* q = Q + d * r;
                const float* g = dO + d * r;
                double qk = 0.0;
                for (int64_t c = 0; c < d; ++c) qk += (double)q[c] * (double)kr[c];
                const double pij = exp(qk * rscale - rmx[r]) / rl[r];
                double gv = 0.0;
                for (int64_t c = 0; c < d; ++c) gv += (double)g[c] * (double)vr[c];
                const double ds = pij * (gv - rD[r]);
                for (int64_t c = 0; c < d; ++c) {
                    dk[c] += ds * (double)q[c] * rscale;
                    dv[c] += pij * (double)g[c];
                }
            }
        }
    }
    free(rmx);
    free(rl);
    free(rD);
    return failed ? -1 : 0;
}

int oracle_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
