/*
 * oracle.c -- plain fp64 CPU oracle for sparse multi-head graph attention.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  It shares nothing with
 * the GPU library: no headers, helpers, tables or kernels.
 *
 * What it computes (destination-sorted CSR: row v lists the sources u of its
 * in-edges u->v; Q, K, V are [N][H][D] with D contiguous):
 *
 *   s_e      = <Q[v,h,:], K[u_e,h,:]> / sqrt(D)            for e in row v
 *   alpha_e  = exp(s_e - m) / sum_e' exp(s_e' - m),  m = max_e s_e
 *   out[v,h] = sum_e alpha_e * V[u_e,h,:]    (0 when v has no in-edges)
 *
 * Sources:
 *  - "Graph Transformer in a Nutshell" (DGL sparse tutorial), section "Sparse
 *    Multi-head Attention": SparseAttn(Q,K,V,A) = softmax((QK^T) o A / sqrt(d)) V,
 *    scores only where A is nonzero (SDDMM), a sparse softmax, then an SpMM.
 *  - "Efficient Sparse Transformer implementation with DGL's builtin
 *    operators", TransLayer.forward: u_dot_v (source key . destination
 *    query), edge_softmax of the scores divided by sqrt(d_qkv), u_mul_e_sum.
 *  - "Graph Transformer theory, derivation and implementation" (Japanese blog),
 *    section reviewing scaled dot-product attention: e_ij = q_i.k_j / sqrt(d_k),
 *    alpha_ij = exp(e_ij) / sum_j' exp(e_ij'), h_i = sum_j alpha_ij v_j; here j
 *    ranges over the in-edges of i only.
 *
 * Readings where the pages are silent:
 *  - the softmax of each destination runs over its in-edges (the tutorial's
 *    Hadamard form read as a logit of -inf, not 0, off the graph);
 *  - each stored edge is its own term (duplicates count twice);
 *  - a destination with no in-edges gets the empty sum, 0;
 *  - the max is subtracted before exp (mathematically a no-op).
 *
 * The algorithm is deliberately plain: per row and head, one pass for all
 * scores and their max, one for the exponentials and their sum, one for the
 * weights and the weighted sum of V rows, all in double.  Inputs are widened
 * to double exactly (fp32 and bf16 values are representable in fp64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

/* element i of a feature array, widened exactly to double */
static double elem(const void* base, int dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float*)base)[i];
    if (dtype == OR_F64) return ((const double*)base)[i];
    /* bf16: the upper 16 bits of an IEEE binary32 */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int bad_dtype(int dtype) { return dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64; }

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* score of edge e (source u) for destination v, head h: dot product over D, then / sqrt(D) */
static double edge_score(const void* Q, const void* K, int dtype, int H, int D, int64_t v, int64_t u, int h) {
    int64_t qo = (v * H + h) * (int64_t)D, ko = (u * H + h) * (int64_t)D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += elem(Q, dtype, qo + d) * elem(K, dtype, ko + d);
    return dot / sqrt((double)D);
}

/*
 * Softmax over the in-edges of one destination for one head, two-pass:
 * s[0..deg) in, a[0..deg) out (a may alias s).
 */
static void row_softmax(const double* s, double* a, int64_t deg) {
    double m = -INFINITY;
    for (int64_t i = 0; i < deg; ++i)
        if (s[i] > m) m = s[i];
    double z = 0.0;
    for (int64_t i = 0; i < deg; ++i) {
        a[i] = exp(s[i] - m);
        z += a[i];
    }
    for (int64_t i = 0; i < deg; ++i) a[i] /= z;
}

/* ------------------------------------------------------------------------ */
/* Stage 1: SDDMM.  scores[e*H + h] = s_e for head h.                        */
/* ------------------------------------------------------------------------ */
int oracle_sddmm(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                 const void* Q, const void* K, double* scores, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || bad_dtype(dtype)) return 1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < N; ++v)
        for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e)
            for (int h = 0; h < H; ++h) scores[e * H + h] = edge_score(Q, K, dtype, H, D, v, indices[e], h);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stage 2: edge softmax per (destination, head).  alpha may alias scores.   */
/* ------------------------------------------------------------------------ */
int oracle_edge_softmax(int64_t N, int64_t E, int H, const int64_t* indptr, const double* scores, double* alpha,
                        int nthreads) {
    if (N < 0 || E < 0 || H < 1) return 1;
    int64_t maxdeg = 0;
    for (int64_t v = 0; v < N; ++v)
        if (indptr[v + 1] - indptr[v] > maxdeg) maxdeg = indptr[v + 1] - indptr[v];
    set_threads(nthreads);
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * (size_t)(maxdeg > 0 ? maxdeg : 1));
#pragma omp for schedule(dynamic, 64)
        for (int64_t v = 0; v < N; ++v) {
            int64_t b = indptr[v], deg = indptr[v + 1] - b;
            for (int h = 0; h < H; ++h) {
                for (int64_t i = 0; i < deg; ++i) buf[i] = scores[(b + i) * H + h];
                row_softmax(buf, buf, deg);
                for (int64_t i = 0; i < deg; ++i) alpha[(b + i) * H + h] = buf[i];
            }
        }
        free(buf);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stage 3: SpMM.  out[v,h,:] = sum_e alpha[e*H+h] * V[u_e,h,:].             */
/* ------------------------------------------------------------------------ */
int oracle_spmm(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                const double* alpha, const void* V, double* out, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || bad_dtype(dtype)) return 1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < N; ++v)
        for (int h = 0; h < H; ++h) {
            double* o = out + (v * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e) {
                double a = alpha[e * H + h];
                int64_t vo = ((int64_t)indices[e] * H + h) * (int64_t)D;
                for (int d = 0; d < D; ++d) o[d] += a * elem(V, dtype, vo + d);
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Whole forward for a list of destination rows: the three stages above,    */
/* applied row by row.  out_rows is [nrows][H][D]; scores_rows and           */
/* alpha_rows (optional) receive the row's edges in CSR order, packed in     */
/* the order the rows are listed: [sum of degrees][H].                       */
/* ------------------------------------------------------------------------ */
int oracle_fwd_rows(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                    const void* Q, const void* K, const void* V, const int64_t* rows, int64_t nrows,
                    double* out_rows, double* scores_rows, double* alpha_rows, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || nrows < 0 || bad_dtype(dtype)) return 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return 1;
    /* packed offset of each listed row's edges */
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows + 1));
    int64_t maxdeg = 0;
    pos[0] = 0;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t deg = indptr[rows[r] + 1] - indptr[rows[r]];
        pos[r + 1] = pos[r] + deg;
        if (deg > maxdeg) maxdeg = deg;
    }
    set_threads(nthreads);
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(maxdeg > 0 ? maxdeg : 1));
        double* a = (double*)malloc(sizeof(double) * (size_t)(maxdeg > 0 ? maxdeg : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t v = rows[r], b = indptr[v], deg = indptr[v + 1] - b;
            for (int h = 0; h < H; ++h) {
                double* o = out_rows + (r * H + h) * (int64_t)D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                /* pass 1: scores (and their max, inside row_softmax) */
                for (int64_t i = 0; i < deg; ++i) s[i] = edge_score(Q, K, dtype, H, D, v, indices[b + i], h);
                /* pass 2: exponentials, their sum, the weights */
                row_softmax(s, a, deg);
                /* pass 3: weighted sum of the source V rows */
                for (int64_t i = 0; i < deg; ++i) {
                    int64_t vo = ((int64_t)indices[b + i] * H + h) * (int64_t)D;
                    for (int d = 0; d < D; ++d) o[d] += a[i] * elem(V, dtype, vo + d);
                    if (scores_rows) scores_rows[(pos[r] + i) * H + h] = s[i];
                    if (alpha_rows) alpha_rows[(pos[r] + i) * H + h] = a[i];
                }
            }
        }
        free(a);
        free(s);
    }
    free(pos);
    return 0;
}

/* Whole forward over every row: out is [N][H][D]; scores/alpha optional [E][H]. */
int oracle_fwd(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
               const void* Q, const void* K, const void* V, double* out, double* scores, double* alpha,
               int nthreads) {
    if (N < 0) return 1;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    for (int64_t v = 0; v < N; ++v) rows[v] = v;
    int rc = oracle_fwd_rows(N, E, H, D, dtype, indptr, indices, Q, K, V, rows, N, out, scores, alpha, nthreads);
    free(rows);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward of the forward above, for a loss L with dL/dout = dO.           */
/*                                                                          */
/* With s_e = q_v.k_u / sqrt(D), alpha_e = exp(s_e - lse_v) and              */
/* lse_v = log sum_e exp(s_e) over the in-edges of v (per head), the chain   */
/* rule through out_v = sum_e alpha_e v_u and the softmax gives:             */
/*   dV_u    = sum over out-edges e = (u->v) of alpha_e dO_v                 */
/*   da_e    = dO_v . v_u                                                    */
/*   delta_v = sum over in-edges e of v of alpha_e da_e  (= dO_v . out_v)    */
/*   ds_e    = alpha_e (da_e - delta_v)                                      */
/*   dQ_v    = sum over in-edges of ds_e k_u / sqrt(D)                       */
/*   dK_u    = sum over out-edges of ds_e q_v / sqrt(D)                      */
/* (the softmax Jacobian is diag(alpha) - alpha alpha^T).  Every stored edge */
/* is its own term.  Rows without in-edges have lse = -inf and contribute    */
/* nothing.                                                                  */
/* ------------------------------------------------------------------------ */

/*
 * Per destination row and head: lse (natural log) and delta = sum alpha da.
 * lse = -inf and delta = 0 for rows without in-edges.  lse and delta are [N][H].
 */
int oracle_row_stats(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                     const void* Q, const void* K, const void* V, const void* dO, double* lse, double* delta,
                     int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || bad_dtype(dtype)) return 1;
    int64_t maxdeg = 0;
    for (int64_t v = 0; v < N; ++v)
        if (indptr[v + 1] - indptr[v] > maxdeg) maxdeg = indptr[v + 1] - indptr[v];
    set_threads(nthreads);
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(maxdeg > 0 ? maxdeg : 1));
#pragma omp for schedule(dynamic, 64)
        for (int64_t v = 0; v < N; ++v) {
            int64_t b = indptr[v], deg = indptr[v + 1] - b;
            for (int h = 0; h < H; ++h) {
                double m = -INFINITY, z = 0.0, dl = 0.0;
                for (int64_t i = 0; i < deg; ++i) {
                    s[i] = edge_score(Q, K, dtype, H, D, v, indices[b + i], h);
                    if (s[i] > m) m = s[i];
                }
                for (int64_t i = 0; i < deg; ++i) z += exp(s[i] - m);
                double l = deg > 0 ? m + log(z) : -INFINITY;
                int64_t go = (v * H + h) * (int64_t)D;
                for (int64_t i = 0; i < deg; ++i) {
                    double a = exp(s[i] - l);
                    int64_t vo = ((int64_t)indices[b + i] * H + h) * (int64_t)D;
                    double da = 0.0;
                    for (int d = 0; d < D; ++d) da += elem(dO, dtype, go + d) * elem(V, dtype, vo + d);
                    dl += a * da;
                }
                lse[v * H + h] = l;
                delta[v * H + h] = dl;
            }
        }
        free(s);
    }
    return 0;
}

/* dQ for the listed destination rows: out is [nrows][H][D]. */
int oracle_dq_rows(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                   const void* Q, const void* K, const void* V, const void* dO, const double* lse,
                   const double* delta, const int64_t* rows, int64_t nrows, double* dq, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || nrows < 0 || bad_dtype(dtype)) return 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return 1;
    const double rs = 1.0 / sqrt((double)D);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t v = rows[r];
        for (int h = 0; h < H; ++h) {
            double* o = dq + (r * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            int64_t go = (v * H + h) * (int64_t)D;
            for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e) {
                int64_t u = indices[e];
                int64_t uo = (u * H + h) * (int64_t)D; /* row u of K and of V */
                double a = exp(edge_score(Q, K, dtype, H, D, v, u, h) - lse[v * H + h]);
                double da = 0.0;
                for (int d = 0; d < D; ++d) da += elem(dO, dtype, go + d) * elem(V, dtype, uo + d);
                double ds = a * (da - delta[v * H + h]);
                for (int d = 0; d < D; ++d) o[d] += ds * elem(K, dtype, uo + d) * rs;
            }
        }
    }
    return 0;
}

/*
 * dK and dV for the listed source nodes, using the transposed graph: for
 * source u, t_indices[t_indptr[u] .. t_indptr[u+1]) are the destinations of
 * its out-edges.  dk and dv are [nsrc][H][D].
 */
int oracle_dkv_sources(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* t_indptr,
                       const int32_t* t_indices, const void* Q, const void* K, const void* V, const void* dO,
                       const double* lse, const double* delta, const int64_t* srcs, int64_t nsrc, double* dk,
                       double* dv, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || nsrc < 0 || bad_dtype(dtype)) return 1;
    for (int64_t r = 0; r < nsrc; ++r)
        if (srcs[r] < 0 || srcs[r] >= N) return 1;
    const double rs = 1.0 / sqrt((double)D);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nsrc; ++r) {
        int64_t u = srcs[r];
        for (int h = 0; h < H; ++h) {
            double* ok = dk + (r * H + h) * (int64_t)D;
            double* ov = dv + (r * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) ok[d] = ov[d] = 0.0;
            int64_t uo = (u * H + h) * (int64_t)D;
            for (int64_t j = t_indptr[u]; j < t_indptr[u + 1]; ++j) {
                int64_t v = t_indices[j];
                int64_t vo = (v * H + h) * (int64_t)D;
                double a = exp(edge_score(Q, K, dtype, H, D, v, u, h) - lse[v * H + h]);
                double da = 0.0;
                for (int d = 0; d < D; ++d) da += elem(dO, dtype, vo + d) * elem(V, dtype, uo + d);
                double ds = a * (da - delta[v * H + h]);
                for (int d = 0; d < D; ++d) {
                    ov[d] += a * elem(dO, dtype, vo + d);
                    ok[d] += ds * elem(Q, dtype, vo + d) * rs;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Graph construction.  "Graph Transformer in a Nutshell", section "Graph   */
/* Transformer Model": GTModel.forward stacks the (src, dst) pairs of       */
/* g.edges() into one sparse adjacency matrix and hands it to every layer. */
/* The attention consumes it grouped by destination (the CSR above); the    */
/* backward also grouped by source (the transpose).                         */
/* ------------------------------------------------------------------------ */

/*
 * COO -> destination-sorted CSR by a counting sort: count the in-degrees,
 * take their running sum as indptr, then walk the edges in COO order and put
 * each one at the next free slot of its destination's row.  Row v thus lists
 * the sources of v's in-edges in COO order; perm[p] (if non-NULL) is the COO
 * id of the edge at CSR position p.  src in [0, n_src), dst in [0, n_dst);
 * indptr has n_dst + 1 entries.  Returns 1 for an id out of range.
 */
int oracle_coo_to_csr(int64_t n_dst, int64_t n_src, int64_t E, const int32_t* src, const int32_t* dst,
                      int64_t* indptr, int32_t* indices, int64_t* perm) {
    if (n_dst < 0 || n_src < 0 || E < 0) return 1;
    for (int64_t e = 0; e < E; ++e)
        if (src[e] < 0 || src[e] >= n_src || dst[e] < 0 || dst[e] >= n_dst) return 1;
    for (int64_t v = 0; v <= n_dst; ++v) indptr[v] = 0;
    for (int64_t e = 0; e < E; ++e) indptr[dst[e] + 1] += 1;
    for (int64_t v = 0; v < n_dst; ++v) indptr[v + 1] += indptr[v];
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_dst > 0 ? n_dst : 1));
    if (!next) return 2;
    for (int64_t v = 0; v < n_dst; ++v) next[v] = indptr[v];
    for (int64_t e = 0; e < E; ++e) {
        int64_t p = next[dst[e]]++;
        indices[p] = src[e];
        if (perm) perm[p] = e;
    }
    free(next);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Logit variants and attention dropout.                                    */
/*  - additive bias: "Graph Transformer theory, derivation and              */
/*    implementation", section on the shortest-path bias and degree         */
/*    encoding (Graphormer type), spatial encoding: a learnable scalar is   */
/*    added to each logit, e_ij = q_i.k_j / sqrt(d_k) + b.  Here any bias   */
/*    per (edge, head), bias[e*H + h].                                      */
/*  - edge weights: "Graph Transformer in a Nutshell", section "Sparse      */
/*    Multi-head Attention": A takes values in [0, 1] and the scaled logit  */
/*    is the Hadamard product (QK^T) o A / sqrt(d), so a weighted edge      */
/*    multiplies its scaled dot product: s_e = w_e <q_v, k_u> / sqrt(D)      */
/*    (+ bias).  The softmax still runs over the stored edges only.         */
/*  - dropout: the gist's TransLayer.forward applies drop_att to the edge  */
/*    softmax's output.  In training an attention weight is dropped with    */
/*    probability p and the kept ones are divided by 1 - p; the softmax's   */
/*    normaliser is unchanged.  The keep decision for (edge e, head h) uses */
/*    word i = e*H + h of the counter-based generator Philox4x64-10         */
/*    (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as  */
/*    1, 2, 3", SC 2011): block i/4 + 1 under key (seed, 0), word i mod 4;  */
/*    the weight is kept iff the word's upper 32 bits are >= floor(p 2^32). */
/* ------------------------------------------------------------------------ */

static uint64_t philox_word(uint64_t seed, uint64_t i) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = i / 4 + 1, c1 = 0, c2 = 0, c3 = 0, k0 = seed, k1 = 0;
    for (int r = 0; r < 10; ++r) {
        unsigned __int128 p0 = (unsigned __int128)M0 * c0, p1 = (unsigned __int128)M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += W0;
        k1 += W1;
    }
    switch (i % 4) {
        case 0: return c0;
        case 1: return c1;
        case 2: return c2;
        default: return c3;
    }
}

uint64_t oracle_philox_word(uint64_t seed, uint64_t i) { return philox_word(seed, i); }

/* dropout multiplier of (edge e, head h): 0 or 1 / (1 - p); 1 when p == 0 */
static double drop_scale(double p, uint64_t seed, int64_t e, int H, int h) {
    if (p <= 0.0) return 1.0;
    uint32_t thresh = (uint32_t)floor(p * 4294967296.0);
    uint32_t hi = (uint32_t)(philox_word(seed, (uint64_t)e * (uint64_t)H + (uint64_t)h) >> 32);
    return hi >= thresh ? 1.0 / (1.0 - p) : 0.0;
}

/* logit of edge e (source u) for destination v, head h, with the variants */
static double edge_logit(const void* Q, const void* K, int dtype, int H, int D, int64_t v, int64_t u, int h,
                         int64_t e, const float* bias, const float* ew) {
    double s = edge_score(Q, K, dtype, H, D, v, u, h);
    if (ew) s *= (double)ew[e];
    if (bias) s += (double)bias[e * H + h];
    return s;
}

static int bad_p(double p) { return !(p >= 0.0 && p < 1.0); }

/*
 * Forward with the variants for the listed destination rows: out
 * [nrows][H][D] and (if non-NULL) lse [nrows][H] of the logits.
 */
int oracle_fwd_rows_ex(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                       const void* Q, const void* K, const void* V, const float* bias, const float* ew, double drop_p,
                       uint64_t seed, const int64_t* rows, int64_t nrows, double* out, double* lse, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || nrows < 0 || bad_dtype(dtype) || bad_p(drop_p)) return 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return 1;
    int64_t maxdeg = 0;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t deg = indptr[rows[r] + 1] - indptr[rows[r]];
        if (deg > maxdeg) maxdeg = deg;
    }
    set_threads(nthreads);
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(maxdeg > 0 ? maxdeg : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t v = rows[r], b = indptr[v], deg = indptr[v + 1] - b;
            for (int h = 0; h < H; ++h) {
                double* o = out + (r * H + h) * (int64_t)D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                double m = -INFINITY, z = 0.0;
                for (int64_t i = 0; i < deg; ++i) {
                    s[i] = edge_logit(Q, K, dtype, H, D, v, indices[b + i], h, b + i, bias, ew);
                    if (s[i] > m) m = s[i];
                }
                for (int64_t i = 0; i < deg; ++i) z += exp(s[i] - m);
                for (int64_t i = 0; i < deg; ++i) {
                    double a = exp(s[i] - m) / z * drop_scale(drop_p, seed, b + i, H, h);
                    int64_t uo = ((int64_t)indices[b + i] * H + h) * (int64_t)D;
                    for (int d = 0; d < D; ++d) o[d] += a * elem(V, dtype, uo + d);
                }
                if (lse) lse[r * H + h] = deg > 0 ? m + log(z) : -INFINITY;
            }
        }
        free(s);
    }
    return 0;
}

/*
 * Backward with the variants.  With alpha_e = exp(s_e - lse_v), the dropout
 * multiplier c_e and da_e = dO_v . v_u:
 *   delta_v = sum alpha_e c_e da_e (= dO_v . out_v)
 *   ds_e    = alpha_e (c_e da_e - delta_v)         (= dL/dbias_e)
 *   dQ_v    = sum over in-edges  ds_e w_e k_u / sqrt(D)
 *   dK_u    = sum over out-edges ds_e w_e q_v / sqrt(D)
 *   dV_u    = sum over out-edges alpha_e c_e dO_v
 *   dw_e    = sum over heads ds_e <q_v, k_u> / sqrt(D)
 * row_stats_ex: lse and delta [N][H] of every row.
 */
int oracle_row_stats_ex(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                        const void* Q, const void* K, const void* V, const void* dO, const float* bias, const float* ew,
                        double drop_p, uint64_t seed, double* lse, double* delta, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || bad_dtype(dtype) || bad_p(drop_p)) return 1;
    int64_t maxdeg = 0;
    for (int64_t v = 0; v < N; ++v)
        if (indptr[v + 1] - indptr[v] > maxdeg) maxdeg = indptr[v + 1] - indptr[v];
    set_threads(nthreads);
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(maxdeg > 0 ? maxdeg : 1));
#pragma omp for schedule(dynamic, 64)
        for (int64_t v = 0; v < N; ++v) {
            int64_t b = indptr[v], deg = indptr[v + 1] - b;
            for (int h = 0; h < H; ++h) {
                double m = -INFINITY, z = 0.0, dl = 0.0;
                for (int64_t i = 0; i < deg; ++i) {
                    s[i] = edge_logit(Q, K, dtype, H, D, v, indices[b + i], h, b + i, bias, ew);
                    if (s[i] > m) m = s[i];
                }
                for (int64_t i = 0; i < deg; ++i) z += exp(s[i] - m);
                double l = deg > 0 ? m + log(z) : -INFINITY;
                int64_t go = (v * H + h) * (int64_t)D;
                for (int64_t i = 0; i < deg; ++i) {
                    double a = exp(s[i] - l) * drop_scale(drop_p, seed, b + i, H, h);
                    int64_t uo = ((int64_t)indices[b + i] * H + h) * (int64_t)D;
                    double da = 0.0;
                    for (int d = 0; d < D; ++d) da += elem(dO, dtype, go + d) * elem(V, dtype, uo + d);
                    dl += a * da;
                }
                lse[v * H + h] = l;
                delta[v * H + h] = dl;
            }
        }
        free(s);
    }
    return 0;
}

/*
 * dQ [nrows][H][D] of the listed destination rows; for their edges also
 * dbias[e*H + h] and dw[e] when those are non-NULL (full-size arrays; other
 * entries are left as they are).
 */
int oracle_dq_rows_ex(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* indptr, const int32_t* indices,
                      const void* Q, const void* K, const void* V, const void* dO, const float* bias, const float* ew,
                      double drop_p, uint64_t seed, const double* lse, const double* delta, const int64_t* rows,
                      int64_t nrows, double* dq, double* dbias, double* dw, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || nrows < 0 || bad_dtype(dtype) || bad_p(drop_p)) return 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return 1;
    const double rs = 1.0 / sqrt((double)D);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t v = rows[r];
        for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e)
            if (dw) dw[e] = 0.0;
        for (int h = 0; h < H; ++h) {
            double* o = dq + (r * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            int64_t go = (v * H + h) * (int64_t)D;
            for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e) {
                int64_t u = indices[e];
                int64_t uo = (u * H + h) * (int64_t)D;
                double dot = edge_score(Q, K, dtype, H, D, v, u, h);
                double w = ew ? (double)ew[e] : 1.0;
                double a = exp(edge_logit(Q, K, dtype, H, D, v, u, h, e, bias, ew) - lse[v * H + h]);
                double da = 0.0;
                for (int d = 0; d < D; ++d) da += elem(dO, dtype, go + d) * elem(V, dtype, uo + d);
                double ds = a * (drop_scale(drop_p, seed, e, H, h) * da - delta[v * H + h]);
                for (int d = 0; d < D; ++d) o[d] += ds * w * elem(K, dtype, uo + d) * rs;
                if (dbias) dbias[e * H + h] = ds;
                if (dw) dw[e] += ds * dot;
            }
        }
    }
    return 0;
}

/*
 * dK, dV [nsrc][H][D] of the listed sources over the source-sorted graph;
 * t_perm[j] is the destination-CSR position of out-edge j (the edge id that
 * bias, weights and the dropout words are indexed by).
 */
int oracle_dkv_sources_ex(int64_t N, int64_t E, int H, int D, int dtype, const int64_t* t_indptr,
                          const int32_t* t_indices, const int32_t* t_perm, const void* Q, const void* K,
                          const void* V, const void* dO, const float* bias, const float* ew, double drop_p,
                          uint64_t seed, const double* lse, const double* delta, const int64_t* srcs, int64_t nsrc,
                          double* dk, double* dv, int nthreads) {
    if (N < 0 || E < 0 || H < 1 || D < 1 || nsrc < 0 || bad_dtype(dtype) || bad_p(drop_p)) return 1;
    for (int64_t r = 0; r < nsrc; ++r)
        if (srcs[r] < 0 || srcs[r] >= N) return 1;
    const double rs = 1.0 / sqrt((double)D);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nsrc; ++r) {
        int64_t u = srcs[r];
        for (int h = 0; h < H; ++h) {
            double* ok = dk + (r * H + h) * (int64_t)D;
            double* ov = dv + (r * H + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) ok[d] = ov[d] = 0.0;
            int64_t uo = (u * H + h) * (int64_t)D;
            for (int64_t j = t_indptr[u]; j < t_indptr[u + 1]; ++j) {
                int64_t v = t_indices[j], e = t_perm[j];
                int64_t vo = (v * H + h) * (int64_t)D;
                double w = ew ? (double)ew[e] : 1.0;
                double c = drop_scale(drop_p, seed, e, H, h);
                double a = exp(edge_logit(Q, K, dtype, H, D, v, u, h, e, bias, ew) - lse[v * H + h]);
                double da = 0.0;
                for (int d = 0; d < D; ++d) da += elem(dO, dtype, vo + d) * elem(V, dtype, uo + d);
                double ds = a * (c * da - delta[v * H + h]);
                for (int d = 0; d < D; ++d) {
                    ov[d] += a * c * elem(dO, dtype, vo + d);
                    ok[d] += ds * w * elem(Q, dtype, vo + d) * rs;
                }
            }
        }
    }
    return 0;
}
