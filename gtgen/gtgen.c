/*
 * gtgen.c -- seeded synthetic inputs for sparse multi-head graph attention.
 *
 * This module only makes inputs: graphs (as COO or destination-sorted CSR)
 * and Q/K/V feature arrays.  It holds none of the attention arithmetic, so
 * both the CPU oracle and the GPU library can be fed from it.
 *
 * Randomness is counter based: value i of stream s under seed k is a pure
 * function of (k, s, i), so results do not depend on thread count or on the
 * order in which values are drawn.  The hash is the SplitMix64 output
 * function (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014), applied to a Weyl sequence keyed by (seed, stream).
 *
 * Normals come from the Box-Muller transform (two uniforms -> two normals).
 * Bounded integers use the multiply-high method (Lemire, 2019).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed + 0x632BE59BD9B4E019ull) ^ (stream * 0xD1B54A32D192ED03ull + 1));
}

/* value i of the keyed Weyl sequence */
static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* uniform double in [0,1) with 53 random bits */
static inline double u01(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

/* uniform integer in [0,n) by the multiply-high method */
static inline uint64_t below(uint64_t x, uint64_t n) {
    return (uint64_t)(((unsigned __int128)x * n) >> 64);
}

uint64_t gtgen_u64(uint64_t seed, uint64_t stream, uint64_t i) { return draw(stream_key(seed, stream), i); }

/* ------------------------------------------------------------------------ */
/* Feature arrays                                                            */
/* ------------------------------------------------------------------------ */

static inline void box_muller(uint64_t key, uint64_t pair, double* z0, double* z1) {
    uint64_t a = draw(key, 2 * pair), b = draw(key, 2 * pair + 1);
    double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0,1] so log is finite */
    double u2 = u01(b);
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

/* out[j] = fp32(scale * N(0,1)) for j < n */
void gtgen_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double scale, float* out) {
    uint64_t key = stream_key(seed, stream);
    int64_t npair = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npair; ++p) {
        double z0, z1;
        box_muller(key, (uint64_t)p, &z0, &z1);
        out[2 * p] = (float)(scale * z0);
        if (2 * p + 1 < n) out[2 * p + 1] = (float)(scale * z1);
    }
}

/* round an fp32 value to bf16 bits, nearest-even (inputs here are finite) */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* out[j] = bf16_rne(fp32(N(0,1)) * scale) for j < n, as raw bf16 bits */
void gtgen_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double scale, uint16_t* out) {
    uint64_t key = stream_key(seed, stream);
    int64_t npair = (n + 1) / 2;
    float fs = (float)scale;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npair; ++p) {
        double z0, z1;
        box_muller(key, (uint64_t)p, &z0, &z1);
        out[2 * p] = f32_to_bf16_rne((float)z0 * fs);
        if (2 * p + 1 < n) out[2 * p + 1] = f32_to_bf16_rne((float)z1 * fs);
    }
}

/* out[j] = uniform double in [lo, hi) */
void gtgen_uniform_f64(uint64_t seed, uint64_t stream, int64_t n, double lo, double hi, double* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = lo + (hi - lo) * u01(draw(key, (uint64_t)j));
}

/* ------------------------------------------------------------------------ */
/* Graphs                                                                    */
/* ------------------------------------------------------------------------ */

/* E directed edges with src and dst uniform and iid over [0,N). */
void gtgen_random_coo(uint64_t seed, uint64_t stream, int64_t N, int64_t E, int32_t* src, int32_t* dst) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < E; ++e) {
        src[e] = (int32_t)below(draw(key, 2 * (uint64_t)e), (uint64_t)N);
        dst[e] = (int32_t)below(draw(key, 2 * (uint64_t)e + 1), (uint64_t)N);
    }
}

/*
 * Stable counting sort of a COO edge list by destination: indptr[v]..indptr[v+1]
 * lists the in-edges of v in their original COO order; indices holds sources.
 * perm (optional) receives the COO position of each CSR edge.
 */
void gtgen_coo_to_dst_csr(int64_t N, int64_t E, const int32_t* src, const int32_t* dst, int64_t* indptr,
                          int32_t* indices, int64_t* perm) {
    for (int64_t v = 0; v <= N; ++v) indptr[v] = 0;
    for (int64_t e = 0; e < E; ++e) indptr[dst[e] + 1]++;
    for (int64_t v = 0; v < N; ++v) indptr[v + 1] += indptr[v];
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    for (int64_t v = 0; v < N; ++v) fill[v] = indptr[v];
    for (int64_t e = 0; e < E; ++e) {
        int64_t pos = fill[dst[e]]++;
        indices[pos] = src[e];
        if (perm) perm[pos] = e;
    }
    free(fill);
}

/* CSR from a per-destination degree array; each edge's source is uniform over [0,N). */
void gtgen_csr_from_degrees(uint64_t seed, uint64_t stream, int64_t N, const int64_t* deg, int64_t* indptr,
                            int32_t* indices) {
    indptr[0] = 0;
    for (int64_t v = 0; v < N; ++v) indptr[v + 1] = indptr[v] + deg[v];
    int64_t E = indptr[N];
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < E; ++e) indices[e] = (int32_t)below(draw(key, (uint64_t)e), (uint64_t)N);
}

/* Fisher-Yates permutation of [0,n) driven by the counter stream. */
void gtgen_permutation(uint64_t seed, uint64_t stream, int64_t n, int64_t* perm) {
    uint64_t key = stream_key(seed, stream);
    for (int64_t i = 0; i < n; ++i) perm[i] = i;
    for (int64_t i = n - 1; i > 0; --i) {
        int64_t j = (int64_t)below(draw(key, (uint64_t)i), (uint64_t)(i + 1));
        int64_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
}

/*
 * Power-law in-degrees: K ~ Zipf(alpha), P(K = k) = k^-alpha / zeta(alpha) for
 * k >= 1, clipped to cap (draws above cap become cap).  Nodes are visited in a
 * random order and given inverse-CDF draws until the running total reaches E
 * (the last draw is cut short); every later node gets degree 0.  Returns the
 * number of edges assigned (E unless the N draws sum to less).
 */
int64_t gtgen_degrees_zipf(uint64_t seed, uint64_t stream_perm, uint64_t stream_draw, int64_t N, int64_t E,
                           double alpha, int64_t cap, int64_t* deg) {
    double* cdf = (double*)malloc(sizeof(double) * (size_t)cap);
    /* zeta(alpha) by Euler-Maclaurin: partial sum to cap-1 plus the tail terms */
    double M = (double)cap, partial = 0.0;
    for (int64_t k = 1; k < cap; ++k) partial += pow((double)k, -alpha);
    double zeta = partial + pow(M, 1.0 - alpha) / (alpha - 1.0) + 0.5 * pow(M, -alpha) +
                  alpha * pow(M, -alpha - 1.0) / 12.0;
    double acc = 0.0;
    for (int64_t k = 1; k < cap; ++k) {
        acc += pow((double)k, -alpha);
        cdf[k - 1] = acc / zeta;
    }
    cdf[cap - 1] = 1.0; /* all mass at k >= cap is clipped to cap */
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    gtgen_permutation(seed, stream_perm, N, order);
    uint64_t key = stream_key(seed, stream_draw);
    for (int64_t v = 0; v < N; ++v) deg[v] = 0;
    int64_t total = 0;
    for (int64_t i = 0; i < N && total < E; ++i) {
        double u = u01(draw(key, (uint64_t)i));
        /* smallest k with cdf[k-1] > u */
        int64_t lo = 0, hi = cap - 1;
        while (lo < hi) {
            int64_t mid = (lo + hi) / 2;
            if (cdf[mid] > u) hi = mid;
            else lo = mid + 1;
        }
        int64_t k = lo + 1;
        if (total + k > E) k = E - total;
        deg[order[i]] = k;
        total += k;
    }
    free(order);
    free(cdf);
    return total;
}

typedef struct {
    double frac;
    int64_t id;
} frac_item;

static int cmp_frac_desc(const void* a, const void* b) {
    const frac_item* x = (const frac_item*)a;
    const frac_item* y = (const frac_item*)b;
    if (x->frac > y->frac) return -1;
    if (x->frac < y->frac) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

/*
 * Log-normal in-degrees with the given mean and log-space shape sigma
 * (mu = ln(mean) - sigma^2/2), integerised by the largest-remainder method so
 * that they sum to exactly E (ties go to the lower node id).
 */
void gtgen_degrees_lognormal(uint64_t seed, uint64_t stream, int64_t N, int64_t E, double mean, double sigma,
                             int64_t* deg) {
    double mu = log(mean) - 0.5 * sigma * sigma;
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    uint64_t key = stream_key(seed, stream);
    int64_t npair = (N + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npair; ++p) {
        double z0, z1;
        box_muller(key, (uint64_t)p, &z0, &z1);
        x[2 * p] = exp(mu + sigma * z0);
        if (2 * p + 1 < N) x[2 * p + 1] = exp(mu + sigma * z1);
    }
    double sum = 0.0;
    for (int64_t v = 0; v < N; ++v) sum += x[v];
    frac_item* fr = (frac_item*)malloc(sizeof(frac_item) * (size_t)N);
    int64_t total = 0;
    for (int64_t v = 0; v < N; ++v) {
        double q = x[v] * (double)E / sum;
        double f = floor(q);
        deg[v] = (int64_t)f;
        total += deg[v];
        fr[v].frac = q - f;
        fr[v].id = v;
    }
    int64_t rem = E - total;
    if (rem > 0) {
        qsort(fr, (size_t)N, sizeof(frac_item), cmp_frac_desc);
        for (int64_t i = 0; i < rem && i < N; ++i) deg[fr[i].id] += 1;
    }
    free(fr);
    free(x);
}

/* ------------------------------------------------------------------------ */
/* Batched molecule-like graphs                                              */
/* ------------------------------------------------------------------------ */

/*
 * ngraphs small graphs, node counts uniform on [nmin, nmax].  Each is a random
 * recursive tree (node i joins a uniform earlier node) plus round_half_up(n/10)
 * extra edges between uniform non-adjacent distinct pairs.  Every undirected
 * edge is stored in both directions; graphs are offset into one block-diagonal
 * graph.  With src == NULL only the sizes are returned in *N_out and *E_out.
 */
void gtgen_molecules(uint64_t seed, uint64_t stream, int64_t ngraphs, int64_t nmin, int64_t nmax, int64_t* N_out,
                     int64_t* E_out, int32_t* src, int32_t* dst) {
    uint64_t key = stream_key(seed, stream);
    uint64_t ctr = 0;
    int64_t nbase = 0, e = 0;
    uint8_t* adj = (uint8_t*)malloc((size_t)(nmax * nmax));
    for (int64_t g = 0; g < ngraphs; ++g) {
        int64_t n = nmin + (int64_t)below(draw(key, ctr++), (uint64_t)(nmax - nmin + 1));
        memset(adj, 0, (size_t)(n * n));
        for (int64_t i = 1; i < n; ++i) {
            int64_t p = (int64_t)below(draw(key, ctr++), (uint64_t)i);
            adj[p * n + i] = adj[i * n + p] = 1;
            if (src) {
                src[e] = (int32_t)(nbase + p); dst[e] = (int32_t)(nbase + i); ++e;
                src[e] = (int32_t)(nbase + i); dst[e] = (int32_t)(nbase + p); ++e;
            } else {
                e += 2;
            }
        }
        int64_t extra = (n + 5) / 10; /* round_half_up(n / 10) */
        int64_t possible = n * (n - 1) / 2 - (n - 1);
        if (extra > possible) extra = possible;
        for (int64_t k = 0; k < extra;) {
            int64_t a = (int64_t)below(draw(key, ctr++), (uint64_t)n);
            int64_t b = (int64_t)below(draw(key, ctr++), (uint64_t)n);
            if (a == b || adj[a * n + b]) continue;
            adj[a * n + b] = adj[b * n + a] = 1;
            if (src) {
                src[e] = (int32_t)(nbase + a); dst[e] = (int32_t)(nbase + b); ++e;
                src[e] = (int32_t)(nbase + b); dst[e] = (int32_t)(nbase + a); ++e;
            } else {
                e += 2;
            }
            ++k;
        }
        nbase += n;
    }
    free(adj);
    *N_out = nbase;
    *E_out = e;
}
