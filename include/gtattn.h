/*
 * gtattn.h -- C ABI of libgtattn: sparse multi-head graph attention on one
 * AMD Instinct MI355X (gfx950): the fused forward and its unfused stages, the
 * backward, logit options (bias, edge weights, dropout), the head-innermost
 * feature layout, and graph construction and plans on the device.
 *
 * The operation.  For a directed graph stored as a destination-sorted CSR and
 * per-node features Q, K, V of H heads x D dims, every edge u->v and head h
 * gets the score
 *
 *     s = <Q[v,h,:], K[u,h,:]> / sqrt(D)
 *
 * (an SDDMM: scores are computed only where the adjacency matrix is nonzero);
 * the scores of each destination's in-edges are normalised by a softmax,
 *
 *     alpha = exp(s - m) / sum exp(s' - m),   m = max over the in-edges of v,
 *
 * and the output is the alpha-weighted sum of the source rows of V (an SpMM):
 *
 *     out[v,h,:] = sum over in-edges u->v of alpha * V[u,h,:].
 *
 * Sources: "Graph Transformer in a Nutshell" (DGL sparse-matrix tutorial),
 * section "Sparse Multi-head Attention" (SparseAttn equation; batched SDDMM,
 * sparse softmax and SpMM over heads); the gist "Efficient Sparse Transformer
 * implementation with DGL's builtin operators", TransLayer.forward (u_dot_v,
 * edge_softmax of e / sqrt(d_qkv), u_mul_e_sum, features viewed as (N, h, d));
 * the blog "Graph Transformer theory, derivation and implementation",
 * scaled dot-product attention review (per-node e_ij, alpha_ij, h_i).
 *
 * Conventions fixed here where the pages leave them open:
 *  - the softmax of a destination runs over its in-edges only (off-graph
 *    pairs take no part: a logit of -inf, not 0);
 *  - every stored edge is its own term, so a duplicated edge counts twice;
 *  - a destination with no in-edges gets out = 0 (the empty sum);
 *  - the d under the square root is the per-head dimension D.
 *
 * Layouts (all arrays dense, row-major, no padding):
 *  - indptr  int64[N+1], indptr[0] = 0, indptr[N] = E, non-decreasing;
 *  - indices int32[E]: indices[e] in [0, N) is the SOURCE of edge e, whose
 *    destination is the row v with indptr[v] <= e < indptr[v+1];
 *  - Q, K, V, out: [N][H][D], D contiguous, element type given by dtype;
 *  - scores, alpha: float32 [E][H], in CSR edge order.
 *
 * Pointers.  Every array pointer is a DEVICE pointer on the current HIP
 * device, allocated and owned by the caller, who keeps it alive until the
 * work enqueued on `stream` has finished.  The library keeps no caller
 * pointer after a call returns.  It owns its internal scratch (work lists
 * and the partial results of split rows): one buffer per (device, stream),
 * grown on demand in the stream's order (the old buffer released with
 * hipFreeAsync and the new one taken with hipMallocAsync on that stream,
 * from the device's default memory pool), so no call waits for the device.
 * The buffer stays allocated until gt_scratch_release.
 *
 * Execution.  Calls enqueue kernels on `stream` (NULL = the null stream) and
 * return without waiting for them; gt_validate_csr is the exception.  Every
 * element of every output is written, including the zeros of destinations
 * without in-edges, so outputs need no clearing.  Results are deterministic:
 * two calls on the same inputs give bit-identical outputs.  Calls on
 * different streams may run concurrently, from any host threads.  Calls on
 * one stream share its scratch and must not be made from several host
 * threads at once: one call growing the buffer would free it under another
 * call that is still enqueuing work on it.
 *
 * Graph capture.  The compute calls without a plan (gt_sparse_mha_fwd*,
 * gt_sparse_mha_bwd*, gt_sddmm, gt_edge_softmax, gt_spmm) enqueue kernels
 * only: no memset, no host synchronisation, no event.  They may be captured
 * into a HIP graph once the capturing stream's scratch is large enough, which
 * one call of the same size on that stream before the capture ensures (else
 * the capture would record the scratch's allocation).  The graph then replays
 * with the results of the eager calls, bit for bit.  gt_sparse_mha_fwd_noalloc
 * needs no warm-up.  Calls on a plan record an event for the plan's release
 * and are not for capture.
 *
 * Errors.  Arguments are checked before anything is enqueued; on a non-OK
 * status nothing was launched.  No exception or abort crosses the ABI.
 *  GT_EINVAL       a NULL array with N > 0 (or E > 0 for indices/scores/
 *                  alpha), N < 0, E < 0, H < 1, D < 1, N >= 2^31, or an
 *                  invalid configuration value;
 *  GT_EUNSUPPORTED an unknown dtype, H > 64 or D > 256;
 *  GT_ENOMEM       the scratch buffer (or a plan) could not be allocated;
 *                  also every allocation while the environment variable
 *                  GT_TEST_FAIL_ALLOC is set to a value other than "" or
 *                  "0" (a test hook: the call returns before any HIP call);
 *  GT_EHIP         a HIP runtime or launch error (gt_last_error() has it).
 * Special sizes: N = 0 is a no-op returning GT_OK; E = 0 writes zeros.
 * The CSR's contents are not checked on the hot path (a malformed CSR is
 * undefined behaviour); gt_validate_csr checks them for tests and debugging.
 * Non-finite inputs are outside the contract.
 */
#ifndef GTATTN_H
#define GTATTN_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and out.  bf16 inputs are accumulated in fp32 and
 * the bf16 output is rounded to nearest-even.  scores/alpha are always fp32. */
typedef enum { GT_F32 = 0, GT_BF16 = 1 } gt_dtype;

typedef enum { GT_OK = 0, GT_EINVAL = 1, GT_EUNSUPPORTED = 2, GT_ENOMEM = 3, GT_EHIP = 4 } gt_status;

/*
 * Fused forward: out = SpMM(edge_softmax(SDDMM(Q, K))) in one pass over the
 * edges; the E x H score and weight arrays never reach memory.  Follows the
 * SparseMHA forward of "Graph Transformer in a Nutshell" (bsddmm, softmax,
 * bspmm) and TransLayer.forward of the DGL builtin-operator gist.
 */
int gt_sparse_mha_fwd(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                      void* out, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream);

/*
 * gt_sparse_mha_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and result, with no hipMalloc, hipFree or
 * other allocating call.  The split-row work lists and partial results go to
 * a file-scope device array of 160 MiB, which every GPU the library runs on
 * holds until the process ends, instead of the per-stream scratch.  The split
 * threshold (gt_config_chunk_edges) is doubled, up to 64 times, until the
 * work lists and partials fit; while it is unchanged, out is bit-identical to
 * gt_sparse_mha_fwd's (at the automatic threshold and 16 in-edges per node on
 * average: up to about 70M edges for 8 heads of 64 features, 120M for 8 heads
 * of 32; each doubling about doubles that).  Inputs that do not fit
 * even at 64 times the threshold return GT_EUNSUPPORTED, before anything is
 * enqueued (gt_last_error() gives the bytes needed).  All calls on one GPU
 * share the array, which keeps the last call's contents; nothing in it needs
 * clearing (each call resets its work-list counters with a kernel).  Calls
 * that overlap on one GPU (several streams, or several host threads) race
 * for the array: the caller must order them.
 */
int gt_sparse_mha_fwd_noalloc(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K,
                              const void* V, void* out, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                              hipStream_t stream);

/*
 * Fused forward that also saves, for the backward, the natural-log
 * log-sum-exp of every destination's scores:
 *     lse[v][h] = log sum over in-edges of exp(s)    (float32 [N][H]),
 * -inf for a destination without in-edges.  out is as gt_sparse_mha_fwd's,
 * bit for bit.  GT_EINVAL also for a NULL lse with N > 0.
 */
int gt_sparse_mha_fwd_lse(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                          void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                          hipStream_t stream);

/*
 * Backward of the fused forward: the gradients that loss.backward() takes
 * through bsddmm, softmax and bspmm in the training loop of "Graph
 * Transformer in a Nutshell" (section "Training").  With alpha recomputed as
 * exp(s - lse) and dout = dL/dout, per edge e = (u -> v) and head h:
 *     delta[v] = <dout[v], out[v]>,  ds_e = alpha_e (<dout[v], V[u]> - delta[v])
 *     dQ[v] = sum over in-edges of ds_e K[u] / sqrt(D)
 *     dK[u] = sum over out-edges of ds_e Q[v] / sqrt(D)
 *     dV[u] = sum over out-edges of alpha_e dout[v]
 * (the chain rule through the row softmax, whose Jacobian is
 * diag(alpha) - alpha alpha^T).
 * Inputs: the destination-sorted CSR (indptr, indices) of the forward and the
 * same graph sorted by source, t_indptr int64[N+1] / t_indices int32[E]
 * holding the DESTINATION of each out-edge (the transpose; duplicated edges
 * appear as often as in the forward); Q, K, V, out and lse as the forward
 * took and left them; dout [N][H][D].  Outputs dQ, dK, dV [N][H][D], every
 * element written (zeros for nodes without in- or out-edges).  All feature
 * arrays share dtype; accumulation is fp32.  The transpose is trusted like
 * the CSR: that it matches (indptr, indices) is not checked.  No atomics:
 * results are deterministic.  Scratch: the per-stream buffer also holds,
 * per (destination, head), delta and lse in the base-2 scale (two floats,
 * 8 * N * H bytes).  Errors as for gt_sparse_mha_fwd.
 */
int gt_sparse_mha_bwd(const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr, const int32_t* t_indices,
                      const void* Q, const void* K, const void* V, const void* out, const void* dout, const float* lse,
                      void* dQ, void* dK, void* dV, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                      hipStream_t stream);

/*
 * SDDMM stage: scores[e][h] = <Q[v,h,:], K[u_e,h,:]> / sqrt(D) for every edge
 * e = (u_e -> v).  The DGL gist's u_dot_v (source key with destination query)
 * followed by its division by sqrt(d_qkv); the tutorial's bsddmm.
 */
int gt_sddmm(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, float* scores, int64_t N,
             int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream);

/*
 * Edge-softmax stage: alpha[e][h] = exp(scores[e][h] - m) / sum exp(scores[e'][h] - m)
 * over the in-edges e' of e's destination, m their maximum.  The gist's
 * edge_softmax, normalised per destination; the tutorial's sparse softmax.
 * alpha may equal scores (in place).
 */
int gt_edge_softmax(const int64_t* indptr, const float* scores, float* alpha, int64_t N, int64_t E, int32_t H,
                    hipStream_t stream);

/*
 * SpMM stage: out[v,h,:] = sum over in-edges e of v of alpha[e][h] * V[u_e,h,:],
 * zero for destinations without in-edges.  The gist's u_mul_e_sum; the
 * tutorial's bspmm.  alpha need not be normalised.
 */
int gt_spmm(const int64_t* indptr, const int32_t* indices, const float* alpha, const void* V, void* out, int64_t N,
            int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream);

/*
 * Checks a CSR on the device: indptr[0] == 0, indptr[N] == E, indptr
 * non-decreasing, every index in [0, N).  Synchronises `stream`.  Returns
 * GT_OK for a valid graph, GT_EINVAL otherwise (gt_last_error() says what).
 */
int gt_validate_csr(const int64_t* indptr, const int32_t* indices, int64_t N, int64_t E, hipStream_t stream);

/*
 * Logit variants and attention dropout.
 *  - bias (float32 [E][H], CSR edge order, or NULL) is added to each logit:
 *    the shortest-path bias of "Graph Transformer theory, derivation and
 *    implementation" (section on the Graphormer-type shortest-path bias and
 *    degree encoding: a learnable scalar added to e_ij), or any other
 *    relative encoding given per edge and head;
 *  - edge_weight (float32 [E], or NULL) multiplies the scaled dot product:
 *    A's values in the Hadamard product (QK^T) o A / sqrt(d) of "Graph
 *    Transformer in a Nutshell" (section "Sparse Multi-head Attention").
 *    The softmax still runs over the stored edges only;
 *  - dropout_p in [0, 1): the drop_att of the gist's TransLayer.forward in
 *    training.  Each weight alpha[e][h] is zeroed with probability p and the
 *    kept ones are divided by 1 - p; the normaliser is the full softmax's.
 *    Keep decisions come from the counter-based generator Philox4x64-10
 *    (Salmon et al., SC 2011) under key (dropout_seed, 0): word i = e*H + h
 *    is word i mod 4 of counter block (i/4 + 1, 0, 0, 0) (the stream of
 *    numpy.random.Philox(key=(seed, 0))), and the weight is kept iff the
 *    word's upper 32 bits are >= floor(p * 2^32) (so p < 2^-32 drops
 *    nothing and no 1/(1 - p) is applied).  The same seed gives the same
 *    mask in the forward and the backward.
 * So s[e][h] = edge_weight[e] * <Q[v,h,:], K[u,h,:]> / sqrt(D) + bias[e][h].
 */
typedef struct {
    const float* bias;
    const float* edge_weight;
    double dropout_p;
    uint64_t dropout_seed;
} gt_logit_opts;

/* gt_sparse_mha_fwd_lse with options (opts NULL: none; lse may be NULL). */
int gt_sparse_mha_fwd_ex(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                         void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                         const gt_logit_opts* opts, hipStream_t stream);

/*
 * gt_sparse_mha_bwd with options.  With c_e the dropout multiplier (0 or
 * 1/(1 - p)) and w_e the edge weight: ds_e = alpha_e (c_e <dout[v], V[u]> -
 * delta[v]); dQ and dK sums carry w_e; dV[u] sums alpha_e c_e dout[v].
 * Optional outputs: dbias (float32 [E][H], = ds) and dweight (float32 [E],
 * = sum over heads of ds <Q[v], K[u]> / sqrt(D)).  t_perm (int32[E]) gives,
 * for each entry of the transpose, its position in the CSR; it is required
 * (GT_EINVAL) when bias, edge weights or dropout are on.
 */
int gt_sparse_mha_bwd_ex(const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr,
                         const int32_t* t_indices, const int32_t* t_perm, const void* Q, const void* K, const void* V,
                         const void* out, const void* dout, const float* lse, void* dQ, void* dK, void* dV,
                         float* dbias, float* dweight, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                         const gt_logit_opts* opts, hipStream_t stream);

/*
 * Feature layouts.  GT_LAYOUT_NHD: [N][H][D], D contiguous (the gist's
 * (N, h, d) view; every other entry point).  GT_LAYOUT_NDH: [N][D][H], head
 * innermost, as "Graph Transformer in a Nutshell" reshapes q, k, v to
 * [N, dh, nh] in SparseMHA.forward.  The layout applies to Q, K, V, out,
 * dout, dQ, dK and dV; lse, bias and the other arrays are unchanged.
 * gt_sparse_mha_fwd_layout / gt_sparse_mha_bwd_layout are gt_sparse_mha_fwd_ex
 * / gt_sparse_mha_bwd_ex with a layout argument (GT_EINVAL for an unknown
 * one).  For GT_LAYOUT_NDH, without logit options (and without dbias /
 * dweight), kernels of their own serve shapes where H is a multiple of the
 * 16-byte vector (4 fp32 or 8 bf16 elements) with a power-of-two quotient and
 * a row fits 256 vectors (4 KB), when they are the faster route: always when
 * [N][H][D] rows would take one wave per head (heads neither whole 16-byte
 * vectors nor whole 8- or 4-byte words of at most 32 per head, 64 per row);
 * for heads of whole words (fp32 D = 10) the forward always and the backward
 * below 65,536 edges, where the copies' launches cost more than the
 * cross-lane sums this layout needs; for heads of 16-byte vectors the forward
 * when a row's gathers are large against those sums.  Everything else goes
 * through [N][H][D] copies in the per-stream scratch (transposed on the
 * device), with results bit-identical to the [N][H][D] calls.
 *
 * (The tutorial also normalises along A[src, dst]'s rows, i.e. over each
 * source's out-edges with the source's query: that is these calls on the
 * transposed graph, e.g. a plan built from (dst, src) pairs.)
 */
typedef enum { GT_LAYOUT_NHD = 0, GT_LAYOUT_NDH = 1 } gt_layout;
int gt_sparse_mha_fwd_layout(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K,
                             const void* V, void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D,
                             int32_t dtype, int32_t layout, const gt_logit_opts* opts, hipStream_t stream);
int gt_sparse_mha_bwd_layout(const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr,
                             const int32_t* t_indices, const int32_t* t_perm, const void* Q, const void* K,
                             const void* V, const void* out, const void* dout, const float* lse, void* dQ, void* dK,
                             void* dV, float* dbias, float* dweight, int64_t N, int64_t E, int32_t H, int32_t D,
                             int32_t dtype, int32_t layout, const gt_logit_opts* opts, hipStream_t stream);

/*
 * Graph construction on the device.  "Graph Transformer in a Nutshell",
 * section "Graph Transformer Model": GTModel.forward stacks the (src, dst)
 * pairs of g.edges() into one sparse adjacency matrix and hands it to every
 * layer.  These calls build that structure once, on the GPU, in the forms the
 * attention needs; results are unique (stable grouping) and deterministic.
 *
 * gt_coo_to_csr: COO edge arrays src, dst (int32[E], edge i = src[i] ->
 * dst[i]) to the destination-sorted CSR: indptr int64[n_dst + 1], indices
 * int32[E] (sources), each row's edges in COO order; perm (nullable) int32[E]
 * gets the COO id of the edge at each CSR position.  Ids must lie in
 * [0, n_src) and [0, n_dst); ids outside give an unspecified (but in-bounds)
 * result, which gt_validate_csr detects.  GT_EUNSUPPORTED for E >= 2^31.
 * Uses the per-stream scratch; asynchronous.
 */
int gt_coo_to_csr(const int32_t* src, const int32_t* dst, int64_t n_dst, int64_t n_src, int64_t E, int64_t* indptr,
                  int32_t* indices, int32_t* perm, hipStream_t stream);

/*
 * A plan: a graph prepared once and reused by every layer and step.  It owns
 * device copies of the destination-sorted CSR (n_dst rows whose in-edges come
 * from n_src source nodes), with GT_PLAN_TRANSPOSE also the source-sorted
 * graph that the backward needs (t_indptr int64[n_src + 1], t_indices
 * int32[E] holding destinations, each source's out-edges in CSR order, and
 * t_perm int32[E], the CSR position of each of those out-edges), and
 * the list of rows split into chunks (at the split threshold current when
 * the plan is built).  n_src != n_dst describes a shard of destination rows
 * whose sources index a larger K/V: Q, out, lse, dout, dQ have n_dst rows;
 * K, V, dK, dV have n_src rows.
 *
 * gt_plan_create copies a caller CSR; gt_plan_create_coo builds it from COO
 * arrays as gt_coo_to_csr does.  Both allocate the plan's device memory with
 * hipMallocAsync on `stream` (so they are not for graph capture), enqueue
 * the construction on `stream` and return without waiting: the plan is ready
 * for work on `stream`, and for other streams once they are ordered after
 * it.  The library keeps no caller pointer.  Every call on a plan records an
 * event on its stream; gt_plan_destroy releases the plan's memory in stream
 * order behind all of them (the null stream waits for those events, then
 * hipFreeAsync), without waiting on the host.  Work of the caller's own that
 * reads arrays taken from gt_plan_info must therefore be finished, or be
 * enqueued before a library call on the plan on the same stream, when the
 * plan is destroyed; and since the release goes on the null stream,
 * gt_plan_destroy must not be called while a stream capture is under way.
 * gt_plan_info returns the plan's sizes and device arrays (owned by the
 * plan; t_* are NULL without GT_PLAN_TRANSPOSE); any output pointer may be
 * NULL.  gt_plan_copy_graph
 * copies the plan's graph into caller device arrays of those sizes (any may
 * be NULL; asking for t_* of a plan without a transpose is GT_EINVAL),
 * enqueued on `stream`.
 * Errors: GT_EINVAL for negative sizes, node counts >= 2^31, NULL arrays or
 * unknown flags; GT_EUNSUPPORTED for E >= 2^31 or too many chunks; GT_ENOMEM.
 */
typedef struct gt_plan_s* gt_plan;
typedef enum { GT_PLAN_TRANSPOSE = 1 } gt_plan_flags;
int gt_plan_create(const int64_t* indptr, const int32_t* indices, int64_t n_dst, int64_t n_src, int64_t E,
                   int32_t flags, hipStream_t stream, gt_plan* plan);
int gt_plan_create_coo(const int32_t* src, const int32_t* dst, int64_t n_dst, int64_t n_src, int64_t E,
                       int32_t flags, hipStream_t stream, gt_plan* plan);
int gt_plan_destroy(gt_plan plan);
int gt_plan_info(gt_plan plan, int64_t* n_dst, int64_t* n_src, int64_t* E, const int64_t** indptr,
                 const int32_t** indices, const int64_t** t_indptr, const int32_t** t_indices,
                 const int32_t** t_perm);
int gt_plan_copy_graph(gt_plan plan, int64_t* indptr, int32_t* indices, int64_t* t_indptr, int32_t* t_indices,
                       int32_t* t_perm, hipStream_t stream);

/*
 * gt_sparse_mha_fwd_ex / gt_sparse_mha_bwd_ex on a plan: the same kernels
 * and results (bit for bit, for the same graph and split threshold), without
 * rebuilding the split-row list each call.  lse, opts, dbias and dweight may
 * be NULL.
 * The backward needs a plan built with GT_PLAN_TRANSPOSE (GT_EINVAL
 * otherwise).  The plan must belong to the current device.
 */
int gt_sparse_mha_fwd_plan(gt_plan plan, const void* Q, const void* K, const void* V, void* out, float* lse,
                           int32_t H, int32_t D, int32_t dtype, const gt_logit_opts* opts, hipStream_t stream);
int gt_sparse_mha_bwd_plan(gt_plan plan, const void* Q, const void* K, const void* V, const void* out,
                           const void* dout, const float* lse, void* dQ, void* dK, void* dV, float* dbias,
                           float* dweight, int32_t H, int32_t D, int32_t dtype, const gt_logit_opts* opts,
                           hipStream_t stream);

/*
 * Measurement aid, not part of the attention: the achievable rate of its
 * gathers.  In "Graph Transformer in a Nutshell", section "Sparse Multi-head
 * Attention", every nonzero (v, u) of the adjacency matrix reads row u of K
 * (SDDMM) and row u of V (SpMM).  gt_calib_gather reads exactly those rows
 * for the E edges of `indices` (int32 [E], values in [0, n_rows)), in CSR
 * order, with the 16-byte loads and lane layout of the fused kernel, and
 * does nothing else with them.  Every 32-bit word read is XOR-folded into
 * *checksum (device memory owned by the caller, who sets it beforehand; 0
 * for the checksum alone), so the result is the XOR over edges of the words
 * of rows K[u] and V[u] and shows that each row was read whole.  K and V are
 * n_rows rows of row_bytes bytes (512, 1024 or 2048: for example bf16 8 x 32,
 * fp32 8 x 32, fp32 8 x 64), 16-byte aligned.  Asynchronous on `stream`.
 * GT_EUNSUPPORTED for another row size or misaligned K or V, GT_EINVAL for
 * negative sizes or a NULL array with E > 0.  Index values are not checked.
 */
int gt_calib_gather(const int32_t* indices, int64_t E, const void* K, const void* V, int64_t n_rows,
                    int32_t row_bytes, uint32_t* checksum, hipStream_t stream);

/* Static text for a status code. */
const char* gt_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* gt_last_error(void);

/*
 * Tuning and testing knobs, process-wide, read at each call.
 *  GT_CFG_CHUNK_EDGES  rows with more in-edges than this are split into
 *                      chunks of this many edges, processed in parallel and
 *                      merged exactly (valid 1 .. 2^30; 0, the default, for
 *                      automatic: 2,048 edges on graphs of 2^23 edges or
 *                      more, 512 on smaller graphs and in gt_edge_softmax).
 * gt_config_set returns GT_EINVAL for an unknown key or an invalid value;
 * gt_config_get returns the configured value (-1 for an unknown key).
 * gt_config_chunk_edges returns the threshold a call on a graph of E edges
 * uses, the configured one or the automatic one (softmax != 0: that of
 * gt_edge_softmax); -1 for E < 0.  The threshold changes results only in
 * the order of rounding; since the automatic one depends on E, a shard of a
 * graph (or a batch of a different size) can take another threshold than the
 * whole graph: configure one where the two must agree bit for bit.
 */
typedef enum { GT_CFG_CHUNK_EDGES = 0 } gt_config_key;
int gt_config_set(int32_t key, int64_t value);
int64_t gt_config_get(int32_t key);
int64_t gt_config_chunk_edges(int64_t E, int32_t softmax);

/*
 * The scratch buffer of `stream` on the current device: gt_scratch_release
 * releases it in the stream's order (hipFreeAsync on `stream`, after the
 * work already enqueued there) and forgets it (the next call on the stream
 * allocates afresh); GT_OK also when the stream has none.  Call it before
 * destroying a stream that the library has used, or to return the memory
 * (up to 8 feature arrays' worth for the head-innermost backward).
 * gt_scratch_bytes gives the buffer's current size (0 if none, -1 if the
 * current device cannot be read).  The same threading rule as for the other
 * calls on a stream applies.
 */
int gt_scratch_release(hipStream_t stream);
int64_t gt_scratch_bytes(hipStream_t stream);

/*
 * Kernel timing for measurement.  gt_profile_begin(capacity) makes the next
 * `capacity` calls of gt_sparse_mha_fwd record HIP events, on the stream they
 * launch on, around their attention kernels (the fused kernel and the merge
 * of split rows, which writes those rows' outputs) and around the whole call
 * (with the work-list kernel).  gt_profile_end waits for those events and
 * returns the summed kernel time,
 * the summed call time (milliseconds) and the number of calls recorded, then
 * stops recording.  Not for concurrent use from several threads.
 */
int gt_profile_begin(int32_t capacity);
int gt_profile_end(double* kernel_ms, double* call_ms, int64_t* calls);

#ifdef __cplusplus
}
#endif

#endif /* GTATTN_H */
