// plan.hip -- device-side work list (heavy rows and their chunks) and the
// CSR validity check.
#include <algorithm>

#include "kernels.hpp"

namespace gt {

__global__ void reset_kernel(PlanCounters* c) {
    if (threadIdx.x < 64) reinterpret_cast<uint32_t*>(c)[threadIdx.x] = 0;
}

// A row with more than `chunk` in-edges gets a slot in the heavy-row list and
// a contiguous range of chunk item ids; the chunk table maps each id back to
// (row, chunk index, heavy slot).  Every other row goes into the row order, by
// degree bin (order_bin), each bin's rows in index order within a block.
// Slot and block order depend on scheduling, but no result does: each row and
// chunk is computed on its own, and the merges read a row's chunks in chunk
// order.  A block takes kPlanThreads * kPlanRows consecutive rows (each thread
// kPlanRows consecutive ones), adds up its heavy rows, chunks and bin counts
// with a block-wide prefix scan and takes its ranges with one atomic per
// counter.  The counters are hot words that every block updates at the
// coherent memory side, so the fewer the atomics the better.  A graph of at
// most kPlanBlockRows rows goes to plan_small_kernel instead: one block, no
// reset launch, no row order.
constexpr int kPlanThreads = 1024;
constexpr int kPlanRows = 8;
static_assert((int64_t)kPlanThreads * kPlanRows == kPlanBlockRows, "one plan block's rows");
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanCounts = 2 + kOrderBins;  // heavy rows, chunks, rows of each bin

// The degrees of the thread's rows (-1 past the end).
__device__ __forceinline__ void plan_degrees(const int64_t* __restrict__ indptr, int64_t N, int64_t v0,
                                             int64_t (&deg)[kPlanRows]) {
    int64_t ip[kPlanRows + 1];
#pragma unroll
    for (int k = 0; k <= kPlanRows; ++k) ip[k] = v0 + k <= N ? indptr[v0 + k] : 0;
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) deg[k] = v0 + k < N ? ip[k + 1] - ip[k] : -1;
}

// Exclusive block-wide prefix of the thread's counts: out[i] is the sum of
// cnt[i] over the threads before this one; tot[i] the block's total.
__device__ __forceinline__ void block_prefix(const uint32_t (&cnt)[kPlanCounts], uint32_t (&out)[kPlanCounts],
                                             uint32_t (&tot)[kPlanCounts], uint32_t (*s_w)[kPlanCounts]) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    uint32_t inc[kPlanCounts];
#pragma unroll
    for (int i = 0; i < kPlanCounts; ++i) inc[i] = cnt[i];
    for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
        for (int i = 0; i < kPlanCounts; ++i) {
            const uint32_t x = __shfl_up(inc[i], off, kWave);
            if (lane >= off) inc[i] += x;
        }
    }
    if (lane == kWave - 1)
#pragma unroll
        for (int i = 0; i < kPlanCounts; ++i) s_w[wid][i] = inc[i];
    __syncthreads();
    if (threadIdx.x < kPlanCounts) {  // exclusive prefix over the waves, kept in place; the total at the end
        const int i = threadIdx.x;
        uint32_t t = 0;
        for (int w = 0; w < kPlanWaves; ++w) {
            const uint32_t c = s_w[w][i];
            s_w[w][i] = t;
            t += c;
        }
        s_w[kPlanWaves][i] = t;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPlanCounts; ++i) {
        out[i] = s_w[wid][i] + inc[i] - cnt[i];
        tot[i] = s_w[kPlanWaves][i];
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int64_t* __restrict__ indptr, int64_t N, Plan p) {
    __shared__ uint32_t s_w[kPlanWaves + 1][kPlanCounts], s_base[kPlanCounts];
    const int64_t v0 = ((int64_t)blockIdx.x * kPlanThreads + threadIdx.x) * kPlanRows;
    int64_t deg[kPlanRows];
    plan_degrees(indptr, N, v0, deg);
    uint32_t nch[kPlanRows], cnt[kPlanCounts];
#pragma unroll
    for (int i = 0; i < kPlanCounts; ++i) cnt[i] = 0;
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        nch[k] = deg[k] > p.chunk ? (uint32_t)((deg[k] + p.chunk - 1) / p.chunk) : 0u;
        cnt[0] += nch[k] ? 1u : 0u;
        cnt[1] += nch[k];
        if (deg[k] >= 0 && !nch[k])
#pragma unroll
            for (int b = 0; b < kOrderBins; ++b) cnt[2 + b] += order_bin(deg[k]) == b ? 1u : 0u;
    }
    uint32_t pre[kPlanCounts], tot[kPlanCounts];
    block_prefix(cnt, pre, tot, s_w);
    if (threadIdx.x < kPlanCounts) {
        const int i = threadIdx.x;
        uint32_t* ctr = i == 0 ? &p.counters->nheavy : i == 1 ? &p.counters->nchunks : &p.counters->bin_total[i - 2];
        s_base[i] = tot[i] && i < 2 ? atomicAdd(ctr, tot[i]) : 0u;
        if (i >= 2 && tot[i]) atomicAdd(ctr, tot[i]);
    }
    __syncthreads();
    uint32_t hs = s_base[0] + pre[0];
    uint32_t cb = s_base[1] + pre[1];
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        if (deg[k] < 0 || !nch[k]) continue;
        const int32_t v = (int32_t)(v0 + k);
        // a valid CSR never trips this (the host sizes both tables for it); a
        // malformed one must not write past them
        if ((int64_t)hs >= p.max_heavy || (int64_t)cb + nch[k] > p.max_chunks) return;
        p.heavy[hs] = HeavyRow{v, (int32_t)nch[k], (int64_t)cb};
        for (uint32_t i = 0; i < nch[k]; ++i) p.chunks[cb + i] = ChunkRef{v, (int32_t)i, (int32_t)hs, 0};
        ++hs;
        cb += nch[k];
    }
}

// Graphs of at most one plan block of rows: one block lists the heavy rows
// and their chunks, taking slots with LDS atomics, and leaves the rows in
// index order.  Small graphs gained nothing from the degree order, and the
// block-wide scan the order needs cost more than the attention it plans for
// (a 4k-row molecule batch: 8.0 us of plan for 4.4 us of fused kernel).
// Slot order depends on scheduling; no result does.
__global__ __launch_bounds__(kPlanThreads) void plan_small_kernel(const int64_t* __restrict__ indptr, int64_t N,
                                                                  Plan p) {
    __shared__ uint32_t s_heavy, s_chunks, s_bad;
    if (threadIdx.x == 0) s_heavy = s_chunks = s_bad = 0u;
    int64_t deg[kPlanRows];  // rows k * kPlanThreads + thread: coalesced loads, all issued up front
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        const int64_t v = (int64_t)k * kPlanThreads + threadIdx.x;
        deg[k] = v < N ? indptr[v + 1] - indptr[v] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        if (deg[k] <= p.chunk) continue;
        const int32_t v = (int32_t)(k * kPlanThreads + threadIdx.x);
        const uint32_t nch = (uint32_t)((deg[k] + p.chunk - 1) / p.chunk);
        const uint32_t hs = atomicAdd(&s_heavy, 1u);
        const uint32_t cb = atomicAdd(&s_chunks, nch);
        // a valid CSR never trips this (the host sizes both tables for it); a
        // malformed one must not write past them, and then lists nothing
        if ((int64_t)hs >= p.max_heavy || (int64_t)cb + nch > p.max_chunks) {
            s_bad = 1u;
            continue;
        }
        p.heavy[hs] = HeavyRow{v, (int32_t)nch, (int64_t)cb};
        for (uint32_t i = 0; i < nch; ++i) p.chunks[cb + i] = ChunkRef{v, (int32_t)i, (int32_t)hs, 0};
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        p.counters->nheavy = s_bad ? 0u : s_heavy;
        p.counters->nchunks = s_bad ? 0u : s_chunks;
    }
}

// Several blocks: the row order, once plan_kernel has counted every bin.
// Each block places its rows of bin b at the bin's start (the rows of the
// longer bins) plus what the blocks before it in this launch placed.
__global__ __launch_bounds__(kPlanThreads) void order_kernel(const int64_t* __restrict__ indptr, int64_t N, Plan p) {
    __shared__ uint32_t s_w[kPlanWaves + 1][kPlanCounts], s_base[kPlanCounts];
    const int64_t v0 = ((int64_t)blockIdx.x * kPlanThreads + threadIdx.x) * kPlanRows;
    int64_t deg[kPlanRows];
    plan_degrees(indptr, N, v0, deg);
    uint32_t cnt[kPlanCounts];
#pragma unroll
    for (int i = 0; i < kPlanCounts; ++i) cnt[i] = 0;
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k)
        if (deg[k] >= 0 && deg[k] <= p.chunk)
#pragma unroll
            for (int b = 0; b < kOrderBins; ++b) cnt[2 + b] += order_bin(deg[k]) == b ? 1u : 0u;
    uint32_t pre[kPlanCounts], tot[kPlanCounts];
    block_prefix(cnt, pre, tot, s_w);
    if (threadIdx.x < kOrderBins) {
        const int b = threadIdx.x;
        uint32_t start = 0;
        for (int c = 0; c < b; ++c) start += p.counters->bin_total[c];
        s_base[2 + b] = start + (tot[2 + b] ? atomicAdd(&p.counters->bin_cursor[b], tot[2 + b]) : 0u);
    }
    __syncthreads();
    uint32_t ob[kOrderBins];
#pragma unroll
    for (int b = 0; b < kOrderBins; ++b) ob[b] = s_base[2 + b] + pre[2 + b];
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        if (deg[k] < 0 || deg[k] > p.chunk) continue;
        const int b = order_bin(deg[k]);
        uint32_t pos = 0;
#pragma unroll
        for (int c = 0; c < kOrderBins; ++c)
            if (c == b) pos = ob[c]++;
        if ((int64_t)pos < p.n_order) p.order[pos] = (int32_t)(v0 + k);
    }
}

hipError_t launch_plan(const Args& a, hipStream_t s) {
    if (a.plan.max_heavy == 0) return hipSuccess;  // no row can be split: nothing to list, rows in index order
    const int64_t per_block = (int64_t)kPlanThreads * kPlanRows;
    const unsigned blocks = (unsigned)((a.N + per_block - 1) / per_block);
    if (blocks == 1) {  // one block sets the counters itself: no reset, no order
        plan_small_kernel<<<1, kPlanThreads, 0, s>>>(a.indptr, a.N, a.plan);
        return hipGetLastError();
    }
    // several blocks add to the counters: clear them first
    reset_kernel<<<1, 64, 0, s>>>(a.plan.counters);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    plan_kernel<<<blocks, kPlanThreads, 0, s>>>(a.indptr, a.N, a.plan);
    err = hipGetLastError();
    if (err != hipSuccess || !a.plan.order) return err;
    order_kernel<<<blocks, kPlanThreads, 0, s>>>(a.indptr, a.N, a.plan);
    return hipGetLastError();
}

// ------------------------------------------------------------ additive merges of split rows
// (the unfused SpMM and both passes of the backward)
// Chunk partials of a heavy row are [chunk][width] with width = regions * HD;
// region r of each is added over the row's chunks, in chunk order, and goes
// to dst_r scaled by scale_r.  A wave per (heavy row, slice of kMergeCols
// columns) at a time; chunks are read kMergeUnroll at a time so that many
// loads are in flight (one wave walks up to E / chunk partials of a hub row).
constexpr int kMergeCols = kWave * 4;
constexpr int kMergeUnroll = 8;

template <int DT>
__global__ __launch_bounds__(kBlock) void sum_merge_kernel(const Args a, int regions, void* dst0, float scale0,
                                                           void* dst1, float scale1) {
    using VT = Vec<DT>;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nheavy = min(a.plan.max_heavy, (int64_t)a.plan.counters->nheavy);
    const int64_t HD = (int64_t)a.H * a.D;
    const int64_t width = HD * regions;
    const int64_t j0 = (int64_t)blockIdx.y * kMergeCols;
    int64_t col[4];
    bool in[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        col[t] = j0 + lane + t * kWave;
        in[t] = col[t] < width;
    }
    for (int64_t hs = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         hs < nheavy; hs += (int64_t)gridDim.x * kWavesPerBlock) {
        const HeavyRow hr = a.plan.heavy[hs];
        const float* pa = a.plan.pacc + hr.base * width;
        float A[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int i0 = 0; i0 < hr.nch; i0 += kMergeUnroll) {
            float x[kMergeUnroll][4];
#pragma unroll
            for (int i = 0; i < kMergeUnroll; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    x[i][t] = (i0 + i < hr.nch && in[t]) ? pa[(int64_t)(i0 + i) * width + col[t]] : 0.0f;
#pragma unroll
            for (int i = 0; i < kMergeUnroll; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t) A[t] += x[i][t];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (!in[t]) continue;
            const int r = col[t] >= HD;  // regions <= 2
            VT::store_scalar(r ? dst1 : dst0, (int64_t)hr.row * HD + col[t] - r * HD, A[t] * (r ? scale1 : scale0));
        }
    }
}

// The grid strides over the heavy rows listed by the plan, capped at
// kMergeGridX blocks in x, as in the forward's merge.
template <int DT>
static hipError_t launch_sum_merge_dt(const Args& a, int regions, void* dst0, float scale0, void* dst1, float scale1,
                                      hipStream_t s) {
    if (a.plan.max_heavy == 0) return hipSuccess;
    const unsigned gx =
        (unsigned)std::min<int64_t>((a.plan.max_heavy + kWavesPerBlock - 1) / kWavesPerBlock, kMergeGridX);
    const unsigned gy = (unsigned)((regions * (int64_t)a.H * a.D + kMergeCols - 1) / kMergeCols);
    sum_merge_kernel<DT><<<dim3(gx, gy), dim3(kBlock), 0, s>>>(a, regions, dst0, scale0, dst1, scale1);
    return hipGetLastError();
}

hipError_t launch_sum_merge(const Args& a, int regions, void* dst0, float scale0, void* dst1, float scale1,
                            hipStream_t s) {
    return a.dtype == kF32 ? launch_sum_merge_dt<kF32>(a, regions, dst0, scale0, dst1, scale1, s)
                           : launch_sum_merge_dt<kBF16>(a, regions, dst0, scale0, dst1, scale1, s);
}

// ------------------------------------------------------------ validation
enum : uint32_t { kBadFirst = 1, kBadLast = 2, kDecreasing = 4, kIndexRange = 8 };

__global__ void clear_flags_kernel(uint32_t* flags) {
    if (threadIdx.x == 0) *flags = 0;
}

__global__ __launch_bounds__(256) void validate_kernel(const int64_t* __restrict__ indptr,
                                                       const int32_t* __restrict__ indices, int64_t N, int64_t E,
                                                       uint32_t* flags) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t f = 0;
    if (t0 == 0) {
        if (indptr[0] != 0) f |= kBadFirst;
        if (indptr[N] != E) f |= kBadLast;
    }
    for (int64_t v = t0; v < N; v += stride)
        if (indptr[v + 1] < indptr[v]) f |= kDecreasing;
    for (int64_t e = t0; e < E; e += stride) {
        const int32_t u = indices[e];
        if (u < 0 || (int64_t)u >= N) f |= kIndexRange;
    }
    if (f) atomicOr(flags, f);
}

hipError_t launch_validate(const int64_t* indptr, const int32_t* indices, int64_t N, int64_t E, uint32_t* flags,
                           hipStream_t s) {
    clear_flags_kernel<<<1, 64, 0, s>>>(flags);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    validate_kernel<<<1024, 256, 0, s>>>(indptr, indices, N, E, flags);
    return hipGetLastError();
}

}  // namespace gt
