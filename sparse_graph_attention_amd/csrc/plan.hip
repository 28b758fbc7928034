// plan.hip -- device-side work list (heavy rows and their chunks) and the
// CSR validity check.
#include <algorithm>

#include "kernels.hpp"

namespace gt {

__global__ void reset_kernel(PlanCounters* c) {
    if (threadIdx.x == 0) {
        c->nheavy = 0;
        c->nchunks = 0;
    }
}

// A row with more than `chunk` in-edges gets a slot in the heavy-row list and
// a contiguous range of chunk item ids; the chunk table maps each id back to
// (row, chunk index, heavy slot).  Slot order depends on scheduling, but each
// chunk's result does not, and the merges read a row's chunks in chunk order,
// so outputs are deterministic.  A block takes kPlanThreads * kPlanRows rows
// (each thread kPlanRows of them, kPlanThreads apart, so that loads
// coalesce), adds up its heavy rows and chunks with a block-wide prefix scan
// and takes its ranges with one atomic per counter.  The counters are hot
// words that every block updates at the coherent memory side, so the fewer
// the atomics the better: one pair per 8,192 rows.  A graph of at most that
// many rows has one block, which writes the counters itself, so small graphs
// need no reset launch before it.
constexpr int kPlanThreads = 1024;
constexpr int kPlanRows = 8;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int64_t* __restrict__ indptr, int64_t N, Plan p) {
    constexpr int kWaves = kPlanThreads / kWave;
    __shared__ uint32_t s_h[kWaves], s_c[kWaves], s_base[2];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const int64_t v0 = (int64_t)blockIdx.x * kPlanThreads * kPlanRows + threadIdx.x;
    uint32_t nch[kPlanRows];
    uint32_t hcnt = 0, ccnt = 0;
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        const int64_t v = v0 + (int64_t)k * kPlanThreads;
        const int64_t deg = v < N ? indptr[v + 1] - indptr[v] : 0;
        nch[k] = deg > p.chunk ? (uint32_t)((deg + p.chunk - 1) / p.chunk) : 0u;
        hcnt += nch[k] ? 1u : 0u;
        ccnt += nch[k];
    }
    uint32_t hin = hcnt, cin = ccnt;  // inclusive prefix sums over the wave
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t h = __shfl_up(hin, off, kWave), c = __shfl_up(cin, off, kWave);
        if (lane >= off) {
            hin += h;
            cin += c;
        }
    }
    if (lane == kWave - 1) {
        s_h[wid] = hin;
        s_c[wid] = cin;
    }
    __syncthreads();
    if (threadIdx.x == 0) {  // exclusive prefix over the waves, then the block's ranges
        uint32_t ht = 0, ct = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t h = s_h[w], c = s_c[w];
            s_h[w] = ht;
            s_c[w] = ct;
            ht += h;
            ct += c;
        }
        if (gridDim.x == 1) {  // the only block: it sets the counters (no reset ran)
            p.counters->nheavy = ht;
            p.counters->nchunks = ct;
            s_base[0] = s_base[1] = 0u;
        } else {
            s_base[0] = ht ? atomicAdd(&p.counters->nheavy, ht) : 0u;
            s_base[1] = ht ? atomicAdd(&p.counters->nchunks, ct) : 0u;
        }
    }
    __syncthreads();
    if (hcnt == 0) return;
    uint32_t hs = s_base[0] + s_h[wid] + hin - hcnt;
    uint32_t cb = s_base[1] + s_c[wid] + cin - ccnt;
#pragma unroll
    for (int k = 0; k < kPlanRows; ++k) {
        if (!nch[k]) continue;
        // a valid CSR never trips this (the host sizes both tables for it); a
        // malformed one must not write past them
        if ((int64_t)hs >= p.max_heavy || (int64_t)cb + nch[k] > p.max_chunks) return;
        const int32_t v = (int32_t)(v0 + (int64_t)k * kPlanThreads);
        p.heavy[hs] = HeavyRow{v, (int32_t)nch[k], (int64_t)cb};
        for (uint32_t i = 0; i < nch[k]; ++i) p.chunks[cb + i] = ChunkRef{v, (int32_t)i, (int32_t)hs, 0};
        ++hs;
        cb += nch[k];
    }
}

hipError_t launch_plan(const Args& a, hipStream_t s) {
    if (a.plan.max_heavy == 0) return hipSuccess;  // no row can be split: nothing to list
    const int64_t per_block = (int64_t)kPlanThreads * kPlanRows;
    if (a.N > per_block) {  // several blocks add to the counters: clear them first
        reset_kernel<<<1, 64, 0, s>>>(a.plan.counters);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    plan_kernel<<<(unsigned)((a.N + per_block - 1) / per_block), kPlanThreads, 0, s>>>(a.indptr, a.N, a.plan);
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
