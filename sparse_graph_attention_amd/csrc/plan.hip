// plan.hip -- device-side work list (heavy rows and their chunks) and the
// CSR validity check.
#include "kernels.hpp"

namespace gt {

__global__ void reset_kernel(PlanCounters* c) {
    if (threadIdx.x == 0) {
        c->nheavy = 0;
        c->nchunks = 0;
    }
}

// One thread per row.  A row with more than `chunk` in-edges gets a slot in
// the heavy-row list and a contiguous range of chunk item ids; the chunk
// table maps each id back to (row, chunk index, heavy slot).  Slot order
// depends on scheduling, but each chunk's result does not, and the merges
// read a row's chunks in chunk order, so outputs are deterministic.
// The wave adds up its heavy rows and chunks with a prefix scan and takes
// its ranges with one atomic per counter (64x fewer atomics on two hot words).
__global__ __launch_bounds__(256) void plan_kernel(const int64_t* __restrict__ indptr, int64_t N, Plan p) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const int64_t deg = v < N ? indptr[v + 1] - indptr[v] : 0;
    const bool heavy = deg > p.chunk;
    const int64_t nch = heavy ? (deg + p.chunk - 1) / p.chunk : 0;
    uint32_t hin = heavy ? 1u : 0u, cin = (uint32_t)nch;  // inclusive prefix sums over the wave
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t h = __shfl_up(hin, off, 64), c = __shfl_up(cin, off, 64);
        if (lane >= off) {
            hin += h;
            cin += c;
        }
    }
    const uint32_t htot = __shfl(hin, 63, 64), ctot = __shfl(cin, 63, 64);
    if (htot == 0) return;
    uint32_t hb = 0, cb = 0;
    if (lane == 0) {
        hb = atomicAdd(&p.counters->nheavy, htot);
        cb = atomicAdd(&p.counters->nchunks, ctot);
    }
    hb = __shfl(hb, 0, 64);
    cb = __shfl(cb, 0, 64);
    if (!heavy) return;
    const uint32_t hs = hb + hin - 1;
    const uint32_t base = cb + cin - (uint32_t)nch;
    // a valid CSR never trips these (the host sizes both tables for it); a
    // malformed one must not write past them
    if ((int64_t)hs >= p.max_heavy || (int64_t)base + nch > p.max_chunks) return;
    p.heavy[hs] = HeavyRow{(int32_t)v, (int32_t)nch, (int64_t)base};
    for (int64_t i = 0; i < nch; ++i) p.chunks[base + i] = ChunkRef{(int32_t)v, (int32_t)i, (int32_t)hs, 0};
}

hipError_t launch_plan(const Args& a, hipStream_t s) {
    if (a.plan.max_heavy == 0) return hipSuccess;  // no row can be split: nothing to list
    reset_kernel<<<1, 64, 0, s>>>(a.plan.counters);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    plan_kernel<<<(unsigned)((a.N + 255) / 256), 256, 0, s>>>(a.indptr, a.N, a.plan);
    return hipGetLastError();
}

// ------------------------------------------------------------ additive merges of split rows
// (the unfused SpMM and both passes of the backward)
// Chunk partials of a heavy row are [chunk][width] with width = regions * HD;
// region r of each is added over the row's chunks, in chunk order, and goes
// to dst_r scaled by scale_r.  One wave per (heavy row, slice of kMergeCols
// columns); chunks are read kMergeUnroll at a time so that many loads are in
// flight (one wave walks up to E / chunk partials of a hub row).
constexpr int kMergeCols = kWave * 4;
constexpr int kMergeUnroll = 8;

template <int DT>
__global__ __launch_bounds__(kBlock) void sum_merge_kernel(const Args a, int regions, void* dst0, float scale0,
                                                           void* dst1, float scale1) {
    using VT = Vec<DT>;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t hs = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (hs >= a.plan.max_heavy || hs >= (int64_t)a.plan.counters->nheavy) return;
    const HeavyRow hr = a.plan.heavy[hs];
    const int64_t HD = (int64_t)a.H * a.D;
    const int64_t width = HD * regions;
    const int64_t j0 = (int64_t)blockIdx.y * kMergeCols;
    const float* pa = a.plan.pacc + hr.base * width;
    int64_t col[4];
    bool in[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        col[t] = j0 + lane + t * kWave;
        in[t] = col[t] < width;
    }
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

template <int DT>
static hipError_t launch_sum_merge_dt(const Args& a0, int regions, void* dst0, float scale0, void* dst1, float scale1,
                                      hipStream_t s) {
    if (a0.plan.max_heavy == 0) return hipSuccess;
    return for_slices(a0, a0.plan.max_heavy, [&](const Args& a, unsigned gx) {
        const unsigned gy = (unsigned)((regions * (int64_t)a.H * a.D + kMergeCols - 1) / kMergeCols);
        sum_merge_kernel<DT><<<dim3(gx, gy), dim3(kBlock), 0, s>>>(a, regions, dst0, scale0, dst1, scale1);
    });
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
