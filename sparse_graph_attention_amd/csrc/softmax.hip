// softmax.hip -- edge-softmax stage:
//   alpha[e][h] = exp(s[e][h] - m) / sum exp(s[e'][h] - m) over the in-edges
//   e' of e's destination, m their maximum.
//
// "Graph Transformer in a Nutshell", section "Sparse Multi-head Attention"
// (the sparse softmax over each row of the attention matrix); the DGL
// builtin-operator gist's edge_softmax, read as normalising over each
// destination's in-edges.  One wave per work item, three passes over the
// item's scores (max, sum of exponentials, weights).  A chunk of a heavy row
// only leaves its (max, sum); the row's chunks are merged in chunk order and
// a last pass over the chunks writes the weights.
#include "kernels.hpp"

namespace gt {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float expd(float s, float m) { return exp2_((s - m) * kLog2e); }

// Max and sum over the lanes that share a head (lanes congruent mod `hstride`).
__device__ __forceinline__ float wave_max_stride(float x, int hstride) {
    for (int off = hstride; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}
__device__ __forceinline__ float wave_sum_stride(float x, int hstride) {
    for (int off = hstride; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Per-(item) statistics and, for whole rows, the weights.
__global__ __launch_bounds__(kBlock) void softmax_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    it.e0 = uniform64(it.e0);
    it.e1 = uniform64(it.e1);
    if (it.e1 == it.e0) return;
    const int H = a.H;
    const float* s = a.scores_in;  // may alias alpha_out (in place)
    float* alpha = a.alpha_out;

    if ((kWave % H) == 0) {
        // lane j covers flat elements e0*H + j + 64t; its head is j mod H
        const int64_t i0 = it.e0 * H, i1 = it.e1 * H;
        float m = -INFINITY;
        for (int64_t i = i0 + lane; i < i1; i += kWave) m = fmaxf(m, s[i]);
        m = wave_max_stride(m, H);
        float l = 0.0f;
        for (int64_t i = i0 + lane; i < i1; i += kWave) l += expd(s[i], m);
        l = wave_sum_stride(l, H);
        if (it.slot < 0) {
            for (int64_t i = i0 + lane; i < i1; i += kWave) alpha[i] = expd(s[i], m) / l;
        } else if (lane < H) {
            a.plan.pm[it.slot * H + lane] = m;
            a.plan.pl[it.slot * H + lane] = l;
        }
    } else {
        for (int h = 0; h < H; ++h) {
            float m = -INFINITY;
            for (int64_t e = it.e0 + lane; e < it.e1; e += kWave) m = fmaxf(m, s[e * H + h]);
            m = wave_max_stride(m, 1);
            float l = 0.0f;
            for (int64_t e = it.e0 + lane; e < it.e1; e += kWave) l += expd(s[e * H + h], m);
            l = wave_sum_stride(l, 1);
            if (it.slot < 0) {
                for (int64_t e = it.e0 + lane; e < it.e1; e += kWave) alpha[e * H + h] = expd(s[e * H + h], m) / l;
            } else if (lane == 0) {
                a.plan.pm[it.slot * H + h] = m;
                a.plan.pl[it.slot * H + h] = l;
            }
        }
    }
}

// One wave per heavy row, lane h < H per head: merge the chunks' (max, sum) in chunk order.
__global__ __launch_bounds__(kBlock) void softmax_merge_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t hs = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H;
    if (hs >= a.plan.max_heavy || hs >= (int64_t)a.plan.counters->nheavy || lane >= H) return;
    const HeavyRow hr = a.plan.heavy[hs];
    float M = -INFINITY;
    for (int i = 0; i < hr.nch; ++i) M = fmaxf(M, a.plan.pm[(hr.base + i) * H + lane]);
    float L = 0.0f;
    for (int i = 0; i < hr.nch; ++i)
        L += a.plan.pl[(hr.base + i) * H + lane] * expd(a.plan.pm[(hr.base + i) * H + lane], M);
    a.plan.hstat[(hs * H + lane) * 2 + 0] = M;
    a.plan.hstat[(hs * H + lane) * 2 + 1] = L;
}

// One wave per chunk item: weights from the merged statistics of its row.
__global__ __launch_bounds__(kBlock) void softmax_chunk_norm_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.plan.max_chunks || item >= (int64_t)a.plan.counters->nchunks) return;
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int H = a.H;
    const float* s = a.scores_in;  // may alias alpha_out (in place)
    const float* st = a.plan.hstat + (int64_t)it.hslot * H * 2;
    for (int64_t i = it.e0 * H + lane; i < it.e1 * H; i += kWave) {
        const int h = (int)(i % H);
        a.alpha_out[i] = expd(s[i], st[2 * h]) / st[2 * h + 1];
    }
}

hipError_t launch_softmax(const Args& a, hipStream_t s) {
    const dim3 block(kBlock);
    hipError_t err = for_slices(a, a.items, [&](const Args& as, unsigned gx) {
        softmax_kernel<<<gx, block, 0, s>>>(as);
    });
    if (err != hipSuccess || a.plan.max_heavy == 0) return err;
    err = for_slices(a, a.plan.max_heavy, [&](const Args& as, unsigned gx) {
        softmax_merge_kernel<<<gx, block, 0, s>>>(as);
    });
    if (err != hipSuccess) return err;
    return for_slices(a, a.plan.max_chunks, [&](const Args& as, unsigned gx) {
        softmax_chunk_norm_kernel<<<gx, block, 0, s>>>(as);
    });
}

}  // namespace gt
