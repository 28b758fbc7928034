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
#include <algorithm>

#include "kernels.hpp"

namespace gt {

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

// Elements per lane kept in registers when a whole item fits (0: none).
// Rows: 16 x 64 scores (128 edges of 8 heads), few registers so that many
// waves hide the latency of the short rows' loads.  Chunks need only their
// statistics, which one streaming pass gives: no cache, more waves.
#ifndef GT_SOFTMAX_ROW_CACHE
#define GT_SOFTMAX_ROW_CACHE 16
#endif
#ifndef GT_SOFTMAX_CHUNK_CACHE
#define GT_SOFTMAX_CHUNK_CACHE 0
#endif
constexpr int kRowCache = GT_SOFTMAX_ROW_CACHE;
constexpr int kChunkCache = GT_SOFTMAX_CHUNK_CACHE;
// Loads in flight per lane in the streaming loops.
#ifndef GT_SOFTMAX_CHUNK_BATCH
#define GT_SOFTMAX_CHUNK_BATCH 16
#endif
constexpr int kBatch = 8;
constexpr int kChunkBatch = GT_SOFTMAX_CHUNK_BATCH;

// One wave over edges [e0, e1) of one destination: the statistics of a chunk
// (slot >= 0), or the weights of a whole row (slot < 0).  Items larger than
// the cache are streamed: one pass for the maximum and the sum together (the
// sum rescaled whenever the lane's maximum grows), and for a row a second
// pass that writes the weights.
template <int kCache, int kB>
__device__ __forceinline__ void softmax_wave(const Args& a, int64_t e0, int64_t e1, int64_t slot, int lane) {
    const int H = a.H;
    const float* s = a.scores_in;  // may alias alpha_out (in place)
    float* alpha = a.alpha_out;
    if ((kWave % H) == 0) {
        // lane j covers flat elements e0*H + j + 64t; its head is j mod H
        const int64_t i0 = e0 * H, i1 = e1 * H;
        if (kCache > 0 && i1 - i0 <= (int64_t)kWave * kCache) {
            // the whole item fits in registers: one read, all loads in flight at once
            constexpr int kC = kCache > 0 ? kCache : 1;
            float v[kC];
#pragma unroll
            for (int t = 0; t < kC; ++t) {
                const int64_t i = i0 + lane + (int64_t)t * kWave;
                v[t] = i < i1 ? s[i] : -INFINITY;
            }
            float m = -INFINITY;
#pragma unroll
            for (int t = 0; t < kC; ++t) m = fmaxf(m, v[t]);
            m = wave_max_stride(m, H);
            float l = 0.0f;
#pragma unroll
            for (int t = 0; t < kC; ++t) {
                v[t] = v[t] == -INFINITY ? 0.0f : expd(v[t], m);
                l += v[t];
            }
            l = wave_sum_stride(l, H);
            if (slot < 0) {
#pragma unroll
                for (int t = 0; t < kC; ++t) {
                    const int64_t i = i0 + lane + (int64_t)t * kWave;
                    if (i < i1) alpha[i] = v[t] / l;
                }
            } else if (lane < H) {
                a.plan.pm[slot * H + lane] = m;
                a.plan.pl[slot * H + lane] = l;
            }
            return;
        }
        // larger items: the lane's running maximum and its sum of exp(s - max)
        float m = -INFINITY, l = 0.0f;
        for (int64_t ib = i0 + lane; ib < i1; ib += (int64_t)kWave * kB) {
            float v[kB];
#pragma unroll
            for (int t = 0; t < kB; ++t) v[t] = ib + t * kWave < i1 ? s[ib + t * kWave] : -INFINITY;
            float mb = v[0];
#pragma unroll
            for (int t = 1; t < kB; ++t) mb = fmaxf(mb, v[t]);
            if (mb > m) {
                l = m == -INFINITY ? 0.0f : l * expd(m, mb);
                m = mb;
            }
#pragma unroll
            for (int t = 0; t < kB; ++t) l += v[t] == -INFINITY ? 0.0f : expd(v[t], m);
        }
        // the lanes of a head: their sums rescaled to the head's maximum
        const float M = wave_max_stride(m, H);
        l = m == -INFINITY ? 0.0f : l * expd(m, M);
        m = M;
        l = wave_sum_stride(l, H);
        if (slot < 0) {
            for (int64_t ib = i0 + lane; ib < i1; ib += (int64_t)kWave * kBatch) {
                float v[kBatch];
#pragma unroll
                for (int t = 0; t < kBatch; ++t) v[t] = ib + t * kWave < i1 ? s[ib + t * kWave] : 0.0f;
#pragma unroll
                for (int t = 0; t < kBatch; ++t)
                    if (ib + t * kWave < i1) alpha[ib + t * kWave] = expd(v[t], m) / l;
            }
        } else if (lane < H) {
            a.plan.pm[slot * H + lane] = m;
            a.plan.pl[slot * H + lane] = l;
        }
    } else {
        for (int h = 0; h < H; ++h) {
            float m = -INFINITY;
            for (int64_t e = e0 + lane; e < e1; e += kWave) m = fmaxf(m, s[e * H + h]);
            m = wave_max_stride(m, 1);
            float l = 0.0f;
            for (int64_t e = e0 + lane; e < e1; e += kWave) l += expd(s[e * H + h], m);
            l = wave_sum_stride(l, 1);
            if (slot < 0) {
                for (int64_t e = e0 + lane; e < e1; e += kWave) alpha[e * H + h] = expd(s[e * H + h], m) / l;
            } else if (lane == 0) {
                a.plan.pm[slot * H + h] = m;
                a.plan.pl[slot * H + h] = l;
            }
        }
    }
}

// Rows of at most this many in-edges are done by one lane per (row, head).
#ifndef GT_SOFTMAX_SMALL_DEG
#define GT_SOFTMAX_SMALL_DEG 16
#endif
constexpr int kSmallDeg = GT_SOFTMAX_SMALL_DEG;

// Chunks of heavy rows: their statistics only (one wave per chunk item).
__global__ __launch_bounds__(kBlock) void softmax_chunk_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.plan.max_chunks) return;
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    softmax_wave<kChunkCache, kChunkBatch>(a, uniform64(it.e0), uniform64(it.e1), it.slot, lane);
}

// Rows that are not split.  When H divides 64 an item is a block of 64/H
// consecutive rows with lane j on (row j/H, head j%H): rows of degree <=
// kSmallDeg are done by their own lanes, larger ones by the whole wave, one
// by one.  Otherwise an item is one row.
__global__ __launch_bounds__(kBlock) void softmax_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H;
    if ((kWave % H) != 0) {
        Item it;
        if (!resolve_item(a.plan, a.indptr, a.N, item + a.plan.max_chunks, it)) return;
        const int64_t e0 = uniform64(it.e0), e1 = uniform64(it.e1);
        if (e1 > e0) softmax_wave<kRowCache, kBatch>(a, e0, e1, -1, lane);
        return;
    }
    const int rpw = kWave / H;
    const int64_t r0 = item * rpw;
    if (r0 >= a.N) return;
    const int64_t r = r0 + lane / H;
    const int h = lane % H;
    int64_t b = 0, e = 0;
    if (r < a.N) {
        b = a.indptr[r];
        e = a.indptr[r + 1];
    }
    const int64_t deg = e - b;
    // rows above the split threshold belong to the chunk kernels: in place,
    // writing their weights here would overwrite scores those kernels read
    if (deg > 0 && deg <= kSmallDeg && deg <= a.plan.chunk) {
        // the lane's (row, head) scores in registers: one read with all loads in flight
        const float* s = a.scores_in;  // may alias alpha_out (in place)
        float v[kSmallDeg];
#pragma unroll
        for (int t = 0; t < kSmallDeg; ++t) v[t] = t < deg ? s[(b + t) * H + h] : -INFINITY;
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < kSmallDeg; ++t) m = fmaxf(m, v[t]);
        float l = 0.0f;
#pragma unroll
        for (int t = 0; t < kSmallDeg; ++t) {
            v[t] = t < deg ? expd(v[t], m) : 0.0f;
            l += v[t];
        }
#pragma unroll
        for (int t = 0; t < kSmallDeg; ++t)
            if (t < deg) a.alpha_out[(b + t) * H + h] = v[t] / l;
    }
    uint64_t big = __ballot(h == 0 && deg > kSmallDeg && deg <= a.plan.chunk);
    while (big) {
        const int j = __builtin_ctzll(big);
        big &= big - 1;
        const int64_t row = r0 + j / H;
        softmax_wave<kRowCache, kBatch>(a, a.indptr[row], a.indptr[row + 1], -1, lane);
    }
}

// The chunks' (max, sum) of each heavy row, merged per head.  A wave per
// heavy row at a time, striding over the rows the plan lists (the grid is
// capped at kMergeGridX blocks; the host only knows an upper bound of heavy
// rows).  When H divides 64, lane j takes head j % H of chunks j / H,
// j / H + 64 / H, ... and the lanes of a head combine their partial (max, sum)
// by xor shuffles, in a fixed order; otherwise lane h < H walks its head's
// chunks in order.
__global__ __launch_bounds__(kBlock) void softmax_merge_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int H = a.H;
    const int64_t nheavy = min(a.plan.max_heavy, (int64_t)a.plan.counters->nheavy);
    for (int64_t hs = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         hs < nheavy; hs += (int64_t)gridDim.x * kWavesPerBlock) {
        const HeavyRow hr = a.plan.heavy[hs];
        const float* pm = a.plan.pm + hr.base * H;
        const float* pl = a.plan.pl + hr.base * H;
        if ((kWave % H) == 0) {
            const int h = lane % H, cpw = kWave / H;
            float m = -INFINITY, l = 0.0f;
            for (int i = lane / H; i < hr.nch; i += cpw) {  // every chunk has edges: its max is finite
                const float mi = pm[(int64_t)i * H + h], li = pl[(int64_t)i * H + h];
                const float mn = fmaxf(m, mi);
                l = l * (m == -INFINITY ? 0.0f : expd(m, mn)) + li * expd(mi, mn);
                m = mn;
            }
            const float M = wave_max_stride(m, H);
            const float L = wave_sum_stride(m == -INFINITY ? 0.0f : l * expd(m, M), H);
            if (lane < H) {
                a.plan.hstat[(hs * H + h) * 2 + 0] = M;
                a.plan.hstat[(hs * H + h) * 2 + 1] = L;
            }
        } else if (lane < H) {
            float M = -INFINITY;
            for (int i = 0; i < hr.nch; ++i) M = fmaxf(M, pm[(int64_t)i * H + lane]);
            float L = 0.0f;
            for (int i = 0; i < hr.nch; ++i) L += pl[(int64_t)i * H + lane] * expd(pm[(int64_t)i * H + lane], M);
            a.plan.hstat[(hs * H + lane) * 2 + 0] = M;
            a.plan.hstat[(hs * H + lane) * 2 + 1] = L;
        }
    }
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
    const int64_t i0 = it.e0 * H, i1 = it.e1 * H;
    if ((kWave % H) == 0) {
        // the lane's head is fixed (i0 and the stride are multiples of H)
        const int h = lane % H;
        const float M = st[2 * h], L = st[2 * h + 1];
        for (int64_t ib = i0 + lane; ib < i1; ib += (int64_t)kWave * kBatch) {
            float v[kBatch];
#pragma unroll
            for (int t = 0; t < kBatch; ++t) v[t] = ib + t * kWave < i1 ? s[ib + t * kWave] : 0.0f;
#pragma unroll
            for (int t = 0; t < kBatch; ++t)
                if (ib + t * kWave < i1) a.alpha_out[ib + t * kWave] = expd(v[t], M) / L;
        }
    } else {
        for (int64_t i = i0 + lane; i < i1; i += kWave) {
            const int h = (int)(i % H);
            a.alpha_out[i] = expd(s[i], st[2 * h]) / st[2 * h + 1];
        }
    }
}

hipError_t launch_softmax(const Args& a, hipStream_t s) {
    const dim3 block(kBlock);
    const int64_t rows = (kWave % a.H) == 0 ? (a.N + kWave / a.H - 1) / (kWave / a.H) : a.N;
    hipError_t err = for_slices(a, rows, [&](const Args& as, unsigned gx) {
        softmax_kernel<<<gx, block, 0, s>>>(as);
    });
    if (err != hipSuccess || a.plan.max_heavy == 0) return err;
    err = for_slices(a, a.plan.max_chunks, [&](const Args& as, unsigned gx) {
        softmax_chunk_kernel<<<gx, block, 0, s>>>(as);
    });
    if (err != hipSuccess) return err;
    softmax_merge_kernel<<<(unsigned)std::min<int64_t>((a.plan.max_heavy + kWavesPerBlock - 1) / kWavesPerBlock,
                                                        kMergeGridX),
                           block, 0, s>>>(a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return for_slices(a, a.plan.max_chunks, [&](const Args& as, unsigned gx) {
        softmax_chunk_norm_kernel<<<gx, block, 0, s>>>(as);
    });
}

}  // namespace gt
