// common.hpp -- device helpers and the work plan shared by the gfx950 kernels.
//
// Work decomposition.  A destination row with at most `chunk` in-edges is one
// work item, handled by one wavefront.  A heavier row (power-law hubs) is cut
// into chunks of `chunk` consecutive edges; each chunk is its own item and
// leaves a partial result in scratch, and a merge kernel combines the chunks
// of a row in chunk order, so results do not depend on scheduling.  The list
// of heavy rows and of their chunks is built on the device by the plan kernel
// (no host synchronisation); kernels are launched over an upper bound of the
// item count and surplus waves exit at once.  Item ids [0, max_chunks) are
// chunks, dispatched first so the longest work starts first; item ids
// [max_chunks, max_chunks + N) are rows, taken through the plan's row order
// (rows grouped by degree bin, longest first) when the plan made one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef GT_WAVES_PER_BLOCK
#define GT_WAVES_PER_BLOCK 4
#endif
#ifndef GT_F32_D64_U
#define GT_F32_D64_U 4  // edges in flight per wave, fp32 rows of 8 heads x 64
#endif
#ifndef GT_BF16_D32_U
#define GT_BF16_D32_U 2  // edges in flight per half-wave, bf16 rows of 8 heads x 32 (8 waves per SIMD)
#endif
#ifndef GT_SDDMM_F32_U
#define GT_SDDMM_F32_U 4  // unfused stages, fp32 8 x 64 and bf16 8 x 32 rows: edges in flight per group
#endif
#ifndef GT_SDDMM_BF16_U
#define GT_SDDMM_BF16_U 8
#endif
#ifndef GT_SPMM_F32_U
#define GT_SPMM_F32_U 4
#endif
#ifndef GT_SPMM_BF16_U
#define GT_SPMM_BF16_U 4
#endif
#ifndef GT_PARTIAL_XL_U
#define GT_PARTIAL_XL_U 2  // rows that end before their last lane group, with logit options: edges in flight
#endif
#ifndef GT_UNFUSED_NTL
#define GT_UNFUSED_NTL 0  // fp32 gathers of arrays over 1 GB with the non-temporal hint (measured slower)
#endif
#ifndef GT_BWD_F32_DQ_U
#define GT_BWD_F32_DQ_U 4  // backward, fp32 8 x 64: destination pass, plain logits
#endif
#ifndef GT_BWD_F32_DKV_U
#define GT_BWD_F32_DKV_U 4  // source pass, plain logits
#endif
#ifndef GT_BWD_BF16_DQ_U
#define GT_BWD_BF16_DQ_U 2  // backward, bf16 8 x 32: destination pass, plain logits (8 waves per SIMD)
#endif
#ifndef GT_BWD_BF16_DQ_XL2_U
#define GT_BWD_BF16_DQ_XL2_U 2  // backward, bf16 8 x 32: destination pass with dropout
#endif
#ifndef GT_BWD_BF16_DKV_U
#define GT_BWD_BF16_DKV_U 2  // source pass, plain logits (6 waves per SIMD)
#endif
#ifndef GT_BWD_BF16_DKV_XL1_U
#define GT_BWD_BF16_DKV_XL1_U 2  // source pass with bias or edge weights
#endif
#ifndef GT_NDH_F32_U
#define GT_NDH_F32_U 4  // head-innermost forward, fp32 rows of 65 to 128 vectors: edges in flight
#endif
#ifndef GT_BF16_NTL
#define GT_BF16_NTL 0  // bf16 8 x 32 forward: gathers with the non-temporal hint (measured slower)
#endif
#ifndef GT_BF16_D32_XL2_U
#define GT_BF16_D32_XL2_U 4  // the same with dropout
#endif
#ifndef GT_BWD_BF16_DQ_XL1_U
#define GT_BWD_BF16_DQ_XL1_U 2  // backward, bf16 8 x 32: destination pass with bias or edge weights
#endif
#ifndef GT_BWD_BF16_DKV_XL2_U
#define GT_BWD_BF16_DKV_XL2_U 2  // source pass with dropout
#endif
#ifndef GT_BF16_D32_XL1_U
#define GT_BF16_D32_XL1_U 2  // the same with bias or edge weights (7 waves per SIMD)
#endif

namespace gt {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = GT_WAVES_PER_BLOCK;
constexpr int kBlock = kWave * kWavesPerBlock;

enum : int { kF32 = 0, kBF16 = 1 };

// Degree bins of the row order, longest rows first: (256, chunk], (64, 256],
// (16, 64], (4, 16], [1, 4], and rows without in-edges.  Waves that take rows
// of like length run together, the write-heavy short and empty rows last.
constexpr int kOrderBins = 6;
__device__ __forceinline__ int order_bin(int64_t deg) {
    return deg > 256 ? 0 : deg > 64 ? 1 : deg > 16 ? 2 : deg > 4 ? 3 : deg > 0 ? 4 : 5;
}

// Rows one plan block takes.  Graphs of at most this many rows are planned by
// a single block and keep their rows in index order.
constexpr int64_t kPlanBlockRows = 8192;

struct PlanCounters {
    uint32_t nheavy;                  // heavy rows listed
    uint32_t nchunks;                 // chunk items listed
    uint32_t bin_total[kOrderBins];   // unsplit rows of each degree bin
    uint32_t bin_cursor[kOrderBins];  // rows placed in each bin's part of the order so far
    uint32_t pad[64 - 2 - 2 * kOrderBins];  // keep the following arrays 256-byte aligned
};

struct HeavyRow {
    int32_t row;
    int32_t nch;   // number of chunks
    int64_t base;  // first chunk item id; the row's chunks are base .. base+nch-1
};

struct ChunkRef {
    int32_t row;
    int32_t idx;    // chunk index within the row
    int32_t hslot;  // index of the row in the heavy-row list
    int32_t pad;
};

// Device view of the scratch buffer of one call.
struct Plan {
    PlanCounters* counters;
    HeavyRow* heavy;     // [max_heavy]
    ChunkRef* chunks;    // [max_chunks]
    float* pm;           // [max_chunks][H] running max of a chunk (log2 domain)
    float* pl;           // [max_chunks][H] sum of exponentials of a chunk
    float* pacc;         // [max_chunks][H*D] unnormalised weighted sum of a chunk
    float* hstat;        // [max_heavy][H][2] merged (max, sum) of a heavy row
    int32_t* order;      // [n_order] the unsplit rows by degree bin (nullptr: rows in index order)
    int64_t n_order;     // N when the plan orders the rows, else 0
    int64_t max_heavy;
    int64_t max_chunks;
    int64_t chunk;       // edges per chunk; rows with more edges are split
};

// What one wavefront works on.
struct Item {
    int64_t row;
    int64_t e0, e1;  // edge range [e0, e1)
    int64_t slot;    // chunk item id (partial results) or -1 for a whole row
    int32_t hslot;   // heavy-row index for chunks
};

__device__ __forceinline__ int64_t uniform64(int64_t x) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The item of the calling wave; false when the wave has nothing to do.
__device__ __forceinline__ bool resolve_item(const Plan& p, const int64_t* __restrict__ indptr, int64_t N,
                                             int64_t item, Item& it) {
    if (item < p.max_chunks) {
        const int64_t n = (int64_t)p.counters->nchunks;  // written by the plan kernel, an earlier launch
        if (item >= n) return false;
        ChunkRef c = p.chunks[item];
        int64_t b = indptr[c.row], e = indptr[c.row + 1];
        it.row = c.row;
        it.e0 = b + (int64_t)c.idx * p.chunk;
        it.e1 = it.e0 + p.chunk < e ? it.e0 + p.chunk : e;
        it.slot = item;
        it.hslot = c.hslot;
        return true;
    }
    int64_t row = item - p.max_chunks;
    if (p.order) {  // rows by degree bin; the list holds every row that is not split
        const PlanCounters* c = p.counters;
        int64_t listed = 0;
#pragma unroll
        for (int b = 0; b < kOrderBins; ++b) listed += c->bin_total[b];
        if (row >= listed) return false;
        row = p.order[row];
    } else if (row >= N) {
        return false;
    }
    it.row = row;
    it.e0 = indptr[row];
    it.e1 = indptr[row + 1];
    if (it.e1 - it.e0 > p.chunk) return false;  // heavy: its chunks do the work
    it.slot = -1;
    it.hslot = -1;
    return true;
}

// Source ids of the U edges a group takes from the batch starting at eb:
// edges eb + grp + j*epw, clamped into the item so that every load is valid
// (the caller masks the clamped ones).  Unconditional loads issue back to
// back; with one group per wave they are scalar loads.
template <int U>
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ idx, int64_t eb, int grp, int epw, int64_t e1,
                                         int32_t (&u)[U]) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int64_t ee = eb + grp + (int64_t)j * epw;
        u[j] = idx[ee < e1 ? ee : e1 - 1];
    }
}

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Natural log-sum-exp of a row's scores from the running state of the
// log2-domain softmax: max m (log2 units) and sum l of 2^(s - m).
__device__ __forceinline__ float lse_of(float m, float l) { return l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY; }

// exp2(a - b) with exp2(-inf - x) = 0 also when b is -inf
__device__ __forceinline__ float rescale(float a, float b) { return a == -INFINITY ? 0.0f : exp2_(a - b); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- cross-lane

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <- lane 15-i within 16

// Sum over aligned segments of `seg` lanes (a power of two <= 64); every lane
// of a segment ends with the same bits (each step adds a commutative pair).
__device__ __forceinline__ float seg_sum(float x, int seg) {
    if (seg >= 2) x += dpp<kQuadXor1>(x);
    if (seg >= 4) x += dpp<kQuadXor2>(x);
    if (seg >= 8) x += dpp<kRowHalfMirror>(x);
    if (seg >= 16) x += dpp<kRowMirror>(x);
    if (seg >= 32) x += __shfl_xor(x, 16, 64);
    if (seg >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

template <int SEG>
__device__ __forceinline__ float seg_sum_c(float x) {
    if constexpr (SEG >= 2) x += dpp<kQuadXor1>(x);
    if constexpr (SEG >= 4) x += dpp<kQuadXor2>(x);
    if constexpr (SEG >= 8) x += dpp<kRowHalfMirror>(x);
    if constexpr (SEG >= 16) x += dpp<kRowMirror>(x);
    if constexpr (SEG >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (SEG >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// ---------------------------------------------------------------- dropout words
//
// Attention dropout ("Efficient Sparse Transformer implementation with DGL's
// builtin operators", TransLayer.forward: drop_att on the edge softmax) draws
// its keep decisions from the counter-based generator Philox4x64-10 (Salmon,
// Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): word i of the stream under key (seed, 0) is word i mod 4 of the
// block whose counter is (i / 4 + 1, 0, 0, 0).  Ten rounds of two 64x64->128
// bit products; the key is bumped by the two Weyl constants after each round.
// philox_block_hi gives the upper 32 bits of the four words of one block.
__device__ __forceinline__ void philox_block_hi(uint64_t seed, uint64_t ctr, uint32_t out[4]) {
    uint64_t c0 = ctr, c1 = 0, c2 = 0, c3 = 0, k0 = seed, k1 = 0;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t a0 = 0xD2E7470EE14C6C93ull * c0, h0 = __umul64hi(0xD2E7470EE14C6C93ull, c0);
        const uint64_t a2 = 0xCA5A826395121157ull * c2, h2 = __umul64hi(0xCA5A826395121157ull, c2);
        c0 = h2 ^ c1 ^ k0;
        c1 = a2;
        c2 = h0 ^ c3 ^ k1;
        c3 = a0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
    out[0] = (uint32_t)(c0 >> 32);
    out[1] = (uint32_t)(c1 >> 32);
    out[2] = (uint32_t)(c2 >> 32);
    out[3] = (uint32_t)(c3 >> 32);
}

// Upper 32 bits of word i of the stream.
__device__ __forceinline__ uint32_t philox_hi32(uint64_t seed, uint64_t i) {
    uint32_t w[4];
    philox_block_hi(seed, i / 4 + 1, w);
    const uint32_t k = (uint32_t)(i & 3);
    return k == 0 ? w[0] : k == 1 ? w[1] : k == 2 ? w[2] : w[3];
}

// Keep decisions of a batch of edges, computed once per wave: a batch has
// nslots edge slots (slot k = group + j * edges-per-wave), and slot k's edge
// needs the words of indices pos(k) * H + h.  The blocks involved are spread
// over the lanes, bpe blocks per slot (lane L -> slot L / bpe, block L % bpe,
// in rounds of 64 lanes); each lane keeps its block's four keep bits.  One
// Philox evaluation per round replaces one per (edge, vector) per lane.
constexpr int kDropRounds = 2;

struct DropBatch {
    uint32_t kb[kDropRounds];
    int rounds;
};

// Blocks per slot: all heads of an edge (hsel < 0), or one head.
__device__ __forceinline__ int drop_bpe(int H, int hsel) {
    return hsel >= 0 ? 1 : (H % 4 == 0 ? H / 4 : (H + 3) / 4 + 1);
}

__device__ __forceinline__ int64_t drop_first_block(int64_t pos, int H, int hsel) {
    return hsel >= 0 ? (pos * H + hsel) / 4 : (pos * H) / 4;
}

// Batches whose keep bits one evaluation covers in a hot instance (edges per
// wave epw, U per group, hc heads per edge), when a pass takes its edges in
// consecutive positions: as many as fill one round of 64 lanes, so that the
// wave's Philox work is not repeated for every batch with most lanes idle.
constexpr int drop_batches_per_eval(int epw, int U, int hc) {
    return 64 / (epw * U * (hc % 4 == 0 ? hc / 4 : (hc + 3) / 4 + 1)) > 1
               ? 64 / (epw * U * (hc % 4 == 0 ? hc / 4 : (hc + 3) / 4 + 1))
               : 1;
}

// Whether a batch fits the rounds (else each lane draws its own words).
__device__ __forceinline__ bool drop_batched(int H, int hsel, int nslots) {
    return nslots * drop_bpe(H, hsel) <= 64 * kDropRounds;
}

// pos_of(k) must be called by every lane (it may use cross-lane shuffles).
template <typename PosOf>
__device__ __forceinline__ void drop_batch_init(DropBatch& d, uint64_t seed, uint32_t thresh, int H, int hsel,
                                                int nslots, int lane, PosOf pos_of) {
    const int bpe = drop_bpe(H, hsel);
    d.rounds = (nslots * bpe + 63) >> 6;
#pragma unroll
    for (int r = 0; r < kDropRounds; ++r) {
        d.kb[r] = 0;
        if (r < d.rounds) {
            const int L = r * 64 + lane;
            const int k = L / bpe, m = L - k * bpe;
            const int64_t pos = pos_of(k < nslots ? k : 0);
            if (k < nslots) {
                uint32_t w[4];
                philox_block_hi(seed, (uint64_t)(drop_first_block(pos, H, hsel) + m) + 1, w);
                d.kb[r] = (uint32_t)(w[0] >= thresh) | (uint32_t)(w[1] >= thresh) << 1 |
                          (uint32_t)(w[2] >= thresh) << 2 | (uint32_t)(w[3] >= thresh) << 3;
            }
        }
    }
}

// The dropout multiplier (0 or scale) of slot k (edge at CSR position pos),
// head h.  Every lane must call it (cross-lane shuffles).
__device__ __forceinline__ float drop_mult(const DropBatch& d, float scale, int H, int hsel, int k, int64_t pos,
                                           int h) {
    const int bpe = drop_bpe(H, hsel);
    const int64_t i = pos * H + h;
    const int L = k * bpe + (int)(i / 4 - drop_first_block(pos, H, hsel));
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < kDropRounds; ++r)
        if (r < d.rounds) {
            const uint32_t t = (uint32_t)__shfl((int)d.kb[r], L & 63, 64);
            if ((L >> 6) == r) bits = t;
        }
    return (bits >> (i & 3)) & 1u ? scale : 0.0f;
}

// ---------------------------------------------------------------- per-edge inputs of a batch
//
// A batch's edge slots k = group + j * edges-per-wave are the consecutive
// edges eb + k of the pass's edge order, so per-edge inputs (bias [E][per],
// weights [E]) of a batch are one contiguous run: the wave loads it 64 values
// at a time (one coalesced load per 64 values instead of one per edge and
// lane vector) and hands each value to the lanes that need it by a shuffle.
constexpr int kSlotRounds = 4;  // shapes known only at run time

template <int R>
struct SlotBatch {
    float v[R];
    int rounds;
};

__device__ __forceinline__ bool slot_batched(int nslots, int per) { return nslots * per <= 64 * kSlotRounds; }

// Values src[(eb + k) * per + h] for the batch's nslots slots; those past the
// item's last edge e1 read as 0.  R bounds the rounds of 64 values.
template <int R>
__device__ __forceinline__ void slot_batch_load(SlotBatch<R>& b, const float* __restrict__ src, int64_t eb, int64_t e1,
                                                int nslots, int per, int lane) {
    b.rounds = (nslots * per + 63) >> 6;
    const int64_t lim = (e1 - eb) * per;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        b.v[r] = 0.0f;
        if (r < b.rounds) {
            const int i = r * 64 + lane;
            if (i < lim) b.v[r] = src[eb * per + i];
        }
    }
}

// The same for slots at scattered edge positions: value (k, h) is
// src[pos_of(k) * per + h] for the nvalid first slots (0 past them).
// pos_of(k) must be called by every lane (it may use cross-lane shuffles).
template <int R, typename PosOf>
__device__ __forceinline__ void slot_batch_load_at(SlotBatch<R>& b, const float* __restrict__ src, int64_t nvalid,
                                                   int nslots, int per, int lane, PosOf pos_of) {
    b.rounds = (nslots * per + 63) >> 6;
    const int64_t lim = nvalid * per;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        b.v[r] = 0.0f;
        if (r < b.rounds) {
            const int i = r * 64 + lane;
            const int k = i / per;
            const int64_t pos = pos_of(k < nslots ? k : 0);
            if (i < lim) b.v[r] = src[pos * per + (i - k * per)];
        }
    }
}

// Value i = k * per + h of the batch; every lane must call it.
template <int R>
__device__ __forceinline__ float slot_batch_get(const SlotBatch<R>& b, int i) {
    if constexpr (R == 1) return __shfl(b.v[0], i & 63, 64);
    float x = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (r < b.rounds) {
            const float t = __shfl(b.v[r], i & 63, 64);
            if ((i >> 6) == r) x = t;
        }
    return x;
}

// ---------------------------------------------------------------- 16-byte vectors

struct alignas(16) U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 ld16(const void* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return U4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ void st16(void* p, U4 v) {
    *reinterpret_cast<uint4*>(p) = make_uint4(v.x, v.y, v.z, v.w);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming variants: the non-temporal hint marks data that will not be reused soon.
__device__ __forceinline__ U4 ld16_nt(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return U4{v.x, v.y, v.z, v.w};
}

// One float with the non-temporal hint (streamed output, not re-read soon).
__device__ __forceinline__ void st_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ void st16_nt(void* p, U4 v) {
    u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// Elements held by one lane per 16-byte vector.
template <int DT>
struct Vec;

template <>
struct Vec<kF32> {
    static constexpr int n = 4;
    static constexpr int bytes = 4;
    __device__ static __forceinline__ void unpack(const U4& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    __device__ static __forceinline__ U4 pack(const float* f) {
        return U4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
    __device__ static __forceinline__ float scalar(const void* base, int64_t i) {
        return reinterpret_cast<const float*>(base)[i];
    }
    __device__ static __forceinline__ void store_scalar(void* base, int64_t i, float f) {
        reinterpret_cast<float*>(base)[i] = f;
    }
};

template <>
struct Vec<kBF16> {
    static constexpr int n = 8;
    static constexpr int bytes = 2;
    __device__ static __forceinline__ void unpack(const U4& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
        f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
        f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    __device__ static __forceinline__ U4 pack(const float* f) {
        return U4{bf16_bits(f[0]) | (bf16_bits(f[1]) << 16), bf16_bits(f[2]) | (bf16_bits(f[3]) << 16),
                  bf16_bits(f[4]) | (bf16_bits(f[5]) << 16), bf16_bits(f[6]) | (bf16_bits(f[7]) << 16)};
    }
    __device__ static __forceinline__ float scalar(const void* base, int64_t i) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
    }
    __device__ static __forceinline__ void store_scalar(void* base, int64_t i, float f) {
        reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)bf16_bits(f);
    }
};

// Lane words of 8 or 4 bytes (the word layout: heads that are a whole number
// of such words but not of 16-byte vectors, e.g. fp32 heads of 10 elements).
template <int DT, int WB>
struct Word {
    static constexpr int NW = WB / 4;                      // 32-bit parts
    static constexpr int EW = DT == kF32 ? NW : 2 * NW;   // elements
    uint32_t w[NW];
};

template <int DT, int WB>
__device__ __forceinline__ Word<DT, WB> ldw(const char* p) {
    Word<DT, WB> r;
    if constexpr (WB == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else {
        r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    return r;
}

template <int DT, int WB>
__device__ __forceinline__ Word<DT, WB> zero_word() {
    Word<DT, WB> r;
#pragma unroll
    for (int i = 0; i < Word<DT, WB>::NW; ++i) r.w[i] = 0;
    return r;
}

template <int DT, int WB>
__device__ __forceinline__ void unpack_word(const Word<DT, WB>& x, float* f) {
#pragma unroll
    for (int i = 0; i < Word<DT, WB>::NW; ++i) {
        if constexpr (DT == kF32) {
            f[i] = __uint_as_float(x.w[i]);
        } else {
            f[2 * i] = bf16_lo(x.w[i]);
            f[2 * i + 1] = bf16_hi(x.w[i]);
        }
    }
}

// Stores EW elements with the non-temporal hint (rows written once).
template <int DT, int WB>
__device__ __forceinline__ void stw_nt(char* p, const float* f) {
    uint32_t w[Word<DT, WB>::NW];
#pragma unroll
    for (int i = 0; i < Word<DT, WB>::NW; ++i)
        w[i] = DT == kF32 ? __float_as_uint(f[i]) : (bf16_bits(f[2 * i]) | (bf16_bits(f[2 * i + 1]) << 16));
    if constexpr (WB == 8) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        u32x2 v = {w[0], w[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
    } else {
        __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
    }
}

// ---------------------------------------------------------------- lane layouts
//
// Vector layout: a node row of H*D elements is R = H*D*bytes/16 vectors of
// 16 bytes.  Lanes per head LPH = D*bytes/16 (a power of two), so a vector
// never straddles two heads.  A group of G lanes (power of two) covers one
// edge's row in NC vectors per lane, lane j of the group holding vectors
// c*G + j, c < NC; a wave runs 64/G groups, each on its own edges.
//
// Scalar layout (any D, one head per wave): a group of G = pow2ceil(D)
// lanes (at most 64) covers one head of one edge, lane j holding elements
// j + k*G, k < KD; a wave runs 64/G groups.
struct VecShape {
    int G;     // lanes per edge group
    int lph;   // lanes per head
    int R;     // 16-byte vectors per node row
};

}  // namespace gt
