// kernels.hpp -- host-side launchers of the gfx950 kernels (one translation
// unit per stage) and the argument block they share.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"

namespace gt {

struct Args {
    const int64_t* indptr;
    const int32_t* indices;
    const void* Q;
    const void* K;
    const void* V;
    void* out;
    const float* scores_in;
    float* scores_out;
    const float* alpha_in;
    float* alpha_out;
    int64_t N, E;
    int64_t n_gather;  // rows of the arrays the pass gathers by index (K and V: the source count)
    int H, D, dtype;
    float qscale;  // fused and backward: log2(e)/sqrt(D); SDDMM: 1/sqrt(D)
    float kscale;  // backward: 1/sqrt(D)
    // training: the forward's log-sum-exp and the backward's inputs/outputs
    float* lse_out;      // [N][H], natural log; written by the forward when non-null
    const float* lse_in; // [N][H]
    const void* O;       // the forward's output
    const void* dO;      // gradient of the loss with respect to the output
    float2* stats;       // [N][H] scratch: (lse in log2 units, delta = dO . O) per destination and head
    void* dQ;
    void* dK;
    void* dV;
    // logit variants and attention dropout (the "extended logit" kernels; all
    // off when bias == ew == nullptr, drop_thresh == 0 and no dbias/dew)
    const float* bias;      // [E][H] added to the natural-log logit, CSR edge order
    const float* ew;        // [E] multiplies the scaled dot product
    uint64_t drop_seed;     // Philox4x64-10 key
    uint32_t drop_thresh;   // keep iff the word's upper 32 bits >= this; 0: no dropout
    float drop_scale;       // 1 / (1 - p)
    const int32_t* t_perm;  // source pass: CSR position of each out-edge
    float* dbias;           // backward output [E][H] or nullptr
    float* dew;             // backward output [E] or nullptr
    float* dew_part;        // scratch [E][H]: per-head terms of dew (scalar layout)
    Plan plan;
    // lane layout (chosen on the host)
    int vec;       // 1: 16-byte vector layout, 0: scalar layout
    int G;         // lanes per edge group
    int lph;       // vector layout: lanes per head
    int R;         // vector layout: lane slots per node row (H * lph)
    int vph;       // vector layout: 16-byte vectors per head in memory (lph = pow2ceil(vph))
    int Rm;        // vector layout: 16-byte vectors per node row in memory (H * vph)
    int NC;        // vector layout: vectors per lane
    int KD;        // scalar layout: elements per lane
    int ndh;       // features are [N][D][H] (head innermost); vec = 2 selects fused_ndh_kernel
    int wb;        // word layout (vec = 3): bytes per lane word (4 or 8); vph words per head
    // grid
    int64_t items;      // max_chunks + N
    int64_t item_base;  // first item of the current launch slice
};

// Per node, src [A][B] -> dst [B][A] (elementwise; bf16 moved as 16-bit words).
hipError_t launch_transpose_rows(const void* src, void* dst, int64_t N, int A, int B, int dtype, hipStream_t s);


// Calls f(wb, lph) with std::integral_constant arguments for the word layout's
// instances (vec = 3): lane words of 8 or 4 bytes, 1 .. 32 lane slots per head.
template <typename F>
inline bool for_word_layout(const Args& a, F&& f) {
    using std::integral_constant;
    auto go = [&](auto wb) {
        switch (a.lph) {
            case 1: f(wb, integral_constant<int, 1>{}); return true;
            case 2: f(wb, integral_constant<int, 2>{}); return true;
            case 4: f(wb, integral_constant<int, 4>{}); return true;
            case 8: f(wb, integral_constant<int, 8>{}); return true;
            case 16: f(wb, integral_constant<int, 16>{}); return true;
            case 32: f(wb, integral_constant<int, 32>{}); return true;
            default: return false;
        }
    };
    return a.wb == 8 ? go(integral_constant<int, 8>{}) : a.wb == 4 ? go(integral_constant<int, 4>{}) : false;
}

// Whether a launch needs the extended-logit kernels.
inline bool extended(const Args& a) { return a.bias || a.ew || a.drop_thresh || a.dbias || a.dew; }

// Blocks in x of the merges of split rows, which stride over the heavy rows.
constexpr int64_t kMergeGridX = 1024;

// Items per launch slice: keeps gridDim.x * blockDim.x below 2^32.
constexpr int64_t kSliceItems = (int64_t)1 << 24;

// Launches `fn(args_with_item_base, grid_x)` over [0, items) in slices.
template <typename F>
inline hipError_t for_slices(Args a, int64_t items, F fn) {
    for (int64_t b = 0; b < items; b += kSliceItems) {
        a.item_base = b;
        const int64_t n = items - b < kSliceItems ? items - b : kSliceItems;
        fn(a, (unsigned)((n + kWavesPerBlock - 1) / kWavesPerBlock));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// Whole rows of 32 to 256 vectors (R == NC * G) get kernel instances
// with the lane layout known at compile time for every head width: the
// run-time layout works out each item's lane groups and heads with integer
// divisions and masks every vector.  Calls f(NC, U, G, LPH) with
// std::integral_constant arguments (U: edges in flight per lane group) and
// returns true, or returns false when the layout has no such instance.
// Every lane slot of a row holds a vector: no lane idles past the row's end,
// and heads are a power of two of vectors (no padding slots).
inline bool full_rows(const Args& a) { return a.R == a.NC * a.G && a.vph == a.lph; }

// The table of compile-time lane layouts (see for_fixed_layout).
template <typename F>
inline bool fixed_layout_table(const Args& a, F&& f) {
    using std::integral_constant;
    if (a.G == 64 && (a.NC == 3 || a.NC == 4)) {  // rows of up to 192 or 256 vectors
        using U = integral_constant<int, 2>;
        using G = integral_constant<int, 64>;
        auto go = [&](auto nc) {
            switch (a.lph) {
                case 8: f(nc, U{}, G{}, integral_constant<int, 8>{}); return true;
                case 16: f(nc, U{}, G{}, integral_constant<int, 16>{}); return true;
                case 32: f(nc, U{}, G{}, integral_constant<int, 32>{}); return true;
                case 64: f(nc, U{}, G{}, integral_constant<int, 64>{}); return true;
                default: return false;
            }
        };
        return a.NC == 3 ? go(integral_constant<int, 3>{}) : go(integral_constant<int, 4>{});
    }
    if (a.G == 64 && a.NC == 2) {
        using N = integral_constant<int, 2>;
        using U = integral_constant<int, 4>;
        using G = integral_constant<int, 64>;
        switch (a.lph) {
            case 8: f(N{}, U{}, G{}, integral_constant<int, 8>{}); return true;
            case 16: f(N{}, U{}, G{}, integral_constant<int, 16>{}); return true;
            case 32: f(N{}, U{}, G{}, integral_constant<int, 32>{}); return true;
            case 64: f(N{}, U{}, G{}, integral_constant<int, 64>{}); return true;
            default: return false;
        }
    }
    if (a.NC == 1 && (a.G == 64 || a.G == 32)) {
        using N = integral_constant<int, 1>;
        using U = integral_constant<int, 8>;
        if (a.G == 64) {
            using G = integral_constant<int, 64>;
            switch (a.lph) {
                case 4: f(N{}, U{}, G{}, integral_constant<int, 4>{}); return true;
                case 8: f(N{}, U{}, G{}, integral_constant<int, 8>{}); return true;
                case 16: f(N{}, U{}, G{}, integral_constant<int, 16>{}); return true;
                case 32: f(N{}, U{}, G{}, integral_constant<int, 32>{}); return true;
                default: return false;
            }
        }
        using G = integral_constant<int, 32>;
        switch (a.lph) {
            case 4: f(N{}, U{}, G{}, integral_constant<int, 4>{}); return true;
            case 8: f(N{}, U{}, G{}, integral_constant<int, 8>{}); return true;
            case 16: f(N{}, U{}, G{}, integral_constant<int, 16>{}); return true;
            default: return false;
        }
    }
    return false;
}

template <typename F>
inline bool for_fixed_layout(const Args& a, F&& f) {
    return full_rows(a) && fixed_layout_table(a, f);
}

// The same table for the other rows: lane slots past the row's end, or
// padded heads (vph < lph).  The instances keep the run-time masks of idle
// slots and the true row stride, with lane groups and head widths known at
// compile time.
template <typename F>
inline bool for_fixed_partial_layout(const Args& a, F&& f) {
    return !full_rows(a) && fixed_layout_table(a, f);
}

// Plan: clears the counters and lists heavy rows and their chunks.
hipError_t launch_plan(const Args& a, hipStream_t s);
// Fused forward over all items, then the merge of split rows.
hipError_t launch_fused(const Args& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_fused_merge(const Args& a, hipStream_t s);
// Unfused stages.
hipError_t launch_sddmm(const Args& a, hipStream_t s);
hipError_t launch_softmax(const Args& a, hipStream_t s);
hipError_t launch_spmm(const Args& a, hipStream_t s);
// Backward: dQ (and delta) over the destination-sorted graph, then dK and dV
// over the source-sorted one (a.indptr/a.indices/a.plan describe that graph).
hipError_t launch_bwd_dq(const Args& a, hipStream_t s);
// Split rows whose chunk partials add up ([chunk][regions * H * D] floats in
// a.plan.pacc): region r of the sum, times scale_r, goes to row hr.row of dst_r.
hipError_t launch_sum_merge(const Args& a, int regions, void* dst0, float scale0, void* dst1, float scale1,
                            hipStream_t s);
hipError_t launch_bwd_dkv(const Args& a, hipStream_t s);
// Graph construction (graph.hip).  A stable LSD radix sort of n uint32 keys
// below 2^key_bits carrying uint32 values (vals_in == nullptr: each key's
// input position) and, when vals2_in is non-null, a second value array.
// scratch holds sort_scratch_bytes(n, vals2_in != nullptr) bytes; the sorted
// values land in vals_final / vals2_final when those are non-null, else in
// scratch; *keys_sorted etc. point at the results.
int key_bits_for(int64_t nkeys);
size_t sort_scratch_bytes(int64_t n, bool two_values);
hipError_t radix_sort(const uint32_t* keys_in, const uint32_t* vals_in, const uint32_t* vals2_in, int64_t n,
                      int key_bits, void* scratch, uint32_t* vals_final, uint32_t* vals2_final, hipStream_t s,
                      const uint32_t** keys_sorted, const uint32_t** vals_sorted, const uint32_t** vals2_sorted);
// offsets[v] = number of sorted keys below v, v in [0, nrows].
hipError_t launch_lower_bounds(const uint32_t* keys, int64_t n, int64_t nrows, int64_t* offsets, hipStream_t s);
// rows[p] = the row of CSR position p.
hipError_t launch_row_of_position(const int64_t* indptr, int64_t nrows, int64_t n, uint32_t* rows, hipStream_t s);
// Grouping by key in one launch, for n <= 16,384 items (group_small_fits):
// offsets[nrows + 1] and out[j] = the value of the j-th item in key order
// (stable); perm[j] = its input position when perm is non-null.  The value of
// item e is vals[e], or with row_indptr non-null the row holding position e
// of that CSR of row_n (< 2^18) rows, perm then required.
bool group_small_fits(int64_t n, int64_t row_n);
hipError_t launch_group_small(const uint32_t* keys, const uint32_t* vals, const int64_t* row_indptr, int64_t row_n,
                              int64_t n, int64_t nrows, int64_t* offsets, uint32_t* out, uint32_t* perm,
                              hipStream_t s);
// Measurement aid (calib.hip): the K and V rows of every edge, read as the
// fused kernel reads them, XOR-folded into *sink.  row_bytes 512, 1024 or 2048.
hipError_t launch_calib_gather(const int32_t* indices, int64_t E, const void* K, const void* V, int64_t n_rows,
                               int row_bytes, uint32_t* sink, hipStream_t s);
// CSR check: writes error flags into *flags (device memory, cleared first).
hipError_t launch_validate(const int64_t* indptr, const int32_t* indices, int64_t N, int64_t E, uint32_t* flags,
                           hipStream_t s);

inline unsigned blocks_for(int64_t waves) { return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

}  // namespace gt
