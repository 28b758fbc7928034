// spmm.hip -- SpMM stage: out[v,h,:] = sum over in-edges e of v of alpha[e][h] * V[u_e,h,:].
//
// "Graph Transformer in a Nutshell", section "Sparse Multi-head Attention"
// (bspmm of the sparse attention matrix with V); the DGL builtin-operator
// gist's u_mul_e_sum.  Same lane layouts and work items as the fused kernel.
// Chunks of heavy rows leave partial sums; the merge (launch_sum_merge) adds
// them in chunk order.
#include "kernels.hpp"

namespace gt {

// G_ and LPH_ non-zero: a hot instance whose lane layout is known at compile
// time, with every lane active (R == NC * G).  It reads a batch's weights
// (epw * U edges x H heads, contiguous in [E][H]) as one run of 64 values
// per load and hands each lane its weights by shuffles, instead of one
// narrow load per (edge, block of heads).  NTL: V gathers with the
// non-temporal hint.
template <int DT, int NC, int U, int G_ = 0, int LPH_ = 0, bool NTL = false>
__global__ __launch_bounds__(kBlock) void spmm_vec_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr int VN = VT::n;
    constexpr bool kHot = G_ > 0 && LPH_ > 0;
    constexpr int kH = kHot ? NC * (G_ / LPH_) : 1;                    // heads
    constexpr int kR = kHot ? ((kWave / G_) * U * kH + kWave - 1) / kWave : 1;  // loads of 64 weights per batch
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    it.row = uniform64(it.row);
    it.e0 = uniform64(it.e0);
    it.e1 = uniform64(it.e1);

    const int G = kHot ? G_ : a.G, lph = kHot ? LPH_ : a.lph;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    // hot instances have no idle lane slots (heads of a power of two of vectors)
    const int vph = kHot ? lph : a.vph;
    const int64_t rowbytes = (int64_t)(kHot ? a.R : a.Rm) * 16;

    bool act[NC];
    int head[NC], moff[NC];  // moff: byte offset of the lane slot's vector in a row
    float acc[NC][VN];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vi = c * G + gl;
        const bool in_row = kHot || vi < a.R;  // a slot of some head (it may idle)
        act[c] = in_row && (vi & (lph - 1)) < vph;
        head[c] = in_row ? vi / lph : 0;
        moff[c] = kHot ? vi * 16 : (head[c] * vph + (vi & (lph - 1))) * 16;
#pragma unroll
        for (int k = 0; k < VN; ++k) acc[c][k] = 0.0f;
    }
    const char* Vb = (const char*)a.V;
    const int64_t e0 = it.e0, e1 = it.e1;
    int32_t un[U];
    if (e1 > e0) load_ids<U>(a.indices, e0, grp, epw, e1, un);
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            ok[j] = eb + grp + (int64_t)j * epw < e1;
            u[j] = un[j];
        }
        U4 vr[U][NC];
        float al[U][NC];
        SlotBatch<kR> ab;
        // weights past the item's last edge read as 0
        if constexpr (kHot) slot_batch_load(ab, a.alpha_in, eb, e1, epw * U, kH, lane);
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bool go = ok[j] && act[c];
                const char* p = Vb + (int64_t)u[j] * rowbytes + moff[c];
                vr[j][c] = go ? (NTL ? ld16_nt(p) : ld16(p)) : U4{0, 0, 0, 0};
                if constexpr (!kHot) al[j][c] = go ? a.alpha_in[(eb + grp + (int64_t)j * epw) * a.H + head[c]] : 0.0f;
            }
        if constexpr (kHot)
#pragma unroll
            for (int j = 0; j < U; ++j)
#pragma unroll
                for (int c = 0; c < NC; ++c) al[j][c] = slot_batch_get(ab, (grp + j * epw) * kH + head[c]);
        // the next batch's source ids load behind this batch's gathers
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(a.indices, nb, grp, epw, e1, un);
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float vf[VN];
                VT::unpack(vr[j][c], vf);
#pragma unroll
                for (int k = 0; k < VN; ++k) acc[c][k] = __builtin_fmaf(al[j][c], vf[k], acc[c][k]);
            }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VN; ++k) acc[c][k] += __shfl_xor(acc[c][k], off, kWave);
    if (grp != 0) return;
    if (it.slot < 0) {
        char* orow = (char*)a.out + it.row * rowbytes;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (act[c]) {
                if (kHot)
                    st16_nt(orow + moff[c], VT::pack(acc[c]));
                else
                    st16(orow + moff[c], VT::pack(acc[c]));
            }
    } else {
        const int64_t HD = (int64_t)a.H * a.D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (!act[c]) continue;
            float* pa = a.plan.pacc + it.slot * HD + (int64_t)(moff[c] / 16) * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) st16(pa + k, Vec<kF32>::pack(&acc[c][k]));
        }
    }
}

template <int DT, int KD, int U>
__global__ __launch_bounds__(kBlock) void spmm_scalar_kernel(const Args a) {
    using VT = Vec<DT>;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y;
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    it.row = uniform64(it.row);
    it.e0 = uniform64(it.e0);
    it.e1 = uniform64(it.e1);

    const int G = a.G, D = a.D;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int64_t HD = (int64_t)a.H * D;
    const int64_t hoff = (int64_t)h * D;
    bool act[KD];
    float acc[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        act[k] = gl + k * G < D;
        acc[k] = 0.0f;
    }
    for (int64_t e = it.e0 + grp; e < it.e1; e += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
        float al[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t ee = e + (int64_t)j * epw;
            ok[j] = ee < it.e1;
            u[j] = ok[j] ? a.indices[ee] : 0;
            al[j] = ok[j] ? a.alpha_in[ee * a.H + h] : 0.0f;
        }
        float vv[U][KD];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k)
                vv[j][k] = (ok[j] && act[k]) ? VT::scalar(a.V, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k) acc[k] = __builtin_fmaf(al[j], vv[j][k], acc[k]);
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[k] += __shfl_xor(acc[k], off, kWave);
    if (grp != 0) return;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        if (!act[k]) continue;
        if (it.slot < 0)
            VT::store_scalar(a.out, it.row * HD + hoff + gl + k * G, acc[k]);
        else
            a.plan.pacc[it.slot * HD + hoff + gl + k * G] = acc[k];
    }
}

// One wave per heavy row: out = sum of the chunks' partial sums, in chunk order.
template <int DT>
static hipError_t launch_spmm_dt(const Args& a0, hipStream_t s) {
    const dim3 block(kBlock);
    hipError_t err;
    if (a0.vec) {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx);
            const bool full = full_rows(a);
            // gathers streamed past the caches when V is far larger than the Infinity Cache
            const bool stream_v = a.n_gather * (int64_t)a.Rm * 16 > ((int64_t)1 << 30);
            if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && a.H == 8 && full) {
                if (stream_v && GT_UNFUSED_NTL)
                    spmm_vec_kernel<DT, 2, GT_SPMM_F32_U, 64, 16, true><<<grid, block, 0, s>>>(a);
                else
                    spmm_vec_kernel<DT, 2, GT_SPMM_F32_U, 64, 16, false><<<grid, block, 0, s>>>(a);
                return;
            }
            if (DT == kBF16 && a.NC == 1 && a.G == 32 && a.lph == 4 && a.H == 8 && full) {
                spmm_vec_kernel<DT, 1, GT_SPMM_BF16_U, 32, 4, false><<<grid, block, 0, s>>>(a);
                return;
            }
            if (for_fixed_layout(a, [&](auto nc, auto u, auto g, auto lph) {
                    spmm_vec_kernel<DT, nc, u, g, lph, false><<<grid, block, 0, s>>>(a);
                }))
                return;
            switch (a.NC) {
                case 1: spmm_vec_kernel<DT, 1, 8><<<grid, block, 0, s>>>(a); break;
                case 2: spmm_vec_kernel<DT, 2, 4><<<grid, block, 0, s>>>(a); break;
                case 3: spmm_vec_kernel<DT, 3, 2><<<grid, block, 0, s>>>(a); break;
                default: spmm_vec_kernel<DT, 4, 2><<<grid, block, 0, s>>>(a); break;
            }
        });
    } else {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx, a.H);
            switch (a.KD) {
                case 1: spmm_scalar_kernel<DT, 1, 8><<<grid, block, 0, s>>>(a); break;
                case 2: spmm_scalar_kernel<DT, 2, 8><<<grid, block, 0, s>>>(a); break;
                case 3: spmm_scalar_kernel<DT, 3, 4><<<grid, block, 0, s>>>(a); break;
                default: spmm_scalar_kernel<DT, 4, 4><<<grid, block, 0, s>>>(a); break;
            }
        });
    }
    if (err != hipSuccess) return err;
    return launch_sum_merge(a0, 1, a0.out, 1.0f, nullptr, 0.0f, s);
}

hipError_t launch_spmm(const Args& a, hipStream_t s) {
    return a.dtype == kF32 ? launch_spmm_dt<kF32>(a, s) : launch_spmm_dt<kBF16>(a, s);
}

}  // namespace gt
