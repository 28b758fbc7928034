// sddmm.hip -- SDDMM stage: scores[e][h] = <Q[v,h,:], K[u_e,h,:]> / sqrt(D).
//
// "Graph Transformer in a Nutshell", section "Sparse Multi-head Attention":
// the product QK^T is formed only at the nonzeros of the adjacency matrix,
// batched over heads; the DGL builtin-operator gist's u_dot_v followed by
// its division by sqrt(d_qkv).  Same lane layouts and work items as the fused
// kernel; chunks of heavy rows are independent here (no merge).
#include "kernels.hpp"

namespace gt {

// G_ and LPH_ non-zero: a hot instance whose lane layout is known at compile
// time, with every lane active (R == NC * G).  It writes a batch's scores
// (epw * U edges x H heads, contiguous in [E][H]) with one coalesced store
// per 64 of them instead of one narrow store per (edge, block of heads).
// NTL: K gathers with the non-temporal hint.
template <int DT, int NC, int U, int G_ = 0, int LPH_ = 0, bool NTL = false>
__global__ __launch_bounds__(kBlock) void sddmm_vec_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr int VN = VT::n;
    constexpr bool kHot = G_ > 0 && LPH_ > 0;
    constexpr int kHPC = kHot ? G_ / LPH_ : 1;             // heads per block of G vectors
    constexpr int kH = NC * kHPC;                          // heads
    constexpr int kEPW = kHot ? kWave / G_ : 1;            // edge groups per wave
    constexpr int kS = kEPW * U * kH;                      // scores per batch
    constexpr int kP = kHot ? (U * NC + LPH_ - 1) / LPH_ : 1;  // registers the batch packs into
    constexpr int kStores = (kS + kWave - 1) / kWave;
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

    float q[NC][VN];
    bool act[NC], writer[NC];
    int head[NC], moff[NC];  // moff: byte offset of the lane slot's vector in a row
    const char* qrow = (const char*)a.Q + it.row * rowbytes;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vi = c * G + gl;
        act[c] = kHot || (vi < a.R && (vi & (lph - 1)) < vph);
        writer[c] = act[c] && (vi & (lph - 1)) == 0;
        head[c] = vi / lph;
        moff[c] = kHot ? vi * 16 : (head[c] * vph + (vi & (lph - 1))) * 16;
        if (act[c]) {
            VT::unpack(ld16(qrow + moff[c]), q[c]);
        } else {
#pragma unroll
            for (int k = 0; k < VN; ++k) q[c][k] = 0.0f;
        }
    }
    const char* Kb = (const char*)a.K;
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
        U4 kr[U][NC];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const char* p = Kb + (int64_t)u[j] * rowbytes + moff[c];
                kr[j][c] = (ok[j] && act[c]) ? (NTL ? ld16_nt(p) : ld16(p)) : U4{0, 0, 0, 0};
            }
        // the next batch's source ids load behind this batch's gathers
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(a.indices, nb, grp, epw, e1, un);
        float dd[U][NC];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float kf[VN];
                VT::unpack(kr[j][c], kf);
                float d = 0.0f;
#pragma unroll
                for (int k = 0; k < VN; ++k) d = __builtin_fmaf(q[c][k], kf[k], d);
                // every lane of the head's segment ends with the same sum
                dd[j][c] = kHot ? seg_sum_c<LPH_>(d) : seg_sum(d, lph);
                if (!kHot && ok[j] && writer[c])
                    st_nt(&a.scores_out[(eb + grp + (int64_t)j * epw) * a.H + head[c]], dd[j][c] * a.qscale);
            }
        if constexpr (kHot) {
            // pack: in each (group, head) segment, the lane at position k holds
            // value i = p * LPH + k of register p, value i being (j, c) = (i / NC, i % NC)
            const int kpos = gl & (LPH_ - 1);
            float x[kP];
#pragma unroll
            for (int p = 0; p < kP; ++p) {
                x[p] = 0.0f;
#pragma unroll
                for (int i = p * LPH_; i < (p + 1) * LPH_ && i < U * NC; ++i)
                    if (kpos == i - p * LPH_) x[p] = dd[i / NC][i % NC];
            }
            // slot s of the batch is edge eb + s / H (= eb + grp + j * epw), head s % H
            const int64_t lim = (e1 - eb) * kH;
#pragma unroll
            for (int r = 0; r < kStores; ++r) {
                const int s = r * kWave + lane;
                const int ke = s / kH, h = s % kH;
                const int j = ke / kEPW, g2 = ke % kEPW;
                const int i = j * NC + h / kHPC;
                const int src = (g2 * G_ + (h % kHPC) * LPH_ + i % LPH_) & (kWave - 1);
                float val = 0.0f;
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    const float t = __shfl(x[p], src, kWave);
                    if (p == i / LPH_) val = t;
                }
                if (s < kS && s < lim) st_nt(&a.scores_out[eb * kH + s], val * a.qscale);
            }
        }
    }
}

template <int DT, int KD, int U>
__global__ __launch_bounds__(kBlock) void sddmm_scalar_kernel(const Args a) {
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
    float q[KD];
    bool act[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = gl + k * G;
        act[k] = d < D;
        q[k] = act[k] ? VT::scalar(a.Q, it.row * HD + hoff + d) : 0.0f;
    }
    for (int64_t e = it.e0 + grp; e < it.e1; e += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t ee = e + (int64_t)j * epw;
            ok[j] = ee < it.e1;
            u[j] = ok[j] ? a.indices[ee] : 0;
        }
        float kv[U][KD];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k)
                kv[j][k] = (ok[j] && act[k]) ? VT::scalar(a.K, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float d = 0.0f;
#pragma unroll
            for (int k = 0; k < KD; ++k) d = __builtin_fmaf(q[k], kv[j][k], d);
            d = seg_sum(d, G);
            if (ok[j] && gl == 0) st_nt(&a.scores_out[(e + (int64_t)j * epw) * a.H + h], d * a.qscale);
        }
    }
}

template <int DT>
static hipError_t launch_sddmm_dt(const Args& a0, hipStream_t s) {
    const dim3 block(kBlock);
    if (a0.vec) {
        return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx);
            const bool full = full_rows(a);
            // gathers streamed past the caches when K is far larger than the Infinity Cache
            const bool stream_k = a.n_gather * (int64_t)a.Rm * 16 > ((int64_t)1 << 30);
            if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && a.H == 8 && full) {
                if (stream_k && GT_UNFUSED_NTL)
                    sddmm_vec_kernel<DT, 2, GT_SDDMM_F32_U, 64, 16, true><<<grid, block, 0, s>>>(a);
                else
                    sddmm_vec_kernel<DT, 2, GT_SDDMM_F32_U, 64, 16, false><<<grid, block, 0, s>>>(a);
                return;
            }
            if (DT == kBF16 && a.NC == 1 && a.G == 32 && a.lph == 4 && a.H == 8 && full) {
                sddmm_vec_kernel<DT, 1, GT_SDDMM_BF16_U, 32, 4, false><<<grid, block, 0, s>>>(a);
                return;
            }
            if (for_fixed_layout(a, [&](auto nc, auto u, auto g, auto lph) {
                    sddmm_vec_kernel<DT, nc, u, g, lph, false><<<grid, block, 0, s>>>(a);
                }))
                return;
            switch (a.NC) {
                case 1: sddmm_vec_kernel<DT, 1, 8><<<grid, block, 0, s>>>(a); break;
                case 2: sddmm_vec_kernel<DT, 2, 4><<<grid, block, 0, s>>>(a); break;
                case 3: sddmm_vec_kernel<DT, 3, 4><<<grid, block, 0, s>>>(a); break;
                default: sddmm_vec_kernel<DT, 4, 2><<<grid, block, 0, s>>>(a); break;
            }
        });
    }
    return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
        const dim3 grid(gx, a.H);
        switch (a.KD) {
            case 1: sddmm_scalar_kernel<DT, 1, 8><<<grid, block, 0, s>>>(a); break;
            case 2: sddmm_scalar_kernel<DT, 2, 8><<<grid, block, 0, s>>>(a); break;
            case 3: sddmm_scalar_kernel<DT, 3, 4><<<grid, block, 0, s>>>(a); break;
            default: sddmm_scalar_kernel<DT, 4, 4><<<grid, block, 0, s>>>(a); break;
        }
    });
}

hipError_t launch_sddmm(const Args& a, hipStream_t s) {
    return a.dtype == kF32 ? launch_sddmm_dt<kF32>(a, s) : launch_sddmm_dt<kBF16>(a, s);
}

}  // namespace gt
