// sddmm.hip -- SDDMM stage: scores[e][h] = <Q[v,h,:], K[u_e,h,:]> / sqrt(D).
//
// "Graph Transformer in a Nutshell", section "Sparse Multi-head Attention":
// the product QK^T is formed only at the nonzeros of the adjacency matrix,
// batched over heads; the DGL builtin-operator gist's u_dot_v followed by
// its division by sqrt(d_qkv).  Same lane layouts and work items as the fused
// kernel; chunks of heavy rows are independent here (no merge).
#include "kernels.hpp"

namespace gt {

template <int DT, int NC, int U>
__global__ __launch_bounds__(kBlock) void sddmm_vec_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr int VN = VT::n;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    it.row = uniform64(it.row);
    it.e0 = uniform64(it.e0);
    it.e1 = uniform64(it.e1);

    const int G = a.G, lph = a.lph;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int64_t rowbytes = (int64_t)a.R * 16;

    float q[NC][VN];
    bool act[NC], writer[NC];
    int head[NC];
    const char* qrow = (const char*)a.Q + it.row * rowbytes;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vi = c * G + gl;
        act[c] = vi < a.R;
        writer[c] = act[c] && (vi & (lph - 1)) == 0;
        head[c] = vi / lph;
        if (act[c]) {
            VT::unpack(ld16(qrow + vi * 16), q[c]);
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
            for (int c = 0; c < NC; ++c)
                kr[j][c] = (ok[j] && act[c]) ? ld16(Kb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : U4{0, 0, 0, 0};
        // the next batch's source ids load behind this batch's gathers
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(a.indices, nb, grp, epw, e1, un);
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float kf[VN];
                VT::unpack(kr[j][c], kf);
                float d = 0.0f;
#pragma unroll
                for (int k = 0; k < VN; ++k) d = __builtin_fmaf(q[c][k], kf[k], d);
                d = seg_sum(d, lph);
                if (ok[j] && writer[c]) a.scores_out[(eb + grp + (int64_t)j * epw) * a.H + head[c]] = d * a.qscale;
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
            if (ok[j] && gl == 0) a.scores_out[(e + (int64_t)j * epw) * a.H + h] = d * a.qscale;
        }
    }
}

template <int DT>
static hipError_t launch_sddmm_dt(const Args& a0, hipStream_t s) {
    const dim3 block(kBlock);
    if (a0.vec) {
        return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx);
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
