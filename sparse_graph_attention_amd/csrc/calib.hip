// calib.hip -- measurement aid: the K and V row gathers of the attention
// alone, for the achievable-rate ceiling beside the HBM peak.
//
// "Graph Transformer in a Nutshell", section "Sparse Multi-head Attention":
// every nonzero (v, u) of the adjacency matrix reads row u of K (the SDDMM)
// and row u of V (the SpMM).  This kernel reads exactly those rows, in CSR
// edge order, with the lane layout and 16-byte loads of the fused kernel's
// hot instances, and does nothing else with them: it folds every loaded word
// into an XOR checksum so that no load can be dropped, and the checksum lets
// a test confirm that each edge's rows were read whole.
#include <algorithm>

#include "kernels.hpp"

namespace gt {

namespace {

// Each wave reads a contiguous span of edges, sized so that the launch has
// about kCalibWaves waves: spans of 512 .. 16384 edges measured fastest at
// 3,700 .. 3,900 waves on both large benchmark graphs (about 15 per CU),
// up to 8% faster than 512-edge spans; far fewer waves starve the CUs.
constexpr int64_t kCalibWaves = 4096;
constexpr int kCalibU = 4;  // edges in flight per lane group

// G lanes per edge, NC 16-byte vectors per lane (row = NC * G vectors).
template <int NC, int G, bool NTL>
__global__ __launch_bounds__(kBlock) void calib_gather_kernel(const int32_t* __restrict__ indices, int64_t E,
                                                              int64_t span, const char* __restrict__ K,
                                                              const char* __restrict__ V, uint32_t* sink) {
    constexpr int epw = kWave / G;
    constexpr int64_t rowbytes = (int64_t)NC * G * 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int grp = lane / G, gl = lane & (G - 1);
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t e0 = wave * span;
    const int64_t e1 = e0 + span < E ? e0 + span : E;
    uint32_t x = 0;
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * kCalibU) {
        U4 kr[kCalibU][NC], vr[kCalibU][NC];
#pragma unroll
        for (int j = 0; j < kCalibU; ++j) {
            const int64_t e = eb + grp + (int64_t)j * epw;
            const bool ok = e < e1;
            const int64_t u = ok ? indices[e] : 0;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const char* pk = K + u * rowbytes + (c * G + gl) * 16;
                const char* pv = V + u * rowbytes + (c * G + gl) * 16;
                kr[j][c] = ok ? (NTL ? ld16_nt(pk) : ld16(pk)) : U4{0, 0, 0, 0};
                vr[j][c] = ok ? (NTL ? ld16_nt(pv) : ld16(pv)) : U4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int j = 0; j < kCalibU; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                x ^= kr[j][c].x ^ kr[j][c].y ^ kr[j][c].z ^ kr[j][c].w ^ vr[j][c].x ^ vr[j][c].y ^ vr[j][c].z ^
                     vr[j][c].w;
    }
    for (int off = 1; off < kWave; off <<= 1) x ^= (uint32_t)__shfl_xor((int)x, off, kWave);
    if (lane == 0 && e0 < E) atomicXor(sink, x);
}

template <int NC, int G>
void launch_calib(const int32_t* indices, int64_t E, const void* K, const void* V, bool ntl, uint32_t* sink,
                  hipStream_t s) {
    const int64_t span = std::max<int64_t>(64, (E / kCalibWaves + 63) / 64 * 64);
    const int64_t waves = (E + span - 1) / span;
    const unsigned grid = (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    if (ntl)
        calib_gather_kernel<NC, G, true><<<grid, kBlock, 0, s>>>(indices, E, span, (const char*)K, (const char*)V,
                                                                  sink);
    else
        calib_gather_kernel<NC, G, false><<<grid, kBlock, 0, s>>>(indices, E, span, (const char*)K, (const char*)V,
                                                                   sink);
}

}  // namespace

hipError_t launch_calib_gather(const int32_t* indices, int64_t E, const void* K, const void* V, int64_t n_rows,
                               int row_bytes, uint32_t* sink, hipStream_t s) {
    if (E == 0) return hipSuccess;
    // streamed like the fused kernel's fp32 hot instance when K and V exceed 1 GB
    const bool ntl = row_bytes == 2048 && 2 * n_rows * (int64_t)row_bytes > ((int64_t)1 << 30);
    switch (row_bytes) {
        case 512: launch_calib<1, 32>(indices, E, K, V, false, sink, s); break;
        case 1024: launch_calib<1, 64>(indices, E, K, V, false, sink, s); break;
        case 2048: launch_calib<2, 64>(indices, E, K, V, ntl, sink, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gt
