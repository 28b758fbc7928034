// bwd.hip -- backward of the fused sparse multi-head attention on gfx950.
//
// With s_e = <q_v, k_u>/sqrt(D), alpha_e = exp(s_e - lse_v) (lse saved by the
// forward) and out_v = sum_e alpha_e v_u, the chain rule through the softmax
// (Jacobian diag(alpha) - alpha alpha^T) gives, per head:
//   da_e    = dO_v . v_u
//   delta_v = sum over in-edges of alpha_e da_e = dO_v . out_v
//   ds_e    = alpha_e (da_e - delta_v)
//   dQ_v    = sum over in-edges of v of ds_e k_u / sqrt(D)
//   dK_u    = sum over out-edges of u of ds_e q_v / sqrt(D)
//   dV_u    = sum over out-edges of u of alpha_e dO_v
// The training loop that the "Graph Transformer in a Nutshell" tutorial runs
// (loss.backward() through bsddmm, softmax and bspmm) needs exactly these.
//
// Two passes, each with the forward's lane layouts and work items, and no
// float atomics (results are deterministic):
//  1. destination-sorted graph, one wave per row or chunk: gathers k_u and v_u
//     per in-edge, recomputes alpha from lse, accumulates dQ; writes delta.
//  2. source-sorted graph (the caller's transposed CSR), one wave per source
//     or chunk: gathers q_v and dO_v per out-edge, recomputes alpha and ds
//     from lse_v and delta_v, accumulates dK and dV.
// Chunks of split rows leave partial sums that a merge adds in chunk order.
#include <algorithm>

#include "kernels.hpp"

// The two passes' launchers compile as separate objects (bwd_dq.hip and
// bwd_dkv.hip include this file with GT_BWD_PART 1 and 2) so that their many
// kernel instances build in parallel; 0 compiles both.
#ifndef GT_BWD_PART
#define GT_BWD_PART 0
#endif

namespace gt {

// ------------------------------------------------------------ dQ, vector layout
// Template parameters as for the forward's fused_vec_kernel (G_, LPH_, FULL).
template <int DT, int NC, int U, int G_, int LPH_, int FULL, int XL, bool NTL = false>
__global__ __launch_bounds__(kBlock) void bwd_dq_vec_kernel(const Args a) {
    using VT = Vec<DT>;
    // hot instances: the heads per edge are known, so the batched dropout
    // words always fit and the per-lane fallback compiles away
    constexpr int kHc = (G_ && LPH_ && FULL) ? NC * G_ / LPH_ : 0;
    constexpr bool kBatched =
        kHc > 0 && (kWave / (G_ ? G_ : kWave)) * U * (kHc % 4 == 0 ? kHc / 4 : (kHc + 3) / 4 + 1) <= 64 * kDropRounds;
    constexpr int kDropMB = kBatched ? drop_batches_per_eval(kWave / (G_ ? G_ : kWave), U, kHc) : 1;
    constexpr bool kSlots = kHc > 0 && (kWave / (G_ ? G_ : kWave)) * U * kHc <= 64 * kSlotRounds;
    // rounds of 64 values for a batch's bias and weights (exact for the hot instances)
    constexpr int kBR = kSlots ? ((kWave / G_) * U * kHc + 63) / 64 : kSlotRounds;
    constexpr int kWR = kSlots ? ((kWave / G_) * U + 63) / 64 : kSlotRounds;
    constexpr int VN = VT::n;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t row = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);

    const int G = G_ ? G_ : a.G;
    const int lph = LPH_ ? LPH_ : a.lph;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    // FULL 1: no idle lane slots; 2: every slot in a head, heads padded (vph < lph);
    // 0: slots past the row's end too
    const int vph = FULL == 1 ? lph : a.vph;
    const int64_t rowbytes = (int64_t)(FULL == 1 ? a.R : a.Rm) * 16;
    const int64_t HD = (int64_t)a.H * a.D;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);

    // row data: q, dO, and per head delta = dO . out and lse (log2 units)
    float q[NC][VN], g[NC][VN], dl[NC], ls[NC];
    bool act[NC];
    int head[NC], moff[NC];  // moff: byte offset of the lane slot's vector in a row
    const char* qrow = (const char*)a.Q + row * rowbytes;
    const char* grow = (const char*)a.dO + row * rowbytes;
    const char* orow = (const char*)a.O + row * rowbytes;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vi = c * G + gl;
        const bool in_row = FULL || vi < a.R;  // a slot of some head (it may idle)
        act[c] = in_row && (vi & (lph - 1)) < vph;
        head[c] = in_row ? vi / lph : 0;
        moff[c] = FULL == 1 ? vi * 16 : (head[c] * vph + (vi & (lph - 1))) * 16;
        const U4 zero{0, 0, 0, 0};
        VT::unpack(act[c] ? ld16(qrow + moff[c]) : zero, q[c]);
        VT::unpack(act[c] ? ld16(grow + moff[c]) : zero, g[c]);
        float o[VN];
        VT::unpack(act[c] ? ld16(orow + moff[c]) : zero, o);
        float d = 0.0f;
#pragma unroll
        for (int k = 0; k < VN; ++k) d = __builtin_fmaf(g[c][k], o[k], d);
        dl[c] = LPH_ ? seg_sum_c<LPH_>(d) : seg_sum(d, lph);
        ls[c] = in_row ? a.lse_in[row * a.H + vi / lph] * kLog2e : 0.0f;
    }
    float acc[NC][VN];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < VN; ++k) acc[c][k] = 0.0f;

    const char* Kb = (const char*)a.K;
    const char* Vb = (const char*)a.V;
    DropBatch db;
    int dph = 0;  // position of the batch among those its keep bits were drawn for
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U, dph = dph + 1 == kDropMB ? 0 : dph + 1) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        auto ej = [&](int j) -> int64_t { return ok[j] ? eb + grp + (int64_t)j * epw : e0; };
        float xw[U], xb[U][NC];
        SlotBatch<kBR> bb;
        SlotBatch<kWR> wb;
        bool sb = false;
        if constexpr (XL) {  // ahead of the gathers: waiting for them never waits for a gather
            sb = kSlots || slot_batched(epw * U, a.H);
            if (sb) {
                if (a.bias) slot_batch_load(bb, a.bias, eb, e1, epw * U, a.H, lane);
                if (a.ew) slot_batch_load(wb, a.ew, eb, e1, epw * U, 1, lane);
            } else {
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    xw[j] = a.ew ? a.ew[ej(j)] : 1.0f;
#pragma unroll
                    for (int c = 0; c < NC; ++c) xb[j][c] = a.bias ? a.bias[ej(j) * a.H + head[c]] * kLog2e : 0.0f;
                }
            }
        }
        U4 kr[U][NC], vr[U][NC];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                kr[j][c] = (ok[j] && act[c]) ? (NTL ? ld16_nt(Kb + (int64_t)u[j] * rowbytes + moff[c]) : ld16(Kb + (int64_t)u[j] * rowbytes + moff[c])) : U4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                vr[j][c] = (ok[j] && act[c]) ? (NTL ? ld16_nt(Vb + (int64_t)u[j] * rowbytes + moff[c]) : ld16(Vb + (int64_t)u[j] * rowbytes + moff[c])) : U4{0, 0, 0, 0};
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
        bool bdrop = false;
        if constexpr (XL) {
            bdrop = XL == 2 && (kBatched || drop_batched(a.H, -1, epw * U));
            // one evaluation covers kDropMB consecutive batches (consecutive edges)
            if (bdrop && dph == 0)
                drop_batch_init(db, a.drop_seed, a.drop_thresh, a.H, -1, kDropMB * epw * U, lane,
                                [&](int k) { return eb + k; });
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float tw = 0.0f;  // extended: sum over this lane's heads of ds * <q, k> / sqrt(D)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float kf[VN], vf[VN];
                VT::unpack(kr[j][c], kf);
                VT::unpack(vr[j][c], vf);
                float sd = 0.0f, dd = 0.0f;
#pragma unroll
                for (int k = 0; k < VN; ++k) {
                    sd = __builtin_fmaf(q[c][k], kf[k], sd);
                    dd = __builtin_fmaf(g[c][k], vf[k], dd);
                }
                sd = (LPH_ ? seg_sum_c<LPH_>(sd) : seg_sum(sd, lph)) * a.qscale;
                dd = LPH_ ? seg_sum_c<LPH_>(dd) : seg_sum(dd, lph);
                if constexpr (XL) {
                    const float raw = sd;
                    const int k = grp + j * epw;
                    const float w = sb ? (a.ew ? slot_batch_get(wb, k) : 1.0f) : xw[j];
                    const float b = sb ? (a.bias ? slot_batch_get(bb, k * a.H + head[c]) * kLog2e : 0.0f) : xb[j][c];
                    sd = __builtin_fmaf(sd, w, b);
                    const float p = ok[j] ? exp2_(sd - ls[c]) : 0.0f;
                    float keep = 1.0f;
                    if (XL == 2 && (kBatched || bdrop))
                        keep = drop_mult(db, a.drop_scale, a.H, -1, dph * epw * U + grp + j * epw, ej(j), head[c]);
                    else if (XL == 2 && !kBatched)
                        keep = philox_hi32(a.drop_seed, (uint64_t)ej(j) * a.H + head[c]) >= a.drop_thresh
                                   ? a.drop_scale : 0.0f;
                    const float ds = p * (keep * dd - dl[c]);
                    const bool lead = ok[j] && act[c] && (gl & (lph - 1)) == 0;
                    if (a.dbias && lead) a.dbias[ej(j) * a.H + head[c]] = ds;
                    if (lead) tw = __builtin_fmaf(ds, raw * kLn2, tw);
                    const float dsw = ds * w;
#pragma unroll
                    for (int k = 0; k < VN; ++k) acc[c][k] = __builtin_fmaf(dsw, kf[k], acc[c][k]);
                } else {
                    const float p = ok[j] ? exp2_(sd - ls[c]) : 0.0f;
                    const float ds = p * (dd - dl[c]);
#pragma unroll
                    for (int k = 0; k < VN; ++k) acc[c][k] = __builtin_fmaf(ds, kf[k], acc[c][k]);
                }
            }
            if constexpr (XL)
                if (a.dew) {
                    tw = seg_sum(tw, G);  // over the group's heads
                    if (ok[j] && gl == 0) a.dew[ej(j)] = tw;
                }
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VN; ++k) acc[c][k] += __shfl_xor(acc[c][k], off, kWave);
    if (grp != 0) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (!act[c]) continue;
        const int vi = c * G + gl;
        if ((vi & (lph - 1)) == 0) a.stats[row * a.H + vi / lph] = make_float2(ls[c], dl[c]);
        if (it.slot < 0) {
            float o[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) o[k] = acc[c][k] * a.kscale;
            st16_nt((char*)a.dQ + row * rowbytes + moff[c], VT::pack(o));
        } else {
            float* pa = a.plan.pacc + it.slot * HD + (int64_t)(moff[c] / 16) * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) st16(pa + k, Vec<kF32>::pack(&acc[c][k]));
        }
    }
}

// ------------------------------------------------------------ dK, dV, vector layout
// a.indptr / a.indices are the source-sorted graph: item rows are sources u,
// "edges" are their out-edges with the destination v in a.indices.
template <int DT, int NC, int U, int G_, int LPH_, int FULL, int XL>
__global__ __launch_bounds__(kBlock) void bwd_dkv_vec_kernel(const Args a) {
    using VT = Vec<DT>;
    // hot instances: the heads per edge are known, so the batched dropout
    // words always fit and the per-lane fallback compiles away
    constexpr int kHc = (G_ && LPH_ && FULL) ? NC * G_ / LPH_ : 0;
    constexpr bool kBatched =
        kHc > 0 && (kWave / (G_ ? G_ : kWave)) * U * (kHc % 4 == 0 ? kHc / 4 : (kHc + 3) / 4 + 1) <= 64 * kDropRounds;
    constexpr int kDropMB = kBatched ? drop_batches_per_eval(kWave / (G_ ? G_ : kWave), U, kHc) : 1;
    constexpr bool kSlots = kHc > 0 && (kWave / (G_ ? G_ : kWave)) * U * kHc <= 64 * kSlotRounds;
    // rounds of 64 values for a batch's bias and weights (exact for the hot instances)
    constexpr int kBR = kSlots ? ((kWave / G_) * U * kHc + 63) / 64 : kSlotRounds;
    constexpr int kWR = kSlots ? ((kWave / G_) * U + 63) / 64 : kSlotRounds;
    constexpr int VN = VT::n;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t src = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);

    const int G = G_ ? G_ : a.G;
    const int lph = LPH_ ? LPH_ : a.lph;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    // FULL 1: no idle lane slots; 2: every slot in a head, heads padded (vph < lph);
    // 0: slots past the row's end too
    const int vph = FULL == 1 ? lph : a.vph;
    const int64_t rowbytes = (int64_t)(FULL == 1 ? a.R : a.Rm) * 16;
    const int64_t HD = (int64_t)a.H * a.D;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U], pn[U];  // destinations and (extended) their CSR positions
    if (e1 > e0) {
        load_ids<U>(idx, e0, grp, epw, e1, un);
        if constexpr (XL) load_ids<U>(a.t_perm, e0, grp, epw, e1, pn);
    }

    float kk[NC][VN], vv[NC][VN];
    bool act[NC];
    int head[NC], moff[NC];  // moff: byte offset of the lane slot's vector in a row
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vi = c * G + gl;
        const bool in_row = FULL || vi < a.R;  // a slot of some head (it may idle)
        act[c] = in_row && (vi & (lph - 1)) < vph;
        head[c] = in_row ? vi / lph : 0;
        moff[c] = FULL == 1 ? vi * 16 : (head[c] * vph + (vi & (lph - 1))) * 16;
        const U4 zero{0, 0, 0, 0};
        VT::unpack(act[c] ? ld16((const char*)a.K + src * rowbytes + moff[c]) : zero, kk[c]);
        VT::unpack(act[c] ? ld16((const char*)a.V + src * rowbytes + moff[c]) : zero, vv[c]);
    }
    float dk[NC][VN], dv[NC][VN];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < VN; ++k) dk[c][k] = dv[c][k] = 0.0f;
    // per-head values of an edge are loaded by lane h of the group for head h
    // (H <= G in this layout) and handed to the lanes of head h by a shuffle
    const int hsrc = gl < a.H ? gl : 0;
    const int gbase = grp * G;

    const char* Qb = (const char*)a.Q;
    const char* Gb = (const char*)a.dO;
    DropBatch db;
    int dph = 0;  // position of the batch among those its keep bits were drawn for
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U, dph = dph + 1 == kDropMB ? 0 : dph + 1) {
        int32_t u[U], ep[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            if constexpr (XL) ep[j] = pn[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        // per-edge inputs at the out-edges' CSR positions ep (prefetched with
        // the destinations): the batch's positions go round the lanes by
        // shuffles, each lane loading one value per round
        float xw[U], xb[U][NC];
        SlotBatch<kBR> bb;
        SlotBatch<kWR> wb;
        bool sb = false;
        if constexpr (XL) {
            sb = kSlots || slot_batched(epw * U, a.H);
            if (sb) {
                auto pos_of = [&](int k) -> int64_t {  // slot k: ep[k / epw] of group k % epw
                    int64_t r = 0;
#pragma unroll
                    for (int jj = 0; jj < U; ++jj) {
                        const int v = __shfl(ep[jj], (k % epw) * G, kWave);
                        if (jj == k / epw) r = v;
                    }
                    return r;
                };
                if (a.bias) slot_batch_load_at(bb, a.bias, e1 - eb, epw * U, a.H, lane, pos_of);
                if (a.ew) slot_batch_load_at(wb, a.ew, e1 - eb, epw * U, 1, lane, pos_of);
            } else {
#pragma unroll
                for (int j = 0; j < U; ++j) {  // a clamped slot's ep is still a valid position
                    xw[j] = a.ew ? a.ew[ep[j]] : 1.0f;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        xb[j][c] = a.bias ? a.bias[(int64_t)ep[j] * a.H + head[c]] * kLog2e : 0.0f;
                }
            }
        }
        U4 qr[U][NC], gr[U][NC];
        float2 st[U];  // the destination's (lse, delta) of head hsrc: one 8-byte load per edge
#pragma unroll
        for (int j = 0; j < U; ++j) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bool go = ok[j] && act[c];
                qr[j][c] = go ? ld16(Qb + (int64_t)u[j] * rowbytes + moff[c]) : U4{0, 0, 0, 0};
                gr[j][c] = go ? ld16(Gb + (int64_t)u[j] * rowbytes + moff[c]) : U4{0, 0, 0, 0};
            }
            st[j] = ok[j] ? a.stats[(int64_t)u[j] * a.H + hsrc] : make_float2(0.0f, 0.0f);
        }
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) {
            load_ids<U>(idx, nb, grp, epw, e1, un);
            if constexpr (XL) load_ids<U>(a.t_perm, nb, grp, epw, e1, pn);
        }
        bool bdrop = false;
        if constexpr (XL) {
            bdrop = XL == 2 && (kBatched || drop_batched(a.H, -1, epw * U));
            // one evaluation covers kDropMB consecutive batches, whose CSR
            // positions are the run t_perm[eb ..] (read directly); for a single
            // batch, slot k's position sits in ep[k / epw] of group k % epw
            if (bdrop && dph == 0)
                drop_batch_init(db, a.drop_seed, a.drop_thresh, a.H, -1, kDropMB * epw * U, lane, [&](int k) {
                    int64_t r = 0;
                    if constexpr (kDropMB > 1) {
                        r = a.t_perm[eb + k < e1 ? eb + k : e1 - 1];
                    } else {
#pragma unroll
                        for (int jj = 0; jj < U; ++jj) {
                            const int v = __shfl(ep[jj], (k % epw) * G, kWave);
                            if (jj == k / epw) r = v;
                        }
                    }
                    return r;
                });
        }
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float qf[VN], gf[VN];
                VT::unpack(qr[j][c], qf);
                VT::unpack(gr[j][c], gf);
                float sd = 0.0f, dd = 0.0f;
#pragma unroll
                for (int k = 0; k < VN; ++k) {
                    sd = __builtin_fmaf(qf[k], kk[c][k], sd);
                    dd = __builtin_fmaf(gf[k], vv[c][k], dd);
                }
                sd = (LPH_ ? seg_sum_c<LPH_>(sd) : seg_sum(sd, lph)) * a.qscale;
                dd = LPH_ ? seg_sum_c<LPH_>(dd) : seg_sum(dd, lph);
                const float lsj = __shfl(st[j].x, gbase + head[c], kWave);
                const float dlj = __shfl(st[j].y, gbase + head[c], kWave);
                if constexpr (XL) {
                    const int k = grp + j * epw;
                    const float w = sb ? (a.ew ? slot_batch_get(wb, k) : 1.0f) : xw[j];
                    const float b = sb ? (a.bias ? slot_batch_get(bb, k * a.H + head[c]) * kLog2e : 0.0f) : xb[j][c];
                    sd = __builtin_fmaf(sd, w, b);
                    const float p = ok[j] ? exp2_(sd - lsj) : 0.0f;
                    float keep = 1.0f;
                    if (XL == 2 && (kBatched || bdrop))
                        keep = drop_mult(db, a.drop_scale, a.H, -1, dph * epw * U + grp + j * epw, ep[j], head[c]);
                    else if (XL == 2 && !kBatched)
                        keep = philox_hi32(a.drop_seed, (uint64_t)ep[j] * a.H + head[c]) >= a.drop_thresh
                                   ? a.drop_scale : 0.0f;
                    const float pk = p * keep;
                    const float dsw = p * (keep * dd - dlj) * w;
#pragma unroll
                    for (int k = 0; k < VN; ++k) {
                        dv[c][k] = __builtin_fmaf(pk, gf[k], dv[c][k]);
                        dk[c][k] = __builtin_fmaf(dsw, qf[k], dk[c][k]);
                    }
                } else {
                    const float p = ok[j] ? exp2_(sd - lsj) : 0.0f;
                    const float ds = p * (dd - dlj);
#pragma unroll
                    for (int k = 0; k < VN; ++k) {
                        dv[c][k] = __builtin_fmaf(p, gf[k], dv[c][k]);
                        dk[c][k] = __builtin_fmaf(ds, qf[k], dk[c][k]);
                    }
                }
            }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                dk[c][k] += __shfl_xor(dk[c][k], off, kWave);
                dv[c][k] += __shfl_xor(dv[c][k], off, kWave);
            }
    if (grp != 0) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (!act[c]) continue;
        if (it.slot < 0) {
            float o[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) o[k] = dk[c][k] * a.kscale;
            st16_nt((char*)a.dK + src * rowbytes + moff[c], VT::pack(o));
            st16_nt((char*)a.dV + src * rowbytes + moff[c], VT::pack(dv[c]));
        } else {
            float* pa = a.plan.pacc + it.slot * 2 * HD + (int64_t)(moff[c] / 16) * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) {
                st16(pa + k, Vec<kF32>::pack(&dk[c][k]));
                st16(pa + HD + k, Vec<kF32>::pack(&dv[c][k]));
            }
        }
    }
}

// ------------------------------------------------------------ scalar layout
// One wave per (item, head h = blockIdx.y); groups of G = pow2ceil(D) lanes,
// lane j holding elements j + k*G, k < KD.
template <int DT, int KD, int U, int XL>
__global__ __launch_bounds__(kBlock) void bwd_dq_scalar_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr bool kBatched = false;  // the batch size depends on D and H: checked at run time
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y;
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t row = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);
    const int G = a.G, D = a.D;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int64_t HD = (int64_t)a.H * D;
    const int64_t hoff = (int64_t)h * D;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);
    float q[KD], g[KD];
    bool act[KD];
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int dd = gl + k * G;
        act[k] = dd < D;
        q[k] = act[k] ? VT::scalar(a.Q, row * HD + hoff + dd) : 0.0f;
        g[k] = act[k] ? VT::scalar(a.dO, row * HD + hoff + dd) : 0.0f;
        d = __builtin_fmaf(g[k], act[k] ? VT::scalar(a.O, row * HD + hoff + dd) : 0.0f, d);
    }
    const float dl = seg_sum(d, G);
    const float ls = a.lse_in[row * a.H + h] * kLog2e;
    float acc[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) acc[k] = 0.0f;
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        auto ej = [&](int j) -> int64_t { return ok[j] ? eb + grp + (int64_t)j * epw : e0; };
        float xw[U], xb[U];
        if constexpr (XL) {
#pragma unroll
            for (int j = 0; j < U; ++j) {
                xw[j] = a.ew ? a.ew[ej(j)] : 1.0f;
                xb[j] = a.bias ? a.bias[ej(j) * a.H + h] * kLog2e : 0.0f;
            }
        }
        float kv[U][KD], vv[U][KD];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                const bool go = ok[j] && act[k];
                kv[j][k] = go ? VT::scalar(a.K, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
                vv[j][k] = go ? VT::scalar(a.V, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
            }
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
        DropBatch db;
        bool bdrop = false;
        if constexpr (XL) {
            bdrop = XL == 2 && (kBatched || drop_batched(a.H, h, epw * U));
            if (bdrop)
                drop_batch_init(db, a.drop_seed, a.drop_thresh, a.H, h, epw * U, lane, [&](int k) { return eb + k; });
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float sd = 0.0f, dd = 0.0f;
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                sd = __builtin_fmaf(q[k], kv[j][k], sd);
                dd = __builtin_fmaf(g[k], vv[j][k], dd);
            }
            sd = seg_sum(sd, G) * a.qscale;
            dd = seg_sum(dd, G);
            if constexpr (XL) {
                const float raw = sd;
                sd = __builtin_fmaf(sd, xw[j], xb[j]);
                const float p = ok[j] ? exp2_(sd - ls) : 0.0f;
                float keep = 1.0f;
                if (XL == 2 && (kBatched || bdrop))
                    keep = drop_mult(db, a.drop_scale, a.H, h, grp + j * epw, ej(j), h);
                else if (XL == 2 && !kBatched)
                    keep = philox_hi32(a.drop_seed, (uint64_t)ej(j) * a.H + h) >= a.drop_thresh ? a.drop_scale : 0.0f;
                const float ds = p * (keep * dd - dl);
                // one wave per head: the per-head terms of dw go to scratch and
                // sum_heads_kernel adds them up in head order
                if (ok[j] && gl == 0) {
                    if (a.dbias) a.dbias[ej(j) * a.H + h] = ds;
                    if (a.dew) a.dew_part[ej(j) * a.H + h] = ds * raw * kLn2;
                }
                const float dsw = ds * xw[j];
#pragma unroll
                for (int k = 0; k < KD; ++k) acc[k] = __builtin_fmaf(dsw, kv[j][k], acc[k]);
            } else {
                const float p = ok[j] ? exp2_(sd - ls) : 0.0f;
                const float ds = p * (dd - dl);
#pragma unroll
                for (int k = 0; k < KD; ++k) acc[k] = __builtin_fmaf(ds, kv[j][k], acc[k]);
            }
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[k] += __shfl_xor(acc[k], off, kWave);
    if (grp != 0) return;
    if (gl == 0) a.stats[row * a.H + h] = make_float2(ls, dl);
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        if (!act[k]) continue;
        if (it.slot < 0)
            VT::store_scalar(a.dQ, row * HD + hoff + gl + k * G, acc[k] * a.kscale);
        else
            a.plan.pacc[it.slot * HD + hoff + gl + k * G] = acc[k];
    }
}

template <int DT, int KD, int U, int XL>
__global__ __launch_bounds__(kBlock) void bwd_dkv_scalar_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr bool kBatched = false;  // the batch size depends on D and H: checked at run time
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y;
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t src = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);
    const int G = a.G, D = a.D;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int64_t HD = (int64_t)a.H * D;
    const int64_t hoff = (int64_t)h * D;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U], pn[U];
    if (e1 > e0) {
        load_ids<U>(idx, e0, grp, epw, e1, un);
        if constexpr (XL) load_ids<U>(a.t_perm, e0, grp, epw, e1, pn);
    }
    float kk[KD], vv[KD], dk[KD], dv[KD];
    bool act[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int dd = gl + k * G;
        act[k] = dd < D;
        kk[k] = act[k] ? VT::scalar(a.K, src * HD + hoff + dd) : 0.0f;
        vv[k] = act[k] ? VT::scalar(a.V, src * HD + hoff + dd) : 0.0f;
        dk[k] = dv[k] = 0.0f;
    }
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U], ep[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            if constexpr (XL) ep[j] = pn[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        float xw[U], xb[U];
        if constexpr (XL) {  // per-edge inputs at the out-edges' CSR positions
#pragma unroll
            for (int j = 0; j < U; ++j) {
                xw[j] = a.ew ? a.ew[ep[j]] : 1.0f;
                xb[j] = a.bias ? a.bias[(int64_t)ep[j] * a.H + h] * kLog2e : 0.0f;
            }
        }
        float qv[U][KD], gv[U][KD], ls[U], dl[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                const bool go = ok[j] && act[k];
                qv[j][k] = go ? VT::scalar(a.Q, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
                gv[j][k] = go ? VT::scalar(a.dO, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
            }
            const float2 t = ok[j] ? a.stats[(int64_t)u[j] * a.H + h] : make_float2(0.0f, 0.0f);
            ls[j] = t.x;
            dl[j] = t.y;
        }
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) {
            load_ids<U>(idx, nb, grp, epw, e1, un);
            if constexpr (XL) load_ids<U>(a.t_perm, nb, grp, epw, e1, pn);
        }
        DropBatch db;
        bool bdrop = false;
        if constexpr (XL) {
            bdrop = XL == 2 && (kBatched || drop_batched(a.H, h, epw * U));
            if (bdrop)
                drop_batch_init(db, a.drop_seed, a.drop_thresh, a.H, h, epw * U, lane, [&](int k) {
                    int64_t r = 0;
#pragma unroll
                    for (int jj = 0; jj < U; ++jj) {
                        const int v = __shfl(ep[jj], (k % epw) * G, kWave);
                        if (jj == k / epw) r = v;
                    }
                    return r;
                });
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float sd = 0.0f, dd = 0.0f;
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                sd = __builtin_fmaf(qv[j][k], kk[k], sd);
                dd = __builtin_fmaf(gv[j][k], vv[k], dd);
            }
            sd = seg_sum(sd, G) * a.qscale;
            dd = seg_sum(dd, G);
            if constexpr (XL) {
                sd = __builtin_fmaf(sd, xw[j], xb[j]);
                const float p = ok[j] ? exp2_(sd - ls[j]) : 0.0f;
                float keep = 1.0f;
                if (XL == 2 && (kBatched || bdrop))
                    keep = drop_mult(db, a.drop_scale, a.H, h, grp + j * epw, ep[j], h);
                else if (XL == 2 && !kBatched)
                    keep = philox_hi32(a.drop_seed, (uint64_t)ep[j] * a.H + h) >= a.drop_thresh ? a.drop_scale : 0.0f;
                const float pk = p * keep;
                const float dsw = p * (keep * dd - dl[j]) * xw[j];
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    dv[k] = __builtin_fmaf(pk, gv[j][k], dv[k]);
                    dk[k] = __builtin_fmaf(dsw, qv[j][k], dk[k]);
                }
            } else {
                const float p = ok[j] ? exp2_(sd - ls[j]) : 0.0f;
                const float ds = p * (dd - dl[j]);
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    dv[k] = __builtin_fmaf(p, gv[j][k], dv[k]);
                    dk[k] = __builtin_fmaf(ds, qv[j][k], dk[k]);
                }
            }
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            dk[k] += __shfl_xor(dk[k], off, kWave);
            dv[k] += __shfl_xor(dv[k], off, kWave);
        }
    if (grp != 0) return;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        if (!act[k]) continue;
        const int64_t o = hoff + gl + k * G;
        if (it.slot < 0) {
            VT::store_scalar(a.dK, src * HD + o, dk[k] * a.kscale);
            VT::store_scalar(a.dV, src * HD + o, dv[k]);
        } else {
            a.plan.pacc[it.slot * 2 * HD + o] = dk[k];
            a.plan.pacc[it.slot * 2 * HD + HD + o] = dv[k];
        }
    }
}

// ------------------------------------------------------------ head-innermost layout
//
// Features [N][D][H]: lane gl of a group holds vectors vi = c * G + gl, c <
// NC, of a row (d = vi / HV, heads (vi % HV) * VN .. +VN-1), as in the
// forward's fused_ndh_kernel; per-head sums add the lane's products over c,
// then run over the lanes with the same gl % HV.  Partials of split rows keep
// the row's [D][H] order; the merge adds them elementwise.

// Sum over the lanes of a group that hold the same heads.
__device__ __forceinline__ float ndh_head_sum(float x, int HV, int G) {
    for (int off = HV; off < G; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

template <int DT, int U, int NC>
__global__ __launch_bounds__(kBlock) void bwd_dq_ndh_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr int VN = VT::n;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t row = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);
    const int G = a.G, HV = a.lph;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int hg = gl & (HV - 1);
    bool act[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) act[c] = c * G + gl < a.R;
    const int64_t rowbytes = (int64_t)a.R * 16;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);
    const U4 zero{0, 0, 0, 0};
    float q[NC][VN], g[NC][VN], dl[VN], ls[VN], acc[NC][VN];
#pragma unroll
    for (int k = 0; k < VN; ++k) dl[k] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t off = row * rowbytes + (c * G + gl) * 16;
        float o[VN];
        VT::unpack(act[c] ? ld16((const char*)a.Q + off) : zero, q[c]);
        VT::unpack(act[c] ? ld16((const char*)a.dO + off) : zero, g[c]);
        VT::unpack(act[c] ? ld16((const char*)a.O + off) : zero, o);
#pragma unroll
        for (int k = 0; k < VN; ++k) {
            dl[k] = __builtin_fmaf(g[c][k], o[k], dl[k]);
            acc[c][k] = 0.0f;
        }
    }
#pragma unroll
    for (int k = 0; k < VN; ++k) {
        dl[k] = ndh_head_sum(dl[k], HV, G);
        ls[k] = a.lse_in[row * a.H + hg * VN + k] * kLog2e;
    }
    const char* Kb = (const char*)a.K;
    const char* Vb = (const char*)a.V;
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        U4 kr[U][NC], vr[U][NC];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                kr[j][c] = (ok[j] && act[c]) ? ld16(Kb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : zero;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                vr[j][c] = (ok[j] && act[c]) ? ld16(Vb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : zero;
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float kf[NC][VN], sd[VN], dd[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) sd[k] = dd[k] = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float vf[VN];
                VT::unpack(kr[j][c], kf[c]);
                VT::unpack(vr[j][c], vf);
#pragma unroll
                for (int k = 0; k < VN; ++k) {
                    sd[k] = __builtin_fmaf(q[c][k], kf[c][k], sd[k]);
                    dd[k] = __builtin_fmaf(g[c][k], vf[k], dd[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                const float s2 = ndh_head_sum(sd[k], HV, G) * a.qscale;
                const float da = ndh_head_sum(dd[k], HV, G);
                const float p = ok[j] ? exp2_(s2 - ls[k]) : 0.0f;
                const float ds = p * (da - dl[k]);
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[c][k] = __builtin_fmaf(ds, kf[c][k], acc[c][k]);
            }
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VN; ++k) acc[c][k] += __shfl_xor(acc[c][k], off, kWave);
    if (grp != 0) return;
    if (gl < HV)  // the lanes of d = 0 (in c = 0) carry each head's (lse, delta) once
#pragma unroll
        for (int k = 0; k < VN; ++k) a.stats[row * a.H + hg * VN + k] = make_float2(ls[k], dl[k]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (!act[c]) continue;
        const int vi = c * G + gl;
        if (it.slot < 0) {
            float r[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) r[k] = acc[c][k] * a.kscale;
            st16_nt((char*)a.dQ + row * rowbytes + vi * 16, VT::pack(r));
        } else {
            float* pa = a.plan.pacc + it.slot * (int64_t)a.H * a.D + (int64_t)vi * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) st16(pa + k, Vec<kF32>::pack(&acc[c][k]));
        }
    }
}

template <int DT, int U, int NC>
__global__ __launch_bounds__(kBlock) void bwd_dkv_ndh_kernel(const Args a) {
    using VT = Vec<DT>;
    constexpr int VN = VT::n;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t src = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);
    const int G = a.G, HV = a.lph;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int hg = gl & (HV - 1);
    bool act[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) act[c] = c * G + gl < a.R;
    const int64_t rowbytes = (int64_t)a.R * 16;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);
    const U4 zero{0, 0, 0, 0};
    float kk[NC][VN], vv[NC][VN], dk[NC][VN], dv[NC][VN];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t off = src * rowbytes + (c * G + gl) * 16;
        VT::unpack(act[c] ? ld16((const char*)a.K + off) : zero, kk[c]);
        VT::unpack(act[c] ? ld16((const char*)a.V + off) : zero, vv[c]);
#pragma unroll
        for (int k = 0; k < VN; ++k) dk[c][k] = dv[c][k] = 0.0f;
    }
    const char* Qb = (const char*)a.Q;
    const char* Gb = (const char*)a.dO;
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        U4 qr[U][NC], gr[U][NC];
        float2 st[U][VN];
#pragma unroll
        for (int j = 0; j < U; ++j) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bool go = ok[j] && act[c];
                qr[j][c] = go ? ld16(Qb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : zero;
                gr[j][c] = go ? ld16(Gb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : zero;
            }
            // the VN (lse, delta) pairs of the lane's heads are contiguous: 16-byte loads
            const char* sp = (const char*)(a.stats + (int64_t)u[j] * a.H + hg * VN);
#pragma unroll
            for (int k = 0; k < VN; k += 2) {
                const U4 t = ok[j] ? ld16(sp + k * 8) : U4{0, 0, 0, 0};
                st[j][k] = make_float2(__uint_as_float(t.x), __uint_as_float(t.y));
                st[j][k + 1] = make_float2(__uint_as_float(t.z), __uint_as_float(t.w));
            }
        }
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float qf[NC][VN], gf[NC][VN], sd[VN], dd[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) sd[k] = dd[k] = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                VT::unpack(qr[j][c], qf[c]);
                VT::unpack(gr[j][c], gf[c]);
#pragma unroll
                for (int k = 0; k < VN; ++k) {
                    sd[k] = __builtin_fmaf(qf[c][k], kk[c][k], sd[k]);
                    dd[k] = __builtin_fmaf(gf[c][k], vv[c][k], dd[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                const float s2 = ndh_head_sum(sd[k], HV, G) * a.qscale;
                const float da = ndh_head_sum(dd[k], HV, G);
                const float p = ok[j] ? exp2_(s2 - st[j][k].x) : 0.0f;
                const float ds = p * (da - st[j][k].y);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    dv[c][k] = __builtin_fmaf(p, gf[c][k], dv[c][k]);
                    dk[c][k] = __builtin_fmaf(ds, qf[c][k], dk[c][k]);
                }
            }
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                dk[c][k] += __shfl_xor(dk[c][k], off, kWave);
                dv[c][k] += __shfl_xor(dv[c][k], off, kWave);
            }
    if (grp != 0) return;
    const int64_t HD = (int64_t)a.H * a.D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (!act[c]) continue;
        const int vi = c * G + gl;
        if (it.slot < 0) {
            float r[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) r[k] = dk[c][k] * a.kscale;
            st16_nt((char*)a.dK + src * rowbytes + vi * 16, VT::pack(r));
            st16_nt((char*)a.dV + src * rowbytes + vi * 16, VT::pack(dv[c]));
        } else {
            float* pa = a.plan.pacc + it.slot * 2 * HD + (int64_t)vi * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) {
                st16(pa + k, Vec<kF32>::pack(&dk[c][k]));
                st16(pa + HD + k, Vec<kF32>::pack(&dv[c][k]));
            }
        }
    }
}

// ------------------------------------------------------------ word layout
//
// [N][H][D] rows whose heads are whole 8- or 4-byte words but not 16-byte
// vectors (fp32 heads of 10 elements: five 8-byte words), laid out as in the
// forward's fused_word_kernel: head h, word j of an edge sit in lane slot
// h * LPH + j of a G-lane group, a per-head sum is a DPP sum over an aligned
// LPH-lane segment, and the 64 / G groups of a wave take different edges.
// Partials of split rows keep the row's [H][D] order.
template <int DT, int WB, int LPH, int U>
__global__ __launch_bounds__(kBlock) void bwd_dq_word_kernel(const Args a) {
    constexpr int EW = Word<DT, WB>::EW;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t row = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);
    const int G = a.G;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int head = gl / LPH, j = gl % LPH;
    const bool hv = head < a.H;
    const bool act = hv && j < a.vph;
    const int64_t rowbytes = (int64_t)a.H * a.vph * WB;
    const int moff = (head * a.vph + j) * WB;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);
    float q[EW], g[EW], o[EW], acc[EW];
    {
        const int64_t off = row * rowbytes + moff;
        unpack_word<DT, WB>(act ? ldw<DT, WB>((const char*)a.Q + off) : zero_word<DT, WB>(), q);
        unpack_word<DT, WB>(act ? ldw<DT, WB>((const char*)a.dO + off) : zero_word<DT, WB>(), g);
        unpack_word<DT, WB>(act ? ldw<DT, WB>((const char*)a.O + off) : zero_word<DT, WB>(), o);
    }
    float dl = 0.0f;
#pragma unroll
    for (int k = 0; k < EW; ++k) {
        dl = __builtin_fmaf(g[k], o[k], dl);
        acc[k] = 0.0f;
    }
    dl = seg_sum_c<LPH>(dl);
    const float ls = hv ? a.lse_in[row * a.H + head] * kLog2e : 0.0f;
    const char* Kb = (const char*)a.K;
    const char* Vb = (const char*)a.V;
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            u[jj] = un[jj];
            ok[jj] = eb + grp + (int64_t)jj * epw < e1;
        }
        Word<DT, WB> kr[U], vr[U];
#pragma unroll
        for (int jj = 0; jj < U; ++jj)
            kr[jj] = (ok[jj] && act) ? ldw<DT, WB>(Kb + (int64_t)u[jj] * rowbytes + moff) : zero_word<DT, WB>();
#pragma unroll
        for (int jj = 0; jj < U; ++jj)
            vr[jj] = (ok[jj] && act) ? ldw<DT, WB>(Vb + (int64_t)u[jj] * rowbytes + moff) : zero_word<DT, WB>();
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            float kf[EW], vf[EW];
            unpack_word<DT, WB>(kr[jj], kf);
            unpack_word<DT, WB>(vr[jj], vf);
            float sd = 0.0f, dd = 0.0f;
#pragma unroll
            for (int k = 0; k < EW; ++k) {
                sd = __builtin_fmaf(q[k], kf[k], sd);
                dd = __builtin_fmaf(g[k], vf[k], dd);
            }
            const float s2 = seg_sum_c<LPH>(sd) * a.qscale;
            const float da = seg_sum_c<LPH>(dd);
            const float p = ok[jj] ? exp2_(s2 - ls) : 0.0f;
            const float ds = p * (da - dl);
#pragma unroll
            for (int k = 0; k < EW; ++k) acc[k] = __builtin_fmaf(ds, kf[k], acc[k]);
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < EW; ++k) acc[k] += __shfl_xor(acc[k], off, kWave);
    if (grp != 0) return;
    if (hv && j == 0) a.stats[row * a.H + head] = make_float2(ls, dl);  // once per head
    if (!act) return;
    if (it.slot < 0) {
        float r[EW];
#pragma unroll
        for (int k = 0; k < EW; ++k) r[k] = acc[k] * a.kscale;
        stw_nt<DT, WB>((char*)a.dQ + row * rowbytes + moff, r);
    } else {
        float* pa = a.plan.pacc + it.slot * (int64_t)a.H * a.D + (int64_t)head * a.D + j * EW;
#pragma unroll
        for (int k = 0; k < EW; ++k) pa[k] = acc[k];
    }
}

template <int DT, int WB, int LPH, int U>
__global__ __launch_bounds__(kBlock) void bwd_dkv_word_kernel(const Args a) {
    constexpr int EW = Word<DT, WB>::EW;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = a.item_base + (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Item it;
    if (!resolve_item(a.plan, a.indptr, a.N, item, it)) return;
    const int64_t src = uniform64(it.row), e0 = uniform64(it.e0), e1 = uniform64(it.e1);
    const int G = a.G;
    const int epw = kWave / G;
    const int grp = lane / G;
    const int gl = lane & (G - 1);
    const int head = gl / LPH, j = gl % LPH;
    const bool hv = head < a.H;
    const bool act = hv && j < a.vph;
    const int64_t rowbytes = (int64_t)a.H * a.vph * WB;
    const int moff = (head * a.vph + j) * WB;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);
    float kk[EW], vv[EW], dk[EW], dv[EW];
    unpack_word<DT, WB>(act ? ldw<DT, WB>((const char*)a.K + src * rowbytes + moff) : zero_word<DT, WB>(), kk);
    unpack_word<DT, WB>(act ? ldw<DT, WB>((const char*)a.V + src * rowbytes + moff) : zero_word<DT, WB>(), vv);
#pragma unroll
    for (int k = 0; k < EW; ++k) dk[k] = dv[k] = 0.0f;
    const char* Qb = (const char*)a.Q;
    const char* Gb = (const char*)a.dO;
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            u[jj] = un[jj];
            ok[jj] = eb + grp + (int64_t)jj * epw < e1;
        }
        Word<DT, WB> qr[U], gr[U];
        float2 st[U];
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            const bool go = ok[jj] && act;
            qr[jj] = go ? ldw<DT, WB>(Qb + (int64_t)u[jj] * rowbytes + moff) : zero_word<DT, WB>();
            gr[jj] = go ? ldw<DT, WB>(Gb + (int64_t)u[jj] * rowbytes + moff) : zero_word<DT, WB>();
            st[jj] = (ok[jj] && hv) ? a.stats[(int64_t)u[jj] * a.H + head] : make_float2(0.0f, 0.0f);
        }
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            float qf[EW], gf[EW];
            unpack_word<DT, WB>(qr[jj], qf);
            unpack_word<DT, WB>(gr[jj], gf);
            float sd = 0.0f, dd = 0.0f;
#pragma unroll
            for (int k = 0; k < EW; ++k) {
                sd = __builtin_fmaf(qf[k], kk[k], sd);
                dd = __builtin_fmaf(gf[k], vv[k], dd);
            }
            const float s2 = seg_sum_c<LPH>(sd) * a.qscale;
            const float da = seg_sum_c<LPH>(dd);
            const float p = ok[jj] ? exp2_(s2 - st[jj].x) : 0.0f;
            const float ds = p * (da - st[jj].y);
#pragma unroll
            for (int k = 0; k < EW; ++k) {
                dv[k] = __builtin_fmaf(p, gf[k], dv[k]);
                dk[k] = __builtin_fmaf(ds, qf[k], dk[k]);
            }
        }
    }
    for (int off = G; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < EW; ++k) {
            dk[k] += __shfl_xor(dk[k], off, kWave);
            dv[k] += __shfl_xor(dv[k], off, kWave);
        }
    if (grp != 0 || !act) return;
    if (it.slot < 0) {
        float r[EW];
#pragma unroll
        for (int k = 0; k < EW; ++k) r[k] = dk[k] * a.kscale;
        stw_nt<DT, WB>((char*)a.dK + src * rowbytes + moff, r);
        stw_nt<DT, WB>((char*)a.dV + src * rowbytes + moff, dv);
    } else {
        const int64_t HD = (int64_t)a.H * a.D;
        float* pa = a.plan.pacc + it.slot * 2 * HD + (int64_t)head * a.D + j * EW;
#pragma unroll
        for (int k = 0; k < EW; ++k) {
            pa[k] = dk[k];
            pa[HD + k] = dv[k];
        }
    }
}

#if GT_BWD_PART != 2
// dw[e] = sum over heads, in head order, of the per-head terms the scalar
// layout's one-head waves left in part[e][h].
__global__ __launch_bounds__(256) void sum_heads_kernel(const float* __restrict__ part, int64_t E, int H,
                                                        float* __restrict__ dw) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    float t = 0.0f;
    for (int h = 0; h < H; ++h) t += part[e * H + h];
    dw[e] = t;
}

#endif

// ------------------------------------------------------------ launchers

// The compile-time layouts (for_fixed_layout) with plain logits.  The
// run-time layout costs the two passes more than it costs the forward
// (power-law graph: fp32 4x128 21.1 -> 18.3 ms, 8x32 11.2 -> 9.0 ms; bf16
// 8x64 13.3 -> 9.9 ms, 16x64 36.2 -> 19.5 ms).
// With logit options the heads per edge are then known too, so bias and
// weights load as batches and dropout draws its keep bits per batch, as in
// the tuned instances (without, a shape off them ran 2-6 times slower: bf16
// 8x64 with dropout 56.9 ms against 9.8 ms plain).  These instances keep
// fewer edges in flight, like the tuned ones: 4 per lane group (2 in the
// source pass of rows of 128 vectors).
#if GT_BWD_PART != 2
template <int DT, int XL>
static bool launch_dq_fixed(const Args& a, dim3 grid, dim3 block, hipStream_t s, bool ntl) {
    if (for_fixed_layout(a, [&](auto nc, auto u, auto g, auto lph) {
            constexpr int U = XL ? (decltype(u)::value < 4 ? decltype(u)::value : 4) : decltype(u)::value;
            if (XL == 0 && DT == kF32 && nc == 2 && ntl)
                bwd_dq_vec_kernel<DT, nc, U, g, lph, true, XL, true><<<grid, block, 0, s>>>(a);
            else
                bwd_dq_vec_kernel<DT, nc, U, g, lph, true, XL><<<grid, block, 0, s>>>(a);
        }))
        return true;
    return for_fixed_partial_layout(a, [&](auto nc, auto u, auto g, auto lph) {
        constexpr int U = XL ? (decltype(u)::value < 4 ? decltype(u)::value : 4) : decltype(u)::value;
        constexpr int U0 = XL ? (U < GT_PARTIAL_XL_U ? U : GT_PARTIAL_XL_U) : U;  // as in the forward
        if (a.R == a.NC * a.G)  // padded heads filling the lane groups: heads per edge known
            bwd_dq_vec_kernel<DT, nc, U, g, lph, 2, XL><<<grid, block, 0, s>>>(a);
        else
            bwd_dq_vec_kernel<DT, nc, U0, g, lph, 0, XL><<<grid, block, 0, s>>>(a);
    });
}

#endif

#if GT_BWD_PART != 1
template <int DT, int XL>
static bool launch_dkv_fixed(const Args& a, dim3 grid, dim3 block, hipStream_t s) {
    if (for_fixed_layout(a, [&](auto nc, auto u, auto g, auto lph) {
            constexpr int U = XL ? (decltype(nc)::value >= 2 ? 2 : 4) : decltype(u)::value;
            bwd_dkv_vec_kernel<DT, nc, U, g, lph, true, XL><<<grid, block, 0, s>>>(a);
        }))
        return true;
    return for_fixed_partial_layout(a, [&](auto nc, auto u, auto g, auto lph) {
        constexpr int U = XL ? (decltype(nc)::value >= 2 ? 2 : 4) : decltype(u)::value;
        if (a.R == a.NC * a.G)  // padded heads filling the lane groups: heads per edge known
            bwd_dkv_vec_kernel<DT, nc, U, g, lph, 2, XL><<<grid, block, 0, s>>>(a);
        else
            bwd_dkv_vec_kernel<DT, nc, U, g, lph, 0, XL><<<grid, block, 0, s>>>(a);
    });
}

#endif

#if GT_BWD_PART != 2
template <int DT, int XL>
static hipError_t launch_dq_dt(const Args& a0, hipStream_t s) {
    const dim3 block(kBlock);
    hipError_t err;
    if (a0.vec == 3) {  // word layout (plain logits only)
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            for_word_layout(a, [&](auto wb, auto lph) {
                bwd_dq_word_kernel<DT, wb, lph, 4><<<dim3(gx), block, 0, s>>>(a);
            });
        });
    } else if (a0.vec == 2) {  // head-innermost layout (plain logits only)
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            switch (a.NC) {
                case 1: bwd_dq_ndh_kernel<DT, DT == kF32 ? 4 : 2, 1><<<dim3(gx), block, 0, s>>>(a); break;
                case 2: bwd_dq_ndh_kernel<DT, DT == kF32 ? 4 : 2, 2><<<dim3(gx), block, 0, s>>>(a); break;
                case 3: bwd_dq_ndh_kernel<DT, 1, 3><<<dim3(gx), block, 0, s>>>(a); break;
                default: bwd_dq_ndh_kernel<DT, 1, 4><<<dim3(gx), block, 0, s>>>(a); break;
            }
        });
    } else if (a0.vec) {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx);
            const bool full = full_rows(a);
            // streamed K/V gathers when K and V are far larger than the Infinity Cache
            const bool stream_kv = 2 * a.n_gather * (int64_t)a.Rm * 16 > ((int64_t)1 << 30);
            if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && full && stream_kv && XL == 0)
                bwd_dq_vec_kernel<DT, 2, GT_BWD_F32_DQ_U, 64, 16, true, XL, true><<<grid, block, 0, s>>>(a);
            else if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && full)
                bwd_dq_vec_kernel<DT, 2, 4, 64, 16, true, XL><<<grid, block, 0, s>>>(a);
            else if (DT == kBF16 && a.NC == 1 && a.G == 32 && a.lph == 4 && full)
                bwd_dq_vec_kernel<DT, 1, XL == 2 ? GT_BWD_BF16_DQ_XL2_U : XL ? GT_BWD_BF16_DQ_XL1_U : GT_BWD_BF16_DQ_U, 32, 4, true, XL><<<grid, block, 0, s>>>(a);
            else if (launch_dq_fixed<DT, XL>(a, grid, block, s, stream_kv))
                ;
            else if (a.NC == 1)
                bwd_dq_vec_kernel<DT, 1, 8, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
            else if (a.NC == 2)
                bwd_dq_vec_kernel<DT, 2, 4, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
            else if (a.NC == 3)
                bwd_dq_vec_kernel<DT, 3, 2, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
            else
                bwd_dq_vec_kernel<DT, 4, 2, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
        });
    } else {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx, a.H);
            switch (a.KD) {
                case 1: bwd_dq_scalar_kernel<DT, 1, 8, XL><<<grid, block, 0, s>>>(a); break;
                case 2: bwd_dq_scalar_kernel<DT, 2, 8, XL><<<grid, block, 0, s>>>(a); break;
                case 3: bwd_dq_scalar_kernel<DT, 3, 4, XL><<<grid, block, 0, s>>>(a); break;
                default: bwd_dq_scalar_kernel<DT, 4, 4, XL><<<grid, block, 0, s>>>(a); break;
            }
        });
        if (err == hipSuccess && XL && a0.dew && a0.E > 0) {
            sum_heads_kernel<<<(unsigned)((a0.E + 255) / 256), 256, 0, s>>>(a0.dew_part, a0.E, a0.H, a0.dew);
            err = hipGetLastError();
        }
    }
    if (err != hipSuccess) return err;
    return launch_sum_merge(a0, 1, a0.dQ, a0.kscale, nullptr, 0.0f, s);
}

#endif

#if GT_BWD_PART != 1
template <int DT, int XL>
static hipError_t launch_dkv_dt(const Args& a0, hipStream_t s) {
    const dim3 block(kBlock);
    hipError_t err;
    if (a0.vec == 3) {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            for_word_layout(a, [&](auto wb, auto lph) {
                bwd_dkv_word_kernel<DT, wb, lph, 4><<<dim3(gx), block, 0, s>>>(a);
            });
        });
    } else if (a0.vec == 2) {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            switch (a.NC) {
                case 1: bwd_dkv_ndh_kernel<DT, DT == kF32 ? 4 : 2, 1><<<dim3(gx), block, 0, s>>>(a); break;
                case 2: bwd_dkv_ndh_kernel<DT, DT == kF32 ? 2 : 1, 2><<<dim3(gx), block, 0, s>>>(a); break;
                case 3: bwd_dkv_ndh_kernel<DT, 1, 3><<<dim3(gx), block, 0, s>>>(a); break;
                default: bwd_dkv_ndh_kernel<DT, 1, 4><<<dim3(gx), block, 0, s>>>(a); break;
            }
        });
    } else if (a0.vec) {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx);
            const bool full = full_rows(a);
            if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && full)
                bwd_dkv_vec_kernel<DT, 2, XL ? 2 : GT_BWD_F32_DKV_U, 64, 16, true, XL><<<grid, block, 0, s>>>(a);
            else if (DT == kBF16 && a.NC == 1 && a.G == 32 && a.lph == 4 && full)
                bwd_dkv_vec_kernel<DT, 1, XL == 2 ? GT_BWD_BF16_DKV_XL2_U : XL == 1 ? GT_BWD_BF16_DKV_XL1_U : GT_BWD_BF16_DKV_U, 32, 4, true, XL><<<grid, block, 0, s>>>(a);
            else if (launch_dkv_fixed<DT, XL>(a, grid, block, s))
                ;
            else if (a.NC == 1)
                bwd_dkv_vec_kernel<DT, 1, 8, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
            else if (a.NC == 2)
                bwd_dkv_vec_kernel<DT, 2, 4, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
            else if (a.NC == 3)
                bwd_dkv_vec_kernel<DT, 3, 2, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
            else
                bwd_dkv_vec_kernel<DT, 4, 2, 0, 0, false, XL><<<grid, block, 0, s>>>(a);
        });
    } else {
        err = for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx, a.H);
            switch (a.KD) {
                case 1: bwd_dkv_scalar_kernel<DT, 1, 8, XL><<<grid, block, 0, s>>>(a); break;
                case 2: bwd_dkv_scalar_kernel<DT, 2, 8, XL><<<grid, block, 0, s>>>(a); break;
                case 3: bwd_dkv_scalar_kernel<DT, 3, 4, XL><<<grid, block, 0, s>>>(a); break;
                default: bwd_dkv_scalar_kernel<DT, 4, 4, XL><<<grid, block, 0, s>>>(a); break;
            }
        });
    }
    if (err != hipSuccess) return err;
    return launch_sum_merge(a0, 2, a0.dK, a0.kscale, a0.dV, 1.0f, s);
}

#endif

// 0: plain logits; 1: bias, edge weights, dbias or dweight; 2: with dropout
[[maybe_unused]] static int xl_level(const Args& a) { return extended(a) ? (a.drop_thresh ? 2 : 1) : 0; }

#if GT_BWD_PART != 2
hipError_t launch_bwd_dq(const Args& a, hipStream_t s) {
    const int xl = xl_level(a);
    if (a.dtype == kF32)
        return xl == 0 ? launch_dq_dt<kF32, 0>(a, s) : xl == 1 ? launch_dq_dt<kF32, 1>(a, s) : launch_dq_dt<kF32, 2>(a, s);
    return xl == 0 ? launch_dq_dt<kBF16, 0>(a, s) : xl == 1 ? launch_dq_dt<kBF16, 1>(a, s) : launch_dq_dt<kBF16, 2>(a, s);
}

#endif

#if GT_BWD_PART != 1
hipError_t launch_bwd_dkv(const Args& a, hipStream_t s) {
    const int xl = xl_level(a);
    if (a.dtype == kF32)
        return xl == 0 ? launch_dkv_dt<kF32, 0>(a, s) : xl == 1 ? launch_dkv_dt<kF32, 1>(a, s) : launch_dkv_dt<kF32, 2>(a, s);
    return xl == 0 ? launch_dkv_dt<kBF16, 0>(a, s) : xl == 1 ? launch_dkv_dt<kBF16, 1>(a, s) : launch_dkv_dt<kBF16, 2>(a, s);
}
#endif

}  // namespace gt
