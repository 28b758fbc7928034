// fused.hip -- fused sparse multi-head attention forward on gfx950.
//
// One wavefront per work item (a destination row, or a chunk of a heavy
// row).  For every in-edge u->v it gathers the source's K row, forms the
// per-head score <q_v, k_u>/sqrt(D) with a segmented cross-lane sum, keeps a
// running maximum m and a running sum l of exp(s - m) per head (rescaling l
// and the accumulator when m grows), gathers the source's V row and adds
// p * v to the accumulator.  The E x H scores and weights live only in
// registers.  At the end out = acc / l, or, for a chunk of a split row, the
// triple (m, l, acc) goes to scratch for the merge kernel below.
//
// The method: "Graph Transformer in a Nutshell", section "Sparse Multi-head
// Attention" (SDDMM, sparse softmax, SpMM); the DGL builtin-operator gist,
// TransLayer.forward (u_dot_v, edge_softmax, u_mul_e_sum).  Computing the
// softmax with a running maximum instead of a separate max pass gives the
// same weights: exp(s - m_old) * exp(m_old - m_new) = exp(s - m_new).
//
// Scores are kept in the log2 domain (each reduced dot product is scaled by
// log2(e)/sqrt(D)) so each exponential is one v_exp_f32.  Partial maxima in
// scratch are also in the log2 domain; only this file reads them.
//
// Memory-level parallelism: each batch of U edges per group issues all its K
// and V gathers at once, and the source ids of the next batch are loaded
// right behind them (unconditional, clamped loads; scalar loads when one
// group spans the wave), so no gather waits on an index load.  Output rows
// are written with the non-temporal hint (never re-read); the fp32 8x64
// instance also gathers K/V that way when K+V exceed 1 GB (measured faster
// there; slower when K/V partly fit the Infinity Cache, and for the 512-byte
// bf16 rows).
#include <algorithm>

#include "kernels.hpp"

namespace gt {

// ------------------------------------------------------------ vector layout
//
// G_ and LPH_ are compile-time lane-group and lanes-per-head sizes when
// nonzero, else read from the arguments.  FULL 1: the row is exactly NC*G
// vectors (no idle lane slot); 2: every slot belongs to a head, but heads
// are padded (vph < lph slots hold vectors); 0: slots may also lie past the
// row's end.  U edges per group are in flight.
template <int DT, int NC, int U, int G_, int LPH_, int FULL, bool NTL, int XL>
__global__ __launch_bounds__(kBlock) void fused_vec_kernel(const Args a) {
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
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);

    float q[NC][VN];
    bool act[NC];
    int head[NC], moff[NC];  // moff: byte offset of the lane slot's vector in a row
    const char* qrow = (const char*)a.Q + row * rowbytes;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vi = c * G + gl;
        const bool in_row = FULL || vi < a.R;  // a slot of some head (it may idle)
        act[c] = in_row && (vi & (lph - 1)) < vph;
        head[c] = in_row ? vi / lph : 0;
        moff[c] = FULL == 1 ? vi * 16 : (head[c] * vph + (vi & (lph - 1))) * 16;
        // unscaled: the scale goes on the reduced score, so nothing waits for Q
        // before the first gathers are issued
        const U4 r = act[c] ? ld16(qrow + moff[c]) : U4{0, 0, 0, 0};
        VT::unpack(r, q[c]);
    }

    float m[NC], l[NC], acc[NC][VN];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        m[c] = -INFINITY;
        l[c] = 0.0f;
#pragma unroll
        for (int k = 0; k < VN; ++k) acc[c][k] = 0.0f;
    }

    const char* Kb = (const char*)a.K;
    const char* Vb = (const char*)a.V;
    DropBatch db;
    // batches one keep-bit evaluation covers: fixed for the hot instances, else
    // as many as one round of 64 lanes holds (rows that end before their last
    // lane group: 8-9% of the forward with dropout, where one round per batch
    // left most lanes idle; the backward passes measured no gain and keep one)
    const int dmb = kBatched ? kDropMB : drop_batches_per_eval(epw, U, a.H);
    int dph = 0;  // position of the batch among those its keep bits were drawn for
    for (int64_t eb = e0; eb < e1; eb += (int64_t)epw * U, dph = dph + 1 == dmb ? 0 : dph + 1) {
        int32_t u[U];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            u[j] = un[j];
            ok[j] = eb + grp + (int64_t)j * epw < e1;
        }
        // extended logits: s = w_e * s + bias[e][h] (log2 units); edge ids
        // clamped into the item like the source ids; loaded ahead of the gathers
        // so that waiting for them never waits for a gather
        auto ej = [&](int j) -> int64_t { return ok[j] ? eb + grp + (int64_t)j * epw : e0; };
        float xw[U], xb[U][NC];
        SlotBatch<kBR> bb;
        SlotBatch<kWR> wb;
        bool sb = false;
        if constexpr (XL) {
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
            // one evaluation covers dmb consecutive batches (consecutive edges)
            if (bdrop && dph == 0)
                drop_batch_init(db, a.drop_seed, a.drop_thresh, a.H, -1, dmb * epw * U, lane,
                                [&](int k) { return eb + k; });
        }

        float s[U][NC];
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float kf[VN];
                VT::unpack(kr[j][c], kf);
                float d = 0.0f;
#pragma unroll
                for (int k = 0; k < VN; ++k) d = __builtin_fmaf(q[c][k], kf[k], d);
                d = (LPH_ ? seg_sum_c<LPH_>(d) : seg_sum(d, lph)) * a.qscale;
                if constexpr (XL) {
                    const int k = grp + j * epw;
                    const float w = sb ? (a.ew ? slot_batch_get(wb, k) : 1.0f) : xw[j];
                    const float b = sb ? (a.bias ? slot_batch_get(bb, k * a.H + head[c]) * kLog2e : 0.0f) : xb[j][c];
                    d = __builtin_fmaf(d, w, b);
                }
                s[j][c] = ok[j] ? d : -INFINITY;
            }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float mb = s[0][c];
#pragma unroll
            for (int j = 1; j < U; ++j) mb = fmaxf(mb, s[j][c]);
            const float mn = fmaxf(m[c], mb);
            const float sc = rescale(m[c], mn);
            l[c] *= sc;
#pragma unroll
            for (int k = 0; k < VN; ++k) acc[c][k] *= sc;
#pragma unroll
            for (int j = 0; j < U; ++j) {
                // a group with no edge left in this batch has mn = -inf: keep p at 0
                const float p = ok[j] ? exp2_(s[j][c] - mn) : 0.0f;
                l[c] += p;
                float pv = p;  // dropout zeroes the weight, not its share of the normaliser
                if constexpr (XL) {
                    if (XL == 2 && (kBatched || bdrop))
                        pv = p * drop_mult(db, a.drop_scale, a.H, -1, dph * epw * U + grp + j * epw, ej(j), head[c]);
                    else if (XL == 2 && !kBatched)
                        pv = philox_hi32(a.drop_seed, (uint64_t)ej(j) * a.H + head[c]) >= a.drop_thresh
                                 ? p * a.drop_scale : 0.0f;
                }
                float vf[VN];
                VT::unpack(vr[j][c], vf);
#pragma unroll
                for (int k = 0; k < VN; ++k) acc[c][k] = __builtin_fmaf(pv, vf[k], acc[c][k]);
            }
            m[c] = mn;
        }
    }

    // fold the edge groups of the wave together (lanes gl, gl+G, ... hold the same vectors)
    for (int off = G; off < kWave; off <<= 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float mo = __shfl_xor(m[c], off, kWave);
            const float lo = __shfl_xor(l[c], off, kWave);
            const float mn = fmaxf(m[c], mo);
            const float sa = rescale(m[c], mn), sb = rescale(mo, mn);
            l[c] = l[c] * sa + lo * sb;
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                const float ao = __shfl_xor(acc[c][k], off, kWave);
                acc[c][k] = acc[c][k] * sa + ao * sb;
            }
            m[c] = mn;
        }
    }
    if (grp != 0) return;

    if (it.slot < 0) {
        char* orow = (char*)a.out + row * rowbytes;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (!act[c]) continue;
            const float inv = l[c] > 0.0f ? 1.0f / l[c] : 0.0f;
            float o[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) o[k] = acc[c][k] * inv;
            st16_nt(orow + moff[c], VT::pack(o));
            const int vi = c * G + gl;
            if (a.lse_out && (vi & (lph - 1)) == 0) a.lse_out[row * a.H + vi / lph] = lse_of(m[c], l[c]);
        }
    } else {
        const int64_t HD = (int64_t)a.H * a.D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (!act[c]) continue;
            const int vi = c * G + gl;
            if ((vi & (lph - 1)) == 0) {
                const int64_t h = it.slot * a.H + vi / lph;
                a.plan.pm[h] = m[c];
                a.plan.pl[h] = l[c];
            }
            float* pa = a.plan.pacc + it.slot * HD + (int64_t)(moff[c] / 16) * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) st16(pa + k, Vec<kF32>::pack(&acc[c][k]));
        }
    }
}

// ------------------------------------------------------------ scalar layout
//
// One wave per (item, head); a group of G = pow2ceil(D) lanes (<= 64) covers
// one edge's head, lane j holding elements j + k*G, k < KD.
template <int DT, int KD, int U, int XL>
__global__ __launch_bounds__(kBlock) void fused_scalar_kernel(const Args a) {
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

    float q[KD];
    bool act[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = gl + k * G;
        act[k] = d < D;
        q[k] = act[k] ? VT::scalar(a.Q, row * HD + hoff + d) : 0.0f;
    }
    float m = -INFINITY, l = 0.0f, acc[KD];
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
            for (int k = 0; k < KD; ++k)
                kv[j][k] = (ok[j] && act[k]) ? VT::scalar(a.K, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k)
                vv[j][k] = (ok[j] && act[k]) ? VT::scalar(a.V, (int64_t)u[j] * HD + hoff + gl + k * G) : 0.0f;
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
        DropBatch db;
        bool bdrop = false;
        if constexpr (XL) {
            bdrop = XL == 2 && (kBatched || drop_batched(a.H, h, epw * U));
            if (bdrop)
                drop_batch_init(db, a.drop_seed, a.drop_thresh, a.H, h, epw * U, lane, [&](int k) { return eb + k; });
        }
        float s[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float d = 0.0f;
#pragma unroll
            for (int k = 0; k < KD; ++k) d = __builtin_fmaf(q[k], kv[j][k], d);
            d = seg_sum(d, G) * a.qscale;
            if constexpr (XL) d = __builtin_fmaf(d, xw[j], xb[j]);
            s[j] = ok[j] ? d : -INFINITY;
        }
        float mb = s[0];
#pragma unroll
        for (int j = 1; j < U; ++j) mb = fmaxf(mb, s[j]);
        const float mn = fmaxf(m, mb);
        const float sc = rescale(m, mn);
        l *= sc;
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[k] *= sc;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const float p = ok[j] ? exp2_(s[j] - mn) : 0.0f;
            l += p;
            float pv = p;
            if constexpr (XL) {
                if (XL == 2 && (kBatched || bdrop))
                    pv = p * drop_mult(db, a.drop_scale, a.H, h, grp + j * epw, ej(j), h);
                else if (XL == 2 && !kBatched)
                    pv = philox_hi32(a.drop_seed, (uint64_t)ej(j) * a.H + h) >= a.drop_thresh ? p * a.drop_scale
                                                                                            : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < KD; ++k) acc[k] = __builtin_fmaf(pv, vv[j][k], acc[k]);
        }
        m = mn;
    }
    for (int off = G; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(m, off, kWave);
        const float lo = __shfl_xor(l, off, kWave);
        const float mn = fmaxf(m, mo);
        const float sa = rescale(m, mn), sb = rescale(mo, mn);
        l = l * sa + lo * sb;
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            const float ao = __shfl_xor(acc[k], off, kWave);
            acc[k] = acc[k] * sa + ao * sb;
        }
        m = mn;
    }
    if (grp != 0) return;
    if (it.slot < 0) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
        for (int k = 0; k < KD; ++k)
            if (act[k]) VT::store_scalar(a.out, row * HD + hoff + gl + k * G, acc[k] * inv);
        if (a.lse_out && gl == 0) a.lse_out[row * a.H + h] = lse_of(m, l);
    } else {
        if (gl == 0) {
            a.plan.pm[it.slot * a.H + h] = m;
            a.plan.pl[it.slot * a.H + h] = l;
        }
#pragma unroll
        for (int k = 0; k < KD; ++k)
            if (act[k]) a.plan.pacc[it.slot * HD + hoff + gl + k * G] = acc[k];
    }
}

// ------------------------------------------------------------ head-innermost layout
//
// Features [N][D][H] ("Graph Transformer in a Nutshell", SparseMHA.forward:
// q, k, v reshaped to [N, dh, nh]).  A 16-byte vector of a row then holds VN
// consecutive heads of one d, so a lane group covers all heads of an edge at
// once: lane gl holds vectors vi = c * G + gl, c < NC (d = vi / HV, heads
// (vi % HV) * VN .. +VN-1, HV = H / VN a power of two, R = D * HV <= 256
// vectors; G = pow2ceil(R) when R <= 64, else 64 with NC = ceil(R / 64)).
// Since G is a multiple of HV, a lane holds the same heads in every c.  A
// head's dot product adds the lane's products over c, then over the lanes
// with the same gl % HV (xor offsets HV .. G/2); every lane keeps VN running
// softmax states, one per head it holds.  For the tutorial's shape (H 8,
// D 10, fp32) a row is 20 vectors, a group 32 lanes and a wave takes two
// edges at a time, where the [N][H][D] layout needs one wave per head with
// 10-element heads.
template <int DT, int U, int NC>
__global__ __launch_bounds__(kBlock) void fused_ndh_kernel(const Args a) {
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
    float q[NC][VN];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        VT::unpack(act[c] ? ld16((const char*)a.Q + row * rowbytes + (c * G + gl) * 16) : U4{0, 0, 0, 0}, q[c]);
    float m[VN], l[VN], acc[NC][VN];
#pragma unroll
    for (int k = 0; k < VN; ++k) {
        m[k] = -INFINITY;
        l[k] = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c][k] = 0.0f;
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
                kr[j][c] = (ok[j] && act[c]) ? ld16(Kb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : U4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                vr[j][c] = (ok[j] && act[c]) ? ld16(Vb + (int64_t)u[j] * rowbytes + (c * G + gl) * 16) : U4{0, 0, 0, 0};
        const int64_t nb = eb + (int64_t)epw * U;
        if (nb < e1) load_ids<U>(idx, nb, grp, epw, e1, un);
        float s[U][VN];
#pragma unroll
        for (int j = 0; j < U; ++j) {
#pragma unroll
            for (int k = 0; k < VN; ++k) s[j][k] = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float kf[VN];
                VT::unpack(kr[j][c], kf);
#pragma unroll
                for (int k = 0; k < VN; ++k) s[j][k] = __builtin_fmaf(q[c][k], kf[k], s[j][k]);
            }
            for (int off = HV; off < G; off <<= 1)
#pragma unroll
                for (int k = 0; k < VN; ++k) s[j][k] += __shfl_xor(s[j][k], off, kWave);
#pragma unroll
            for (int k = 0; k < VN; ++k) s[j][k] = ok[j] ? s[j][k] * a.qscale : -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < VN; ++k) {
            float mb = s[0][k];
#pragma unroll
            for (int j = 1; j < U; ++j) mb = fmaxf(mb, s[j][k]);
            const float mn = fmaxf(m[k], mb);
            const float sc = rescale(m[k], mn);
            l[k] *= sc;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c][k] *= sc;
            m[k] = mn;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float p[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                p[k] = ok[j] ? exp2_(s[j][k] - m[k]) : 0.0f;
                l[k] += p[k];
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float vf[VN];
                VT::unpack(vr[j][c], vf);
#pragma unroll
                for (int k = 0; k < VN; ++k) acc[c][k] = __builtin_fmaf(p[k], vf[k], acc[c][k]);
            }
        }
    }
    for (int off = G; off < kWave; off <<= 1) {
#pragma unroll
        for (int k = 0; k < VN; ++k) {
            const float mo = __shfl_xor(m[k], off, kWave);
            const float lo = __shfl_xor(l[k], off, kWave);
            const float mn = fmaxf(m[k], mo);
            const float sa = rescale(m[k], mn), sb = rescale(mo, mn);
            l[k] = l[k] * sa + lo * sb;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float ao = __shfl_xor(acc[c][k], off, kWave);
                acc[c][k] = acc[c][k] * sa + ao * sb;
            }
            m[k] = mn;
        }
    }
    if (grp != 0) return;
    const bool first_d = gl < HV;  // the lanes of d = 0 (in c = 0) carry each head's (m, l) once
    if (it.slot < 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (!act[c]) continue;
            float o[VN];
#pragma unroll
            for (int k = 0; k < VN; ++k) o[k] = l[k] > 0.0f ? acc[c][k] / l[k] : 0.0f;
            st16_nt((char*)a.out + row * rowbytes + (c * G + gl) * 16, VT::pack(o));
        }
        if (a.lse_out && first_d)
#pragma unroll
            for (int k = 0; k < VN; ++k) a.lse_out[row * a.H + hg * VN + k] = lse_of(m[k], l[k]);
    } else {
        const int64_t HD = (int64_t)a.H * a.D;
        if (first_d)
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                a.plan.pm[it.slot * a.H + hg * VN + k] = m[k];
                a.plan.pl[it.slot * a.H + hg * VN + k] = l[k];
            }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (!act[c]) continue;
            float* pa = a.plan.pacc + it.slot * HD + (int64_t)(c * G + gl) * VN;
#pragma unroll
            for (int k = 0; k < VN; k += 4) st16(pa + k, Vec<kF32>::pack(&acc[c][k]));
        }
    }
}

// ------------------------------------------------------------ word layout
//
// [N][H][D] rows whose heads are a whole number of 8- or 4-byte words but not
// of 16-byte vectors, such as the tutorial's molecule shape (H 8, D 10, fp32:
// 40-byte heads, five 8-byte words).  A head of vph words takes LPH =
// pow2ceil(vph) lane slots, so its dot product is a DPP sum within an aligned
// LPH-lane segment (the slots past vph idle with zeros), and a lane group of
// G = pow2ceil(H * LPH) <= 64 lanes covers all heads of an edge: one wave per
// row, 64 / G edges per step, where the scalar layout takes a wave per
// (row, head) with 4-byte loads.  Plain logits only.
template <int DT, int WB, int LPH, int U>
__global__ __launch_bounds__(kBlock) void fused_word_kernel(const Args a) {
    using W = Word<DT, WB>;
    constexpr int EW = W::EW;
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
    const bool act = head < a.H && j < a.vph;
    const int64_t rowbytes = (int64_t)a.H * a.vph * WB;
    const int moff = (head * a.vph + j) * WB;
    const int32_t* __restrict__ idx = a.indices;

    int32_t un[U];
    if (e1 > e0) load_ids<U>(idx, e0, grp, epw, e1, un);
    float q[EW];
    unpack_word<DT, WB>(act ? ldw<DT, WB>((const char*)a.Q + row * rowbytes + moff) : zero_word<DT, WB>(), q);
    float m = -INFINITY, l = 0.0f, acc[EW];
#pragma unroll
    for (int k = 0; k < EW; ++k) acc[k] = 0.0f;
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
        float sc[U];
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            float kf[EW];
            unpack_word<DT, WB>(kr[jj], kf);
            float d = 0.0f;
#pragma unroll
            for (int k = 0; k < EW; ++k) d = __builtin_fmaf(q[k], kf[k], d);
            d = seg_sum_c<LPH>(d) * a.qscale;
            sc[jj] = ok[jj] ? d : -INFINITY;
        }
        float mb = sc[0];
#pragma unroll
        for (int jj = 1; jj < U; ++jj) mb = fmaxf(mb, sc[jj]);
        const float mn = fmaxf(m, mb);
        const float r = rescale(m, mn);
        l *= r;
#pragma unroll
        for (int k = 0; k < EW; ++k) acc[k] *= r;
#pragma unroll
        for (int jj = 0; jj < U; ++jj) {
            const float p = ok[jj] ? exp2_(sc[jj] - mn) : 0.0f;
            l += p;
            float vf[EW];
            unpack_word<DT, WB>(vr[jj], vf);
#pragma unroll
            for (int k = 0; k < EW; ++k) acc[k] = __builtin_fmaf(p, vf[k], acc[k]);
        }
        m = mn;
    }
    // fold the edge groups of the wave together
    for (int off = G; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(m, off, kWave);
        const float lo = __shfl_xor(l, off, kWave);
        const float mn = fmaxf(m, mo);
        const float sa = rescale(m, mn), sb = rescale(mo, mn);
        l = l * sa + lo * sb;
#pragma unroll
        for (int k = 0; k < EW; ++k) {
            const float ao = __shfl_xor(acc[k], off, kWave);
            acc[k] = acc[k] * sa + ao * sb;
        }
        m = mn;
    }
    if (grp != 0) return;
    const bool first = j == 0 && head < a.H;  // one lane per head carries its (m, l)
    if (it.slot < 0) {
        if (act) {
            float o[EW];
#pragma unroll
            for (int k = 0; k < EW; ++k) o[k] = l > 0.0f ? acc[k] / l : 0.0f;
            stw_nt<DT, WB>((char*)a.out + row * rowbytes + moff, o);
        }
        if (a.lse_out && first) a.lse_out[row * a.H + head] = lse_of(m, l);
    } else {
        if (first) {
            a.plan.pm[it.slot * a.H + head] = m;
            a.plan.pl[it.slot * a.H + head] = l;
        }
        if (act) {
            float* pa = a.plan.pacc + it.slot * (int64_t)a.H * a.D + (int64_t)head * a.D + j * EW;
#pragma unroll
            for (int k = 0; k < EW; ++k) pa[k] = acc[k];
        }
    }
}

// Per node, src [A][B] -> dst [B][A]; grid-stride over the elements, reads
// coalesced.
template <typename T>
__global__ __launch_bounds__(256) void transpose_rows_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t n,
                                                              int A, int B) {
    const int64_t AB = (int64_t)A * B;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t node = i / AB;
        const int r = (int)(i - node * AB);
        const int x = r / B, y = r - x * B;
        dst[node * AB + (int64_t)y * A + x] = src[i];
    }
}

// The same through LDS, for nodes of a whole number of 16-byte vectors: a
// block loads a tile of whole consecutive nodes with 16-byte loads, stores it
// in LDS as [node][A][pitch] 32-bit words (pitch = B padded to an odd count,
// against bank conflicts when read down a column), then writes the
// transposed tile with 16-byte stores, so both sides are coalesced.
constexpr int kTrTileWords = 8192;  // 32 KB of LDS per block

template <typename T>
__global__ __launch_bounds__(256) void transpose_tiles_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                               int64_t N, int A, int B, int pitch, int npt) {
    __shared__ uint32_t lds[kTrTileWords];
    constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte vector
    const int64_t AB = (int64_t)A * B;
    const int nodewords = A * pitch;
    for (int64_t n0 = (int64_t)blockIdx.x * npt; n0 < N; n0 += (int64_t)gridDim.x * npt) {
        const int nn = (int)(N - n0 < npt ? N - n0 : npt);
        const int64_t nvec = nn * AB / VE;
        const char* sp = (const char*)(src + n0 * AB);
        for (int64_t v = threadIdx.x; v < nvec; v += blockDim.x) {
            const U4 w = ld16(sp + v * 16);
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
            const int64_t e = v * VE;
            const int nl = (int)(e / AB);
            const int r = (int)(e - nl * AB);
            int x = r / B, y = r - x * B;  // src [A][B]: row x, column y
#pragma unroll
            for (int i = 0; i < VE; ++i) {
                const uint32_t bits = sizeof(T) == 4 ? wd[i] : (wd[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
                lds[nl * nodewords + x * pitch + y] = bits;
                if (++y == B) {
                    y = 0;
                    ++x;
                }
            }
        }
        __syncthreads();
        char* dp = (char*)(dst + n0 * AB);
        for (int64_t v = threadIdx.x; v < nvec; v += blockDim.x) {
            const int64_t o = v * VE;
            const int nl = (int)(o / AB);
            const int r = (int)(o - nl * AB);
            int y = r / A, x = r - y * A;  // dst [B][A]: row y, column x
            uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < VE; ++i) {
                const uint32_t bits = lds[nl * nodewords + x * pitch + y];
                if (sizeof(T) == 4)
                    wd[i] = bits;
                else
                    wd[i / 2] |= bits << (16 * (i & 1));
                if (++x == A) {
                    x = 0;
                    ++y;
                }
            }
            st16(dp + v * 16, U4{wd[0], wd[1], wd[2], wd[3]});
        }
        __syncthreads();
    }
}

hipError_t launch_transpose_rows(const void* src, void* dst, int64_t N, int A, int B, int dtype, hipStream_t s) {
    const int64_t n = N * A * B;
    if (n == 0) return hipSuccess;
    const int esize = dtype == kF32 ? 4 : 2;
    const int pitch = B % 2 == 0 ? B + 1 : B + 2;
    const bool tiled = ((int64_t)A * B * esize) % 16 == 0 && ((uintptr_t)src & 15) == 0 && ((uintptr_t)dst & 15) == 0 &&
                       (int64_t)A * pitch <= kTrTileWords;
    if (tiled) {
        const int npt = kTrTileWords / (A * pitch);
        const unsigned grid = (unsigned)std::min<int64_t>((N + npt - 1) / npt, (int64_t)1 << 16);
        if (dtype == kF32)
            transpose_tiles_kernel<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, N, A, B, pitch, npt);
        else
            transpose_tiles_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, N, A, B, pitch,
                                                                  npt);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, (int64_t)1 << 20);
    if (dtype == kF32)
        transpose_rows_kernel<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, n, A, B);
    else
        transpose_rows_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, n, A, B);
    return hipGetLastError();
}

// ------------------------------------------------------------ merge of split rows
//
// One wave per heavy row; for each head the row's chunks are combined as
// M = max m_i, L = sum l_i 2^(m_i - M), A = sum acc_i 2^(m_i - M), out = A / L:
// the associative form of the softmax that the running-max loop also uses.
// Lanes run over chunks for (M, L) and over the head's D elements for A,
// which is summed in chunk order.
__device__ __forceinline__ float wave_max(float x) {
    for (int off = 1; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Merges head h of one heavy row (one wave).  The chunk loop is unrolled so
// that eight partial rows are in flight per lane.
template <int DT, int T>
__device__ __forceinline__ void merge_row(const Args& a, const HeavyRow hr, int h, int lane) {
    using VT = Vec<DT>;
    constexpr int UN = 8;
    const int H = a.H, D = a.D, nch = hr.nch;
    const int64_t HD = (int64_t)H * D;
    const float* pm = a.plan.pm + hr.base * H + h;
    const float* pl = a.plan.pl + hr.base * H + h;
    // element (h, d) of a row: h*D + d, or d*H + h in the head-innermost layout
    const int64_t hoff = a.ndh ? h : (int64_t)h * D, dstride = a.ndh ? H : 1;
    const float* pa = a.plan.pacc + hr.base * HD + hoff;
    float M = -INFINITY;
    for (int i = lane; i < nch; i += kWave) M = fmaxf(M, pm[(int64_t)i * H]);
    M = wave_max(M);
    float L = 0.0f;
    for (int i = lane; i < nch; i += kWave) L += pl[(int64_t)i * H] * exp2_(pm[(int64_t)i * H] - M);
    L = wave_sum(L);
    if (a.lse_out && lane == 0) a.lse_out[(int64_t)hr.row * H + h] = lse_of(M, L);
    float A[T];  // D <= 64 * T elements, lane holds d = lane + 64 t
#pragma unroll
    for (int t = 0; t < T; ++t) A[t] = 0.0f;
    for (int ib = 0; ib < nch; ib += kWave) {
        const int i = ib + lane;
        const float wl = i < nch ? exp2_(pm[(int64_t)i * H] - M) : 0.0f;
        const int nb = nch - ib < kWave ? nch - ib : kWave;
        for (int k0 = 0; k0 < nb; k0 += UN) {
            float v[UN][T];
#pragma unroll
            for (int k = 0; k < UN; ++k)
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int d = lane + t * kWave;
                    v[k][t] = (k0 + k < nb && d < D) ? pa[(int64_t)(ib + k0 + k) * HD + d * dstride] : 0.0f;
                }
#pragma unroll
            for (int k = 0; k < UN; ++k) {
                const float w = __shfl(wl, (k0 + k) & (kWave - 1), kWave);
#pragma unroll
                for (int t = 0; t < T; ++t) A[t] = __builtin_fmaf(v[k][t], w, A[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int d = lane + t * kWave;
        if (d < D) VT::store_scalar(a.out, (int64_t)hr.row * HD + hoff + d * dstride, A[t] / L);
    }
}

// A wave per (heavy row, head h = blockIdx.y) at a time, striding over the
// heavy rows listed by the plan.  The grid is capped (kMergeGridX blocks in
// x): the host sizes it for the upper bound of heavy rows, E / (chunk + 1),
// which can be ten times the rows the plan lists, and a wave per bound would
// spend the kernel's time launching waves that exit at once.
template <int DT, int T>
__global__ __launch_bounds__(kBlock) void fused_merge_kernel(const Args a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int h = blockIdx.y;
    const int64_t nheavy = min(a.plan.max_heavy, (int64_t)a.plan.counters->nheavy);
    for (int64_t hs = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         hs < nheavy; hs += (int64_t)gridDim.x * kWavesPerBlock)
        merge_row<DT, T>(a, a.plan.heavy[hs], h, lane);
}

// ------------------------------------------------------------ launchers

// The compile-time layouts (for_fixed_layout) with plain logits: 4-6% on
// the power-law graph against the run-time layout (fp32 4x128, 16x32, 8x32,
// 2x256; bf16 8x64, 16x64, 8x128).  NTL as for the tuned fp32 instance.
// With logit options the heads per edge are known at compile time too, so
// bias and weights load as batches and dropout draws its keep bits per
// batch, as in the tuned instances; 4 edges in flight per lane group.
template <int DT, int XL>
static bool launch_fixed_lph(const Args& a, dim3 grid, dim3 block, hipStream_t s, bool ntl) {
    // fp32 rows of three or four vectors per lane measured 2-3% faster with
    // the run-time layout (12x64, 16x64); bf16 ones 13% slower (16x128)
    if (DT == kF32 && a.NC >= 3) return false;
    if (for_fixed_layout(a, [&](auto nc, auto u, auto g, auto lph) {
            constexpr int U = XL ? (decltype(u)::value < 4 ? decltype(u)::value : 4) : decltype(u)::value;
            if (XL == 0 && DT == kF32 && nc == 2 && ntl)
                fused_vec_kernel<DT, nc, U, g, lph, true, true, XL><<<grid, block, 0, s>>>(a);
            else
                fused_vec_kernel<DT, nc, U, g, lph, true, false, XL><<<grid, block, 0, s>>>(a);
        }))
        return true;
    // rows with idle lane slots
    return for_fixed_partial_layout(a, [&](auto nc, auto u, auto g, auto lph) {
        constexpr int U = XL ? (decltype(u)::value < 4 ? decltype(u)::value : 4) : decltype(u)::value;
        // rows that end early with logit options: the run-time head masks and
        // per-lane dropout state took 141-175 VGPRs at 4 edges in flight (2-3
        // waves per SIMD); 2 in flight keep more waves resident
        constexpr int U0 = XL ? (U < GT_PARTIAL_XL_U ? U : GT_PARTIAL_XL_U) : U;
        if (a.R == a.NC * a.G)  // padded heads filling the lane groups: heads per edge known
            fused_vec_kernel<DT, nc, U, g, lph, 2, false, XL><<<grid, block, 0, s>>>(a);
        else
            fused_vec_kernel<DT, nc, U0, g, lph, 0, false, XL><<<grid, block, 0, s>>>(a);
    });
}

template <int DT, int XL>
static hipError_t launch_fused_dt(const Args& a0, hipStream_t s) {
    const dim3 block(kBlock);
    if (a0.vec == 3) {  // word layout (plain logits only)
        return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            for_word_layout(a, [&](auto wb, auto lph) {
                fused_word_kernel<DT, wb, lph, 4><<<dim3(gx), block, 0, s>>>(a);
            });
        });
    }
    if (a0.vec == 2) {  // head-innermost layout (plain logits only)
        return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            switch (a.NC) {
                case 1: fused_ndh_kernel<DT, 4, 1><<<dim3(gx), block, 0, s>>>(a); break;
                case 2: fused_ndh_kernel<DT, DT == kF32 ? GT_NDH_F32_U : 2, 2><<<dim3(gx), block, 0, s>>>(a); break;
                case 3: fused_ndh_kernel<DT, 2, 3><<<dim3(gx), block, 0, s>>>(a); break;
                default: fused_ndh_kernel<DT, 2, 4><<<dim3(gx), block, 0, s>>>(a); break;
            }
        });
    }
    if (a0.vec) {
        return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
            const dim3 grid(gx);
            const bool full = full_rows(a);
            // Streaming K/V gathers pay off only when K and V are far larger than
            // the 256 MB Infinity Cache; smaller ones are partly served from it.
            const bool stream_kv = 2 * a.n_gather * (int64_t)a.Rm * 16 > ((int64_t)1 << 30);
            if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && full && stream_kv)
                fused_vec_kernel<DT, 2, XL == 2 ? 4 : GT_F32_D64_U, 64, 16, true, true, XL><<<grid, block, 0, s>>>(a);
            else if (DT == kF32 && a.NC == 2 && a.G == 64 && a.lph == 16 && full)
                fused_vec_kernel<DT, 2, XL == 2 ? 4 : GT_F32_D64_U, 64, 16, true, false, XL><<<grid, block, 0, s>>>(a);
            else if (DT == kBF16 && a.NC == 1 && a.G == 32 && a.lph == 4 && full)
                // the extended kernel keeps per-edge inputs live: fewer edges in flight
                fused_vec_kernel<DT, 1, XL == 2 ? GT_BF16_D32_XL2_U : XL == 1 ? GT_BF16_D32_XL1_U : GT_BF16_D32_U, 32, 4, true, GT_BF16_NTL != 0, XL><<<grid, block, 0, s>>>(a);
            else if (launch_fixed_lph<DT, XL>(a, grid, block, s, DT == kF32 && stream_kv))
                ;
            else if (a.NC == 1)
                fused_vec_kernel<DT, 1, 8, 0, 0, false, false, XL><<<grid, block, 0, s>>>(a);
            else if (a.NC == 2)
                fused_vec_kernel<DT, 2, 4, 0, 0, false, false, XL><<<grid, block, 0, s>>>(a);
            else if (a.NC == 3)
                fused_vec_kernel<DT, 3, 2, 0, 0, false, false, XL><<<grid, block, 0, s>>>(a);
            else
                fused_vec_kernel<DT, 4, 2, 0, 0, false, false, XL><<<grid, block, 0, s>>>(a);
        });
    }
    return for_slices(a0, a0.items, [&](const Args& a, unsigned gx) {
        const dim3 grid(gx, a.H);
        switch (a.KD) {
            case 1: fused_scalar_kernel<DT, 1, 8, XL><<<grid, block, 0, s>>>(a); break;
            case 2: fused_scalar_kernel<DT, 2, 8, XL><<<grid, block, 0, s>>>(a); break;
            case 3: fused_scalar_kernel<DT, 3, 4, XL><<<grid, block, 0, s>>>(a); break;
            default: fused_scalar_kernel<DT, 4, 4, XL><<<grid, block, 0, s>>>(a); break;
        }
    });
}

hipError_t launch_fused(const Args& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (ev0) (void)hipEventRecord(ev0, s);
    // 0: plain logits; 1: bias and edge weights; 2: with dropout
    const int xl = extended(a) ? (a.drop_thresh ? 2 : 1) : 0;
    hipError_t err;
    if (a.dtype == kF32)
        err = xl == 0 ? launch_fused_dt<kF32, 0>(a, s) : xl == 1 ? launch_fused_dt<kF32, 1>(a, s) : launch_fused_dt<kF32, 2>(a, s);
    else
        err = xl == 0 ? launch_fused_dt<kBF16, 0>(a, s) : xl == 1 ? launch_fused_dt<kBF16, 1>(a, s) : launch_fused_dt<kBF16, 2>(a, s);
    if (ev1) (void)hipEventRecord(ev1, s);
    return err;
}

hipError_t launch_fused_merge(const Args& a, hipStream_t s) {
    const dim3 block(kBlock);
    const dim3 grid((unsigned)std::min<int64_t>((a.plan.max_heavy + kWavesPerBlock - 1) / kWavesPerBlock, kMergeGridX),
                    a.H);
    const int T = (a.D + kWave - 1) / kWave;
    if (a.dtype == kF32) {
        if (T == 1) fused_merge_kernel<kF32, 1><<<grid, block, 0, s>>>(a);
        else fused_merge_kernel<kF32, 4><<<grid, block, 0, s>>>(a);
    } else {
        if (T == 1) fused_merge_kernel<kBF16, 1><<<grid, block, 0, s>>>(a);
        else fused_merge_kernel<kBF16, 4><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace gt
