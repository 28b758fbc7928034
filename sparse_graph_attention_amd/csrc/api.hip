// api.hip -- the C ABI of libgtattn (declared in include/gtattn.h): argument
// checks, the per-(device, stream) scratch buffer, layout choice and launches.
#include <gtattn.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "kernels.hpp"

using namespace gt;

namespace {

thread_local std::string g_err;
std::atomic<int64_t> g_chunk{512};

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(GT_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// ---------------------------------------------------------------- scratch

struct Scratch {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_scratch_mu;
std::map<std::pair<int, uintptr_t>, Scratch> g_scratch;

// A buffer of at least `bytes` for `stream` on the current device.  Growing it
// waits for the stream (its old buffer may still be in use by queued work).
int get_scratch(hipStream_t stream, size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    Scratch& s = g_scratch[{dev, (uintptr_t)stream}];
    if (s.bytes < bytes) {
        if (s.ptr) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            (void)hipFree(s.ptr);
            s.ptr = nullptr;
            s.bytes = 0;
        }
        size_t want = bytes + bytes / 4;  // headroom against frequent regrowth
        e = hipMalloc(&s.ptr, want);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            s.ptr = nullptr;
            return fail(GT_ENOMEM, "hipMalloc of %zu scratch bytes failed: %s", want, hipGetErrorString(e));
        }
        s.bytes = want;
    }
    *out = s.ptr;
    return GT_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Sizes a plan for a graph of N rows and E edges whose chunk partials are
// `accw` floats wide; returns its scratch bytes (0 when no row can be split,
// except for the counters).
size_t plan_bytes(int64_t N, int64_t E, int H, int64_t accw, Plan& p) {
    const int64_t C = g_chunk.load();
    p.chunk = C;
    p.max_heavy = std::min<int64_t>(N, E / (C + 1));
    p.max_chunks = p.max_heavy ? E / C + p.max_heavy : 0;
    return align256(sizeof(PlanCounters)) + align256(sizeof(HeavyRow) * p.max_heavy) +
           align256(sizeof(ChunkRef) * p.max_chunks) + 2 * align256(sizeof(float) * p.max_chunks * H) +
           align256(sizeof(float) * p.max_chunks * accw) + align256(sizeof(float) * p.max_heavy * H * 2);
}

// Points the plan's arrays into scratch at b (laid out as plan_bytes counts them).
char* carve_plan(char* b, int H, int64_t accw, Plan& p) {
    p.counters = (PlanCounters*)b;               b += align256(sizeof(PlanCounters));
    p.heavy = (HeavyRow*)b;                      b += align256(sizeof(HeavyRow) * p.max_heavy);
    p.chunks = (ChunkRef*)b;                     b += align256(sizeof(ChunkRef) * p.max_chunks);
    p.pm = (float*)b;                            b += align256(sizeof(float) * p.max_chunks * H);
    p.pl = (float*)b;                            b += align256(sizeof(float) * p.max_chunks * H);
    p.pacc = (float*)b;                          b += align256(sizeof(float) * p.max_chunks * accw);
    p.hstat = (float*)b;                         b += align256(sizeof(float) * p.max_heavy * H * 2);
    return b;
}

int check_plan(const Plan& p) {
    if (p.max_chunks >= ((int64_t)1 << 31))
        return fail(GT_EUNSUPPORTED, "too many chunks (%lld); raise GT_CFG_CHUNK_EDGES", (long long)p.max_chunks);
    return GT_OK;
}

// Sizes the plan for (N, E), carves it out of the stream's scratch and lists
// the split rows on the device.
int make_plan(const int64_t* indptr, int64_t N, int64_t E, int H, int D, hipStream_t stream, Args& a) {
    (void)indptr;
    const size_t bytes = plan_bytes(N, E, H, (int64_t)H * D, a.plan);
    int rc = check_plan(a.plan);
    if (rc) return rc;
    a.items = a.plan.max_chunks + N;
    void* base = nullptr;
    rc = get_scratch(stream, bytes, &base);
    if (rc) return rc;
    carve_plan((char*)base, H, (int64_t)H * D, a.plan);
    hipError_t e = launch_plan(a, stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    return GT_OK;
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int pow2ceil(int64_t x) {
    int r = 1;
    while (r < x) r <<= 1;
    return r;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Vector layout when every head is a power-of-two number of 16-byte vectors,
// the row fits in four vectors per lane and the feature arrays are aligned;
// the scalar layout otherwise.
void choose_layout(Args& a, std::initializer_list<const void*> feats) {
    const int bytes = a.dtype == GT_F32 ? 4 : 2;
    const int64_t hb = (int64_t)a.D * bytes;
    bool vec = hb % 16 == 0 && pow2(hb / 16);
    for (const void* p : feats) vec = vec && aligned16(p);
    if (vec) {
        a.lph = (int)(hb / 16);
        a.R = a.H * a.lph;
        if (a.R >= kWave) {
            a.G = kWave;
            a.NC = (a.R + kWave - 1) / kWave;
            vec = a.NC <= 4;
        } else {
            a.G = pow2ceil(a.R);
            a.NC = 1;
        }
    }
    a.vec = vec ? 1 : 0;
    if (!vec) {
        a.G = std::min(kWave, pow2ceil(a.D));
        a.KD = (a.D + a.G - 1) / a.G;
        a.lph = a.R = a.NC = 0;
    }
}

int check_common(int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype) {
    if (N < 0 || E < 0) return fail(GT_EINVAL, "N (%lld) and E (%lld) must be >= 0", (long long)N, (long long)E);
    if (N >= ((int64_t)1 << 31)) return fail(GT_EINVAL, "N (%lld) must be < 2^31", (long long)N);
    if (H < 1 || D < 1) return fail(GT_EINVAL, "H (%d) and D (%d) must be >= 1", H, D);
    if (dtype != GT_F32 && dtype != GT_BF16) return fail(GT_EUNSUPPORTED, "unknown dtype %d", dtype);
    if (H > 64) return fail(GT_EUNSUPPORTED, "H = %d > 64 is not supported", H);
    if (D > 256) return fail(GT_EUNSUPPORTED, "D = %d > 256 is not supported", D);
    return GT_OK;
}

// ---------------------------------------------------------------- profiling

struct Profile {
    bool on = false;
    std::vector<hipEvent_t> ev;  // 4 per call: call start, kernel start, kernel end, call end
    int capacity = 0;
    int used = 0;
};
Profile g_prof;

void release_profile() {
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof = Profile{};
}

}  // namespace

// ==================================================================== C ABI

extern "C" {

const char* gt_status_string(int status) {
    switch (status) {
        case GT_OK: return "ok";
        case GT_EINVAL: return "invalid argument";
        case GT_EUNSUPPORTED: return "unsupported argument";
        case GT_ENOMEM: return "out of device memory";
        case GT_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* gt_last_error(void) { return g_err.c_str(); }

int gt_config_set(int32_t key, int64_t value) {
    if (key != GT_CFG_CHUNK_EDGES) return fail(GT_EINVAL, "unknown configuration key %d", key);
    if (value < 1 || value > ((int64_t)1 << 30)) return fail(GT_EINVAL, "chunk edges %lld out of range", (long long)value);
    g_chunk.store(value);
    return GT_OK;
}

int64_t gt_config_get(int32_t key) { return key == GT_CFG_CHUNK_EDGES ? g_chunk.load() : -1; }

int gt_profile_begin(int32_t capacity) {
    if (capacity < 1) return fail(GT_EINVAL, "profile capacity must be >= 1");
    release_profile();
    g_prof.ev.resize((size_t)capacity * 4, nullptr);
    for (auto& e : g_prof.ev) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
            release_profile();
            return hip_fail(err, "hipEventCreate");
        }
    }
    g_prof.capacity = capacity;
    g_prof.used = 0;
    g_prof.on = true;
    return GT_OK;
}

int gt_profile_end(double* kernel_ms, double* call_ms, int64_t* calls) {
    double kt = 0.0, ct = 0.0;
    const int n = g_prof.used;
    for (int i = 0; i < n; ++i) {
        hipEvent_t* e = &g_prof.ev[(size_t)i * 4];
        hipError_t err = hipEventSynchronize(e[3]);
        if (err != hipSuccess) {
            release_profile();
            return hip_fail(err, "hipEventSynchronize");
        }
        float a = 0.0f, b = 0.0f;
        (void)hipEventElapsedTime(&a, e[1], e[2]);
        (void)hipEventElapsedTime(&b, e[0], e[3]);
        kt += a;
        ct += b;
    }
    release_profile();
    if (kernel_ms) *kernel_ms = kt;
    if (call_ms) *call_ms = ct;
    if (calls) *calls = n;
    return GT_OK;
}

}  // extern "C"

namespace {

int fused_fwd(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V, void* out,
              float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream) {
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0) return GT_OK;
    if (!indptr || !Q || !K || !V || !out) return fail(GT_EINVAL, "NULL array with N > 0");
    if (E > 0 && !indices) return fail(GT_EINVAL, "NULL indices with E > 0");
    Args a{};
    a.indptr = indptr;
    a.indices = indices;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.out = out;
    a.lse_out = lse;
    a.N = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    a.qscale = (float)(1.4426950408889634074 / std::sqrt((double)D));
    choose_layout(a, {Q, K, V, out});

    hipEvent_t* ev = nullptr;
    if (g_prof.on && g_prof.used < g_prof.capacity) ev = &g_prof.ev[(size_t)(g_prof.used++) * 4];
    if (ev) (void)hipEventRecord(ev[0], stream);
    rc = make_plan(indptr, N, E, H, D, stream, a);
    if (rc) return rc;
    hipError_t e = launch_fused(a, stream, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr);
    if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
    if (a.plan.max_heavy) {
        e = launch_fused_merge(a, stream);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
    if (ev) (void)hipEventRecord(ev[3], stream);
    return GT_OK;
}

}  // namespace

extern "C" {

int gt_sparse_mha_fwd(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                      void* out, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream) {
    return fused_fwd(indptr, indices, Q, K, V, out, nullptr, N, E, H, D, dtype, stream);
}

int gt_sparse_mha_fwd_lse(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                          void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                          hipStream_t stream) {
    if (N > 0 && !lse) return fail(GT_EINVAL, "NULL lse with N > 0");
    return fused_fwd(indptr, indices, Q, K, V, out, lse, N, E, H, D, dtype, stream);
}

int gt_sparse_mha_bwd(const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr, const int32_t* t_indices,
                      const void* Q, const void* K, const void* V, const void* out, const void* dout, const float* lse,
                      void* dQ, void* dK, void* dV, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                      hipStream_t stream) {
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0) return GT_OK;
    if (!indptr || !t_indptr || !Q || !K || !V || !out || !dout || !lse || !dQ || !dK || !dV)
        return fail(GT_EINVAL, "NULL array with N > 0");
    if (E > 0 && (!indices || !t_indices)) return fail(GT_EINVAL, "NULL indices with E > 0");
    Args a{};
    a.indices = indices;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = out;
    a.dO = dout;
    a.lse_in = lse;
    a.dQ = dQ;
    a.dK = dK;
    a.dV = dV;
    a.N = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    a.qscale = (float)(1.4426950408889634074 / std::sqrt((double)D));
    a.kscale = (float)(1.0 / std::sqrt((double)D));
    choose_layout(a, {Q, K, V, out, dout, dQ, dK, dV});
    const int64_t HD = (int64_t)H * D;

    // scratch: plan over destinations (dQ partials HD wide), plan over sources
    // (dK and dV partials, 2 HD wide), and delta [N][H]
    Args at = a;
    const size_t b1 = plan_bytes(N, E, H, HD, a.plan);
    const size_t b2 = plan_bytes(N, E, H, 2 * HD, at.plan);
    rc = check_plan(a.plan);
    if (!rc) rc = check_plan(at.plan);
    if (rc) return rc;
    void* base = nullptr;
    rc = get_scratch(stream, b1 + b2 + align256(sizeof(float) * (size_t)N * H), &base);
    if (rc) return rc;
    char* p = carve_plan((char*)base, H, HD, a.plan);
    p = carve_plan(p, H, 2 * HD, at.plan);
    a.delta = at.delta = (float*)p;

    a.indptr = indptr;
    a.indices = indices;
    a.items = a.plan.max_chunks + N;
    at.indptr = t_indptr;
    at.indices = t_indices;
    at.items = at.plan.max_chunks + N;
    hipError_t e = launch_plan(a, stream);
    if (e == hipSuccess) e = launch_plan(at, stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    e = launch_bwd_dq(a, stream);
    if (e != hipSuccess) return hip_fail(e, "dQ kernel launch");
    e = launch_bwd_dkv(at, stream);
    if (e != hipSuccess) return hip_fail(e, "dK/dV kernel launch");
    return GT_OK;
}

int gt_sddmm(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, float* scores, int64_t N,
             int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream) {
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0 || E == 0) return GT_OK;
    if (!indptr || !indices || !Q || !K || !scores) return fail(GT_EINVAL, "NULL array with E > 0");
    Args a{};
    a.indptr = indptr;
    a.indices = indices;
    a.Q = Q;
    a.K = K;
    a.scores_out = scores;
    a.N = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    a.qscale = (float)(1.0 / std::sqrt((double)D));
    choose_layout(a, {Q, K});
    rc = make_plan(indptr, N, E, H, D, stream, a);
    if (rc) return rc;
    hipError_t e = launch_sddmm(a, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "sddmm launch");
}

int gt_edge_softmax(const int64_t* indptr, const float* scores, float* alpha, int64_t N, int64_t E, int32_t H,
                    hipStream_t stream) {
    int rc = check_common(N, E, H, 1, GT_F32);
    if (rc) return rc;
    if (N == 0 || E == 0) return GT_OK;
    if (!indptr || !scores || !alpha) return fail(GT_EINVAL, "NULL array with E > 0");
    Args a{};
    a.indptr = indptr;
    a.scores_in = scores;
    a.alpha_out = alpha;
    a.N = N;
    a.E = E;
    a.H = H;
    a.D = 1;
    a.dtype = GT_F32;
    rc = make_plan(indptr, N, E, H, 1, stream, a);
    if (rc) return rc;
    hipError_t e = launch_softmax(a, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "edge softmax launch");
}

int gt_spmm(const int64_t* indptr, const int32_t* indices, const float* alpha, const void* V, void* out, int64_t N,
            int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream) {
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0) return GT_OK;
    if (!indptr || !V || !out) return fail(GT_EINVAL, "NULL array with N > 0");
    if (E > 0 && (!indices || !alpha)) return fail(GT_EINVAL, "NULL array with E > 0");
    Args a{};
    a.indptr = indptr;
    a.indices = indices;
    a.alpha_in = alpha;
    a.V = V;
    a.out = out;
    a.N = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    choose_layout(a, {V, out});
    rc = make_plan(indptr, N, E, H, D, stream, a);
    if (rc) return rc;
    hipError_t e = launch_spmm(a, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "spmm launch");
}

int gt_validate_csr(const int64_t* indptr, const int32_t* indices, int64_t N, int64_t E, hipStream_t stream) {
    if (N < 0 || E < 0) return fail(GT_EINVAL, "N and E must be >= 0");
    if (N >= ((int64_t)1 << 31)) return fail(GT_EINVAL, "N must be < 2^31");
    if (!indptr) return fail(GT_EINVAL, "NULL indptr");
    if (E > 0 && !indices) return fail(GT_EINVAL, "NULL indices with E > 0");
    void* buf = nullptr;
    int rc = get_scratch(stream, 256, &buf);
    if (rc) return rc;
    hipError_t e = launch_validate(indptr, indices, N, E, (uint32_t*)buf, stream);
    if (e != hipSuccess) return hip_fail(e, "validate launch");
    uint32_t flags = 0;
    e = hipMemcpyAsync(&flags, buf, sizeof flags, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "validate readback");
    if (flags == 0) return GT_OK;
    std::string why;
    if (flags & 1) why += " indptr[0] != 0;";
    if (flags & 2) why += " indptr[N] != E;";
    if (flags & 4) why += " indptr decreases;";
    if (flags & 8) why += " an index is outside [0, N);";
    return fail(GT_EINVAL, "invalid CSR:%s", why.c_str());
}

}  // extern "C"
