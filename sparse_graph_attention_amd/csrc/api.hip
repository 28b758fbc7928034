// api.hip -- the C ABI of libgtattn (declared in include/gtattn.h): argument
// checks, the per-(device, stream) scratch buffer, layout choice and launches.
#include <gtattn.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <new>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "kernels.hpp"

using namespace gt;

namespace {

thread_local std::string g_err;
std::atomic<int64_t> g_chunk{0};  // the configured split threshold; 0: automatic

// The automatic split threshold.  Each chunk of a split row is one wave's
// item, and a wave keeps only a few edges' rows in flight (on its own, some
// 10-20 GB/s at memory latency), so a chunk must stay short against the call
// as a whole.  From 2^23 edges up, the 4,096 waves the chip holds at four a
// SIMD average 2,048 edges each, and 2,048-edge chunks make fewer partials
// and merges than 512-edge ones; below that, chunks stay at 512 edges.  The
// unfused softmax keeps 512: its row kernel gives each row below the
// threshold to one wave, and rows of a few thousand edges would each hold one
// wave for their whole length.
constexpr int64_t kChunkSmall = 512, kChunkLarge = 2048, kChunkLargeFromEdges = (int64_t)1 << 23;

int64_t chunk_for(int64_t E, bool softmax) {
    const int64_t c = g_chunk.load();
    if (c > 0) return c;
    return !softmax && E >= kChunkLargeFromEdges ? kChunkLarge : kChunkSmall;
}

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

// Test hook: with GT_TEST_FAIL_ALLOC set to anything but "" or "0", every
// device allocation the library would make (scratch growth, plans) fails as
// if the device were out of memory: the call returns GT_ENOMEM before any
// HIP call, so nothing is enqueued.
bool alloc_refused() {
    const char* v = getenv("GT_TEST_FAIL_ALLOC");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

struct Scratch {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_scratch_mu;
std::map<std::pair<int, uintptr_t>, Scratch> g_scratch;

// A buffer of at least `bytes` for `stream` on the current device.  Growth
// is stream-ordered: the old buffer goes back to the device's memory pool
// after the work already queued on `stream` (hipFreeAsync), and the new one
// is allocated in the stream's order (hipMallocAsync), so no call waits for
// the device.
int get_scratch(hipStream_t stream, size_t bytes, void** out) {
    if (alloc_refused()) return fail(GT_ENOMEM, "scratch allocation refused (GT_TEST_FAIL_ALLOC is set)");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    Scratch& s = g_scratch[{dev, (uintptr_t)stream}];
    if (s.bytes < bytes) {
        if (s.ptr) {
            e = hipFreeAsync(s.ptr, stream);
            if (e != hipSuccess) return hip_fail(e, "hipFreeAsync of the old scratch");
            s.ptr = nullptr;
            s.bytes = 0;
        }
        size_t want = bytes + bytes / 4;  // headroom against frequent regrowth
        e = hipMallocAsync(&s.ptr, want, stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            s.ptr = nullptr;
            return fail(GT_ENOMEM, "hipMallocAsync of %zu scratch bytes failed: %s", want, hipGetErrorString(e));
        }
        s.bytes = want;
    }
    *out = s.ptr;
    return GT_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A plan has tables (counters, heavy rows, chunk list: built once per graph)
// and partials (per-chunk results, sized by the features: per call).
// Sizes the tables for a graph of N rows and E edges at the current split
// threshold.
void size_plan_at(int64_t N, int64_t E, int64_t C, Plan& p) {
    p.chunk = C;
    p.max_heavy = std::min<int64_t>(N, E / (C + 1));
    p.max_chunks = p.max_heavy ? E / C + p.max_heavy : 0;
    // the row order by degree bin comes with the plan kernel, which runs when
    // a row can be split, on graphs of more than one plan block of rows (for
    // other graphs rows go in index order)
    p.n_order = p.max_heavy && N > kPlanBlockRows ? N : 0;
}

void size_plan(int64_t N, int64_t E, Plan& p) { size_plan_at(N, E, chunk_for(E, false), p); }

size_t table_bytes(const Plan& p) {
    return align256(sizeof(PlanCounters)) + align256(sizeof(HeavyRow) * p.max_heavy) +
           align256(sizeof(ChunkRef) * p.max_chunks) + align256(sizeof(int32_t) * p.n_order);
}

// Partials of chunks `accw` floats wide.
size_t partial_bytes(const Plan& p, int H, int64_t accw) {
    return 2 * align256(sizeof(float) * p.max_chunks * H) + align256(sizeof(float) * p.max_chunks * accw) +
           align256(sizeof(float) * p.max_heavy * H * 2);
}

char* carve_tables(char* b, Plan& p) {
    p.counters = (PlanCounters*)b;               b += align256(sizeof(PlanCounters));
    p.heavy = (HeavyRow*)b;                      b += align256(sizeof(HeavyRow) * p.max_heavy);
    p.chunks = (ChunkRef*)b;                     b += align256(sizeof(ChunkRef) * p.max_chunks);
    p.order = p.n_order ? (int32_t*)b : nullptr; b += align256(sizeof(int32_t) * p.n_order);
    return b;
}

char* carve_partials(char* b, int H, int64_t accw, Plan& p) {
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

// Sizes the plan for (N, E), carves tables and partials out of the stream's
// scratch and lists the split rows on the device.
int make_plan(const int64_t* indptr, int64_t N, int64_t E, int H, int D, hipStream_t stream, Args& a,
              bool softmax = false) {
    (void)indptr;
    size_plan_at(N, E, chunk_for(E, softmax), a.plan);
    int rc = check_plan(a.plan);
    if (rc) return rc;
    const int64_t accw = (int64_t)H * D;
    a.items = a.plan.max_chunks + N;
    void* base = nullptr;
    rc = get_scratch(stream, table_bytes(a.plan) + partial_bytes(a.plan, H, accw), &base);
    if (rc) return rc;
    carve_partials(carve_tables((char*)base, a.plan), H, accw, a.plan);
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

// Vector layout when every head is a whole number of 16-byte vectors, the
// row fits in four lane slots per lane and the feature arrays are aligned;
// the scalar layout otherwise.  A head of vph vectors takes lph =
// pow2ceil(vph) lane slots, so that head sums stay within aligned lane
// segments; the slots past vph idle (for example fp32 D = 48: 12 vectors in
// 16 slots).
void choose_layout(Args& a, std::initializer_list<const void*> feats) {
    const int bytes = a.dtype == GT_F32 ? 4 : 2;
    const int64_t hb = (int64_t)a.D * bytes;
    bool vec = hb % 16 == 0;
    for (const void* p : feats) vec = vec && aligned16(p);
    if (vec) {
        a.vph = (int)(hb / 16);
        a.lph = pow2ceil(a.vph);
        a.Rm = a.H * a.vph;
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
        a.lph = a.R = a.NC = a.vph = a.Rm = 0;
    }
}

// Word layout for plain logits when choose_layout fell back to one wave per
// head: every head a whole number vph of 8-byte (else 4-byte) words, in lph =
// pow2ceil(vph) <= 32 lane slots, all H heads of an edge in one lane group of
// G = pow2ceil(H * lph) <= 64 lanes, the feature arrays aligned to the word.  The
// shape it is for: fp32 heads of 10 elements (five 8-byte words), 8 heads in
// 64 lanes; a wave then takes 1 (row) instead of 8 (row, head) items with
// 4-byte loads.  word_bytes: the word for heads of hb bytes with arrays
// aligned to `align` bytes, 0 if none fits.
int word_bytes(int64_t H, int64_t hb, int align) {
    for (int w : {8, 4})
        if (w <= align && hb % w == 0 && pow2ceil(hb / w) <= 32 && H * pow2ceil(hb / w) <= kWave) return w;
    return 0;
}

bool choose_word_layout(Args& a, std::initializer_list<const void*> feats) {
    if (a.vec || extended(a)) return false;
    const int64_t hb = (int64_t)a.D * (a.dtype == GT_F32 ? 4 : 2);
    uintptr_t bits = 0;
    for (const void* p : feats) bits |= (uintptr_t)p;
    const int wb = word_bytes(a.H, hb, bits % 8 == 0 ? 8 : bits % 4 == 0 ? 4 : 0);
    if (!wb) return false;
    const int64_t vph = hb / wb;
    const int lph = pow2ceil(vph);
    a.vec = 3;
    a.wb = wb;
    a.vph = (int)vph;
    a.lph = lph;
    a.R = a.Rm = a.H * (int)vph;
    a.G = pow2ceil((int64_t)a.H * lph);
    a.NC = 1;
    a.KD = 0;
    return true;
}

// The forward's layout over [N][H][D] rows: vector, else word, else scalar.
void choose_fwd_layout(Args& a, std::initializer_list<const void*> feats) {
    choose_layout(a, feats);
    choose_word_layout(a, feats);
}

// The head-innermost kernels: a 16-byte vector holds VN heads of one d, the
// vectors of a d are a power of two, and a row is at most 256 vectors (a
// lane group of pow2ceil(R) lanes up to 64, then NC = ceil(R / 64) vectors
// per lane of a 64-lane group).
bool choose_layout_ndh(Args& a, std::initializer_list<const void*> feats) {
    const int vn = a.dtype == GT_F32 ? 4 : 8;
    if (a.H % vn != 0 || !pow2(a.H / vn)) return false;
    const int64_t R = (int64_t)a.D * (a.H / vn);
    if (R > 4 * kWave) return false;
    for (const void* p : feats)
        if (!aligned16(p)) return false;
    a.vec = 2;
    a.ndh = 1;
    a.lph = a.vph = a.H / vn;
    a.R = a.Rm = (int)R;
    a.G = R > kWave ? kWave : pow2ceil(R);
    a.NC = (int)((R + a.G - 1) / a.G);
    return true;
}

// Whether the head-innermost kernels beat transposing into [N][H][D], run
// with a layout chosen by choose_fwd_layout.  Their cost is the head sums: a
// lane holds VN heads of one d, so each head's dot product takes VN *
// log2(G / HV) cross-lane shuffles per edge, where [N][H][D] rows sum a head
// in a few DPP steps; the copies cost five transposes in and three out (one
// in and one out for the forward), each a launch.  Measured:
// - heads that [N][H][D] serves only one wave per head: the native kernels;
// - heads that take the word layout in [N][H][D] (fp32 8 x 10): the native
//   forward (molecule batch 17 against 43 us, power-law graph 2.30 against
//   2.65 ms); the backward through copies on large graphs (power-law 5.6
//   against 13.7 ms), natively on small ones, where the launches of the
//   copies outweigh the head sums (molecule batch, 8.5 K edges: 61 against
//   93 us);
// - heads of 16-byte vectors: the forward natively when a row's gathers are
//   large against its shuffles (fp32 8 x 64: 4 KB per edge for 20 shuffles,
//   12.2 against 16.9 ms), through copies when they are not (bf16 8 x 32: 1 KB
//   for 40 shuffles, 19.5 against 11 ms); the backward, with two head sums
//   per edge in each pass, through copies at both of those shapes.
constexpr int64_t kNdhBwdCopiesMinEdges = 1 << 16;

bool ndh_kernels_pay(const Args& a, bool forward) {
    const int64_t hb = (int64_t)a.D * (a.dtype == GT_F32 ? 4 : 2);
    if (!(hb % 16 == 0 && (a.H * (int64_t)pow2ceil(hb / 16) + kWave - 1) / kWave <= 4)) {
        if (!word_bytes(a.H, hb, 8)) return true;
        return forward || a.E < kNdhBwdCopiesMinEdges;
    }
    if (!forward) return false;
    int steps = 0;
    for (int64_t x = a.G / a.lph; x > 1; x >>= 1) ++steps;
    const int shuffles = (a.dtype == GT_F32 ? 4 : 8) * steps;
    return 2 * (int64_t)a.R * 16 >= 128 * (int64_t)shuffles;
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
    std::vector<hipEvent_t> ev;  // 4 per call: call start, kernels start, kernels end, call end
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
    if (value < 0 || value > ((int64_t)1 << 30)) return fail(GT_EINVAL, "chunk edges %lld out of range", (long long)value);
    g_chunk.store(value);
    return GT_OK;
}

int64_t gt_config_get(int32_t key) { return key == GT_CFG_CHUNK_EDGES ? g_chunk.load() : -1; }

int64_t gt_config_chunk_edges(int64_t E, int32_t softmax) { return E < 0 ? -1 : chunk_for(E, softmax != 0); }

int gt_scratch_release(hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch.find({dev, (uintptr_t)stream});
    if (it == g_scratch.end()) return GT_OK;
    e = it->second.ptr ? hipFreeAsync(it->second.ptr, stream) : hipSuccess;
    g_scratch.erase(it);
    return e == hipSuccess ? GT_OK : hip_fail(e, "hipFreeAsync");
}

int64_t gt_scratch_bytes(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch.find({dev, (uintptr_t)stream});
    return it == g_scratch.end() ? 0 : (int64_t)it->second.bytes;
}

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

// The fused forward on a's CSR (a.N rows), features and layout.  Without
// `tables` the plan is built in the stream's scratch; with them (a prebuilt
// plan of this graph) only the chunk partials come from scratch.
int run_fwd(Args& a, const Plan* tables, hipStream_t stream) {
    hipEvent_t* ev = nullptr;
    if (g_prof.on && g_prof.used < g_prof.capacity) ev = &g_prof.ev[(size_t)(g_prof.used++) * 4];
    if (ev) (void)hipEventRecord(ev[0], stream);
    int rc;
    if (tables) {
        const int64_t accw = (int64_t)a.H * a.D;
        a.plan = *tables;
        void* base = nullptr;
        rc = get_scratch(stream, partial_bytes(a.plan, a.H, accw), &base);
        if (rc) return rc;
        carve_partials((char*)base, a.H, accw, a.plan);
        a.items = a.plan.max_chunks + a.N;
    } else {
        rc = make_plan(a.indptr, a.N, a.E, a.H, a.D, stream, a);
        if (rc) return rc;
    }
    // the attention kernels: the fused kernel and the merge of split rows,
    // which writes those rows' outputs
    hipError_t e = launch_fused(a, stream, ev ? ev[1] : nullptr, nullptr);
    if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
    if (a.plan.max_heavy) {
        e = launch_fused_merge(a, stream);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
    if (ev) (void)hipEventRecord(ev[2], stream);
    if (ev) (void)hipEventRecord(ev[3], stream);
    return GT_OK;
}

void set_scales(Args& a) {
    a.qscale = (float)(1.4426950408889634074 / std::sqrt((double)a.D));
    a.kscale = (float)(1.0 / std::sqrt((double)a.D));
}

// Logit variants and dropout from the caller's options (nullptr: none).
int set_options(Args& a, const gt_logit_opts* o) {
    if (!o) return GT_OK;
    const double p = o->dropout_p;
    if (!(p >= 0.0 && p < 1.0)) return fail(GT_EINVAL, "dropout_p = %g is outside [0, 1)", p);
    a.bias = o->bias;
    a.ew = o->edge_weight;
    a.drop_seed = o->dropout_seed;
    a.drop_thresh = (uint32_t)std::floor(p * 4294967296.0);
    a.drop_scale = (float)(1.0 / (1.0 - p));
    return GT_OK;
}

int fused_fwd(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V, void* out,
              float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype, const gt_logit_opts* opts,
              hipStream_t stream) {
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
    a.n_gather = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    set_scales(a);
    rc = set_options(a, opts);
    if (rc) return rc;
    choose_fwd_layout(a, {Q, K, V, out});
    return run_fwd(a, nullptr, stream);
}

// The backward: a over the destination-sorted graph (a.N destinations), at
// over the source-sorted one (at.N sources).  Without tables both plans are
// built in scratch; with them only partials and delta come from scratch.
// Scratch bytes of run_bwd (sizes the plans when no tables are given).
int bwd_scratch_bytes(Args& a, Args& at, const Plan* tables, const Plan* t_tables, size_t* out) {
    const int64_t HD = (int64_t)a.H * a.D;
    size_t bytes = align256(sizeof(float2) * (size_t)a.N * a.H);  // stats
    if (tables) {
        a.plan = *tables;
        at.plan = *t_tables;
    } else {
        size_plan(a.N, a.E, a.plan);
        size_plan(at.N, at.E, at.plan);
        int rc = check_plan(a.plan);
        if (!rc) rc = check_plan(at.plan);
        if (rc) return rc;
        bytes += table_bytes(a.plan) + table_bytes(at.plan);
    }
    bytes += partial_bytes(a.plan, a.H, HD) + partial_bytes(at.plan, a.H, 2 * HD);
    if (a.dew && !a.vec) bytes += align256(sizeof(float) * (size_t)a.E * a.H);
    *out = bytes;
    return GT_OK;
}

// Scratch bytes of run_fwd without tables.
int fwd_scratch_bytes(int64_t N, int64_t E, int H, int D, size_t* out) {
    Plan p{};
    size_plan(N, E, p);
    int rc = check_plan(p);
    if (rc) return rc;
    *out = table_bytes(p) + partial_bytes(p, H, (int64_t)H * D);
    return GT_OK;
}

int run_bwd(Args& a, Args& at, const Plan* tables, const Plan* t_tables, hipStream_t stream) {
    const int64_t HD = (int64_t)a.H * a.D;
    size_t bytes = 0;
    int brc = bwd_scratch_bytes(a, at, tables, t_tables, &bytes);
    if (brc) return brc;
    const bool dew_part = a.dew && !a.vec;  // one-head waves: dw's per-head terms go through scratch
    const size_t part_bytes = dew_part ? align256(sizeof(float) * (size_t)a.E * a.H) : 0;
    void* base = nullptr;
    int rc = get_scratch(stream, bytes, &base);
    if (rc) return rc;
    char* p = (char*)base;
    a.stats = at.stats = (float2*)p;
    p += align256(sizeof(float2) * (size_t)a.N * a.H);
    if (dew_part) {
        a.dew_part = (float*)p;
        p += part_bytes;
    }
    if (!tables) {
        p = carve_tables(p, a.plan);
        p = carve_tables(p, at.plan);
    }
    p = carve_partials(p, a.H, HD, a.plan);
    carve_partials(p, a.H, 2 * HD, at.plan);
    a.items = a.plan.max_chunks + a.N;
    at.items = at.plan.max_chunks + at.N;
    hipError_t e = hipSuccess;
    if (!tables) {
        e = launch_plan(a, stream);
        if (e == hipSuccess) e = launch_plan(at, stream);
        if (e != hipSuccess) return hip_fail(e, "plan launch");
    }
    e = launch_bwd_dq(a, stream);
    if (e != hipSuccess) return hip_fail(e, "dQ kernel launch");
    e = launch_bwd_dkv(at, stream);
    if (e != hipSuccess) return hip_fail(e, "dK/dV kernel launch");
    return GT_OK;
}

// Arguments of the backward over (destination CSR, source CSR) with n_dst
// destinations (rows of Q, out, dout, lse, dQ) and n_src sources (rows of K,
// V, dK, dV).
int bwd_args(Args& a, Args& at, const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr,
             const int32_t* t_indices, const int32_t* t_perm, const void* Q, const void* K, const void* V,
             const void* out, const void* dout, const float* lse, void* dQ, void* dK, void* dV, float* dbias,
             float* dew, int64_t n_dst, int64_t n_src, int64_t E, int32_t H, int32_t D, int32_t dtype,
             const gt_logit_opts* opts) {
    a = Args{};
    a.indptr = indptr;
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
    a.N = n_dst;
    a.n_gather = n_src;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    set_scales(a);
    int rc = set_options(a, opts);
    if (rc) return rc;
    choose_layout(a, {Q, K, V, out, dout, dQ, dK, dV});
    at = a;
    at.indptr = t_indptr;
    at.indices = t_indices;
    at.t_perm = t_perm;
    at.N = n_src;
    at.n_gather = n_dst;
    // the destination pass writes the per-edge gradients; the source pass
    // needs the CSR positions of its out-edges only for per-edge inputs
    a.dbias = dbias;
    a.dew = dew;
    if (choose_word_layout(a, {Q, K, V, out, dout, dQ, dK, dV})) {
        at.vec = a.vec;
        at.wb = a.wb;
        at.vph = a.vph;
        at.lph = a.lph;
        at.R = a.R;
        at.Rm = a.Rm;
        at.G = a.G;
        at.NC = a.NC;
        at.KD = a.KD;
    }
    if (extended(at) && E > 0 && !t_perm)
        return fail(GT_EINVAL, "bias, edge weights or dropout need the transpose's CSR positions (t_perm)");
    return GT_OK;
}

}  // namespace

extern "C" {

int gt_sparse_mha_fwd(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                      void* out, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype, hipStream_t stream) {
    return fused_fwd(indptr, indices, Q, K, V, out, nullptr, N, E, H, D, dtype, nullptr, stream);
}

int gt_sparse_mha_fwd_lse(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                          void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                          hipStream_t stream) {
    if (N > 0 && !lse) return fail(GT_EINVAL, "NULL lse with N > 0");
    return fused_fwd(indptr, indices, Q, K, V, out, lse, N, E, H, D, dtype, nullptr, stream);
}

int gt_sparse_mha_fwd_ex(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K, const void* V,
                         void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                         const gt_logit_opts* opts, hipStream_t stream) {
    return fused_fwd(indptr, indices, Q, K, V, out, lse, N, E, H, D, dtype, opts, stream);
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
    Args a, at;
    rc = bwd_args(a, at, indptr, indices, t_indptr, t_indices, nullptr, Q, K, V, out, dout, lse, dQ, dK, dV, nullptr,
                  nullptr, N, N, E, H, D, dtype, nullptr);
    if (rc) return rc;
    return run_bwd(a, at, nullptr, nullptr, stream);
}

int gt_sparse_mha_bwd_ex(const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr,
                         const int32_t* t_indices, const int32_t* t_perm, const void* Q, const void* K, const void* V,
                         const void* out, const void* dout, const float* lse, void* dQ, void* dK, void* dV,
                         float* dbias, float* dweight, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                         const gt_logit_opts* opts, hipStream_t stream) {
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0) return GT_OK;
    if (!indptr || !t_indptr || !Q || !K || !V || !out || !dout || !lse || !dQ || !dK || !dV)
        return fail(GT_EINVAL, "NULL array with N > 0");
    if (E > 0 && (!indices || !t_indices)) return fail(GT_EINVAL, "NULL indices with E > 0");
    Args a, at;
    rc = bwd_args(a, at, indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse, dQ, dK, dV, dbias,
                  dweight, N, N, E, H, D, dtype, opts);
    if (rc) return rc;
    return run_bwd(a, at, nullptr, nullptr, stream);
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
    a.n_gather = N;
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
    rc = make_plan(indptr, N, E, H, 1, stream, a, true);
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
    a.n_gather = N;
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

int gt_sparse_mha_fwd_layout(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K,
                             const void* V, void* out, float* lse, int64_t N, int64_t E, int32_t H, int32_t D,
                             int32_t dtype, int32_t layout, const gt_logit_opts* opts, hipStream_t stream) {
    if (layout == GT_LAYOUT_NHD) return fused_fwd(indptr, indices, Q, K, V, out, lse, N, E, H, D, dtype, opts, stream);
    if (layout != GT_LAYOUT_NDH) return fail(GT_EINVAL, "unknown layout %d", layout);
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
    a.n_gather = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    set_scales(a);
    rc = set_options(a, opts);
    if (rc) return rc;
    Args an = a;  // the head-innermost kernels' arguments, if they are used
    if (!extended(a) && choose_layout_ndh(an, {Q, K, V, out}) && ndh_kernels_pay(an, true))
        return run_fwd(an, nullptr, stream);
    // other shapes and the logit options: through [N][H][D] copies in scratch,
    // after the plan's part of it
    size_t pb = 0;
    rc = fwd_scratch_bytes(N, E, H, D, &pb);
    if (rc) return rc;
    const size_t fb = align256((size_t)N * H * D * (dtype == GT_F32 ? 4 : 2));
    void* base = nullptr;
    rc = get_scratch(stream, align256(pb) + 4 * fb, &base);
    if (rc) return rc;
    char* t = (char*)base + align256(pb);
    void *Qt = t, *Kt = t + fb, *Vt = t + 2 * fb, *Ot = t + 3 * fb;
    hipError_t e = launch_transpose_rows(Q, Qt, N, D, H, dtype, stream);
    if (e == hipSuccess) e = launch_transpose_rows(K, Kt, N, D, H, dtype, stream);
    if (e == hipSuccess) e = launch_transpose_rows(V, Vt, N, D, H, dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "layout transpose");
    a.Q = Qt;
    a.K = Kt;
    a.V = Vt;
    a.out = Ot;
    choose_fwd_layout(a, {Qt, Kt, Vt, Ot});
    rc = run_fwd(a, nullptr, stream);
    if (rc) return rc;
    e = launch_transpose_rows(Ot, out, N, H, D, dtype, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "layout transpose");
}

int gt_sparse_mha_bwd_layout(const int64_t* indptr, const int32_t* indices, const int64_t* t_indptr,
                             const int32_t* t_indices, const int32_t* t_perm, const void* Q, const void* K,
                             const void* V, const void* out, const void* dout, const float* lse, void* dQ, void* dK,
                             void* dV, float* dbias, float* dweight, int64_t N, int64_t E, int32_t H, int32_t D,
                             int32_t dtype, int32_t layout, const gt_logit_opts* opts, hipStream_t stream) {
    if (layout == GT_LAYOUT_NHD)
        return gt_sparse_mha_bwd_ex(indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse, dQ, dK, dV,
                                    dbias, dweight, N, E, H, D, dtype, opts, stream);
    if (layout != GT_LAYOUT_NDH) return fail(GT_EINVAL, "unknown layout %d", layout);
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0) return GT_OK;
    if (!indptr || !t_indptr || !Q || !K || !V || !out || !dout || !lse || !dQ || !dK || !dV)
        return fail(GT_EINVAL, "NULL array with N > 0");
    if (E > 0 && (!indices || !t_indices)) return fail(GT_EINVAL, "NULL indices with E > 0");
    Args a, at;
    rc = bwd_args(a, at, indptr, indices, t_indptr, t_indices, t_perm, Q, K, V, out, dout, lse, dQ, dK, dV, dbias,
                  dweight, N, N, E, H, D, dtype, opts);
    if (rc) return rc;
    Args an = a;  // the head-innermost kernels' arguments, if they are used
    if (!extended(a) && choose_layout_ndh(an, {Q, K, V, out, dout, dQ, dK, dV}) && ndh_kernels_pay(an, false)) {
        a = an;
        at.vec = a.vec;
        at.ndh = a.ndh;
        at.lph = a.lph;
        at.vph = a.vph;
        at.R = a.R;
        at.Rm = a.Rm;
        at.G = a.G;
        at.NC = a.NC;
        return run_bwd(a, at, nullptr, nullptr, stream);
    }
    // other shapes and the logit options: through [N][H][D] copies, five
    // inputs and three gradients after the backward's own part of the scratch
    const size_t fb = align256((size_t)N * H * D * (dtype == GT_F32 ? 4 : 2));
    const void* src[5] = {Q, K, V, out, dout};
    void* cp[8];
    a.vec = at.vec = 1;  // the copies are aligned; only the dew scratch depends on it, sized below for both cases
    size_t bb = 0;
    rc = bwd_scratch_bytes(a, at, nullptr, nullptr, &bb);
    if (rc) return rc;
    if (dweight) bb += align256(sizeof(float) * (size_t)E * H);
    void* base = nullptr;
    rc = get_scratch(stream, align256(bb) + 8 * fb, &base);
    if (rc) return rc;
    char* t = (char*)base + align256(bb);
    for (int i = 0; i < 8; ++i) cp[i] = t + i * fb;
    hipError_t e = hipSuccess;
    for (int i = 0; i < 5 && e == hipSuccess; ++i) e = launch_transpose_rows(src[i], cp[i], N, D, H, dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "layout transpose");
    rc = bwd_args(a, at, indptr, indices, t_indptr, t_indices, t_perm, cp[0], cp[1], cp[2], cp[3], cp[4], lse, cp[5],
                  cp[6], cp[7], dbias, dweight, N, N, E, H, D, dtype, opts);
    if (rc) return rc;
    rc = run_bwd(a, at, nullptr, nullptr, stream);
    if (rc) return rc;
    void* dst[3] = {dQ, dK, dV};
    for (int i = 0; i < 3 && e == hipSuccess; ++i) e = launch_transpose_rows(cp[5 + i], dst[i], N, H, D, dtype, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "layout transpose");
}

// ------------------------------------------------------------------ allocation-free forward

}  // extern "C"

namespace {

// Scratch of gt_sparse_mha_fwd_noalloc: one file-scope device array, which
// each GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)160 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_static_mu;
std::map<int, void*> g_static_ptr;  // device -> address of its `scratch`

int static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_static_mu);
    auto it = g_static_ptr.find(dev);
    if (it == g_static_ptr.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
        it = g_static_ptr.emplace(dev, p).first;
    }
    *out = it->second;
    return GT_OK;
}

// The split threshold may grow to this multiple of the configured one so that
// a plan fits the static scratch.
constexpr int64_t kNoallocChunkGrowth = 64;

}  // namespace

extern "C" {

int gt_sparse_mha_fwd_noalloc(const int64_t* indptr, const int32_t* indices, const void* Q, const void* K,
                              const void* V, void* out, int64_t N, int64_t E, int32_t H, int32_t D, int32_t dtype,
                              hipStream_t stream) {
    int rc = check_common(N, E, H, D, dtype);
    if (rc) return rc;
    if (N == 0) return GT_OK;
    if (!indptr || !Q || !K || !V || !out) return fail(GT_EINVAL, "NULL array with N > 0");
    if (E > 0 && !indices) return fail(GT_EINVAL, "NULL indices with E > 0");
    // the configured split threshold, doubled until the plan's tables and
    // partials fit the static scratch
    const int64_t HD = (int64_t)H * D;
    const int64_t C0 = chunk_for(E, false);
    Plan p{};
    size_t need = 0;
    for (int64_t C = C0;; C *= 2) {
        size_plan_at(N, E, C, p);
        need = table_bytes(p) + partial_bytes(p, H, HD);
        if (need <= kStaticScratchBytes || C >= C0 * kNoallocChunkGrowth || C >= ((int64_t)1 << 30)) break;
    }
    if (need > kStaticScratchBytes)
        return fail(GT_EUNSUPPORTED,
                    "N = %lld, E = %lld, H x D = %lld need %zu bytes of scratch at a split threshold of %lld "
                    "edges; the allocation-free forward has %zu",
                    (long long)N, (long long)E, (long long)HD, need, (long long)p.chunk, kStaticScratchBytes);
    rc = check_plan(p);
    if (rc) return rc;
    void* base = nullptr;
    rc = static_scratch(&base);
    if (rc) return rc;
    Args a{};
    a.indptr = indptr;
    a.indices = indices;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.out = out;
    a.N = N;
    a.n_gather = N;
    a.E = E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    set_scales(a);
    choose_fwd_layout(a, {Q, K, V, out});
    a.plan = p;
    carve_partials(carve_tables((char*)base, a.plan), H, HD, a.plan);
    a.items = a.plan.max_chunks + N;
    // launch_plan clears the counters with a kernel when several blocks add
    // to them, or its one block writes them: nothing carries over from the
    // last call's contents
    hipError_t e = launch_plan(a, stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    e = launch_fused(a, stream, nullptr, nullptr);
    if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
    if (a.plan.max_heavy) {
        e = launch_fused_merge(a, stream);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
    return GT_OK;
}

// ------------------------------------------------------------------ graph plans

}  // extern "C"

struct gt_plan_s {
    int device = 0;
    int64_t n_dst = 0, n_src = 0, E = 0;
    int flags = 0;
    void* mem = nullptr;
    int64_t* indptr = nullptr;
    int32_t* indices = nullptr;
    int64_t* t_indptr = nullptr;
    int32_t* t_indices = nullptr;
    int32_t* t_perm = nullptr;  // CSR position of each out-edge of the transpose
    Plan tables{};    // split rows of the destination-sorted graph
    Plan t_tables{};  // split rows of the source-sorted graph
    // The streams the plan's memory is used on, each with an event recorded
    // after the last work enqueued there; destruction releases the memory in
    // stream order behind all of them.
    std::mutex mu;
    std::vector<std::pair<hipStream_t, hipEvent_t>> uses;
};

namespace {

int check_graph(int64_t n_dst, int64_t n_src, int64_t E) {
    if (n_dst < 0 || n_src < 0 || E < 0) return fail(GT_EINVAL, "node and edge counts must be >= 0");
    if (n_dst >= ((int64_t)1 << 31) || n_src >= ((int64_t)1 << 31)) return fail(GT_EINVAL, "node counts must be < 2^31");
    if (E >= ((int64_t)1 << 31)) return fail(GT_EUNSUPPORTED, "graph construction needs E < 2^31 (E = %lld)", (long long)E);
    return GT_OK;
}

// Groups E items by key (keys < nrows), stably: offsets[nrows + 1] from the
// sorted keys, and out[j] = vals_src[position of the j-th item]; the sorted
// positions go to perm when it is non-null.  `scratch` holds
// sort_scratch_bytes(E, perm != nullptr).
hipError_t group_by_key(const uint32_t* keys, const uint32_t* vals_src, int64_t E, int64_t nrows, int64_t* offsets,
                        uint32_t* out, uint32_t* perm, void* scratch, hipStream_t s) {
    if (group_small_fits(E, 0)) return launch_group_small(keys, vals_src, nullptr, 0, E, nrows, offsets, out, perm, s);
    const uint32_t *ks = nullptr, *vs = nullptr, *v2s = nullptr;
    hipError_t e = perm ? radix_sort(keys, nullptr, vals_src, E, key_bits_for(nrows), scratch, perm, out, s, &ks, &vs,
                                     &v2s)
                        : radix_sort(keys, vals_src, nullptr, E, key_bits_for(nrows), scratch, out, nullptr, s, &ks,
                                     &vs, nullptr);
    if (e == hipSuccess) e = launch_lower_bounds(ks, E, nrows, offsets, s);
    return e;
}

// Source-sorted copy of a destination-sorted graph in the plan.
int build_transpose(gt_plan_s* P, hipStream_t stream) {
    if (group_small_fits(P->E, P->n_dst)) {  // one launch: rows of positions, sort and offsets together
        hipError_t e = launch_group_small((const uint32_t*)P->indices, nullptr, P->indptr, P->n_dst, P->E, P->n_src,
                                          P->t_indptr, (uint32_t*)P->t_indices, (uint32_t*)P->t_perm, stream);
        return e == hipSuccess ? GT_OK : hip_fail(e, "transpose launch");
    }
    void* base = nullptr;
    const size_t rows_bytes = align256(sizeof(uint32_t) * (size_t)P->E);
    int rc = get_scratch(stream, rows_bytes + sort_scratch_bytes(P->E, true), &base);
    if (rc) return rc;
    uint32_t* rows = (uint32_t*)base;
    hipError_t e = launch_row_of_position(P->indptr, P->n_dst, P->E, rows, stream);
    if (e == hipSuccess)
        e = group_by_key((const uint32_t*)P->indices, rows, P->E, P->n_src, P->t_indptr, (uint32_t*)P->t_indices,
                         (uint32_t*)P->t_perm, (char*)base + rows_bytes, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "transpose launch");
}

// Allocates a plan for (n_dst, n_src, E): CSR, transpose (with
// GT_PLAN_TRANSPOSE) and the split-row tables, in one device allocation
// ordered on `stream`.
int alloc_plan(int64_t n_dst, int64_t n_src, int64_t E, int32_t flags, hipStream_t stream, gt_plan_s** out) {
    if (flags & ~GT_PLAN_TRANSPOSE) return fail(GT_EINVAL, "unknown plan flags 0x%x", flags);
    if (alloc_refused()) return fail(GT_ENOMEM, "plan allocation refused (GT_TEST_FAIL_ALLOC is set)");
    auto* P = new (std::nothrow) gt_plan_s;
    if (!P) return fail(GT_ENOMEM, "host allocation of a plan failed");
    P->n_dst = n_dst;
    P->n_src = n_src;
    P->E = E;
    P->flags = flags;
    const bool tr = flags & GT_PLAN_TRANSPOSE;
    size_plan(n_dst, E, P->tables);
    size_plan(tr ? n_src : 0, tr ? E : 0, P->t_tables);
    int rc = check_plan(P->tables);
    if (!rc) rc = check_plan(P->t_tables);
    hipError_t e = hipSuccess;
    if (!rc) e = hipGetDevice(&P->device);
    if (!rc && e != hipSuccess) rc = hip_fail(e, "hipGetDevice");
    const size_t bytes = align256(sizeof(int64_t) * (size_t)(n_dst + 1)) + align256(sizeof(int32_t) * (size_t)E) +
                         (tr ? align256(sizeof(int64_t) * (size_t)(n_src + 1)) + 2 * align256(sizeof(int32_t) * (size_t)E)
                             : 0) +
                         table_bytes(P->tables) + table_bytes(P->t_tables);
    if (!rc) {
        e = hipMallocAsync(&P->mem, bytes, stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            P->mem = nullptr;
            rc = fail(GT_ENOMEM, "hipMallocAsync of %zu plan bytes failed: %s", bytes, hipGetErrorString(e));
        }
    }
    if (rc) {
        delete P;
        return rc;
    }
    char* b = (char*)P->mem;
    P->indptr = (int64_t*)b;      b += align256(sizeof(int64_t) * (size_t)(n_dst + 1));
    P->indices = (int32_t*)b;     b += align256(sizeof(int32_t) * (size_t)E);
    if (tr) {
        P->t_indptr = (int64_t*)b;   b += align256(sizeof(int64_t) * (size_t)(n_src + 1));
        P->t_indices = (int32_t*)b;  b += align256(sizeof(int32_t) * (size_t)E);
        P->t_perm = (int32_t*)b;     b += align256(sizeof(int32_t) * (size_t)E);
    }
    b = carve_tables(b, P->tables);
    carve_tables(b, P->t_tables);
    *out = P;
    return GT_OK;
}

// With the plan's CSR in place: the transpose if asked for, then the tables.
int finish_plan(gt_plan_s* P, hipStream_t stream) {
    int rc = GT_OK;
    if (P->flags & GT_PLAN_TRANSPOSE) rc = build_transpose(P, stream);
    if (rc) return rc;
    Args a{};
    a.indptr = P->indptr;
    a.N = P->n_dst;
    a.plan = P->tables;
    hipError_t e = launch_plan(a, stream);
    if (e == hipSuccess && (P->flags & GT_PLAN_TRANSPOSE)) {
        a.indptr = P->t_indptr;
        a.N = P->n_src;
        a.plan = P->t_tables;
        e = launch_plan(a, stream);
    }
    return e == hipSuccess ? GT_OK : hip_fail(e, "plan launch");
}

// Records that `stream` has work on the plan's memory enqueued up to now.
int note_use(gt_plan_s* P, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(P->mu);
    hipEvent_t ev = nullptr;
    for (auto& u : P->uses)
        if (u.first == stream) ev = u.second;
    if (!ev) {
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
        P->uses.emplace_back(stream, ev);
    }
    hipError_t e = hipEventRecord(ev, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "hipEventRecord");
}

// Stream-ordered release: the null stream waits for the last recorded work
// of every stream that used the plan, then returns its memory to the pool.
// The host does not wait.
void free_plan(gt_plan_s* P) {
    if (!P) return;
    {
        std::lock_guard<std::mutex> lock(P->mu);
        for (auto& u : P->uses) (void)hipStreamWaitEvent(nullptr, u.second, 0);
        if (P->mem) (void)hipFreeAsync(P->mem, nullptr);
        for (auto& u : P->uses) (void)hipEventDestroy(u.second);
        P->uses.clear();
    }
    delete P;
}

int check_plan_use(const gt_plan_s* P) {
    if (!P) return fail(GT_EINVAL, "NULL plan");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != P->device) return fail(GT_EINVAL, "plan was built on device %d, current device is %d", P->device, dev);
    return GT_OK;
}

}  // namespace

extern "C" {

int gt_coo_to_csr(const int32_t* src, const int32_t* dst, int64_t n_dst, int64_t n_src, int64_t E, int64_t* indptr,
                  int32_t* indices, int32_t* perm, hipStream_t stream) {
    int rc = check_graph(n_dst, n_src, E);
    if (rc) return rc;
    if (!indptr) return fail(GT_EINVAL, "NULL indptr");
    if (E > 0 && (!src || !dst || !indices)) return fail(GT_EINVAL, "NULL COO or indices array with E > 0");
    void* base = nullptr;
    rc = get_scratch(stream, sort_scratch_bytes(E, perm != nullptr), &base);
    if (rc) return rc;
    hipError_t e = group_by_key((const uint32_t*)dst, (const uint32_t*)src, E, n_dst, indptr, (uint32_t*)indices,
                                (uint32_t*)perm, base, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "COO to CSR launch");
}

int gt_plan_create(const int64_t* indptr, const int32_t* indices, int64_t n_dst, int64_t n_src, int64_t E,
                   int32_t flags, hipStream_t stream, gt_plan* plan) {
    if (!plan) return fail(GT_EINVAL, "NULL plan pointer");
    *plan = nullptr;
    int rc = check_graph(n_dst, n_src, E);
    if (rc) return rc;
    if (!indptr) return fail(GT_EINVAL, "NULL indptr");
    if (E > 0 && !indices) return fail(GT_EINVAL, "NULL indices with E > 0");
    gt_plan_s* P = nullptr;
    rc = alloc_plan(n_dst, n_src, E, flags, stream, &P);
    if (rc) return rc;
    hipError_t e = hipMemcpyAsync(P->indptr, indptr, sizeof(int64_t) * (size_t)(n_dst + 1), hipMemcpyDeviceToDevice,
                                  stream);
    if (e == hipSuccess && E > 0)
        e = hipMemcpyAsync(P->indices, indices, sizeof(int32_t) * (size_t)E, hipMemcpyDeviceToDevice, stream);
    rc = e == hipSuccess ? finish_plan(P, stream) : hip_fail(e, "CSR copy");
    const int urc = note_use(P, stream);
    if (!rc) rc = urc;
    if (rc) {
        free_plan(P);
        return rc;
    }
    *plan = P;
    return GT_OK;
}

int gt_plan_create_coo(const int32_t* src, const int32_t* dst, int64_t n_dst, int64_t n_src, int64_t E,
                       int32_t flags, hipStream_t stream, gt_plan* plan) {
    if (!plan) return fail(GT_EINVAL, "NULL plan pointer");
    *plan = nullptr;
    int rc = check_graph(n_dst, n_src, E);
    if (rc) return rc;
    if (E > 0 && (!src || !dst)) return fail(GT_EINVAL, "NULL COO array with E > 0");
    gt_plan_s* P = nullptr;
    rc = alloc_plan(n_dst, n_src, E, flags, stream, &P);
    if (rc) return rc;
    void* base = nullptr;
    rc = get_scratch(stream, sort_scratch_bytes(E, false), &base);
    if (!rc) {
        hipError_t e = group_by_key((const uint32_t*)dst, (const uint32_t*)src, E, n_dst, P->indptr,
                                    (uint32_t*)P->indices, nullptr, base, stream);
        rc = e == hipSuccess ? finish_plan(P, stream) : hip_fail(e, "COO to CSR launch");
    }
    const int urc = note_use(P, stream);
    if (!rc) rc = urc;
    if (rc) {
        free_plan(P);
        return rc;
    }
    *plan = P;
    return GT_OK;
}

int gt_plan_destroy(gt_plan plan) {
    free_plan(plan);
    return GT_OK;
}

int gt_plan_info(gt_plan plan, int64_t* n_dst, int64_t* n_src, int64_t* E, const int64_t** indptr,
                 const int32_t** indices, const int64_t** t_indptr, const int32_t** t_indices,
                 const int32_t** t_perm) {
    if (!plan) return fail(GT_EINVAL, "NULL plan");
    if (n_dst) *n_dst = plan->n_dst;
    if (n_src) *n_src = plan->n_src;
    if (E) *E = plan->E;
    if (indptr) *indptr = plan->indptr;
    if (indices) *indices = plan->indices;
    if (t_indptr) *t_indptr = plan->t_indptr;
    if (t_indices) *t_indices = plan->t_indices;
    if (t_perm) *t_perm = plan->t_perm;
    return GT_OK;
}

int gt_plan_copy_graph(gt_plan plan, int64_t* indptr, int32_t* indices, int64_t* t_indptr, int32_t* t_indices,
                       int32_t* t_perm, hipStream_t stream) {
    int rc = check_plan_use(plan);
    if (rc) return rc;
    if ((t_indptr || t_indices || t_perm) && !(plan->flags & GT_PLAN_TRANSPOSE))
        return fail(GT_EINVAL, "the plan was built without GT_PLAN_TRANSPOSE");
    struct Item {
        void* dst;
        const void* src;
        size_t bytes;
    } items[5] = {{indptr, plan->indptr, sizeof(int64_t) * (size_t)(plan->n_dst + 1)},
                  {indices, plan->indices, sizeof(int32_t) * (size_t)plan->E},
                  {t_indptr, plan->t_indptr, sizeof(int64_t) * (size_t)(plan->n_src + 1)},
                  {t_indices, plan->t_indices, sizeof(int32_t) * (size_t)plan->E},
                  {t_perm, plan->t_perm, sizeof(int32_t) * (size_t)plan->E}};
    for (const Item& it : items) {
        if (!it.dst || it.bytes == 0) continue;
        hipError_t e = hipMemcpyAsync(it.dst, it.src, it.bytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) {
            (void)note_use(plan, stream);
            return hip_fail(e, "plan graph copy");
        }
    }
    return note_use(plan, stream);
}

int gt_sparse_mha_fwd_plan(gt_plan plan, const void* Q, const void* K, const void* V, void* out, float* lse,
                           int32_t H, int32_t D, int32_t dtype, const gt_logit_opts* opts, hipStream_t stream) {
    int rc = check_plan_use(plan);
    if (!rc) rc = check_common(plan->n_dst, plan->E, H, D, dtype);
    if (rc) return rc;
    if (plan->n_dst == 0) return GT_OK;
    if (!Q || !out || (plan->E > 0 && (!K || !V))) return fail(GT_EINVAL, "NULL feature array");
    Args a{};
    a.indptr = plan->indptr;
    a.indices = plan->indices;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.out = out;
    a.lse_out = lse;
    a.N = plan->n_dst;
    a.n_gather = plan->n_src;
    a.E = plan->E;
    a.H = H;
    a.D = D;
    a.dtype = dtype;
    set_scales(a);
    rc = set_options(a, opts);
    if (rc) return rc;
    choose_fwd_layout(a, {Q, K, V, out});
    rc = run_fwd(a, &plan->tables, stream);
    const int urc = note_use(plan, stream);
    return rc ? rc : urc;
}

int gt_sparse_mha_bwd_plan(gt_plan plan, const void* Q, const void* K, const void* V, const void* out,
                           const void* dout, const float* lse, void* dQ, void* dK, void* dV, float* dbias,
                           float* dweight, int32_t H, int32_t D, int32_t dtype, const gt_logit_opts* opts,
                           hipStream_t stream) {
    int rc = check_plan_use(plan);
    if (!rc) rc = check_common(std::max(plan->n_dst, plan->n_src), plan->E, H, D, dtype);
    if (rc) return rc;
    if (!(plan->flags & GT_PLAN_TRANSPOSE)) return fail(GT_EINVAL, "the plan was built without GT_PLAN_TRANSPOSE");
    if (plan->n_dst == 0 && plan->n_src == 0) return GT_OK;
    if ((plan->n_dst > 0 && (!Q || !out || !dout || !lse || !dQ)) || (plan->n_src > 0 && (!K || !V || !dK || !dV)))
        return fail(GT_EINVAL, "NULL array");
    Args a, at;
    rc = bwd_args(a, at, plan->indptr, plan->indices, plan->t_indptr, plan->t_indices, plan->t_perm, Q, K, V, out,
                  dout, lse, dQ, dK, dV, dbias, dweight, plan->n_dst, plan->n_src, plan->E, H, D, dtype, opts);
    if (rc) return rc;
    rc = run_bwd(a, at, &plan->tables, &plan->t_tables, stream);
    const int urc = note_use(plan, stream);
    return rc ? rc : urc;
}

int gt_calib_gather(const int32_t* indices, int64_t E, const void* K, const void* V, int64_t n_rows,
                    int32_t row_bytes, uint32_t* checksum, hipStream_t stream) {
    if (E < 0 || n_rows < 0) return fail(GT_EINVAL, "E and n_rows must be >= 0");
    if (row_bytes != 512 && row_bytes != 1024 && row_bytes != 2048)
        return fail(GT_EUNSUPPORTED, "row_bytes = %d: 512, 1024 or 2048 supported", row_bytes);
    if (E == 0) return GT_OK;
    if (!indices || !K || !V || !checksum) return fail(GT_EINVAL, "NULL array with E > 0");
    if (!aligned16(K) || !aligned16(V)) return fail(GT_EUNSUPPORTED, "K and V must be 16-byte aligned");
    hipError_t e = launch_calib_gather(indices, E, K, V, n_rows, row_bytes, checksum, stream);
    return e == hipSuccess ? GT_OK : hip_fail(e, "calibration gather launch");
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
