// graph.hip -- graph construction on the device: a stable LSD radix sort of
// 32-bit keys carrying one or two arrays of 32-bit values, an exclusive scan,
// and the helpers that turn sorted keys into a CSR (row offsets by binary
// search, the row of each CSR position).
//
// "Graph Transformer in a Nutshell", section "Graph Transformer Model":
// GTModel.forward stacks the (src, dst) pairs of g.edges() into one sparse
// adjacency matrix used by all its layers.  Here that matrix is built once on
// the device, grouped by destination (the attention's CSR) and by source (the
// backward's transpose): a stable sort of the edges by destination id (or
// source id) keeps each row's edges in their input order, so the result is
// unique and bit-reproducible.
//
// Sort pass (8-bit digits, tiles of kSortTile keys per block of 4 waves; the
// values, and an optional second value array, travel with the keys):
//  1. radix_count_kernel: per-tile digit histogram -> hist[digit][tile];
//  2. exclusive scan of hist in that digit-major order -> the first output
//     slot of each (digit, tile);
//  3. radix_scatter_kernel: each wave ranks its keys in input order with a
//     ballot multisplit (lanes with equal digits find each other through one
//     ballot per key bit; the lowest such lane takes their slots with one LDS
//     atomic), then adds the counts of earlier waves of its tile; the tile is
//     rearranged in LDS into (digit, input) order, and consecutive threads
//     write consecutive keys, so each digit's run leaves as one contiguous
//     stretch instead of one scattered 4-byte store per key.
// Keys of equal digit keep their input order, so every pass is stable.  At
// most 16,384 keys are grouped in one launch instead (group_small_kernel).
#include "kernels.hpp"

namespace gt {

namespace {

constexpr int kSortWaves = 4;
constexpr int kSortItems = 16;                              // 64-key chunks per wave
constexpr int kWaveSpan = kWave * kSortItems;               // keys per wave
constexpr int64_t kSortTile = (int64_t)kSortWaves * kWaveSpan;  // keys per block
static_assert(kSortWaves * kWave == 256, "one thread per 8-bit digit in the sort kernels");
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int64_t kScanTile = (int64_t)kScanThreads * kScanItems;

__device__ __forceinline__ uint64_t lanes_below(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

// Lanes of the wave whose key has the same digit (and are in range).
__device__ __forceinline__ uint64_t digit_peers(uint32_t digit, int bits, bool valid) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
        const bool bit = (digit >> b) & 1u;
        const uint64_t ones = __ballot(bit);
        peers &= bit ? ones : ~ones;
    }
    return valid ? peers : 0ull;
}

__global__ __launch_bounds__(kSortWaves * kWave) void radix_count_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                                          int shift, int bits, uint32_t* hist,
                                                                          int64_t ntiles) {
    __shared__ uint32_t cnt[256];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
    cnt[t] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile + (int64_t)w * kWaveSpan;
    const uint32_t mask = (1u << bits) - 1u;
    for (int i = 0; i < kSortItems; ++i) {
        const int64_t e = base + (int64_t)i * kWave + lane;
        const bool valid = e < n;
        const uint32_t d = valid ? (keys[e] >> shift) & mask : 0u;
        const uint64_t peers = digit_peers(d, bits, valid);
        if (valid && (int)__builtin_ctzll(peers) == lane) atomicAdd(&cnt[d], (uint32_t)__builtin_popcountll(peers));
    }
    __syncthreads();
    if (t <= (int)mask) hist[(int64_t)t * ntiles + blockIdx.x] = cnt[t];
}

// IOTA: the values are the keys' input positions.  TWO: a second value array
// travels with the first.
template <bool IOTA, bool TWO>
__global__ __launch_bounds__(kSortWaves * kWave) void radix_scatter_kernel(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, const uint32_t* __restrict__ vals2_in,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint32_t* __restrict__ vals2_out, int64_t n,
    int shift, int bits, const uint32_t* __restrict__ first, int64_t ntiles) {
    __shared__ uint32_t cnt[kSortWaves][256];
    __shared__ uint32_t wsum[kSortWaves];
    __shared__ int64_t gbase[256];           // output slot of the tile's first key of each digit, minus its tile slot
    __shared__ uint32_t sk[kSortTile], sv[kSortTile], sv2[TWO ? kSortTile : 1];  // the tile in (digit, input) order
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
    for (int j = 0; j < kSortWaves; ++j) cnt[j][t] = 0;
    __syncthreads();
    const int64_t tile0 = (int64_t)blockIdx.x * kSortTile;
    const int64_t base = tile0 + (int64_t)w * kWaveSpan;
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t key[kSortItems], val[kSortItems], val2[TWO ? kSortItems : 1], rank[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int64_t e = base + (int64_t)i * kWave + lane;
        const bool valid = e < n;
        key[i] = valid ? keys_in[e] : 0u;
        val[i] = valid ? (IOTA ? (uint32_t)e : vals_in[e]) : 0u;
        if constexpr (TWO) val2[i] = valid ? vals2_in[e] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int64_t e = base + (int64_t)i * kWave + lane;
        const bool valid = e < n;
        const uint32_t d = (key[i] >> shift) & mask;
        const uint64_t peers = digit_peers(d, bits, valid);
        const int leader = valid ? (int)__builtin_ctzll(peers) : lane;
        uint32_t old = 0;
        if (valid && leader == lane) old = atomicAdd(&cnt[w][d], (uint32_t)__builtin_popcountll(peers));
        old = __shfl(old, leader, kWave);
        rank[i] = old + (uint32_t)__builtin_popcountll(peers & lanes_below(lane));
    }
    __syncthreads();
    // thread t = digit t: counts of earlier waves, then the digit's first slot in
    // the tile (exclusive scan of the tile's digit totals over the 256 threads)
    uint32_t tot = 0;
    for (int j = 0; j < kSortWaves; ++j) {
        const uint32_t c = cnt[j][t];
        cnt[j][t] = tot;
        tot += c;
    }
    uint32_t inc = tot;
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    uint32_t start = inc - tot;
    for (int j = 0; j < w; ++j) start += wsum[j];
    for (int j = 0; j < kSortWaves; ++j) cnt[j][t] += start;
    gbase[t] = t <= (int)mask ? (int64_t)first[(int64_t)t * ntiles + blockIdx.x] - start : 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int64_t e = base + (int64_t)i * kWave + lane;
        if (e >= n) continue;
        const uint32_t d = (key[i] >> shift) & mask;
        const uint32_t slot = cnt[w][d] + rank[i];
        sk[slot] = key[i];
        sv[slot] = val[i];
        if constexpr (TWO) sv2[slot] = val2[i];
    }
    __syncthreads();
    // consecutive threads take consecutive slots: each digit's run goes out as
    // one contiguous stretch
    const int count = (int)(n - tile0 < kSortTile ? n - tile0 : kSortTile);
    for (int j = t; j < count; j += kSortWaves * kWave) {
        const uint32_t k = sk[j];
        const int64_t pos = gbase[(k >> shift) & mask] + j;
        keys_out[pos] = k;
        vals_out[pos] = sv[j];
        if constexpr (TWO) vals2_out[pos] = sv2[j];
    }
}

constexpr int kSmallWaves = 16;
constexpr int64_t kSmallSortKeys = (int64_t)kSmallWaves * kWaveSpan;
constexpr int kGapList = 2048;  // long runs of rows without keys, filled by the whole block
constexpr int kLongGap = 64;

// ---------------------------------------------------------------- exclusive scan (uint32)

// Sum of each kScanTile-element tile.
__global__ __launch_bounds__(kScanThreads) void scan_sums_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                                  uint32_t* __restrict__ sums) {
    __shared__ uint32_t part[kScanThreads / kWave];
    const int t = threadIdx.x;
    const int64_t b = (int64_t)blockIdx.x * kScanTile;
    uint32_t s = 0;
    for (int i = 0; i < kScanItems; ++i) {
        const int64_t e = b + (int64_t)i * kScanThreads + t;
        if (e < n) s += in[e];
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    if ((t & (kWave - 1)) == 0) part[t >> 6] = s;
    __syncthreads();
    if (t == 0) {
        uint32_t tot = 0;
        for (int j = 0; j < kScanThreads / kWave; ++j) tot += part[j];
        sums[blockIdx.x] = tot;
    }
}

// out = exclusive scan of in (tile by tile), plus offsets[tile] when given.
// Thread t owns kScanItems consecutive elements; in and out may alias.
__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(const uint32_t* in, uint32_t* out, int64_t n,
                                                                   const uint32_t* __restrict__ offsets) {
    __shared__ uint32_t wsum[kScanThreads / kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
    const int64_t b = (int64_t)blockIdx.x * kScanTile + (int64_t)t * kScanItems;
    uint32_t x[kScanItems];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        x[i] = b + i < n ? in[b + i] : 0u;
        s += x[i];
    }
    uint32_t inc = s;  // inclusive scan of thread sums within the wave
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    uint32_t run = offsets ? offsets[blockIdx.x] : 0u;
    for (int j = 0; j < w; ++j) run += wsum[j];
    run += inc - s;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        if (b + i < n) out[b + i] = run;
        run += x[i];
    }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Scratch (in uint32 words) that scan_exclusive needs for n elements.
int64_t scan_words(int64_t n) {
    int64_t w = 0;
    for (int64_t m = cdiv(n, kScanTile); m > 1; m = cdiv(m, kScanTile)) w += m + 64;
    return w + 64;
}

// In-place exclusive scan of a[0..n) with tmp of scan_words(n) words.
hipError_t scan_exclusive(uint32_t* a, int64_t n, uint32_t* tmp, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t tiles = cdiv(n, kScanTile);
    if (tiles == 1) {
        scan_apply_kernel<<<1, kScanThreads, 0, s>>>(a, a, n, nullptr);
        return hipGetLastError();
    }
    uint32_t* sums = tmp;
    scan_sums_kernel<<<(unsigned)tiles, kScanThreads, 0, s>>>(a, n, sums);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = scan_exclusive(sums, tiles, tmp + tiles + 64, s);
    if (err != hipSuccess) return err;
    scan_apply_kernel<<<(unsigned)tiles, kScanThreads, 0, s>>>(a, a, n, sums);
    return hipGetLastError();
}

// ---------------------------------------------------------------- CSR helpers

// offsets[v] = number of sorted keys below v, for v in [0, nrows]: the row
// offsets of the rows the keys name.  One binary search per row.
__global__ __launch_bounds__(256) void lower_bounds_kernel(const uint32_t* __restrict__ keys, int64_t n, int64_t nrows,
                                                            int64_t* __restrict__ offsets) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v > nrows) return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if ((int64_t)keys[mid] < v)
            lo = mid + 1;
        else
            hi = mid;
    }
    offsets[v] = lo;
}

// rows[p] = the row holding CSR position p.  A wave takes kFillRows
// consecutive rows, lane j loading the offset of row r0 + j (kFillRows + 1
// offsets fit the wave), and its lanes write each row's positions in turn,
// 64 at a time.  Every position is written once, by coalesced stores.  A
// binary search per position, which cost each one a chain of dependent
// loads, took 34 us on a 4k-node molecule batch against 12 us here; on the
// power-law graph, where one wave fills a 50,000-edge row alone, 59 against
// 69 us.
constexpr int kFillRows = kWave - 1;

__global__ __launch_bounds__(256) void fill_rows_kernel(const int64_t* __restrict__ indptr, int64_t nrows,
                                                        uint32_t* __restrict__ rows) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t r0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave * kFillRows;
    if (r0 >= nrows) return;
    const int nr = (int)(nrows - r0 < kFillRows ? nrows - r0 : kFillRows);
    const int64_t off = lane <= nr ? indptr[r0 + lane] : 0;
    for (int j = 0; j < nr; ++j) {
        const int64_t b = __shfl(off, j, kWave), e = __shfl(off, j + 1, kWave);
        for (int64_t p = b + lane; p < e; p += kWave) rows[p] = (uint32_t)(r0 + j);
    }
}

// Grouping by key in one launch for at most kSmallSortKeys items (a batch of
// molecules: 8.5k edges), where the tiled sort takes a launch per pass and
// the row offsets one more, each a few memory round trips long.  One block
// of kSmallWaves waves keeps every item in registers, wave w holding items
// [w * kWaveSpan, (w + 1) * kWaveSpan), and runs the LSD passes one after
// another:
//  1. every wave ranks its keys within their digit (the tiled kernels' ballot
//     multisplit) and counts the digits into cnt[wave][digit];
//  2. thread t = digit t (the first four waves) turns the counts into first
//     slots: the counts of the waves before, plus the keys of lower digits;
//  3. each item goes to LDS at its digit's first slot for its wave plus its
//     rank, and every thread reloads the items of its positions for the next
//     pass.  Equal digits keep their order: slots grow with (wave, item, lane).
// The items carry their input position; after the last pass the block writes
// each item's value, its position (perm) and the row offsets, which it reads
// off the sorted keys (offsets[v] = first position whose key is >= v).
// ROWS: the value of item e is the row holding position e of the CSR
// row_indptr (row_n rows, fewer than 2^18), packed beside the position
// (e < 2^14) through the passes; the rows come from a fill of LDS from
// row_indptr, each thread writing whole rows (a wave per 63 rows, as in
// fill_rows_kernel, was a chain of shuffles per row: 55 us for 4k rows on one
// block's 16 waves).  Otherwise the value is vals[e], gathered at the end.
template <bool ROWS, bool PERM>
__global__ __launch_bounds__(kSmallWaves * kWave) void group_small_kernel(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, const int64_t* __restrict__ row_indptr,
    int64_t row_n, int n, int key_bits, int64_t nrows, int64_t* __restrict__ offsets, uint32_t* __restrict__ out,
    uint32_t* __restrict__ perm) {
    __shared__ uint32_t cnt[kSmallWaves][256];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t sk[kSmallSortKeys], sv[kSmallSortKeys];  // a pass's output, in slot order
    __shared__ uint32_t s_gap[kGapList], s_ngap;                   // positions before long runs of empty rows
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
    const int base = w * kWaveSpan;
    if constexpr (ROWS) {
        for (int64_t r = t; r < row_n; r += kSmallWaves * kWave) {
            const int64_t b = row_indptr[r], e = row_indptr[r + 1];
            for (int64_t q = b; q < e && q < n; ++q) sv[q] = (uint32_t)r;
        }
        __syncthreads();
    }
    uint32_t key[kSortItems], val[kSortItems], rank[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const int e = base + i * kWave + lane;
        const bool valid = e < n;
        key[i] = valid ? keys_in[e] : 0u;
        val[i] = valid ? (ROWS ? (uint32_t)e | (sv[e] << 14) : (uint32_t)e) : 0u;
    }
    const int passes = key_bits > 0 ? (key_bits + 7) / 8 : 1;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        const int bits = key_bits - shift < 8 ? (key_bits - shift > 0 ? key_bits - shift : 1) : 8;
        const uint32_t mask = (1u << bits) - 1u;
        __syncthreads();  // the last pass's reloads (or the row fill's reads) are done
        for (int k = t; k < kSmallWaves * 256; k += kSmallWaves * kWave) (&cnt[0][0])[k] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            const bool valid = base + i * kWave + lane < n;
            const uint32_t d = (key[i] >> shift) & mask;
            const uint64_t peers = digit_peers(d, bits, valid);
            const int leader = valid ? (int)__builtin_ctzll(peers) : lane;
            uint32_t old = 0;
            if (valid && leader == lane) old = atomicAdd(&cnt[w][d], (uint32_t)__builtin_popcountll(peers));
            old = __shfl(old, leader, kWave);
            rank[i] = old + (uint32_t)__builtin_popcountll(peers & lanes_below(lane));
        }
        __syncthreads();
        uint32_t tot = 0, inc = 0;
        if (t < 256) {
            for (int j = 0; j < kSmallWaves; ++j) {
                const uint32_t c = cnt[j][t];
                cnt[j][t] = tot;
                tot += c;
            }
            inc = tot;
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t y = __shfl_up(inc, off, kWave);
                if (lane >= off) inc += y;
            }
            if (lane == kWave - 1) wsum[w] = inc;
        }
        __syncthreads();
        if (t < 256) {
            uint32_t start = inc - tot;
            for (int j = 0; j < w; ++j) start += wsum[j];
            for (int j = 0; j < kSmallWaves; ++j) cnt[j][t] += start;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) {
            if (base + i * kWave + lane < n) {
                const uint32_t slot = cnt[w][(key[i] >> shift) & mask] + rank[i];
                sk[slot] = key[i];
                sv[slot] = val[i];
            }
        }
        __syncthreads();
        if (p + 1 < passes) {
#pragma unroll
            for (int i = 0; i < kSortItems; ++i) {
                const int e = base + i * kWave + lane;
                if (e < n) {
                    key[i] = sk[e];
                    val[i] = sv[e];
                }
            }
        }
    }
    for (int j = t; j < n; j += kSmallWaves * kWave) {
        const uint32_t v = sv[j];
        const uint32_t pos = ROWS ? v & ((1u << 14) - 1u) : v;
        out[j] = ROWS ? v >> 14 : vals_in[pos];
        if constexpr (PERM) perm[j] = pos;
    }
    // Position j writes the offsets of the rows after the previous key up to its
    // own; keys >= nrows (a malformed input) are clamped so that nothing lands
    // past offsets[nrows].  A long run of rows without keys (a shard whose
    // sources start far above row 0) is listed and then written by the whole
    // block, not by one thread; a full list falls back to the thread.
    if (t == 0) s_ngap = 0u;
    __syncthreads();
    for (int j = t; j <= n; j += kSmallWaves * kWave) {
        const int64_t prev = j > 0 ? min((int64_t)sk[j - 1], nrows) : -1;
        const int64_t cur = j < n ? min((int64_t)sk[j], nrows) : nrows;
        if (cur - prev > kLongGap) {
            const uint32_t k = atomicAdd(&s_ngap, 1u);
            if (k < kGapList) {
                s_gap[k] = (uint32_t)j;
                continue;
            }
        }
        for (int64_t v = prev + 1; v <= cur; ++v) offsets[v] = j;
    }
    __syncthreads();
    const uint32_t ng = min(s_ngap, (uint32_t)kGapList);
    for (uint32_t g = 0; g < ng; ++g) {
        const int j = (int)s_gap[g];
        const int64_t prev = j > 0 ? min((int64_t)sk[j - 1], nrows) : -1;
        const int64_t cur = j < n ? min((int64_t)sk[j], nrows) : nrows;
        for (int64_t v = prev + 1 + t; v <= cur; v += kSmallWaves * kWave) offsets[v] = j;
    }
}

unsigned grid256(int64_t n) { return (unsigned)cdiv(n, 256); }

}  // namespace

int key_bits_for(int64_t nkeys) {
    int b = 0;
    while (b < 32 && ((int64_t)1 << b) < nkeys) ++b;
    return b;
}

size_t sort_scratch_bytes(int64_t n, bool two_values) {
    const int64_t tiles = cdiv(n > 0 ? n : 1, kSortTile);
    return sizeof(uint32_t) * (size_t)((two_values ? 6 : 4) * n + 256 * tiles + scan_words(256 * tiles) + 1024);
}

hipError_t radix_sort(const uint32_t* keys_in, const uint32_t* vals_in, const uint32_t* vals2_in, int64_t n,
                      int key_bits, void* scratch, uint32_t* vals_final, uint32_t* vals2_final, hipStream_t s,
                      const uint32_t** keys_sorted, const uint32_t** vals_sorted, const uint32_t** vals2_sorted) {
    const bool two = vals2_in != nullptr;
    const int64_t tiles = cdiv(n > 0 ? n : 1, kSortTile);
    uint32_t* w = (uint32_t*)scratch;
    uint32_t* kb[2] = {w, w + n};
    uint32_t* vb[2] = {w + 2 * n, w + 3 * n};
    uint32_t* v2b[2] = {two ? w + 4 * n : nullptr, two ? w + 5 * n : nullptr};
    uint32_t* hist = w + (two ? 6 : 4) * n;
    uint32_t* tmp = hist + 256 * tiles;
    const int passes = key_bits > 0 ? (key_bits + 7) / 8 : 1;
    const uint32_t* kin = keys_in;
    const uint32_t* vin = vals_in;
    const uint32_t* v2in = vals2_in;
    const unsigned grid = (unsigned)tiles;
    const unsigned block = kSortWaves * kWave;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        const int bits = key_bits - shift < 8 ? (key_bits - shift > 0 ? key_bits - shift : 1) : 8;
        const bool last = p == passes - 1;
        uint32_t* kout = kb[p & 1];
        uint32_t* vout = (last && vals_final) ? vals_final : vb[p & 1];
        uint32_t* v2out = (last && vals2_final) ? vals2_final : v2b[p & 1];
        if (n > 0) {
            radix_count_kernel<<<grid, block, 0, s>>>(kin, n, shift, bits, hist, tiles);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            err = scan_exclusive(hist, ((int64_t)1 << bits) * tiles, tmp, s);
            if (err != hipSuccess) return err;
            if (!vin && two)
                radix_scatter_kernel<true, true><<<grid, block, 0, s>>>(kin, nullptr, v2in, kout, vout, v2out, n,
                                                                         shift, bits, hist, tiles);
            else if (!vin)
                radix_scatter_kernel<true, false><<<grid, block, 0, s>>>(kin, nullptr, nullptr, kout, vout, nullptr,
                                                                          n, shift, bits, hist, tiles);
            else if (two)
                radix_scatter_kernel<false, true><<<grid, block, 0, s>>>(kin, vin, v2in, kout, vout, v2out, n, shift,
                                                                          bits, hist, tiles);
            else
                radix_scatter_kernel<false, false><<<grid, block, 0, s>>>(kin, vin, nullptr, kout, vout, nullptr, n,
                                                                           shift, bits, hist, tiles);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        kin = kout;
        vin = vout;
        v2in = v2out;
    }
    *keys_sorted = kin;
    *vals_sorted = vin;
    if (vals2_sorted) *vals2_sorted = v2in;
    return hipSuccess;
}

hipError_t launch_lower_bounds(const uint32_t* keys, int64_t n, int64_t nrows, int64_t* offsets, hipStream_t s) {
    lower_bounds_kernel<<<grid256(nrows + 1), 256, 0, s>>>(keys, n, nrows, offsets);
    return hipGetLastError();
}

bool group_small_fits(int64_t n, int64_t row_n) { return n > 0 && n <= kSmallSortKeys && row_n < ((int64_t)1 << 18); }

hipError_t launch_group_small(const uint32_t* keys, const uint32_t* vals, const int64_t* row_indptr, int64_t row_n,
                              int64_t n, int64_t nrows, int64_t* offsets, uint32_t* out, uint32_t* perm,
                              hipStream_t s) {
    if (!group_small_fits(n, row_indptr ? row_n : 0)) return hipErrorInvalidValue;
    const int bits = key_bits_for(nrows);
    const dim3 grid(1), block(kSmallWaves * kWave);
    if (row_indptr)
        group_small_kernel<true, true><<<grid, block, 0, s>>>(keys, nullptr, row_indptr, row_n, (int)n, bits, nrows,
                                                              offsets, out, perm);
    else if (perm)
        group_small_kernel<false, true><<<grid, block, 0, s>>>(keys, vals, nullptr, 0, (int)n, bits, nrows, offsets,
                                                               out, perm);
    else
        group_small_kernel<false, false><<<grid, block, 0, s>>>(keys, vals, nullptr, 0, (int)n, bits, nrows, offsets,
                                                                out, nullptr);
    return hipGetLastError();
}

hipError_t launch_row_of_position(const int64_t* indptr, int64_t nrows, int64_t n, uint32_t* rows, hipStream_t s) {
    if (n == 0 || nrows == 0) return hipSuccess;
    const int64_t waves = cdiv(nrows, kFillRows);
    fill_rows_kernel<<<(unsigned)cdiv(waves * kWave, 256), 256, 0, s>>>(indptr, nrows, rows);
    return hipGetLastError();
}

}  // namespace gt
