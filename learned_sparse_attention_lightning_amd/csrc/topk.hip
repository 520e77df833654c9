// topk.hip -- exact per-row top-k selection on gfx950.
//
// S_t = the k candidates s in 0..t with the highest score ("DeepSeek Sparse
// Attention: Learned Token Selection from Scratch", section 3.1), ties broken
// by the lower position; rows with t+1 <= k keep every candidate (section
// 7.2).  Output: the selected positions in ascending order, -1 padded.
//
// All comparisons are on an order-preserving 32-bit key of the fp32 score
// (-0 folded onto +0), so every decision below is exact integer work.
//
// Two paths:
//  * many rows (prefill): one 1024-thread workgroup per row.  The row is
//    cached in LDS when it fits (<= 32768 scores), a threshold search narrows
//    the key range [lo, hi] with <= 2048-bin LDS histograms until it is the
//    single key value tau of the k-th largest score, then one ordered sweep
//    takes every key > tau plus the first `need` keys == tau in position order.
//  * few wide rows (decode): the row is split over many workgroups.
//      hist     per slice, an LDS histogram of the top 12 key bits, merged into
//               a per-row histogram in global memory;
//      scan     every slice finds the digit d1 holding the k-th largest key,
//               writes a bitmap word of "digit > d1" per 32 positions and
//               appends the positions with digit == d1 to a candidate list;
//      resolve  one workgroup per row selects the remaining `need` candidates
//               exactly (ties by lower position), ORs them into the bitmap and
//               compacts the bitmap in position order.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkBins = 2048;
constexpr int kRowCache = 32768;  // scores cached in LDS by the per-row kernel

// wide-row path
constexpr int kWideThreads = 256;
constexpr int kWidePer = 8;                         // consecutive positions per thread
constexpr int kWideSlice = kWideThreads * kWidePer;  // positions per slice workgroup
constexpr int kCandCache = 8192;                     // candidates the resolve keeps in LDS
constexpr int kDigitBits = 12;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kWideMinS = 16384;
constexpr int kWideMaxS = 262144;      // bitmap of one row fits 32 KB of LDS
constexpr int kWideMaxRows = 512;
constexpr int kMetaWords = 16;         // per row: [1] count of keys above digit d1
constexpr int kMaxSlices = kWideMaxS / kWideSlice;  // candidate counts per row (one per slice)
constexpr int kHist2Direct = 256;      // candidates a slice adds to hist2 without LDS staging

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    const uint32_t lo = __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u);
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), lo);
}

// Exclusive prefix sum of v over the workgroup in thread order, and the
// total.  `scratch` holds one word per wave; two barriers.
template <int Waves>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *scratch,
                                                    uint32_t &total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < Waves; ++w) {
        const uint32_t c = scratch[w];
        before += w < wave ? c : 0u;
        sum += c;
    }
    __syncthreads();
    total = sum;
    return before + incl - v;
}

// Exclusive prefix count of a flag (ballot based), same contract.
template <int Waves>
__device__ __forceinline__ uint32_t block_flag_scan(bool flag, uint32_t *scratch,
                                                    uint32_t &total) {
    const int wave = threadIdx.x >> 6;
    const uint64_t m = __ballot(flag);
    if ((threadIdx.x & 63) == 0) scratch[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < Waves; ++w) {
        const uint32_t c = scratch[w];
        before += w < wave ? c : 0u;
        sum += c;
    }
    __syncthreads();
    total = sum;
    return before + lanes_below(m);
}

struct SelectSmem {
    uint32_t hist[kTkBins];
    uint32_t red_lo[kTkWaves], red_hi[kTkWaves];
    uint32_t scan[kTkWaves];
    uint32_t found_bin, found_above;
};

// Smallest and largest of the keys this thread visits, reduced over the
// workgroup (uniform result).  `each(f)` calls f(key) for every key the
// calling thread owns.
template <typename Each>
__device__ void block_key_range(Each each, SelectSmem &sm, uint32_t &lo_out, uint32_t &hi_out) {
    const int tid = threadIdx.x;
    uint32_t lo = 0xffffffffu, hi = 0u;
    each([&](uint32_t u) {
        lo = min(lo, u);
        hi = max(hi, u);
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
    }
    if ((tid & 63) == 0) {
        sm.red_lo[tid >> 6] = lo;
        sm.red_hi[tid >> 6] = hi;
    }
    __syncthreads();
    lo = sm.red_lo[0];
    hi = sm.red_hi[0];
#pragma unroll
    for (int v = 1; v < kTkWaves; ++v) {
        lo = min(lo, sm.red_lo[v]);
        hi = max(hi, sm.red_hi[v]);
    }
    __syncthreads();
    lo_out = lo;
    hi_out = hi;
}

// Key value tau of the need-th largest of the keys visited by `each` (every
// key of the set, over the workgroup), all of which lie in [lo, hi], and how
// many keys equal to tau belong to the top `need` (need_out).  1 <= need <=
// number of keys.  Called by all kTkThreads threads; the result is uniform.
template <typename Each>
__device__ void block_select_in(Each each, uint32_t lo, uint32_t hi, uint32_t need,
                                SelectSmem &sm, uint32_t &tau_out, uint32_t &need_out) {
    const int tid = threadIdx.x;
    while (lo != hi) {  // invariant: keys > hi are taken; need more lie in [lo, hi]
        const uint32_t range = hi - lo;
        int shift = 0;
        while ((range >> shift) >= (uint32_t)kTkBins) ++shift;
        const int nb = (int)(range >> shift) + 1;
        for (int j = tid; j < nb; j += kTkThreads) sm.hist[j] = 0u;
        __syncthreads();
        each([&](uint32_t u) {
            if (u >= lo && u <= hi) atomicAdd(&sm.hist[(u - lo) >> shift], 1u);
        });
        __syncthreads();
        {  // bin holding the need-th largest: suffix counts over thread-owned bin pairs
            constexpr int kPer = kTkBins / kTkThreads;  // 2 bins per thread
            uint32_t hb[kPer], c = 0u;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int bj = tid * kPer + j;
                hb[j] = bj < nb ? sm.hist[bj] : 0u;
                c += hb[j];
            }
            uint32_t tot;
            const uint32_t pre = block_excl_scan<kTkWaves>(c, sm.scan, tot);
            uint32_t run = tot - pre - c;  // keys in bins above this thread's pair
#pragma unroll
            for (int j = kPer - 1; j >= 0; --j) {
                const uint32_t before = run;
                run += hb[j];
                if (before < need && run >= need) {
                    sm.found_bin = (uint32_t)(tid * kPer + j);
                    sm.found_above = before;
                }
            }
        }
        __syncthreads();
        const uint32_t bin = sm.found_bin;
        need -= sm.found_above;
        const uint32_t new_lo = lo + (bin << shift);
        const uint32_t width_m1 = (1u << shift) - 1u;
        hi = (hi - new_lo > width_m1) ? new_lo + width_m1 : hi;
        lo = new_lo;
        __syncthreads();
    }
    tau_out = lo;
    need_out = need;
}

// block_select_in over keys key_at(0..n-1), range found first.
template <typename KeyAt>
__device__ void block_select(KeyAt key_at, int n, uint32_t need, SelectSmem &sm,
                             uint32_t &tau_out, uint32_t &need_out) {
    auto each = [&](auto f) {
        for (int p = threadIdx.x; p < n; p += kTkThreads) f(key_at(p));
    };
    uint32_t lo, hi;
    block_key_range(each, sm, lo, hi);
    block_select_in(each, lo, hi, need, sm, tau_out, need_out);
}

// ------------------------------------------------------- per-row kernel ----
struct RowSmem {
    SelectSmem sel;
    uint32_t cnt_gt[kTkWaves], cnt_eq[kTkWaves];
    __align__(16) uint32_t keys[kRowCache];
};

// One workgroup per row.  A cached row is read with 16-byte loads, four in
// flight per thread, converted to keys on the way into LDS; the threshold
// search and the selection then read LDS only.  The selection gives each
// wave one contiguous segment of positions: a first sweep counts the keys
// above tau and equal to tau per wave, and after one barrier a second sweep
// writes the wave's selected positions in order (ballot prefix counts).
__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int T, int S, int row0, int k, int cur, int ostride, int32_t *__restrict__ idx) {
    __shared__ RowSmem sm;
    const int r = blockIdx.x;
    const int b = blockIdx.y;
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S) - cur;  // last candidate position
    const float *row = scores + (size_t)b * batch_stride + (size_t)r * S;
    int32_t *out = idx + ((size_t)b * T + i) * ostride;
    const int n = t < 0 ? 0 : t + 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    if (n <= k) {  // every candidate is selected
        for (int p = tid; p < k; p += kTkThreads) out[p] = p < n ? p : -1;
        return;
    }
    const bool cached = n <= kRowCache;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    uint32_t lo, hi;
    if (cached) {
        // 16-byte pieces j = tid + kTkThreads * (4 * it + u), four loads in flight
        const int n16 = aligned ? n / 4 : 0;  // whole pieces read as vectors
        uint32_t vlo = 0xffffffffu, vhi = 0u;
        for (int j0 = tid; j0 < n16; j0 += 4 * kTkThreads) {
            f32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kTkThreads;
                if (j < n16) v[u] = reinterpret_cast<const f32x4 *>(row)[j];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kTkThreads;
                if (j < n16) {
                    uint32_t kk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kk[e] = ordered_key(v[u][e]);
                        vlo = min(vlo, kk[e]);
                        vhi = max(vhi, kk[e]);
                    }
                    reinterpret_cast<u32x4 *>(sm.keys)[j] = u32x4{kk[0], kk[1], kk[2], kk[3]};
                }
            }
        }
        for (int p = 4 * n16 + tid; p < n; p += kTkThreads) {
            const uint32_t u = ordered_key(row[p]);
            sm.keys[p] = u;
            vlo = min(vlo, u);
            vhi = max(vhi, u);
        }
        // the range reduction's barriers also publish the keys
        block_key_range([&](auto f) { f(vlo); f(vhi); }, sm.sel, lo, hi);
    }
    auto each = [&](auto f) {
        if (cached) {
            const int n16 = (n + 3) / 4;
            for (int j = tid; j < n16; j += kTkThreads) {
                const u32x4 v = reinterpret_cast<const u32x4 *>(sm.keys)[j];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * j + e < n) f(v[e]);
            }
        } else {
            // a row longer than the cache is re-read on every pass: 16-byte
            // loads, eight in flight per thread, so a pass costs a few memory
            // latencies rather than one per key a thread reads
            constexpr int U = 8;
            const int n16 = aligned ? n / 4 : 0;
            for (int j0 = tid; j0 < n16; j0 += U * kTkThreads) {
                f32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int j = j0 + u * kTkThreads;
                    if (j < n16) v[u] = reinterpret_cast<const f32x4 *>(row)[j];
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (j0 + u * kTkThreads < n16) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) f(ordered_key(v[u][e]));
                    }
            }
            for (int p = 4 * n16 + tid; p < n; p += kTkThreads) f(ordered_key(row[p]));
        }
    };
    if (!cached) block_key_range(each, sm.sel, lo, hi);

    uint32_t tau, need;
    block_select_in(each, lo, hi, (uint32_t)k, sm.sel, tau, need);

    // ordered selection: all keys > tau, plus the first `need` keys == tau
    const int seg = ceil_div(ceil_div(n, kTkWaves), 64) * 64;  // positions per wave
    const int w0 = wave * seg, w1 = min(n, w0 + seg);
    // sweep 1 counts the wave's keys above and at tau; after the barrier,
    // sweep 2 writes the wave's selected positions from the same keys (a
    // cached row's keys stay in registers between the sweeps)
    const int nit = w1 > w0 ? ceil_div(w1 - w0, 64) : 0;
    constexpr int kMaxIt = kRowCache / kTkThreads;  // seg <= 64 * kMaxIt when cached
    uint32_t kv[kMaxIt];
    if (cached) {
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
            const int p = w0 + 64 * it + lane;
            kv[it] = it < nit && p < w1 ? sm.keys[p] : 0u;
        }
    }
    auto sweep = [&](auto body) {
        if (cached) {
#pragma unroll
            for (int it = 0; it < kMaxIt; ++it)
                if (it < nit) body(kv[it], w0 + 64 * it + lane);
        } else {  // keys from memory, eight loads ahead of their use
            constexpr int U = 8;
            for (int it0 = 0; it0 < nit; it0 += U) {
                uint32_t kk[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int p = w0 + 64 * (it0 + u) + lane;
                    kk[u] = it0 + u < nit && p < w1 ? ordered_key(row[p]) : 0u;
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (it0 + u < nit) body(kk[u], w0 + 64 * (it0 + u) + lane);
            }
        }
    };
    uint32_t c_gt = 0u, c_eq = 0u;
    sweep([&](uint32_t u, int p) {
        c_gt += (uint32_t)__popcll(__ballot(p < w1 && u > tau));
        c_eq += (uint32_t)__popcll(__ballot(p < w1 && u == tau));
    });
    if (lane == 0) {
        sm.cnt_gt[wave] = c_gt;
        sm.cnt_eq[wave] = c_eq;
    }
    __syncthreads();
    uint32_t gt_before = 0u, eq_before = 0u;
    for (int v = 0; v < wave; ++v) {
        gt_before += sm.cnt_gt[v];
        eq_before += sm.cnt_eq[v];
    }
    uint32_t written = gt_before + min(eq_before, need), ties = eq_before;
    sweep([&](uint32_t u, int p) {
        const bool gt = p < w1 && u > tau;
        const bool eq = p < w1 && u == tau;
        const uint64_t eqm = __ballot(eq);
        const bool take = gt || (eq && ties + lanes_below(eqm) < need);
        const uint64_t tm = __ballot(take);
        if (take) out[written + lanes_below(tm)] = p;
        written += (uint32_t)__popcll(tm);
        ties += (uint32_t)__popcll(eqm);
    });
}

// ------------------------------------------------------- wide-row path -----
struct WideLayout {
    uint32_t *hist;     // [rows][kDigits]   top 12 key bits, every key
    uint32_t *hist2;    // [rows][kDigits]   key bits 19..8 of the keys whose top 12 bits are d1
    uint32_t *meta;     // [rows][kMetaWords]
    uint32_t *counts;   // [rows][kMaxSlices] candidates found by each slice
    uint32_t *bitmap;   // [rows][words]
    uint2 *cand;        // [rows][S] (key, position); slice i owns [i*slice, (i+1)*slice)
    int words;
};

__host__ __device__ inline size_t wide_row_bytes(int S) {
    const size_t words = (size_t)(S + 31) / 32;
    return (size_t)2 * kDigits * 4 + kMetaWords * 4 + kMaxSlices * 4 + words * 4 +
           (size_t)S * 8 + 16;
}

__host__ __device__ inline WideLayout wide_layout(void *ws, int nrows, int S) {
    WideLayout L;
    char *p = static_cast<char *>(ws);
    L.words = (S + 31) / 32;
    L.hist = reinterpret_cast<uint32_t *>(p);
    p += (size_t)nrows * kDigits * 4;
    L.hist2 = reinterpret_cast<uint32_t *>(p);
    p += (size_t)nrows * kDigits * 4;
    L.meta = reinterpret_cast<uint32_t *>(p);
    p += (size_t)nrows * kMetaWords * 4;
    L.counts = reinterpret_cast<uint32_t *>(p);
    p += (size_t)nrows * kMaxSlices * 4;
    L.bitmap = reinterpret_cast<uint32_t *>(p);
    p += (size_t)nrows * L.words * 4;
    p = reinterpret_cast<char *>(((uintptr_t)p + 15) & ~(uintptr_t)15);
    L.cand = reinterpret_cast<uint2 *>(p);
    return L;
}

// hist, hist2 and meta are contiguous: one sweep clears them
__global__ __launch_bounds__(256) void topk_wide_clear_kernel(uint32_t *hist, uint32_t *meta,
                                                              int nrows) {
    const size_t n1 = (size_t)nrows * kDigits * 2;
    const size_t n2 = (size_t)nrows * kMetaWords;
    for (size_t j = blockIdx.x * 256ull + threadIdx.x; j < n1 + n2; j += (size_t)gridDim.x * 256)
        if (j < n1) hist[j] = 0u;
        else meta[j - n1] = 0u;
}

// Scores of 8 consecutive positions p0..p0+7 of a row as order-preserving
// keys (positions >= n read as 0 and are ignored by the callers).
__device__ __forceinline__ void load8_keys(const float *row, int p0, int n, uint32_t (&u)[8]) {
    if (p0 + 8 <= n && ((uintptr_t)(row + p0) & 15) == 0) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(row + p0);
        const f32x4 c = *reinterpret_cast<const f32x4 *>(row + p0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] = ordered_key(a[e]);
            u[4 + e] = ordered_key(c[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = p0 + e < n ? ordered_key(row[p0 + e]) : 0u;
    }
}

// grid: x = slice, y = row in chunk, z = batch
__global__ __launch_bounds__(kWideThreads) void topk_wide_hist_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int T, int S, int row0, int rows, int k, int cur, WideLayout L) {
    __shared__ uint32_t hist[kDigits];
    const int r = blockIdx.y, b = blockIdx.z;
    const int t = query_pos(q_pos, b, row0 + r, T, S) - cur;
    const int n = t < 0 ? 0 : t + 1;
    const int base = blockIdx.x * kWideSlice;
    if (n <= k || base >= n) return;
    const float *row = scores + (size_t)b * batch_stride + (size_t)r * S;
    for (int j = threadIdx.x; j < kDigits; j += kWideThreads) hist[j] = 0u;
    __syncthreads();
    const int p0 = base + threadIdx.x * kWidePer;
    uint32_t u[8];
    load8_keys(row, p0, n, u);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (p0 + e < n) atomicAdd(&hist[u[e] >> (32 - kDigitBits)], 1u);
    __syncthreads();
    uint32_t *gh = L.hist + ((size_t)b * rows + r) * kDigits;
    for (int j = threadIdx.x; j < kDigits; j += kWideThreads)
        if (hist[j]) atomicAdd(&gh[j], hist[j]);
}

// grid: x = slice, y = row in chunk, z = batch
__global__ __launch_bounds__(kWideThreads) void topk_wide_scan_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int T, int S, int row0, int rows, int k, int cur, WideLayout L) {
    __shared__ uint32_t scratch[kWideThreads / 64];
    __shared__ uint32_t d1_s, above_s;
    __shared__ uint32_t h2[kDigits];  // second-digit counts when a slice has many candidates
    const int r = blockIdx.y, b = blockIdx.z;
    const int t = query_pos(q_pos, b, row0 + r, T, S) - cur;
    const int n = t < 0 ? 0 : t + 1;
    const int base = blockIdx.x * kWideSlice;
    if (n <= k || base >= n) return;
    const size_t rr = (size_t)b * rows + r;
    const uint32_t *gh = L.hist + rr * kDigits;
    const int tid = threadIdx.x;
    const float *row = scores + (size_t)b * batch_stride + (size_t)r * S;
    const int p0 = base + tid * kWidePer;
    uint32_t u[8];
    load8_keys(row, p0, n, u);  // issued early; used after the digit search

    // digit d1 holding the k-th largest key: walk the histogram from the top
    constexpr int per = kDigits / kWideThreads;  // 16 bins per thread
    uint32_t h[per], csum = 0u;
#pragma unroll
    for (int j = 0; j < per; ++j) {
        h[j] = gh[tid * per + j];
        csum += h[j];
    }
    uint32_t total;
    const uint32_t prefix = block_excl_scan<kWideThreads / 64>(csum, scratch, total);
    uint32_t running = total - prefix - csum;  // keys in bins of higher threads
#pragma unroll
    for (int j = per - 1; j >= 0; --j) {
        const uint32_t before = running;
        running += h[j];
        if (before < (uint32_t)k && running >= (uint32_t)k) {
            d1_s = (uint32_t)(tid * per + j);
            above_s = before;
        }
    }
    __syncthreads();
    const uint32_t d1 = d1_s;
    if (blockIdx.x == 0 && tid == 0) L.meta[rr * kMetaWords + 1] = above_s;

    // 8 bits of "digit > d1" per thread; 4 neighbouring lanes form one word.
    // Candidates (digit == d1) go to this slice's own region in position order.
    const int lane = tid & 63;
    uint32_t byte = 0u, cmask = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool valid = p0 + e < n;
        const uint32_t d = u[e] >> (32 - kDigitBits);
        if (valid && d > d1) byte |= 1u << e;
        if (valid && d == d1) cmask |= 1u << e;
    }
    uint32_t ncand;
    uint32_t slot = block_excl_scan<kWideThreads / 64>((uint32_t)__popc(cmask), scratch, ncand);
    uint2 *cand = L.cand + rr * (size_t)S + base;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (cmask & (1u << e)) cand[slot++] = make_uint2(u[e], (uint32_t)(p0 + e));
    if (tid == 0) L.counts[rr * kMaxSlices + blockIdx.x] = ncand;
    // second digit (key bits 19..8) of the candidates; a slice with many of
    // them (ties) aggregates in LDS first so no global counter gets hammered
    uint32_t *gh2 = L.hist2 + rr * kDigits;
    if (ncand <= kHist2Direct) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (cmask & (1u << e)) atomicAdd(&gh2[(u[e] >> 8) & (kDigits - 1)], 1u);
    } else {
        for (int j = tid; j < kDigits; j += kWideThreads) h2[j] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (cmask & (1u << e)) atomicAdd(&h2[(u[e] >> 8) & (kDigits - 1)], 1u);
        __syncthreads();
        for (int j = tid; j < kDigits; j += kWideThreads)
            if (h2[j]) atomicAdd(&gh2[j], h2[j]);
    }
    uint32_t word = byte << (8 * (lane & 3));
    word |= (uint32_t)__shfl_xor((int)word, 1, 64);
    word |= (uint32_t)__shfl_xor((int)word, 2, 64);
    if ((lane & 3) == 0 && p0 < n) L.bitmap[rr * L.words + (p0 >> 5)] = word;
}

constexpr int kMaxTies = 2048;  // members of the final group resolved by rank counting

struct ResolveSmem {
    SelectSmem sel;
    uint32_t scan[kTkWaves];
    uint32_t offs[kMaxSlices + 1];
    uint32_t d2, above2, gsize, gcount;
    uint2 group[kMaxTies];          // (key, position) of the candidates in bin d2
    uint32_t bits[kWideMaxS / 32];
    uint2 cand[kCandCache];
};

// Candidates a thread fetches before the second digit is known: kResolveSub
// threads per slice, kResolveFetch each, so runs of up to 64 candidates a
// slice arrive in a single round of loads.
constexpr int kResolveSub = 16;
constexpr int kResolveFetch = 4;
constexpr int kResolvePairs = kMaxSlices * kResolveSub / kTkThreads;  // (slice, sub) pairs a thread

// grid: x = row in chunk, y = batch
//
// The candidates (keys whose top 12 bits are d1) are split once more by key
// bits 19..8 with the histogram the scan built: d2 is the bin holding the
// need1-th largest candidate, so every candidate above d2 is taken and only
// the few in bin d2 need ordering -- each of them counts the group members
// ahead of it (larger key, or equal key at a lower position).  A group too
// large for that (massive ties) goes through the general threshold search.
__global__ __launch_bounds__(kTkThreads) void topk_wide_resolve_kernel(
    const int32_t *__restrict__ q_pos, int T, int S, int row0, int rows, int k, int cur,
    int ostride, int32_t *__restrict__ idx, WideLayout L) {
    __shared__ ResolveSmem sm;
    const int r = blockIdx.x, b = blockIdx.y;
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S) - cur;
    const int n = t < 0 ? 0 : t + 1;
    int32_t *out = idx + ((size_t)b * T + i) * ostride;
    const int tid = threadIdx.x;
    if (n <= k) {
        for (int p = tid; p < k; p += kTkThreads) out[p] = p < n ? p : -1;
        return;
    }
    const size_t rr = (size_t)b * rows + r;
    const int nw = (n + 31) / 32;
    const int nslices = (n + kWideSlice - 1) / kWideSlice;
    const uint2 *gcand = L.cand + rr * (size_t)S;

    // ---- everything this thread needs from memory, issued up front
    uint32_t bitmap_pre[kWideMaxS / 32 / kTkThreads];
#pragma unroll
    for (int u = 0; u < kWideMaxS / 32 / kTkThreads; ++u) {
        const int w = tid + u * kTkThreads;
        bitmap_pre[u] = w < nw ? L.bitmap[rr * L.words + w] : 0u;
    }
    constexpr int kPer2 = kDigits / kTkThreads;  // 4 second-digit bins per thread
    uint32_t h2[kPer2], c2 = 0u;
#pragma unroll
    for (int j = 0; j < kPer2; ++j) {
        h2[j] = L.hist2[rr * kDigits + tid * kPer2 + j];
        c2 += h2[j];
    }
    const uint32_t need1 = (uint32_t)k - L.meta[rr * kMetaWords + 1];
    uint32_t cnt[kResolvePairs];
    uint2 pre[kResolvePairs][kResolveFetch];
#pragma unroll
    for (int v = 0; v < kResolvePairs; ++v) {
        const int u = tid + v * kTkThreads;
        const int sl = u / kResolveSub, sub = u % kResolveSub;
        cnt[v] = sl < nslices ? L.counts[rr * kMaxSlices + sl] : 0u;
#pragma unroll
        for (int f = 0; f < kResolveFetch; ++f) {
            const uint32_t j = (uint32_t)(sub + kResolveSub * f);
            pre[v][f] = j < cnt[v] ? gcand[(size_t)sl * kWideSlice + j] : make_uint2(0u, 0u);
        }
    }

    // ---- bin d2 of the need1-th largest candidate (histogram walked from the top)
    if (tid == 0) sm.gcount = 0u;
    {
        uint32_t tot;
        const uint32_t before_me = block_excl_scan<kTkWaves>(c2, sm.scan, tot);
        uint32_t running = tot - before_me - c2;
#pragma unroll
        for (int j = kPer2 - 1; j >= 0; --j) {
            const uint32_t before = running;
            running += h2[j];
            if (before < need1 && running >= need1) {
                sm.d2 = (uint32_t)(tid * kPer2 + j);
                sm.above2 = before;
                sm.gsize = h2[j];
            }
        }
    }
    for (int w = tid; w < nw; w += kTkThreads) sm.bits[w] = bitmap_pre[w / kTkThreads];
    __syncthreads();
    const uint32_t d2 = sm.d2;
    const uint32_t need2 = need1 - sm.above2;  // to take from bin d2
    const uint32_t gsize = sm.gsize;

    if (gsize <= (uint32_t)kMaxTies) {
        auto visit = [&](const uint2 c) {
            const uint32_t dg = (c.x >> 8) & (kDigits - 1);
            if (dg > d2) atomicOr(&sm.bits[c.y >> 5], 1u << (c.y & 31));
            else if (dg == d2) {
                const uint32_t slot = atomicAdd(&sm.gcount, 1u);
                if (slot < (uint32_t)kMaxTies) sm.group[slot] = c;
            }
        };
#pragma unroll
        for (int v = 0; v < kResolvePairs; ++v) {
            const int u = tid + v * kTkThreads;
            const int sl = u / kResolveSub, sub = u % kResolveSub;
#pragma unroll
            for (int f = 0; f < kResolveFetch; ++f)
                if ((uint32_t)(sub + kResolveSub * f) < cnt[v]) visit(pre[v][f]);
            // long runs (many candidates in one slice): the rest, one by one
            for (uint32_t j = (uint32_t)(sub + kResolveSub * kResolveFetch); j < cnt[v];
                 j += kResolveSub)
                visit(gcand[(size_t)sl * kWideSlice + j]);
        }
        __syncthreads();
        // rank inside the group: larger key first, then lower position
        for (uint32_t a = tid; a < gsize; a += kTkThreads) {
            const uint2 ca = sm.group[a];
            uint32_t ahead = 0u;
            for (uint32_t g = 0; g < gsize; ++g) {
                const uint2 cg = sm.group[g];
                ahead += (cg.x > ca.x || (cg.x == ca.x && cg.y < ca.y)) ? 1u : 0u;
            }
            if (ahead < need2) atomicOr(&sm.bits[ca.y >> 5], 1u << (ca.y & 31));
        }
    } else {
        // general path: exact threshold among all candidates, ties by position
        if (tid < 64) {  // offsets of the slices' candidate runs
            uint32_t run = 0u;
            for (int s0 = 0; s0 < nslices; s0 += 64) {
                const int sl = s0 + tid;
                uint32_t c = sl < nslices ? L.counts[rr * kMaxSlices + sl] : 0u;
                uint32_t incl = c;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
                    if (tid >= off) incl += o;
                }
                if (sl < nslices) sm.offs[sl] = run + incl - c;
                run += (uint32_t)__shfl((int)incl, 63, 64);
            }
            if (tid == 0) sm.offs[nslices] = run;
        }
        __syncthreads();
        const int m = (int)sm.offs[nslices];
        const bool cached = m <= kCandCache;
        auto cand_global = [&](int j) -> uint2 {  // slice by binary search over the runs
            int lo = 0, hi = nslices - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sm.offs[mid] <= (uint32_t)j) lo = mid;
                else hi = mid - 1;
            }
            return gcand[lo * kWideSlice + (j - (int)sm.offs[lo])];
        };
        if (cached) {
            for (int j = tid; j < m; j += kTkThreads) sm.cand[j] = cand_global(j);
            __syncthreads();
        }
        auto cand_at = [&](int j) -> uint2 { return cached ? sm.cand[j] : cand_global(j); };
        uint32_t tau, need_tau;
        block_select([&](int j) -> uint32_t { return cand_at(j).x; }, m, need1, sm.sel, tau,
                     need_tau);
        uint32_t tie_count;
        {
            uint32_t mine = 0u;
            for (int j = tid; j < m; j += kTkThreads) mine += cand_at(j).x == tau ? 1u : 0u;
            block_excl_scan<kTkWaves>(mine, sm.scan, tie_count);
        }
        uint32_t pos_cut = 0xffffffffu;  // ties at positions <= pos_cut are taken
        if (need_tau < tie_count) {
            uint32_t tau2, need2b;
            block_select(
                [&](int j) -> uint32_t {
                    const uint2 c = cand_at(j);
                    return c.x == tau ? ~c.y : 0u;
                },
                m, need_tau, sm.sel, tau2, need2b);
            pos_cut = ~tau2;
        }
        for (int j = tid; j < m; j += kTkThreads) {
            const uint2 c = cand_at(j);
            if (c.x > tau || (c.x == tau && c.y <= pos_cut))
                atomicOr(&sm.bits[c.y >> 5], 1u << (c.y & 31));
        }
    }
    __syncthreads();

    // ordered compaction: contiguous words per thread, prefix of popcounts
    const int per = (nw + kTkThreads - 1) / kTkThreads;
    const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
    uint32_t cntw = 0u;
    for (int w = w0; w < w1; ++w) cntw += (uint32_t)__popc(sm.bits[w]);
    uint32_t total;
    uint32_t slot = block_excl_scan<kTkWaves>(cntw, sm.scan, total);
    for (int w = w0; w < w1; ++w) {
        uint32_t x = sm.bits[w];
        while (x) {
            const int bit = __builtin_ctz(x);
            x &= x - 1u;
            out[slot++] = w * 32 + bit;
        }
    }
}

// The current-token variant: the selection kernels ran with budget k-1 over
// the positions before t, writing slots 0..k-2 of each k-wide row (ascending,
// -1 after the n_sel = min(k-1, t) selected).  Position t is the largest of
// the set, so it goes right after them; slot k-1 gets -1 when unused.
__global__ __launch_bounds__(256) void topk_current_fix_kernel(
    const int32_t *__restrict__ q_pos, int B, int T, int S, int row0, int rows, int k,
    int32_t *__restrict__ idx) {
    const int g = blockIdx.x * 256 + threadIdx.x;
    if (g >= B * rows) return;
    const int b = g / rows, i = row0 + g % rows;
    const int t = query_pos(q_pos, b, i, T, S);
    int32_t *out = idx + ((size_t)b * T + i) * k;
    if (t < 0) {
        out[k - 1] = -1;
        return;
    }
    const int n_sel = t < k - 1 ? t : k - 1;
    out[n_sel] = t;
    if (n_sel < k - 1) out[k - 1] = -1;
}

// Every candidate selected (at most k of them in every row): positions
// 0..t ascending, then -1.  grid: x = slot block, y = row in chunk, z = batch.
__global__ __launch_bounds__(256) void topk_select_all_kernel(
    const int32_t *__restrict__ q_pos, int T, int S, int row0, int k,
    int32_t *__restrict__ idx) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= k) return;
    const int b = blockIdx.z, i = row0 + blockIdx.y;
    const int t = query_pos(q_pos, b, i, T, S);
    idx[((size_t)b * T + i) * k + p] = p <= t ? p : -1;
}

bool use_wide(int B, int rows, int S) {
    return S >= kWideMinS && S <= kWideMaxS && (long long)B * rows <= kWideMaxRows;
}

}  // namespace

size_t topk_workspace_bytes(int B, int T, int S, int) {
    if (S < kWideMinS || S > kWideMaxS) return 0;
    const long long bt = (long long)B * T;
    const long long nrows = bt < kWideMaxRows ? bt : kWideMaxRows;
    return (size_t)nrows * wide_row_bytes(S) + 64;
}

// Counters of the wide path that must be zero when its first kernel starts
// (the histograms and per-row words at the head of the workspace).
size_t topk_clear_words(int B, int rows, int S) {
    if (!use_wide(B, rows, S)) return 0;
    return (size_t)B * rows * (2 * kDigits + kMetaWords);
}

hipError_t launch_topk(const float *scores, size_t batch_stride, const int32_t *q_pos, int B,
                       int T, int S, int row0, int rows, int k, int32_t *idx, void *workspace,
                       bool workspace_cleared, hipStream_t stream, bool include_current) {
    // the current-token variant selects k-1 among the positions before t
    const int cur = include_current ? 1 : 0;
    const int kk = k - cur;
    if (kk >= 1 && use_wide(B, rows, S) && workspace) {
        const WideLayout L = wide_layout(workspace, B * rows, S);
        const int nrows = B * rows;
        if (!workspace_cleared)
            hipLaunchKernelGGL(topk_wide_clear_kernel,
                               dim3(min(1024, ceil_div(nrows * (2 * kDigits + kMetaWords), 256))),
                               dim3(256), 0, stream, L.hist, L.meta, nrows);
        const dim3 g(ceil_div(S, kWideSlice), rows, B);
        hipLaunchKernelGGL(topk_wide_hist_kernel, g, dim3(kWideThreads), 0, stream, scores,
                           batch_stride, q_pos, T, S, row0, rows, kk, cur, L);
        hipLaunchKernelGGL(topk_wide_scan_kernel, g, dim3(kWideThreads), 0, stream, scores,
                           batch_stride, q_pos, T, S, row0, rows, kk, cur, L);
        hipLaunchKernelGGL(topk_wide_resolve_kernel, dim3(rows, B), dim3(kTkThreads), 0, stream,
                           q_pos, T, S, row0, rows, kk, cur, k, idx, L);
    } else if (kk >= 1) {
        hipLaunchKernelGGL(topk_row_kernel, dim3(rows, B), dim3(kTkThreads), 0, stream, scores,
                           batch_stride, q_pos, T, S, row0, kk, cur, k, idx);
    }
    if (include_current)
        hipLaunchKernelGGL(topk_current_fix_kernel, dim3(ceil_div(B * rows, 256)), dim3(256), 0,
                           stream, q_pos, B, T, S, row0, rows, k, idx);
    return hipGetLastError();
}

hipError_t launch_select_all(const int32_t *q_pos, int B, int T, int S, int row0, int rows,
                             int k, int32_t *idx, hipStream_t stream) {
    hipLaunchKernelGGL(topk_select_all_kernel, dim3(ceil_div(k, 256), rows, B), dim3(256), 0,
                       stream, q_pos, T, S, row0, k, idx);
    return hipGetLastError();
}

}  // namespace dsa
