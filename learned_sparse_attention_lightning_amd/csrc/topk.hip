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
#include <algorithm>
#include <cmath>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkBins = 2048;

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

template <int NT>  // threads of the workgroup
struct SelectSmemT {
    uint32_t hist[kTkBins];
    uint32_t red_lo[NT / 64], red_hi[NT / 64];
    uint32_t scan[NT / 64];
    uint32_t found_bin, found_above, gcount;
};
using SelectSmem = SelectSmemT<kTkThreads>;

// Smallest and largest of the keys this thread visits, reduced over the
// workgroup (uniform result).  `each(f)` calls f(key) for every key the
// calling thread owns.
template <typename Each, int NT>
__device__ void block_key_range(Each each, SelectSmemT<NT> &sm, uint32_t &lo_out,
                                uint32_t &hi_out) {
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
    for (int v = 1; v < NT / 64; ++v) {
        lo = min(lo, sm.red_lo[v]);
        hi = max(hi, sm.red_hi[v]);
    }
    __syncthreads();
    lo_out = lo;
    hi_out = hi;
}

// Keys left in range below which a histogram pass gives way to ranking them
// pairwise.
constexpr uint32_t kRankMax = 256;

// Key value tau of the need-th largest of the keys visited by `each` (every
// key of the set, over the workgroup), all of which lie in [lo, hi], and how
// many keys equal to tau belong to the top `need` (need_out).  1 <= need <=
// number of keys.  Called by all kTkThreads threads; the result is uniform.
// Histogram passes narrow [lo, hi] to the bin holding the need-th largest;
// with Rank, once that bin holds at most kRankMax keys of several values
// they are gathered and each counts the keys above it and at it: the value
// with fewer than need above and at least need at or above is tau.  (Rank is
// taken by the per-row workgroups of rows up to 4096 keys, where it saves a
// pass or two; in the larger workgroups its registers cost occupancy.)
template <bool Rank = false, typename Each, int NT>
__device__ void block_select_in(Each each, uint32_t lo, uint32_t hi, uint32_t need,
                                SelectSmemT<NT> &sm, uint32_t &tau_out, uint32_t &need_out) {
    const int tid = threadIdx.x;
    while (lo != hi) {  // invariant: keys > hi are taken; need more lie in [lo, hi]
        const uint32_t range = hi - lo;
        int shift = 0;
        while ((range >> shift) >= (uint32_t)kTkBins) ++shift;
        const int nb = (int)(range >> shift) + 1;
        for (int j = tid; j < nb; j += NT) sm.hist[j] = 0u;
        __syncthreads();
        each([&](uint32_t u) {
            if (u >= lo && u <= hi) atomicAdd(&sm.hist[(u - lo) >> shift], 1u);
        });
        __syncthreads();
        {  // bin holding the need-th largest: suffix counts over thread-owned bin pairs
            constexpr int kPer = kTkBins / NT;  // bins per thread
            uint32_t hb[kPer], c = 0u;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int bj = tid * kPer + j;
                hb[j] = bj < nb ? sm.hist[bj] : 0u;
                c += hb[j];
            }
            uint32_t tot;
            const uint32_t pre = block_excl_scan<NT / 64>(c, sm.scan, tot);
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
        const uint32_t m = sm.hist[bin];  // keys in the narrowed range
        const uint32_t new_lo = lo + (bin << shift);
        const uint32_t width_m1 = (1u << shift) - 1u;
        hi = (hi - new_lo > width_m1) ? new_lo + width_m1 : hi;
        lo = new_lo;
        __syncthreads();
        if (Rank && lo != hi && m <= kRankMax) {  // uniform
            if (tid == 0) sm.gcount = 0u;
            __syncthreads();
            each([&](uint32_t u) {
                if (u >= lo && u <= hi) {
                    const uint32_t sl = atomicAdd(&sm.gcount, 1u);
                    if (sl < kRankMax) sm.hist[sl] = u;
                }
            });
            __syncthreads();
            for (uint32_t a = tid; a < m; a += NT) {
                const uint32_t ka = sm.hist[a];
                uint32_t gt = 0u, ge = 0u;
                for (uint32_t g = 0; g < m; ++g) {
                    const uint32_t kg = sm.hist[g];
                    gt += kg > ka ? 1u : 0u;
                    ge += kg >= ka ? 1u : 0u;
                }
                if (gt < need && need <= ge) {  // every key equal to tau writes the same
                    sm.found_bin = ka;
                    sm.found_above = gt;
                }
            }
            __syncthreads();
            tau_out = sm.found_bin;
            need_out = need - sm.found_above;
            __syncthreads();
            return;
        }
    }
    tau_out = lo;
    need_out = need;
}

// block_select_in over keys key_at(0..n-1), range found first.
template <bool Rank = false, typename KeyAt, int NT>
__device__ void block_select(KeyAt key_at, int n, uint32_t need, SelectSmemT<NT> &sm,
                             uint32_t &tau_out, uint32_t &need_out) {
    auto each = [&](auto f) {
        for (int p = threadIdx.x; p < n; p += NT) f(key_at(p));
    };
    uint32_t lo, hi;
    block_key_range(each, sm, lo, hi);
    block_select_in<Rank>(each, lo, hi, need, sm, tau_out, need_out);
}

// ------------------------------------------------------- per-row kernel ----
template <int NT, int CACHE>
struct RowSmemT {
    SelectSmemT<NT> sel;
    uint32_t cnt_gt[NT / 64], cnt_eq[NT / 64];
    __align__(16) uint32_t keys[CACHE];
};

// Rows longer than the LDS cache: a threshold from a 1/16 sample of the row
// (runs of 32 consecutive positions, so each sample run is one cache line),
// then one pass over the row that keeps, per wave and in position order, the
// keys at or above it; the exact selection then runs on those candidates
// only, and the row is read about once instead of once per radix pass.
// Exact whenever at least k keys reach the threshold (the k-th largest is
// then among them, with all its ties) and every wave's candidates fit its
// share of the cache; otherwise it returns false with nothing written and
// the caller runs the full passes.
constexpr int kSampleRun = 32;
template <int NT, int CACHE>
__device__ bool sampled_select(const float *__restrict__ row, int n, int k,
                               int32_t *__restrict__ out, RowSmemT<NT, CACHE> &sm) {
    // the two threshold searches rank their last bin in the 512-thread tier,
    // where that fits the registers (elsewhere it spills)
    constexpr bool kSampledRank = NT == 512;
    constexpr int W = NT / 64;
    constexpr int kCap = CACHE / 2 / W;        // candidates per wave
    constexpr int kMaxRuns = CACHE / 2 / kSampleRun;
    uint32_t *ck = sm.keys;                    // [W][kCap] keys (samples first)
    uint32_t *cp = sm.keys + CACHE / 2;        // [W][kCap] positions
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // 1. sample: runs of kSampleRun positions every `stride` (>= 512)
    int stride = 512;
    while (n / stride > kMaxRuns) stride *= 2;
    const int ns = (n / stride) * kSampleRun;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    if (aligned) {  // 16-byte pieces of the runs, every load issued before any is used
        constexpr int kVec = CACHE / 2 / 4 / NT;  // ns <= CACHE / 2
        f32x4 sv[kVec];
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            const int m = 4 * (tid + u * NT);
            sv[u] = m < ns ? *reinterpret_cast<const f32x4 *>(
                                 row + (size_t)(m / kSampleRun) * stride + m % kSampleRun)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            const int m = 4 * (tid + u * NT);
            if (m < ns)
                *reinterpret_cast<u32x4 *>(ck + m) =
                    u32x4{ordered_key(sv[u][0]), ordered_key(sv[u][1]), ordered_key(sv[u][2]),
                          ordered_key(sv[u][3])};
        }
    } else {
        for (int m = tid; m < ns; m += NT)
            ck[m] = ordered_key(row[(size_t)(m / kSampleRun) * stride + m % kSampleRun]);
    }
    __syncthreads();
    // the need_s-th largest sample: 1.25 k of the row's share plus a margin
    const uint32_t need_s =
        (uint32_t)min((long long)ns, (long long)k * ns * 5 / (4LL * n) + 32);
    uint32_t tau_s, unused;
    block_select<kSampledRank>([&](int j) -> uint32_t { return ck[j]; }, ns, need_s, sm.sel, tau_s,
                               unused);
    __syncthreads();  // every thread is done with the samples
    // 2. one pass over the row: each wave keeps its segment's keys >= tau_s,
    // in position order.  Segments are whole multiples of 256 positions, so
    // with an aligned row every 16-byte piece but the row's last lies inside
    // one wave's segment; a lane takes 4 consecutive keys per piece, eight
    // pieces in flight.
    const int seg = ceil_div(ceil_div(n, W), 256) * 256;
    const int w0 = wave * seg, w1 = min(n, w0 + seg);
    uint32_t *myk = ck + wave * kCap, *myp = cp + wave * kCap;
    uint32_t cnt = 0u;
    if (aligned) {
        constexpr int U = 8;
        for (int p0 = w0; p0 < w1; p0 += 256 * U) {
            f32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + 256 * u + 4 * lane;
                if (p + 4 <= w1) {
                    v[u] = *reinterpret_cast<const f32x4 *>(row + p);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[u][e] = p + e < w1 ? row[p + e] : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + 256 * u + 4 * lane;
                uint32_t key[4], take = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    key[e] = ordered_key(v[u][e]);
                    if (p + e < w1 && key[e] >= tau_s) take |= 1u << e;
                }
                // this lane's count and the wave's prefix of counts (three ballots)
                const uint32_t c = (uint32_t)__popc(take);
                const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
                uint32_t slot = cnt + lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (take & (1u << e)) {
                        if (slot < (uint32_t)kCap) {
                            myk[slot] = key[e];
                            myp[slot] = (uint32_t)(p + e);
                        }
                        ++slot;
                    }
                cnt += (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
            }
        }
    } else {
        constexpr int U = 8;
        for (int p0 = w0; p0 < w1; p0 += 64 * U) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + 64 * u + lane;
                v[u] = p < w1 ? row[p] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + 64 * u + lane;
                const uint32_t key = ordered_key(v[u]);
                const bool c = p < w1 && key >= tau_s;
                const uint64_t m = __ballot(c);
                if (c) {
                    const uint32_t slot = cnt + lanes_below(m);
                    if (slot < (uint32_t)kCap) {
                        myk[slot] = key;
                        myp[slot] = (uint32_t)p;
                    }
                }
                cnt += (uint32_t)__popcll(m);
            }
        }
    }
    if (lane == 0) {
        sm.cnt_gt[wave] = cnt;
        sm.cnt_eq[wave] = 0u;
    }
    __syncthreads();
    uint32_t cw[W], total = 0u;
    bool over = false;
#pragma unroll
    for (int v = 0; v < W; ++v) {
        cw[v] = sm.cnt_gt[v];
        over |= cw[v] > (uint32_t)kCap;
        total += cw[v];
    }
    __syncthreads();  // the counts are read before they are reused below
    if (over || total < (uint32_t)k) return false;  // uniform
    // 3. exact threshold among the candidates
    auto each = [&](auto f) {
        for (int j = tid; j < W * kCap; j += NT) {
            const int v = j / kCap;
            if ((uint32_t)(j - v * kCap) < cw[v]) f(ck[j]);
        }
    };
    uint32_t lo, hi, tau, need;
    block_key_range(each, sm.sel, lo, hi);
    block_select_in<kSampledRank>(each, lo, hi, (uint32_t)k, sm.sel, tau, need);
    // 4. in position order (wave regions in order, each in order): all keys
    // > tau and the first `need` keys == tau
    const uint32_t mine = cw[wave];
    uint32_t c_gt = 0u, c_eq = 0u;
    for (uint32_t j0 = 0; j0 < mine; j0 += 64) {
        const uint32_t j = j0 + lane;
        const uint32_t key = j < mine ? myk[j] : 0u;
        c_gt += (uint32_t)__popcll(__ballot(j < mine && key > tau));
        c_eq += (uint32_t)__popcll(__ballot(j < mine && key == tau));
    }
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
    for (uint32_t j0 = 0; j0 < mine; j0 += 64) {
        const uint32_t j = j0 + lane;
        const uint32_t key = j < mine ? myk[j] : 0u;
        const bool gt = j < mine && key > tau;
        const bool eq = j < mine && key == tau;
        const uint64_t eqm = __ballot(eq);
        const bool take = gt || (eq && ties + lanes_below(eqm) < need);
        const uint64_t tm = __ballot(take);
        if (take) out[written + lanes_below(tm)] = (int32_t)myp[j];
        written += (uint32_t)__popcll(tm);
        ties += (uint32_t)__popcll(eqm);
    }
    return true;
}

// One workgroup per row.  A cached row is read with 16-byte loads, four in
// flight per thread, converted to keys on the way into LDS; the threshold
// search and the selection then read LDS only.  The selection gives each
// wave one contiguous segment of positions: a first sweep counts the keys
// above tau and equal to tau per wave, and after one barrier a second sweep
// writes the wave's selected positions in order (ballot prefix counts).
//
// bits (optional, rows no longer than CACHE): the selection also as one bit
// per position, bits[(b * rows + r) * words + p / 32] bit p % 32 (every word
// of the row written, zeros past the candidates), and row_hi[b * rows + r] =
// n - 1 (no selected position lies beyond it; -1 for an empty row).
// The exact top-k of one row of n > k scores (in memory), written to out in
// ascending position order by the NT threads of the workgroup; brow
// (optional) receives the selection as bits, `words` words.
template <int NT, int CACHE>
__device__ void select_row(const float *__restrict__ row, int n, int k, int32_t *__restrict__ out,
                           uint32_t *__restrict__ brow, int words, RowSmemT<NT, CACHE> &sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const bool bits = brow != nullptr;
    if (bits)  // words past the waves' 64-position runs below
        for (int wd = 2 * ((n + 63) / 64) + tid; wd < words; wd += NT) brow[wd] = 0u;
    const bool cached = n <= CACHE;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    if (!cached && !bits && sampled_select(row, n, k, out, sm)) return;
    uint32_t lo, hi;
    if (cached) {
        // 16-byte pieces j = tid + NT * (4 * it + u), four loads in flight
        const int n16 = aligned ? n / 4 : 0;  // whole pieces read as vectors
        uint32_t vlo = 0xffffffffu, vhi = 0u;
        for (int j0 = tid; j0 < n16; j0 += 4 * NT) {
            f32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * NT;
                if (j < n16) v[u] = reinterpret_cast<const f32x4 *>(row)[j];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * NT;
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
        for (int p = 4 * n16 + tid; p < n; p += NT) {
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
            for (int j = tid; j < n16; j += NT) {
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
            for (int j0 = tid; j0 < n16; j0 += U * NT) {
                f32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int j = j0 + u * NT;
                    if (j < n16) v[u] = reinterpret_cast<const f32x4 *>(row)[j];
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (j0 + u * NT < n16) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) f(ordered_key(v[u][e]));
                    }
            }
            for (int p = 4 * n16 + tid; p < n; p += NT) f(ordered_key(row[p]));
        }
    };
    if (!cached) block_key_range(each, sm.sel, lo, hi);

    uint32_t tau, need;
    block_select_in<(CACHE <= 4096)>(each, lo, hi, (uint32_t)k, sm.sel, tau, need);

    // ordered selection: all keys > tau, plus the first `need` keys == tau
    const int seg = ceil_div(ceil_div(n, (NT / 64)), 64) * 64;  // positions per wave
    const int w0 = wave * seg, w1 = min(n, w0 + seg);
    // sweep 1 counts the wave's keys above and at tau; after the barrier,
    // sweep 2 writes the wave's selected positions from the same keys (a
    // cached row's keys stay in registers between the sweeps)
    const int nit = w1 > w0 ? ceil_div(w1 - w0, 64) : 0;
    constexpr int kMaxIt = CACHE / NT;  // seg <= 64 * kMaxIt when cached
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
        if (bits && lane == 0) {  // positions p - lane .. p - lane + 63: two words
            const int wd = (p - lane) / 32;
            brow[wd] = (uint32_t)tm;
            if (wd + 1 < words) brow[wd + 1] = (uint32_t)(tm >> 32);
        }
        written += (uint32_t)__popcll(tm);
        ties += (uint32_t)__popcll(eqm);
    });
}

template <int NT, int CACHE>
__global__ __launch_bounds__(NT) void topk_row_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int T, int S, int row0, int k, int cur, int ostride, int32_t *__restrict__ idx,
    uint32_t *__restrict__ bits, int32_t *__restrict__ row_hi, int words) {
    __shared__ RowSmemT<NT, CACHE> sm;
    // the last rows first: without explicit positions they are the longest,
    // so the short ones fill in at the end rather than trailing behind them
    const int r = gridDim.x - 1 - blockIdx.x;
    const int b = blockIdx.y;
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S) - cur;  // last candidate position
    const float *row = scores + (size_t)b * batch_stride + (size_t)r * S;
    int32_t *out = idx + ((size_t)b * T + i) * ostride;
    const int n = t < 0 ? 0 : t + 1;
    const int tid = threadIdx.x;
    uint32_t *brow = bits ? bits + ((size_t)b * gridDim.x + r) * words : nullptr;
    if (bits && tid == 0) row_hi[(size_t)b * gridDim.x + r] = n - 1;

    if (n <= k) {  // every candidate is selected
        for (int p = tid; p < k; p += NT) out[p] = p < n ? p : -1;
        if (bits)
            for (int wd = tid; wd < words; wd += NT) {
                const int p0 = 32 * wd;
                brow[wd] = p0 + 32 <= n ? 0xffffffffu : p0 >= n ? 0u : (1u << (n - p0)) - 1u;
            }
        return;
    }
    select_row<NT, CACHE>(row, n, k, out, brow, words, sm);
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
            // issued without waiting for the count (only the slice's range
            // decides); entries past the count are read but never visited
            const size_t ci = min((size_t)sl * kWideSlice + j, (size_t)S - 1);
            pre[v][f] = sl < nslices ? gcand[ci] : make_uint2(0u, 0u);
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

// ------------------------------------------------------ partition path -----
// Few wide rows with a budget small against the row (decode): the row's
// 32-position tiles are dealt round-robin to P partitions of 64 tiles, one
// workgroup each, and every workgroup keeps its partition's keys at or above
// a threshold chosen with two rounds of a 256-bin histogram (the partition's
// key range, then the bin where the count crosses) so that at most `cap`
// remain; it records the threshold when it dropped keys.  The kept keys of a
// partition are a prefix of it in the selection order.  Let theta be the
// largest recorded threshold: every dropped key lies below it, so once at
// least k kept keys reach theta the k-th largest kept key is >= theta, no
// dropped key can belong to the top k, and the top k of the kept keys is
// the row's.  The resolve checks exactly that and selects among the kept
// keys; otherwise (a partition holding a large share of the top k, heavy
// ties) it runs the exact per-row selection on the whole row.  Dealing tiles
// round-robin puts a contiguous run of top scores (a local window) at one
// tile per partition.
constexpr int kPartTiles = 64;                         // 32-position tiles per partition
constexpr int kPartKeys = kPartTiles * 32;             // 2048
constexpr int kPartBins = 256;
constexpr int kPartMax = 12288;                        // kept keys a row's resolve holds
constexpr int kPartPieces = kPartMax / 2 / kTkThreads;  // 16-byte pieces per resolve thread
constexpr int kPartMaxP = kWideMaxS / kPartKeys;       // 128
constexpr int kPartTies = 1024;                        // keys equal to tau ranked pairwise
constexpr uint32_t kPartRefineMin = 32;                // crossing bins below this are not refined

struct PartLayout {
    uint2 *meta;  // [rows][P] (kept count, threshold; 0 when nothing was dropped)
    uint2 *cand;  // [rows][P][stride] (key, position) of the kept keys
    int P;        // partitions a row; 0: the partition path does not apply
    int stride;   // slots a partition (even, >= cap)
    int cap;      // keys a partition keeps at most
    uint32_t magic;  // ceil(2^32 / stride): slot / stride = umulhi(slot, magic) for a row's slots
};

// Over a 256-bin histogram hw of fewer than 4096 keys (every lane of the
// wave active): the lowest bin `first` whose keys and those of every bin
// above it number at most `room` (256: the top bin alone holds more); room
// becomes what is left of it for bin first - 1.  Uniform.  The keys in the
// bins of higher lanes come from one ballot per bit of the lanes' counts.
__device__ __forceinline__ void part_first_bin(const uint32_t *hw, int lane, uint32_t &room,
                                               uint32_t &first) {
    const u32x4 hb = reinterpret_cast<const u32x4 *>(hw)[lane];  // bins 4 lane .. + 3
    const uint32_t s4 = hb[0] + hb[1] + hb[2] + hb[3];
    uint32_t higher = 0u;
#pragma unroll
    for (int bit = 0; bit < 12; ++bit) {
        const uint32_t mine = (s4 >> bit) & 1u;
        const uint64_t m = __ballot(mine);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        higher += ((uint32_t)__popcll(m) - below - mine) << bit;
    }
    uint32_t above = higher + s4;  // keys in bins >= 4 lane
    uint32_t at_bin = kPartBins, at_count = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (above <= room && at_bin == (uint32_t)kPartBins) {
            at_bin = 4 * lane + j;
            at_count = above;
        }
        above -= hb[j];
    }
    // the bins that qualify are all those from `first` up: the lowest lane
    // holding one has it
    const uint64_t q = __ballot(at_bin != (uint32_t)kPartBins);
    if (q == 0u) {
        first = kPartBins;
        return;
    }
    const int src = __builtin_ctzll(q);
    first = (uint32_t)__builtin_amdgcn_readlane((int)at_bin, src);
    room -= (uint32_t)__builtin_amdgcn_readlane((int)at_count, src);
}

// Sum, smallest or largest of v over the 64 lanes of a wave, uniform; every
// lane must be active.  DPP within each row of 16 lanes (quad permutations,
// then the half-row and row mirrors), then the four rows' results.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));
    return op(op((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
              op((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// grid: 1-D, 8 * ceil(B * rows / 8) * P workgroups, one a partition.
// Workgroup id mod 8 (its XCD) takes the rows rr = b * rows + r with rr mod 8
// equal to it, the XCD of the row's resolve workgroup.
__global__ __launch_bounds__(256) void topk_part_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int B, int T, int S, int row0, int rows, int k, int cur, PartLayout L) {
    __shared__ __align__(16) uint32_t hist[kPartBins];
    __shared__ uint32_t red[3][4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int jx = (int)(blockIdx.x >> 3);
    const int rr = (int)(blockIdx.x & 7) + 8 * (jx / L.P);
    const int c = jx % L.P;
    if (rr >= B * rows) return;
    const int b = rr / rows, r = rr % rows;
    const int t = query_pos(q_pos, b, row0 + r, T, S) - cur;
    const int n = t < 0 ? 0 : t + 1;
    if (n <= k) return;  // the resolve takes every position
    const float *row = scores + (size_t)b * batch_stride + (size_t)r * S;
    // the thread's 16-byte pieces j = tid and tid + 256 of the partition:
    // piece j holds positions 4 (j % 8) .. + 3 of tile c + P (j / 8)
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    int p0[2];
    f32x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int j = tid + 256 * h;
        p0[h] = 32 * (c + L.P * (j >> 3)) + 4 * (j & 7);
        if (aligned && p0[h] + 4 <= n) {
            v[h] = *reinterpret_cast<const f32x4 *>(row + p0[h]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[h][e] = p0[h] + e < n ? row[p0[h] + e] : 0.0f;
        }
    }
    reinterpret_cast<uint32_t *>(hist)[tid] = 0u;  // 256 bins, one a thread
    uint32_t key[8], valid = 0u, lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        key[e] = ordered_key(v[e >> 2][e & 3]);
        if (p0[e >> 2] + (e & 3) < n) {
            valid |= 1u << e;
            lo = min(lo, key[e]);
            hi = max(hi, key[e]);
        }
    }
    lo = wave_reduce(lo, [](uint32_t a, uint32_t b) { return min(a, b); });
    hi = wave_reduce(hi, [](uint32_t a, uint32_t b) { return max(a, b); });
    uint32_t nvalid =
        wave_reduce((uint32_t)__popc(valid), [](uint32_t a, uint32_t b) { return a + b; });
    if (lane == 0) {
        red[0][wave] = lo;
        red[1][wave] = hi;
        red[2][wave] = nvalid;
    }
    __syncthreads();
    lo = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
    hi = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    nvalid = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    uint64_t theta = 0u;  // keys below it are dropped
    if (nvalid > (uint32_t)L.cap) {  // uniform
        int shift = 0;
        while (((hi - lo) >> shift) >= (uint32_t)kPartBins) ++shift;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (valid & (1u << e)) atomicAdd(&hist[min((key[e] - lo) >> shift, 255u)], 1u);
        __syncthreads();
        // every wave reads the same histogram and reaches the same bin
        uint32_t room = (uint32_t)L.cap, first;
        part_first_bin(hist, lane, room, first);
        theta = (uint64_t)lo + ((uint64_t)first << shift);
        // refine inside bin first - 1 (it holds a key; the bins above it hold
        // cap - room keys) unless it holds few: then keeping only the bins
        // above it loses little (a row of random scores: never refined)
        if (first >= 1 && shift > 0 && hist[first - 1] > kPartRefineMin) {  // uniform
            const uint32_t b1 = first - 1;
            const uint32_t base = lo + (b1 << shift);
            const int s2 = shift > 8 ? shift - 8 : 0;
            __syncthreads();  // every wave has read the histogram
            hist[tid] = 0u;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((valid & (1u << e)) && ((key[e] - lo) >> shift) == b1)
                    atomicAdd(&hist[min((key[e] - base) >> s2, 255u)], 1u);
            __syncthreads();
            uint32_t first2;
            part_first_bin(hist, lane, room, first2);
            theta = (uint64_t)base + ((uint64_t)first2 << s2);
        }
    }
    uint32_t take = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if ((valid & (1u << e)) && (uint64_t)key[e] >= theta) take |= 1u << e;
    // slots: the waves' totals, then a prefix of the lanes' counts (0..8, four ballots)
    const uint32_t cnt = (uint32_t)__popc(take);
    const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u),
                   b3 = __ballot(cnt & 8u);
    const uint32_t wtot = (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2) +
                                     8 * __popcll(b3));
    __syncthreads();  // red is reused
    if (lane == 0) red[0][wave] = wtot;
    __syncthreads();
    uint32_t slot = lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2) +
                    8u * lanes_below(b3);
    uint32_t kept = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        slot += w < wave ? red[0][w] : 0u;
        kept += red[0][w];
    }
    uint2 *dst = L.cand + ((size_t)rr * L.P + c) * (size_t)L.stride;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (take & (1u << e)) {
            if (slot < (uint32_t)L.stride)
                dst[slot] = make_uint2(key[e], (uint32_t)(p0[e >> 2] + (e & 3)));
            ++slot;
        }
    // (more than the slots hold cannot happen; were it to, the partition
    // reports that it dropped every key, and the exact selection runs)
    if (tid == 0)
        L.meta[(size_t)rr * L.P + c] =
            kept > (uint32_t)L.stride
                ? make_uint2(0u, 0xffffffffu)
                : make_uint2(kept,
                             kept < nvalid ? (uint32_t)min(theta, (uint64_t)0xffffffffu) : 0u);
}

// Sum, smallest and largest of the threads' values (uniform results; every
// thread active).  One LDS-only barrier: `red` may be written again only
// after a later barrier (callers alternate two buffers), and global loads in
// flight are not waited for.
__device__ __forceinline__ void block_sum_min_max(uint32_t &s, uint32_t &mn, uint32_t &mx,
                                                  uint32_t (&red)[3][kTkWaves]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    s = wave_reduce(s, [](uint32_t a, uint32_t b) { return a + b; });
    mn = wave_reduce(mn, [](uint32_t a, uint32_t b) { return min(a, b); });
    mx = wave_reduce(mx, [](uint32_t a, uint32_t b) { return max(a, b); });
    if (lane == 0) {
        red[0][wave] = s;
        red[1][wave] = mn;
        red[2][wave] = mx;
    }
    lds_barrier();
    s = 0u;
    mn = 0xffffffffu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        s += red[0][w];
        mn = min(mn, red[1][w]);
        mx = max(mx, red[2][w]);
    }
}

// Exclusive prefix sum over the workgroup in thread order of values below
// 2^Bits, and the total: one ballot per bit within a wave, the waves'
// totals through LDS (one LDS-only barrier; `wsum` reused only after a
// later barrier).
template <int Bits>
__device__ __forceinline__ uint32_t block_excl_scan_small(uint32_t v, uint32_t *wsum,
                                                          uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t below = 0u, wtot = 0u;
#pragma unroll
    for (int bit = 0; bit < Bits; ++bit) {
        const uint64_t m = __ballot((v >> bit) & 1u);
        below += lanes_below(m) << bit;
        wtot += (uint32_t)__popcll(m) << bit;
    }
    if (lane == 0) wsum[wave] = wtot;
    lds_barrier();
    uint32_t before = 0u, sum = 0u;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        const uint32_t c = wsum[w];
        before += w < wave ? c : 0u;
        sum += c;
    }
    total = sum;
    return before + below;
}

struct PartSmem {
    SelectSmem sel;
    uint32_t red[2][3][kTkWaves];
    uint32_t wsum[2][kTkWaves];
    uint32_t cnt[kPartMaxP];  // kept keys of each partition
    uint32_t nties;
    uint2 ties[kPartTies];
    uint32_t bits[kWideMaxS / 32];
};
// the exact per-row selection, when the kept keys do not decide, reuses it
union PartResolveSmem {
    PartSmem p;
    RowSmemT<kTkThreads, 16384> row;
};

// grid: x = row in chunk, y = batch (workgroup id b * rows + r: the XCD that
// ran the row's partitions)
__global__ __launch_bounds__(kTkThreads) void topk_part_resolve_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int T, int S, int row0, int rows, int k, int cur, int ostride, int32_t *__restrict__ idx,
    PartLayout L) {
    __shared__ PartResolveSmem smu;
    PartSmem &sm = smu.p;
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
    const int P = L.P, stride = L.stride;
    const int nslots = P * stride;
    const u32x4 *cp = reinterpret_cast<const u32x4 *>(L.cand + rr * (size_t)nslots);

    // ---- every load up front: the partitions' counts and thresholds, and
    // all their slots (two per 16-byte piece; slots past a count are ignored)
    // (unconditional, clamped into the row's slots, so that the waits count
    // each load: the counts first, the slots after; pieces past the slots
    // are never used)
    uint2 mt = L.meta[rr * P + min(tid, P - 1)];
    u32x4 cv[kPartPieces];
#pragma unroll
    for (int u = 0; u < kPartPieces; ++u) cv[u] = cp[min(tid + u * kTkThreads, nslots / 2 - 1)];
    if (tid >= P) mt = make_uint2(0u, 0u);
    // while they are in flight: clear the bitmap, the histogram, the group
    // (the barriers below are LDS-only, so the loads stay in flight)
    const int nw = (n + 31) / 32;
    for (int w = tid; w < nw; w += kTkThreads) sm.bits[w] = 0u;
    for (int j = tid; j < kTkBins; j += kTkThreads) sm.sel.hist[j] = 0u;
    if (tid == 0) sm.nties = 0u;
    if (tid < P) sm.cnt[tid] = mt.x;
    uint32_t unused_s = 0u, unused_mn = 0xffffffffu, theta = mt.y;
    block_sum_min_max(unused_s, unused_mn, theta, sm.red[0]);  // also publishes the above

    // ---- the kept keys at or above theta
    uint32_t vmask = 0u, nkeys = 0u, lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int u = 0; u < kPartPieces; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = 2 * (tid + u * kTkThreads) + e;
            if (q < nslots) {
                const int c = (int)__umulhi((uint32_t)q, L.magic);  // q / stride
                const uint32_t key = cv[u][2 * e], p = cv[u][2 * e + 1];
                if ((uint32_t)(q - c * stride) < sm.cnt[c] && p < (uint32_t)n && key >= theta) {
                    vmask |= 1u << (2 * u + e);
                    ++nkeys;
                    lo = min(lo, key);
                    hi = max(hi, key);
                }
            }
        }
    block_sum_min_max(nkeys, lo, hi, sm.red[1]);
    if (nkeys < (uint32_t)k) {  // uniform: a dropped key may belong to the top k
        __syncthreads();
        select_row<kTkThreads, 16384>(scores + (size_t)b * batch_stride + (size_t)r * S, n, k,
                                      out, nullptr, 0, smu.row);
        return;
    }
    auto each = [&](auto f) {
#pragma unroll
        for (int u = 0; u < kPartPieces; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                if (vmask & (1u << (2 * u + e))) f(cv[u][2 * e], cv[u][2 * e + 1]);
    };
    auto set_bit = [&](uint32_t p) { atomicOr(&sm.bits[p >> 5], 1u << (p & 31)); };

    // ---- one histogram pass over [lo, hi]: bin d holds the k-th largest
    int shift = 0;
    while (((hi - lo) >> shift) >= (uint32_t)kTkBins) ++shift;
    each([&](uint32_t key, uint32_t) { atomicAdd(&sm.sel.hist[(key - lo) >> shift], 1u); });
    lds_barrier();
    {
        constexpr int kPer = kTkBins / kTkThreads;
        uint32_t hb[kPer], c = 0u;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            hb[j] = sm.sel.hist[tid * kPer + j];
            c += hb[j];
        }
        uint32_t tot;  // the kept keys: fewer than 2^14
        const uint32_t pre = block_excl_scan_small<14>(c, sm.wsum[0], tot);
        uint32_t run = tot - pre - c;  // keys in the bins of later threads
#pragma unroll
        for (int j = kPer - 1; j >= 0; --j) {
            const uint32_t before = run;
            run += hb[j];
            if (before < (uint32_t)k && run >= (uint32_t)k) {
                sm.sel.found_bin = (uint32_t)(tid * kPer + j);
                sm.sel.found_above = before;
            }
        }
    }
    lds_barrier();
    const uint32_t d = sm.sel.found_bin;
    const uint32_t need = (uint32_t)k - sm.sel.found_above;  // keys to take from bin d

    // ---- the bins above d are taken; bin d's keys are gathered and ranked
    // (larger key first, then lower position)
    each([&](uint32_t key, uint32_t p) {
        const uint32_t bin = (key - lo) >> shift;
        if (bin > d) {
            set_bit(p);
        } else if (bin == d) {
            const uint32_t s = atomicAdd(&sm.nties, 1u);
            if (s < (uint32_t)kPartTies) sm.ties[s] = make_uint2(key, p);
        }
    });
    lds_barrier();
    const uint32_t m = sm.nties;
    if (m <= (uint32_t)kPartTies) {
        for (uint32_t a = tid; a < m; a += kTkThreads) {
            const uint2 ca = sm.ties[a];
            uint32_t ahead = 0u;
            for (uint32_t g = 0; g < m; ++g) {
                const uint2 cg = sm.ties[g];
                ahead += (cg.x > ca.x || (cg.x == ca.x && cg.y < ca.y)) ? 1u : 0u;
            }
            if (ahead < need) set_bit(ca.y);
        }
    } else {  // a crowded bin: exact threshold among its keys, then ties by position
        const uint32_t blo = lo + (d << shift);
        const uint32_t bhi = hi - blo > (1u << shift) - 1u ? blo + ((1u << shift) - 1u) : hi;
        auto eachd = [&](auto f) {
            each([&](uint32_t key, uint32_t) {
                if (((key - lo) >> shift) == d) f(key);
            });
        };
        uint32_t tau, need_tau;
        block_select_in(eachd, blo, bhi, need, sm.sel, tau, need_tau);
        uint32_t nt = 0u, unused_mn2 = 0xffffffffu, unused_mx2 = 0u;
        each([&](uint32_t key, uint32_t) { nt += key == tau ? 1u : 0u; });
        block_sum_min_max(nt, unused_mn2, unused_mx2, sm.red[0]);
        uint32_t pos_cut = 0xffffffffu;  // ties at positions <= pos_cut are taken
        if (need_tau < nt) {
            auto each2 = [&](auto f) {
                each([&](uint32_t key, uint32_t p) { f(key == tau ? ~p : 0u); });
            };
            uint32_t lo2, hi2, tau2, need2;
            block_key_range(each2, sm.sel, lo2, hi2);
            block_select_in(each2, lo2, hi2, need_tau, sm.sel, tau2, need2);
            pos_cut = ~tau2;
        }
        each([&](uint32_t key, uint32_t p) {
            if (((key - lo) >> shift) == d && (key > tau || (key == tau && p <= pos_cut)))
                set_bit(p);
        });
    }
    __syncthreads();

    // ---- ordered compaction: contiguous words per thread, prefix of popcounts
    const int per = (nw + kTkThreads - 1) / kTkThreads;
    const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
    uint32_t cntw = 0u;
    for (int w = w0; w < w1; ++w) cntw += (uint32_t)__popc(sm.bits[w]);
    uint32_t total;  // per <= 8 words a thread: at most 256
    uint32_t slot = block_excl_scan_small<9>(cntw, sm.wsum[1], total);
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

// Partition plan of a wide launch with budget k (P = 0 in the result: the
// path does not apply): P partitions of 2048 positions a row.  A partition
// keeps at most cap keys, about k / P of which belong to the top k of a
// random row: cap leaves six standard deviations and a margin above that,
// and at least 40 so that a window of consecutive top positions (one
// 32-position tile per partition) fits; the kept keys of a row must fit the
// resolve's registers (kPartMax).  The layout sits at the head of the wide
// path's workspace, which is larger.
PartLayout part_plan(void *ws, int nrows, int S, int k) {
    PartLayout L{};
    const int P = ceil_div(S, kPartKeys);
    if (k < 1 || P > kPartMaxP) return L;
    const double mu = (double)k / P;
    int cap = (int)std::ceil(mu + 6.0 * std::sqrt(mu) + 8.0);
    cap = (std::max(cap, 40) + 7) & ~7;
    const int stride = cap;  // even
    if ((long long)P * cap > kPartMax || cap >= kPartKeys) return L;
    const size_t meta_bytes = ((size_t)nrows * P * sizeof(uint2) + 15) & ~(size_t)15;
    if (15 + meta_bytes + (size_t)nrows * P * stride * sizeof(uint2) >
        (size_t)nrows * wide_row_bytes(S) + 64)
        return L;  // not reached for S >= kWideMinS; the layout must fit the workspace
    // both arrays 16-byte aligned (the resolve reads the slots as 16-byte
    // pieces); the workspace's 64 spare bytes cover the padding
    const uintptr_t m = ((uintptr_t)ws + 15) & ~(uintptr_t)15;
    L.meta = reinterpret_cast<uint2 *>(m);
    L.cand = reinterpret_cast<uint2 *>(m + meta_bytes);
    L.P = P;
    L.stride = stride;
    L.cap = cap;
    L.magic = (uint32_t)(((1ull << 32) + stride - 1) / stride);
    return L;
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
size_t topk_clear_words(int B, int rows, int S, int k, bool include_current) {
    const int kk = k - (include_current ? 1 : 0);
    if (!use_wide(B, rows, S) || kk < 1 || part_plan(nullptr, B * rows, S, kk).P > 0) return 0;
    return (size_t)B * rows * (2 * kDigits + kMetaWords);
}

bool topk_writes_bitmap(int B, int rows, int S, int k, bool include_current) {
    // per-row kernel with every row in its LDS cache (a longer row writes the
    // bitmap only through the full passes, not the faster sampled path)
    return !include_current && k >= 1 && !use_wide(B, rows, S) && S <= 16384;
}

hipError_t launch_topk(const float *scores, size_t batch_stride, const int32_t *q_pos, int B,
                       int T, int S, int row0, int rows, int k, int32_t *idx, void *workspace,
                       bool workspace_cleared, hipStream_t stream, bool include_current,
                       uint32_t *bits, int32_t *row_hi) {
    // the current-token variant selects k-1 among the positions before t
    const int cur = include_current ? 1 : 0;
    const int kk = k - cur;
    const int words = (S + 31) / 32;
    if (bits && !(topk_writes_bitmap(B, rows, S, k, include_current) && row_hi))
        return hipErrorInvalidValue;
    const PartLayout PL =
        kk >= 1 && use_wide(B, rows, S) && workspace ? part_plan(workspace, B * rows, S, kk)
                                                     : PartLayout{};
    if (PL.P > 0) {
        const int nwg = 8 * ceil_div(B * rows, 8) * PL.P;
        hipLaunchKernelGGL(topk_part_kernel, dim3(nwg), dim3(256), 0, stream, scores,
                           batch_stride, q_pos, B, T, S, row0, rows, kk, cur, PL);
        hipLaunchKernelGGL(topk_part_resolve_kernel, dim3(rows, B), dim3(kTkThreads), 0, stream,
                           scores, batch_stride, q_pos, T, S, row0, rows, kk, cur, k, idx, PL);
    } else if (kk >= 1 && use_wide(B, rows, S) && workspace) {
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
        // the longest row of the launch picks the workgroup: short rows go to
        // small workgroups with small caches, several rows a CU at once; rows
        // past 16384 keys take the sampled path of the 16384-key tier (two
        // workgroups a CU), which beat caching them in a 128 KB workgroup
        const long long n_max = q_pos ? S : std::min<long long>(S, (long long)S - T + row0 + rows);
        if (n_max <= 4096)
            hipLaunchKernelGGL((topk_row_kernel<256, 4096>), dim3(rows, B), dim3(256), 0, stream,
                               scores, batch_stride, q_pos, T, S, row0, kk, cur, k, idx, bits, row_hi,
                               words);
        else if (n_max <= 8192)
            hipLaunchKernelGGL((topk_row_kernel<256, 8192>), dim3(rows, B), dim3(256), 0, stream,
                               scores, batch_stride, q_pos, T, S, row0, kk, cur, k, idx, bits, row_hi,
                               words);
        else
            hipLaunchKernelGGL((topk_row_kernel<512, 16384>), dim3(rows, B), dim3(512), 0, stream,
                               scores, batch_stride, q_pos, T, S, row0, kk, cur, k, idx, bits, row_hi,
                               words);
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
