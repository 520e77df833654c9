// topk.hip -- exact per-row top-k selection on gfx950.
//
// S_t = the k candidates s in 0..t with the highest score ("DeepSeek Sparse
// Attention: Learned Token Selection from Scratch", section 3.1), ties broken
// by the lower position; rows with t+1 <= k keep every candidate (section
// 7.2).  Output: the selected positions in ascending order, -1 padded.
//
// Method (one workgroup of 1024 threads per row):
//  1. map each score to an order-preserving 32-bit key (-0 folded onto +0);
//  2. threshold search on the key range: a block-wide min/max, then at most
//     three passes of a <=2048-bin LDS histogram over the current key range
//     [lo, hi] (bins are key >> shift, so binning is exact integer work);
//     each pass keeps only the bin holding the k-th largest key, until the
//     range is one key value tau.  `need` counts how many keys equal to tau
//     are still to be taken;
//  3. one ordered compaction sweep: tiles of 1024 consecutive positions, a
//     ballot/prefix count gives each tied position its rank among ties (lower
//     positions first) and each selected position its output slot, so the
//     output is ascending and identical run to run.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkBins = 2048;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    const uint32_t lo = __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u);
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), lo);
}

// Exclusive prefix count of `flag` over the workgroup in thread order, and
// the workgroup total.  `scratch` holds kTkWaves entries; two barriers.
__device__ __forceinline__ uint32_t block_flag_scan(bool flag, uint32_t *scratch,
                                                    uint32_t &total) {
    const int wave = threadIdx.x >> 6;
    const uint64_t m = __ballot(flag);
    const uint32_t in_wave = lanes_below(m);
    if ((threadIdx.x & 63) == 0) scratch[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int v = 0; v < kTkWaves; ++v) {
        const uint32_t c = scratch[v];
        before += v < wave ? c : 0u;
        sum += c;
    }
    __syncthreads();
    total = sum;
    return before + in_wave;
}

__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(
    const float *__restrict__ scores, size_t batch_stride, const int32_t *__restrict__ q_pos,
    int T, int S, int row0, int k, int32_t *__restrict__ idx) {
    __shared__ uint32_t hist[kTkBins];
    __shared__ uint32_t red_lo[kTkWaves], red_hi[kTkWaves];
    __shared__ uint32_t scan_scratch[kTkWaves];
    __shared__ uint32_t found_bin, found_above;

    const int r = blockIdx.x;
    const int b = blockIdx.y;
    const int i = row0 + r;
    const int t = query_pos(q_pos, b, i, T, S);
    const float *row = scores + (size_t)b * batch_stride + (size_t)r * S;
    int32_t *out = idx + ((size_t)b * T + i) * k;
    const int n = t < 0 ? 0 : t + 1;
    const int tid = threadIdx.x;

    if (n <= k) {  // every candidate is selected
        for (int p = tid; p < k; p += kTkThreads) out[p] = p < n ? p : -1;
        return;
    }

    // ---- 1. key range of the row
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int p = tid; p < n; p += kTkThreads) {
        const uint32_t u = ordered_key(row[p]);
        lo = min(lo, u);
        hi = max(hi, u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
    }
    if ((tid & 63) == 0) {
        red_lo[tid >> 6] = lo;
        red_hi[tid >> 6] = hi;
    }
    __syncthreads();
    lo = red_lo[0];
    hi = red_hi[0];
#pragma unroll
    for (int v = 1; v < kTkWaves; ++v) {
        lo = min(lo, red_lo[v]);
        hi = max(hi, red_hi[v]);
    }

    // ---- 2. narrow [lo, hi] to the single key value of the k-th largest
    uint32_t need = (uint32_t)k;  // still to take from keys inside [lo, hi]
    while (lo != hi) {
        const uint32_t range = hi - lo;
        int shift = 0;
        while ((range >> shift) >= (uint32_t)kTkBins) ++shift;
        const int nb = (int)(range >> shift) + 1;
        for (int j = tid; j < nb; j += kTkThreads) hist[j] = 0u;
        __syncthreads();
        for (int p = tid; p < n; p += kTkThreads) {
            const uint32_t u = ordered_key(row[p]);
            if (u >= lo && u <= hi) atomicAdd(&hist[(u - lo) >> shift], 1u);
        }
        __syncthreads();
        if (tid < 64) {  // one wave scans the bins from the top
            uint32_t above = 0u;
            int top = nb - 1;
            bool done = false;
            while (!done && top >= 0) {
                const int j = top - tid;
                uint32_t c = j >= 0 ? hist[j] : 0u;
                // inclusive scan over lanes (lane 0 = highest bin)
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t o = (uint32_t)__shfl_up((int)c, off, 64);
                    if (tid >= off) c += o;
                }
                const uint32_t incl = above + c;
                const uint64_t hit = __ballot(j >= 0 && incl >= need);
                if (hit) {
                    const int first = __builtin_ctzll(hit);
                    if (tid == first) {
                        found_bin = (uint32_t)j;
                        found_above = incl - hist[j];
                    }
                    done = true;
                } else {
                    above += (uint32_t)__shfl((int)c, 63, 64);
                    top -= 64;
                }
            }
        }
        __syncthreads();
        const uint32_t bin = found_bin;
        need -= found_above;
        const uint32_t new_lo = lo + (bin << shift);
        const uint32_t width_m1 = (shift >= 32) ? 0xffffffffu : ((1u << shift) - 1u);
        const uint32_t new_hi = (hi - new_lo > width_m1) ? new_lo + width_m1 : hi;
        lo = new_lo;
        hi = new_hi;
        __syncthreads();
    }
    const uint32_t tau = lo;

    // ---- 3. ordered compaction: all keys > tau, plus the first `need` ties
    uint32_t written = 0u, ties_seen = 0u;
    for (int base = 0; base < n; base += kTkThreads) {
        const int p = base + tid;
        const uint32_t u = p < n ? ordered_key(row[p]) : 0u;
        const bool gt = p < n && u > tau;
        const bool eq = p < n && u == tau;
        uint32_t eq_total;
        const uint32_t eq_rank = block_flag_scan(eq, scan_scratch, eq_total);
        const bool take = gt || (eq && ties_seen + eq_rank < need);
        uint32_t take_total;
        const uint32_t slot = block_flag_scan(take, scan_scratch, take_total);
        if (take) out[written + slot] = p;
        written += take_total;
        ties_seen += eq_total;
    }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_topk(const float *scores, size_t batch_stride, const int32_t *q_pos, int B,
                       int T, int S, int row0, int rows, int k, int32_t *idx, void *,
                       hipStream_t stream) {
    dim3 grid(rows, B);
    hipLaunchKernelGGL(topk_row_kernel, grid, dim3(kTkThreads), 0, stream, scores, batch_stride,
                       q_pos, T, S, row0, k, idx);
    return hipGetLastError();
}

}  // namespace dsa
