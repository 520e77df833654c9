// kl.hip -- forward value of the indexer's distillation loss over a selected
// set ("DeepSeek Sparse Attention: Learned Token Selection from Scratch",
// sections 5.2-5.4 and 6.2), MLA latent form and MHA form.
//
// For query row t with selected set S_t and per-head log-sum-exp lse_h of
// the scaled logits over S_t (what the attention step writes), the target is
// the head mean of the attention weights,
//   p_s = (1/H) sum_h exp(scale * q_h . c_s - lse_h),   s in S_t,
// and the loss is KL(p || softmax over S_t of I[t,s]).  The logits are
// recomputed on the matrix cores (the QK half of the attention; the value
// products are not needed), summed over heads in registers, and each lane
// folds the entries it owns into a running (max, sum-exp, sums) state.
#include <math.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kKlWaves = 4;
constexpr int kKlThreads = kKlWaves * kWave;
constexpr int kKlDqk = 576;                    // latent row: key width
constexpr int kKlSteps = kKlDqk / 16;          // 32x32x16 products per head/entry tile
constexpr int kKlGroup = 9;                    // k-steps per prefetch group
constexpr int kKlGroups = kKlSteps / kKlGroup;
constexpr int kKlPieces = kKlDqk * 2 / 16;     // 16-byte pieces of one query row
// Query rows in LDS with a 16-byte pad: the 16 lanes of one 16-byte read
// phase start 36 dwords apart (mod 64 banks), so no two share a bank.
constexpr int kQPitch = kKlDqk * 2 + 16;
static_assert(kKlSteps % kKlGroup == 0, "prefetch groups must tile the key width");

// Per-lane running state of one row's divergence terms over the entries the
// lane owns: m = max I, z = sum exp(I - m), P = sum p, A = sum p log p,
// Bd = sum p (I - m).
struct KlState {
    float m, z, P, A, Bd;
};

__device__ __forceinline__ void kl_push(KlState &st, float p, float I) {
    if (I > st.m) {  // new maximum: rebase the sums taken against the old one
        if (st.m != -INFINITY) {
            st.z *= __expf(st.m - I);
            st.Bd -= st.P * (I - st.m);
        }
        st.m = I;
    }
    st.z += __expf(I - st.m);
    st.P += p;
    if (p > 0.f) st.A += p * __logf(p);
    st.Bd += p * (I - st.m);
}

__device__ __forceinline__ KlState kl_merge(KlState a, KlState b) {
    if (b.m == -INFINITY) return a;
    if (a.m == -INFINITY) return b;
    KlState r;
    r.m = fmaxf(a.m, b.m);
    r.z = a.z * __expf(a.m - r.m) + b.z * __expf(b.m - r.m);
    r.P = a.P + b.P;
    r.A = a.A + b.A;
    r.Bd = a.Bd - a.P * (r.m - a.m) + b.Bd - b.P * (r.m - b.m);
    return r;
}

__device__ __forceinline__ float load_as_float(const float *p) { return *p; }
__device__ __forceinline__ float load_as_float(const uint16_t *p) {
    return __uint_as_float((uint32_t)*p << 16);
}
// 16 bytes of keys to fp32: four floats or eight bf16
__device__ __forceinline__ void unpack16(u32x4 raw, float (&out)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(raw[j]);
}
__device__ __forceinline__ void unpack16(u32x4 raw, float (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[2 * j] = __uint_as_float(raw[j] << 16);
        out[2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ KlState kl_shfl_xor(KlState s, int mask) {
    return {__shfl_xor(s.m, mask), __shfl_xor(s.z, mask), __shfl_xor(s.P, mask),
            __shfl_xor(s.A, mask), __shfl_xor(s.Bd, mask)};
}

// One workgroup per query row (grid x = row in launch, y = batch).  The
// row's query block (H x 576 bf16) sits in LDS; each wave takes pairs of
// 32-entry tiles: per 16-wide k-step it gathers the two tiles' key pieces
// from memory (one 16-byte load per lane and tile, a group ahead) and
// multiplies them with the HT head tiles read from LDS.
template <int HT>
__global__ __launch_bounds__(kKlThreads, 1) void mla_indexer_kl_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const float *__restrict__ lse,
    const float *__restrict__ scores, int T, int S, int k, float scale,
    float *__restrict__ loss) {
    constexpr int H = 32 * HT;
    __shared__ __attribute__((aligned(16))) unsigned char qs[H * kQPitch];
    __shared__ __attribute__((aligned(16))) float lse2[H];
    __shared__ KlState red[kKlWaves];

    const int i = blockIdx.x, b = blockIdx.y;
    const size_t row = (size_t)b * T + i;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, half = lane >> 5;
    constexpr float kLog2e = 1.4426950408889634f;

    const uint16_t *qrow = q + row * (size_t)H * kKlDqk;
    {  // every load of the query block in flight before the first LDS write
        constexpr int kQIters = H * kKlPieces / kKlThreads;
        static_assert(H * kKlPieces % kKlThreads == 0, "query pieces must tile the workgroup");
        u32x4 qv[kQIters];
#pragma unroll
        for (int it = 0; it < kQIters; ++it) {
            const int p = tid + it * kKlThreads;
            const int h = p / kKlPieces, c = p - h * kKlPieces;
            qv[it] = *reinterpret_cast<const u32x4 *>(qrow + (size_t)h * kKlDqk + c * 8);
        }
#pragma unroll
        for (int it = 0; it < kQIters; ++it) {
            const int p = tid + it * kKlThreads;
            const int h = p / kKlPieces, c = p - h * kKlPieces;
            *reinterpret_cast<u32x4 *>(qs + h * kQPitch + c * 16) = qv[it];
        }
    }
    for (int h = tid; h < H; h += kKlThreads) lse2[h] = lse[row * H + h] * kLog2e;
    __syncthreads();

    const float c1 = scale * kLog2e;
    const int32_t *sel = idx + row * (size_t)k;
    const float *irow = scores + row * (size_t)S;
    const char *kbase = reinterpret_cast<const char *>(kv + (size_t)b * S * kKlDqk) + half * 16;
    KlState st = {-INFINITY, 0.f, 0.f, 0.f, 0.f};

    const int npairs = (k + 63) / 64;
    auto sel_at = [&](int e) -> int { return e < k ? sel[e] : -1; };
    auto kptr = [&](int s) { return kbase + (size_t)(s < 0 ? 0 : s) * (kKlDqk * 2); };
    bf16x8 bg[2][kKlGroup][2];
    auto load_group = [&](bf16x8 (&dst)[kKlGroup][2], const char *p0, const char *p1, int g) {
#pragma unroll
        for (int j = 0; j < kKlGroup; ++j) {
            dst[j][0] = *reinterpret_cast<const bf16x8 *>(p0 + (g * kKlGroup + j) * 32);
            dst[j][1] = *reinterpret_cast<const bf16x8 *>(p1 + (g * kKlGroup + j) * 32);
        }
    };
    // the selection of a wave's next pair is in flight while the current pair
    // is multiplied
    int pr = wave;
    int s0 = -1, s1 = -1, sme = -1;
    if (pr < npairs) {
        s0 = sel_at(pr * 64 + n);
        s1 = sel_at(pr * 64 + 32 + n);
        sme = sel_at(pr * 64 + lane);
    }
    for (; pr < npairs; pr += kKlWaves) {
        const int nx = pr + kKlWaves;
        int s0n = -1, s1n = -1, smen = -1;
        if (nx < npairs) {
            s0n = sel_at(nx * 64 + n);
            s1n = sel_at(nx * 64 + 32 + n);
            smen = sel_at(nx * 64 + lane);
        }
        const char *k0 = kptr(s0), *k1 = kptr(s1);
        if (__ballot(sme >= 0) == 0) {  // the whole pair is unused
            s0 = s0n, s1 = s1n, sme = smen;
            continue;
        }
        const float Ime = sme >= 0 ? irow[sme] : 0.f;
        load_group(bg[0], k0, k1, 0);

        f32x16 acc[HT][2];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht][0] = acc[ht][1] = f32x16{};
#pragma unroll
        for (int g = 0; g < kKlGroups; ++g) {
            if (g + 1 < kKlGroups) load_group(bg[(g + 1) & 1], k0, k1, g + 1);
#pragma unroll
            for (int j = 0; j < kKlGroup; ++j) {
                const int ks = g * kKlGroup + j;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        qs + (ht * 32 + n) * kQPitch + ks * 32 + half * 16);
                    acc[ht][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bg[g & 1][j][0],
                                                                        acc[ht][0], 0, 0, 0);
                    acc[ht][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bg[g & 1][j][1],
                                                                        acc[ht][1], 0, 0, 0);
                }
            }
        }

        // acc[ht][e][j]: head ht*32 + 8*(j/4) + 4*half + j%4, entry e*32 + n
        float pa0 = 0.f, pa1 = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lse2[ht * 32 + 8 * jj + 4 * half]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pa0 += exp2f(fmaf(acc[ht][0][4 * jj + r], c1, -l4[r]));
                    pa1 += exp2f(fmaf(acc[ht][1][4 * jj + r], c1, -l4[r]));
                }
            }
        }
        // lanes 0-31 finish entry n of tile 0, lanes 32-63 entry n of tile 1
        const float recv = __shfl_xor(half ? pa0 : pa1, 32);
        const float p = ((half ? pa1 : pa0) + recv) * (1.0f / H);
        if (sme >= 0) kl_push(st, p, Ime);
        s0 = s0n, s1 = s1n, sme = smen;
    }

#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) st = kl_merge(st, kl_shfl_xor(st, mask));
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0) {
        KlState r = red[0];
        for (int w = 1; w < kKlWaves; ++w) r = kl_merge(r, red[w]);
        // sum over S_t of (p/P) (log(p/P) - I + log sum exp I)
        loss[row] = r.P > 0.f ? r.A / r.P - __logf(r.P) - r.Bd / r.P + __logf(r.z) : 0.f;
    }
}


// MHA form: every head has its own key row, so the logits are 2-operand dot
// products per (entry, head) rather than one shared-operand product.  One
// workgroup per query row, one lane per selected entry: the lane streams its
// entry's H key rows (16-byte loads) against the query block, broadcast from
// LDS as fp32, and sums exp(scale q_h.K[s,h] - lse_h) over the heads.
constexpr int kMhaKlThreads = 256;
constexpr int kMhaKlMaxH = 64;
constexpr int kMhaKlMaxD = 128;

template <typename Tin>
__global__ __launch_bounds__(kMhaKlThreads) void mha_indexer_kl_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ K, const int32_t *__restrict__ idx,
    const float *__restrict__ lse, const float *__restrict__ scores, int T, int S, int H, int D,
    int k, float scale, float *__restrict__ loss) {
    __shared__ __attribute__((aligned(16))) float qf[kMhaKlMaxH * kMhaKlMaxD];
    __shared__ float lse2[kMhaKlMaxH];
    __shared__ KlState red[kMhaKlThreads / kWave];
    const int i = blockIdx.x, b = blockIdx.y;
    const size_t row = (size_t)b * T + i;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int kPer = 16 / sizeof(Tin);  // elements per 16-byte load

    const Tin *qrow = q + row * (size_t)H * D;
    for (int e = tid; e < H * D; e += kMhaKlThreads) qf[e] = load_as_float(qrow + e);
    for (int h = tid; h < H; h += kMhaKlThreads) lse2[h] = lse[row * H + h] * kLog2e;
    __syncthreads();

    const float c1 = scale * kLog2e;
    const int32_t *sel = idx + row * (size_t)k;
    const float *irow = scores + row * (size_t)S;
    KlState st = {-INFINITY, 0.f, 0.f, 0.f, 0.f};
    for (int e = tid; e < k; e += kMhaKlThreads) {
        const int s = sel[e];
        if (s < 0) continue;
        const Tin *krow = K + ((size_t)b * S + s) * (size_t)H * D;
        float pacc = 0.f;
        for (int h = 0; h < H; ++h) {
            const Tin *kh = krow + (size_t)h * D;
            const float *qh = qf + h * D;
            float dot = 0.f;
            for (int d0 = 0; d0 < D; d0 += kPer) {
                const u32x4 raw = *reinterpret_cast<const u32x4 *>(kh + d0);
                float kv[kPer];
                unpack16(raw, kv);
#pragma unroll
                for (int j = 0; j < kPer; ++j) dot = fmaf(qh[d0 + j], kv[j], dot);
            }
            pacc += exp2f(fmaf(dot, c1, -lse2[h]));
        }
        kl_push(st, pacc / (float)H, irow[s]);
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) st = kl_merge(st, kl_shfl_xor(st, mask));
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0) {
        KlState r = red[0];
        for (int w = 1; w < kMhaKlThreads / kWave; ++w) r = kl_merge(r, red[w]);
        loss[row] = r.P > 0.f ? r.A / r.P - __logf(r.P) - r.Bd / r.P + __logf(r.z) : 0.f;
    }
}

}  // namespace

bool indexer_kl_supported(const dsa_attn_desc_t &d) {
    if (d.form == DSA_MHA)
        return (d.dtype == DSA_BF16 || d.dtype == DSA_F32) && (d.d_qk == 64 || d.d_qk == 128) &&
               d.num_heads <= kMhaKlMaxH;
    return d.form == DSA_MLA && d.dtype == DSA_BF16 && d.d_qk == kKlDqk &&
           (d.num_heads == 32 || d.num_heads == 64 || d.num_heads == 128);
}

hipError_t launch_indexer_kl(const dsa_attn_desc_t &d, const void *q, const void *kv,
                             const int32_t *idx, const float *lse, const float *scores, int B,
                             int T, int S, int k, float *loss, hipStream_t stream) {
    const dim3 grid(T, B);
    if (d.form == DSA_MHA) {
        if (d.dtype == DSA_BF16)
            hipLaunchKernelGGL(mha_indexer_kl_kernel<uint16_t>, grid, dim3(kMhaKlThreads), 0,
                               stream, static_cast<const uint16_t *>(q),
                               static_cast<const uint16_t *>(kv), idx, lse, scores, T, S,
                               d.num_heads, d.d_qk, k, d.scale, loss);
        else
            hipLaunchKernelGGL(mha_indexer_kl_kernel<float>, grid, dim3(kMhaKlThreads), 0,
                               stream, static_cast<const float *>(q),
                               static_cast<const float *>(kv), idx, lse, scores, T, S,
                               d.num_heads, d.d_qk, k, d.scale, loss);
        return hipGetLastError();
    }
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(kv);
    switch (d.num_heads) {
        case 32:
            hipLaunchKernelGGL(mla_indexer_kl_kernel<1>, grid, dim3(kKlThreads), 0, stream, qq,
                               kk, idx, lse, scores, T, S, k, d.scale, loss);
            break;
        case 64:
            hipLaunchKernelGGL(mla_indexer_kl_kernel<2>, grid, dim3(kKlThreads), 0, stream, qq,
                               kk, idx, lse, scores, T, S, k, d.scale, loss);
            break;
        default:
            hipLaunchKernelGGL(mla_indexer_kl_kernel<4>, grid, dim3(kKlThreads), 0, stream, qq,
                               kk, idx, lse, scores, T, S, k, d.scale, loss);
            break;
    }
    return hipGetLastError();
}

}  // namespace dsa
