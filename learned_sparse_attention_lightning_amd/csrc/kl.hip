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
#include "kl_schedule.h"

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

// kl_push when `take`, else no change, without a branch: a value loaded
// for a pair that only a branch consumed could be moved into that branch,
// i.e. next to its use, where its memory latency is no longer hidden.
__device__ __forceinline__ void kl_push_if(KlState &st, bool take, float p, float I) {
    const bool first = st.m == -INFINITY;
    const float mn = fmaxf(st.m, I);
    const float zr = first ? 0.f : st.z * __expf(st.m - mn);
    const float bshift = first ? 0.f : st.P * (mn - st.m);
    const float plogp = p > 0.f ? p * __logf(p) : 0.f;
    const KlState nx = {mn, zr + __expf(I - mn), st.P + p, st.A + plogp,
                        st.Bd - bshift + p * (I - mn)};
    st.m = take ? nx.m : st.m;
    st.z = take ? nx.z : st.z;
    st.P = take ? nx.P : st.P;
    st.A = take ? nx.A : st.A;
    st.Bd = take ? nx.Bd : st.Bd;
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

// MHA masked-dense form (bf16, d_qk 64 or 128, 8 or 16 heads, a selection
// that covers a large share of the causal prefix): the target p_s of every
// key of the causal area is computed on the matrix cores and the bitmap of
// the selection decides which keys enter the loss.  Workgroup = 32 query
// rows x one range of 256 keys (a split) x every head: wave w multiplies
// heads HPW w .. HPW w + HPW-1 (their query fragments in registers, B
// operand) with the key rows of one 32-key tile at a time (A operand; each
// head-tile's rows are loaded with whole-row 16-byte pieces into one of two
// register sets, which is refilled two head-tiles ahead as soon as it has
// passed through a wave-private LDS tile into the operand layout),
// and adds exp2(S^T scale log2e - lse_h log2e) over its heads; the eight
// waves' sums meet in LDS (one barrier a tile, two buffers), where each
// thread takes 2 (key, query) pairs and folds the selected ones into its
// running KL state.  The splits of a row are merged by a second kernel.
// Each key range is taken by one XCD (the workgroup order is described in
// the kernel), so its keys stay in that XCD's L2.
constexpr int kDkWaves = 8;
constexpr int kDkThreads = kDkWaves * kWave;
constexpr int kDkQ = kl::kQ;                  // query rows per workgroup
constexpr int kDkKeys = kl::kKeys;            // keys per tile
constexpr int kDkSplitTiles = kl::kSplitTiles;  // tiles per split (256 keys)
constexpr int kDkRing = 2;          // register sets of key fragments (loads two head-tiles ahead)
constexpr int kDkAhead = 3;         // tiles whose scores and selection words are in flight

__device__ __forceinline__ __amdgpu_buffer_rsrc_t kl_buffer(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int D, int HPW>
__global__ __launch_bounds__(kDkThreads, 1) void mha_kl_dense_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint32_t *__restrict__ bits, const int32_t *__restrict__ row_hi,
    const float *__restrict__ lse, const float *__restrict__ scores, int T, int S, float scale,
    int nqb, int nsplit, int per_xcd, KlState *__restrict__ part) {
    constexpr int H = kDkWaves * HPW;
    constexpr int KS = D / 16;  // 16-dim k-steps
    constexpr int P = D / 8;                 // 16-byte pieces of a key's head row
    constexpr int NL = kDkKeys * P / kWave;  // loads of a head-tile per lane
    constexpr int kPitch = D * 2 + 16;       // LDS row pitch: rows 4 banks apart
    __shared__ float red[2][kDkWaves][16][kWave];  // per-wave sums of a tile, two buffers
    __shared__ KlState fin[kDkWaves][kDkQ];
    __shared__ __align__(16) uint8_t ktile[kDkWaves][kDkKeys * kPitch];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    // workgroup -> (batch, key split, query block): each XCD keeps its own
    // key ranges in its L2 with equal shares of the causal triangle, the
    // causal pairs first in runs, longest first (kl_schedule.h)
    const kl::Work wk = kl::work_of(blockIdx.x, T, S, nqb, nsplit, per_xcd);
    if (wk.split < 0) return;  // past this XCD's share
    const int b = wk.b, split = wk.split, qb = wk.qb;
    const int words = (S + 31) / 32;
    const int my_r = qb * kDkQ + l32;  // this lane's query row (queries are lanes mod 32)
    const bool live = my_r < T;
    const int rr = live ? my_r : T - 1;
    const size_t row = (size_t)b * T + rr;
    int hi = live ? row_hi[row] : -1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hi = max(hi, __shfl_xor(hi, off, 64));
    hi = __builtin_amdgcn_readfirstlane(hi);  // equal in every lane: keep it scalar
    const int ntiles = hi < 0 ? 0 : hi / kDkKeys + 1;  // the same in every wave
    const int t0 = split * kDkSplitTiles;
    const int t1 = min(ntiles, t0 + kDkSplitTiles);
    const int njt = t1 > t0 ? (t1 - t0) * HPW : 0;  // head-tiles of this wave
    if (njt == 0) {  // nothing selected in the split by any row of the block
        if (wave == 0 && half == 0 && live)
            part[row * nsplit + split] = KlState{-INFINITY, 0.f, 0.f, 0.f, 0.f};
        return;
    }

    constexpr float kLog2e = 1.4426950408889634f;
    const float c1 = scale * kLog2e;
    // query fragments (B operand): lane (query l32, half) holds dims 16 ks + 8 half .. +8
    bf16x8 qf[HPW][KS];
    float lse2[HPW];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        const uint16_t *qp = q + (row * H + wave * HPW + h) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[h][ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
        lse2[h] = lse[row * H + wave * HPW + h] * kLog2e;
    }
    // key rows of head-tile j (head wave*HPW + j%HPW): load i of a lane is
    // piece q % P of tile key q / P, q = 64 i + lane, so one instruction reads
    // whole rows.  Buffer loads over this batch's keys: the lane's offset is
    // fixed, the tile, head and load index only move the scalar offset, and
    // keys past the cache read as zeros (never selected).
    constexpr uint32_t kRow = (uint32_t)H * D * 2;  // bytes of one key (every head)
    const __amdgpu_buffer_rsrc_t krs = kl_buffer(K + (size_t)b * S * H * D, (uint32_t)S * kRow);
    const uint32_t kvoff = (uint32_t)(lane / P) * kRow + 16u * (uint32_t)(lane % P);
    auto load_kt = [&](int j, u32x4 (&dst)[NL]) {
        const uint32_t t = (uint32_t)(t0 + j / HPW);
        const uint32_t hh = (uint32_t)(wave * HPW + j % HPW);
        const uint32_t base = t * kDkKeys * kRow + hh * D * 2;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            dst[i] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           krs, kvoff, base + (uint32_t)i * (kWave / P) * kRow, 0));
    };
    // through the wave's LDS tile into the A operand: lane (key l32, half)
    // holds dims 16 ks + 8 half .. +8 (reads 4 banks apart a row: no conflict)
    uint8_t *kt = ktile[wave];
    auto to_operand = [&](const u32x4 (&src)[NL], bf16x8 (&af)[KS]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int qq = kWave * i + lane;
            *reinterpret_cast<u32x4 *>(kt + (qq / P) * kPitch + 16 * (qq % P)) = src[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            af[ks] = *reinterpret_cast<const bf16x8 *>(kt + l32 * kPitch + (16 * ks + 8 * half) * 2);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // the next head-tile's writes come after these reads
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // the pairs this thread folds: lane L = `lane`, registers 2 wave, 2 wave + 1
    // of every wave's tile sums: query l32, keys kin and kin + 1 of the tile
    const int kin = 8 * (wave >> 1) + 4 * half + 2 * (wave & 1);
    // scores and selection words of the block's rows, over buffers that end
    // at the block's last row (lanes past it read zeros)
    const size_t brow0 = (size_t)b * T + (size_t)qb * kDkQ;
    const uint32_t brows = (uint32_t)min(kDkQ, T - qb * kDkQ);
    const __amdgpu_buffer_rsrc_t srs = kl_buffer(scores + brow0 * S, brows * (uint32_t)S * 4u);
    const __amdgpu_buffer_rsrc_t brs = kl_buffer(bits + brow0 * words, brows * (uint32_t)words * 4u);
    const uint32_t svoff = ((uint32_t)l32 * (uint32_t)S + (uint32_t)kin) * 4u;
    const uint32_t bvoff = (uint32_t)l32 * (uint32_t)words * 4u;
    KlState st = {-INFINITY, 0.f, 0.f, 0.f, 0.f};
    u32x4 kr[kDkRing][NL];
    f32x16 pacc = {};
    // Scores and selection words of this thread's pairs, TPB tiles ahead: the
    // scores come from memory once, so their latency is the longest of the
    // loop's.  The split's tiles are unrolled completely, so every ring slot
    // is a fixed register set: no copies of registers with loads in flight
    // (such a copy waits for every load issued before it).
    constexpr int TPB = kDkAhead;
    float isc[TPB][2];
    uint32_t ibw[TPB];
    auto fetch_pairs = [&](int slot, int t) {
        const uint32_t so = (uint32_t)t * kDkKeys * 4u;
        ibw[slot] = __builtin_amdgcn_raw_buffer_load_b32(brs, bvoff, (uint32_t)t * 4u, 0);
        isc[slot][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, svoff, so, 0));
        isc[slot][1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, svoff + 4u, so, 0));
    };
    // A split shorter than kDkSplitTiles tiles (the diagonal one) computes
    // its last head-tile again in place of the missing ones and does not
    // fold them: every load and barrier of the unrolled tiles is then
    // unconditional, so the wait for one head-tile's fragments counts only
    // the loads issued before them.
    auto tile_done = [&](int t, bool valid, int slot) {
        const int par = t & 1;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) red[par][wave][rg][lane] = pacc[rg];
        pacc = f32x16{};
        const uint32_t bw = ibw[slot];
        const float i0 = isc[slot][0], i1 = isc[slot][1];
        fetch_pairs(slot, min(t + TPB, t1 - 1));
        lds_barrier();
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int v = 0; v < kDkWaves; ++v) {
            s0 += red[par][v][2 * wave][lane];
            s1 += red[par][v][2 * wave + 1][lane];
        }
        const bool fold = valid && live;
        kl_push_if(st, fold && ((bw >> kin) & 1u), s0 * (1.0f / H), i0);
        kl_push_if(st, fold && ((bw >> (kin + 1)) & 1u), s1 * (1.0f / H), i1);
    };
    if (njt > 0) {  // uniform over the workgroup
#pragma unroll
        for (int i = 0; i < TPB; ++i) fetch_pairs(i, min(t0 + i, t1 - 1));
        load_kt(0, kr[0]);
        load_kt(min(1, njt - 1), kr[1]);
        // Head-tile j's products go to acc[j & 1] and its exponentials are
        // taken after head-tile j+1's products are issued: the matrix cores
        // and the VALU work on different head-tiles.
        constexpr int NJ = kDkSplitTiles * HPW;
        f32x16 acc[2];
        auto products = [&](int j) {
            bf16x8 af[KS];
            to_operand(kr[j % kDkRing], af);
            load_kt(min(j + 2, njt - 1), kr[j % kDkRing]);
            f32x16 a = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qf[j % HPW][ks], a, 0, 0, 0);
            acc[j & 1] = a;
        };
        auto weights = [&](int j) {
            const int h = j % HPW;
#pragma unroll
            for (int rg = 0; rg < 16; ++rg)
                pacc[rg] += __builtin_amdgcn_exp2f(fmaf(acc[j & 1][rg], c1, -lse2[h]));
            if (h == HPW - 1) tile_done(t0 + min(j, njt - 1) / HPW, j < njt, (j / HPW) % TPB);
        };
        products(0);
#pragma unroll
        for (int j = 1; j < NJ; ++j) {
            products(j);
            weights(j - 1);
        }
        weights(NJ - 1);
    }
    // this row's state: lanes l32 and l32 + 32 of every wave hold parts of it
    st = kl_merge(st, kl_shfl_xor(st, 32));
    if (half == 0) fin[wave][l32] = st;
    __syncthreads();
    if (wave == 0 && half == 0 && live) {
        KlState r = fin[0][l32];
#pragma unroll
        for (int v = 1; v < kDkWaves; ++v) r = kl_merge(r, fin[v][l32]);
        part[row * nsplit + split] = r;
    }
}

// Loss of each row from the states of its splits.
__global__ __launch_bounds__(256) void kl_split_merge_kernel(const KlState *__restrict__ part,
                                                             int rows, int nsplit,
                                                             float *__restrict__ loss) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    KlState m = part[(size_t)r * nsplit];
    for (int s = 1; s < nsplit; ++s) m = kl_merge(m, part[(size_t)r * nsplit + s]);
    loss[r] = m.P > 0.f ? m.A / m.P - __logf(m.P) - m.Bd / m.P + __logf(m.z) : 0.f;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The masked-dense form: bf16, d_qk 64 or 128, 8 or 16 heads, S within the
// bitmap's reach, and a selection of at least a quarter of the keys.
bool kl_dense_path(const dsa_attn_desc_t &d, int S, int k) {
    return d.form == DSA_MHA && d.dtype == DSA_BF16 && (d.d_qk == 64 || d.d_qk == 128) &&
           (d.num_heads == 8 || d.num_heads == 16) && S <= 65536 && 4LL * k >= (long long)S;
}

int kl_splits(int S) { return kl::splits_of(S); }

}  // namespace

size_t kl_workspace_bytes(const dsa_attn_desc_t &d, int B, int T, int S, int k) {
    if (!kl_dense_path(d, S, k)) return 0;
    const size_t rows = (size_t)B * T;
    const size_t words = (size_t)(S + 31) / 32;
    return align256(rows * words * 4) + align256(rows * 4) +
           align256(rows * kl_splits(S) * sizeof(KlState));
}

bool indexer_kl_supported(const dsa_attn_desc_t &d) {
    if (d.form == DSA_MHA)
        return (d.dtype == DSA_BF16 || d.dtype == DSA_F32) && (d.d_qk == 64 || d.d_qk == 128) &&
               d.num_heads <= kMhaKlMaxH;
    return d.form == DSA_MLA && d.dtype == DSA_BF16 && d.d_qk == kKlDqk &&
           (d.num_heads == 32 || d.num_heads == 64 || d.num_heads == 128);
}

hipError_t launch_indexer_kl(const dsa_attn_desc_t &d, const void *q, const void *kv,
                             const int32_t *idx, const float *lse, const float *scores, int B,
                             int T, int S, int k, float *loss, void *workspace,
                             hipStream_t stream) {
    const dim3 grid(T, B);
    if (workspace && kl_dense_path(d, S, k)) {
        const size_t rows = (size_t)B * T;
        const size_t words = (size_t)(S + 31) / 32;
        char *ws = static_cast<char *>(workspace);
        uint32_t *bits = reinterpret_cast<uint32_t *>(ws);
        int32_t *row_hi = reinterpret_cast<int32_t *>(ws + align256(rows * words * 4));
        KlState *part = reinterpret_cast<KlState *>(ws + align256(rows * words * 4) +
                                                    align256(rows * 4));
        hipError_t e = launch_selection_bitmap(idx, B, T, S, 0, T, k, bits, row_hi, stream);
        if (e != hipSuccess) return e;
        const int nqb = kl::blocks_of(T);
        const int nsplit = kl_splits(S);
        const int per_xcd = kl::per_xcd(nqb, nsplit);
        const dim3 g((unsigned)((long long)B * per_xcd * kl::kXcds));
        const uint16_t *qq = static_cast<const uint16_t *>(q);
        const uint16_t *kk = static_cast<const uint16_t *>(kv);
        if (d.d_qk == 128 && d.num_heads == 16)
            hipLaunchKernelGGL((mha_kl_dense_kernel<128, 2>), g, dim3(kDkThreads), 0, stream, qq,
                               kk, bits, row_hi, lse, scores, T, S, d.scale, nqb, nsplit, per_xcd, part);
        else if (d.d_qk == 128)
            hipLaunchKernelGGL((mha_kl_dense_kernel<128, 1>), g, dim3(kDkThreads), 0, stream, qq,
                               kk, bits, row_hi, lse, scores, T, S, d.scale, nqb, nsplit, per_xcd, part);
        else if (d.num_heads == 16)
            hipLaunchKernelGGL((mha_kl_dense_kernel<64, 2>), g, dim3(kDkThreads), 0, stream, qq,
                               kk, bits, row_hi, lse, scores, T, S, d.scale, nqb, nsplit, per_xcd, part);
        else
            hipLaunchKernelGGL((mha_kl_dense_kernel<64, 1>), g, dim3(kDkThreads), 0, stream, qq,
                               kk, bits, row_hi, lse, scores, T, S, d.scale, nqb, nsplit, per_xcd, part);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kl_split_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256),
                           0, stream, part, (int)rows, nsplit, loss);
        return hipGetLastError();
    }
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
