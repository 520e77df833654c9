// attention_mha.hip -- MHA-form sparse attention on gfx950 matrix cores, for
// dense selections (prefill, k a large share of the causal prefix).
//
//   out[t,h] = sum_{s in S_t} softmax_s( scale * q[t,h] . K[s,h] ) V[s,h]
// ("DeepSeek Sparse Attention: Learned Token Selection from Scratch",
// sections 3.3 and 10.1; per-head K and V rows, one selected set S_t per query
// shared by every head).  When k is a large fraction of the t+1 candidates
// the page notes that the masked-dense form does little extra work
// (section 9.3): here every (32-query block, 32-key tile) of the causal area
// up to the block's last selected key is computed with MFMA and the
// probabilities of unselected keys are forced to 0, which gives exactly the
// softmax over S_t.
//
//   mha_bitmap_kernel  idx -> one bit per (row, key) and the row's largest
//                      selected position
//   mha_dense_kernel   one wave = 32 query rows x one head:
//       S^T = K(32 keys) . Q^T(32 queries) over d (v_mfma_f32_32x32x16_bf16,
//       the query block in registers as the B operand), bitmap mask, online
//       softmax in fp32 per query lane (lazy reference max), P (bf16) to LDS,
//       O[32 queries, d] += P . V with V read by the LDS transpose read.
//       Waves are independent (no workgroup barriers); the next tile's K and V
//       are loaded into registers while the current one is multiplied.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kQb = 32;            // query rows per wave
constexpr int kKt = 32;            // keys per tile
constexpr int kMaxS = 65536;       // bitmap row of a row kept in LDS (8 KB)
constexpr float kRescaleLog2 = 8.0f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct MhaTile {
    static constexpr int row_bytes = D * 2;
    // K: pitch = odd multiple of 16 bytes -> the 16 rows read by 16 lanes
    // (b128 operand reads) start on 16 different bank groups.
    static constexpr int k_pitch = row_bytes + 16;
    // V: pitch = row + 64 bytes (a 16-dword bank shift) -> the 4 rows of one
    // transpose read, and the two 16-lane groups served together, hit
    // disjoint banks.
    static constexpr int v_pitch = row_bytes + 64;
    static constexpr int pieces = row_bytes / 16;         // 16-byte pieces a row
    static constexpr int loads = kKt * pieces / 64;       // wave loads a tile (K or V)
    static constexpr int p_pitch = kKt * 2 + 16;          // P row [query][key] bf16
    static constexpr int k_bytes = kKt * k_pitch;         // also holds P
    static constexpr int v_bytes = kKt * v_pitch;
    static_assert(kKt * p_pitch <= k_bytes, "P fits the K tile");
};

__global__ __launch_bounds__(256) void mha_bitmap_kernel(const int32_t *__restrict__ idx, int T,
                                                         int S, int row0, int rows, int k,
                                                         uint32_t *__restrict__ bits,
                                                         int32_t *__restrict__ row_hi) {
    __shared__ uint32_t w[kMaxS / 32];
    __shared__ int hi_s;
    const int r = blockIdx.x, b = blockIdx.y;
    const int words = (S + 31) / 32;
    for (int j = threadIdx.x; j < words; j += 256) w[j] = 0u;
    if (threadIdx.x == 0) hi_s = -1;
    __syncthreads();
    const int32_t *sel = idx + ((size_t)b * T + row0 + r) * k;
    int hi = -1;
    for (int e = threadIdx.x; e < k; e += 256) {
        const int s = sel[e];
        if (s >= 0 && s < S) {
            atomicOr(&w[s >> 5], 1u << (s & 31));
            hi = max(hi, s);
        }
    }
    atomicMax(&hi_s, hi);
    __syncthreads();
    uint32_t *out = bits + ((size_t)b * rows + r) * words;
    for (int j = threadIdx.x; j < words; j += 256) out[j] = w[j];
    if (threadIdx.x == 0) row_hi[(size_t)b * rows + r] = hi_s;
}

template <typename Tout>
__device__ __forceinline__ void mha_store(Tout *p, float v);
template <>
__device__ __forceinline__ void mha_store<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void mha_store<uint16_t>(uint16_t *p, float v) {
    *p = (uint16_t)f32_to_bf16_bits(v);
}

// grid: 1-D over (batch, query block, head) in units of 4 waves
template <int D, typename Tout>
__global__ __launch_bounds__(256, 2) void mha_dense_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const uint32_t *__restrict__ bits,
    const int32_t *__restrict__ row_hi, int T, int S, int H, float scale, int row0, int rows,
    int B, Tout *__restrict__ out, float *__restrict__ lse) {
    typedef MhaTile<D> Mt;
    constexpr int KS = D / 16;   // k-steps of S, and 32-wide output tiles of O is D / 32
    constexpr int DT = D / 32;
    __shared__ __align__(16) uint8_t ktile[4][Mt::k_bytes];
    __shared__ __align__(16) uint8_t vtile[4][Mt::v_bytes];
    __shared__ float xq[4][kQb];  // per-query values handed from the S to the O layout

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int nqb = (rows + kQb - 1) / kQb;
    const long long unit = (long long)blockIdx.x * 4 + wave;
    if (unit >= (long long)B * nqb * H) return;
    const int h = (int)(unit % H);
    const int qb = (int)((unit / H) % nqb);
    const int b = (int)(unit / ((long long)H * nqb));
    uint8_t *kt = ktile[wave];
    uint8_t *vt = vtile[wave];
    float *xw = xq[wave];

    const int words = (S + 31) / 32;
    const int my_r = qb * kQb + l32;                 // this lane's query row (in the launch)
    const bool my_live = my_r < rows;
    const int rr = my_live ? my_r : rows - 1;
    const uint32_t *my_bits = bits + ((size_t)b * rows + rr) * words;
    int hi = my_live ? row_hi[(size_t)b * rows + rr] : -1;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) hi = max(hi, __shfl_xor(hi, off, 32));
    const int ntiles = hi < 0 ? 0 : hi / kKt + 1;    // uniform: max over the 32 rows

    // query block (B operand): lane (query l32, half) holds dims 16 ks + 8 half .. +8
    bf16x8 qb_reg[KS];
    {
        const uint16_t *qp = q + (((size_t)b * T + row0 + rr) * H + h) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb_reg[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
    }
    f32x16 o[DT];
#pragma unroll
    for (int c = 0; c < DT; ++c) o[c] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const float sl2 = scale * 1.4426950408889634f;

    const size_t head_stride = (size_t)H * D;  // elements between consecutive positions
    const uint16_t *kb = kc + ((size_t)b * S * H + h) * D;
    const uint16_t *vb = vc + ((size_t)b * S * H + h) * D;
    u32x4 gk[Mt::loads], gv[Mt::loads];
    uint32_t mw_next = 0u;
    auto load_tile = [&](int j) {  // keys past S re-read key S-1 (masked anyway)
#pragma unroll
        for (int m = 0; m < Mt::loads; ++m) {
            const int pq = lane + 64 * m;
            const int key = min(j * kKt + pq / Mt::pieces, S - 1);
            const size_t off = (size_t)key * head_stride + (pq % Mt::pieces) * 8;
            gk[m] = *reinterpret_cast<const u32x4 *>(kb + off);
            gv[m] = *reinterpret_cast<const u32x4 *>(vb + off);
        }
        mw_next = my_bits[min(j, words - 1)];
    };
    if (ntiles > 0) load_tile(0);

    // transpose-read lane address (see attention_mla.hip): row key0 + j/4, column col0 + 4 (j%4)
    const int trj = lane & 15, trg = lane >> 4;
    const int vrow = 8 * (trg >> 1) + (trj >> 2);
    const int vcol = (16 * (trg & 1) + 4 * (trj & 3)) * 2;

    for (int j = 0; j < ntiles; ++j) {
        // park tile j, start tile j+1
#pragma unroll
        for (int m = 0; m < Mt::loads; ++m) {
            const int pq = lane + 64 * m;
            const int key = pq / Mt::pieces, pc = pq % Mt::pieces;
            *reinterpret_cast<u32x4 *>(kt + key * Mt::k_pitch + pc * 16) = gk[m];
            *reinterpret_cast<u32x4 *>(vt + key * Mt::v_pitch + pc * 16) = gv[m];
        }
        const uint32_t mw = mw_next;
        if (j + 1 < ntiles) load_tile(j + 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // S^T: register rg holds key 8 (rg/4) + 4 half + rg%4, query l32
        bf16x8 af[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            af[ks] = *reinterpret_cast<const bf16x8 *>(kt + l32 * Mt::k_pitch +
                                                       (16 * ks + 8 * half) * 2);
        f32x16 sacc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qb_reg[ks], sacc, 0, 0, 0);
        float tmax = -INFINITY;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
            const int key = 8 * (rg >> 2) + 4 * half + (rg & 3);
            const float x = (mw >> key) & 1u ? sacc[rg] * sl2 : -INFINITY;
            sacc[rg] = x;
            tmax = fmaxf(tmax, x);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        float corr = 1.0f;
        if (tmax > m_run + kRescaleLog2) {
            corr = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - tmax);
            m_run = tmax;
        }
        const float m_ref = m_run;
        float ps0 = 0.0f, ps1 = 0.0f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // every lane has read the K tile; P overwrites it
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint8_t *prow = kt + l32 * Mt::p_pitch;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pv[e] = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sacc[4 * g + e] - m_ref);
            ps0 += pv[0] + pv[1];
            ps1 += pv[2] + pv[3];
            const bf16x4 pk = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
            *reinterpret_cast<bf16x4 *>(prow + (8 * g + 4 * half) * 2) = pk;
        }
        l_run = l_run * corr + (ps0 + ps1);
        const bool rescale = __ballot(corr != 1.0f) != 0;
        if (rescale && half == 0) xw[l32] = corr;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // O layout: register rg holds query 8 (rg/4) + 4 half + rg%4, dim 32 c + l32
        if (rescale) {
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) {
                const float cr = xw[8 * (rg >> 2) + 4 * half + (rg & 3)];
#pragma unroll
                for (int c = 0; c < DT; ++c) o[c][rg] *= cr;
            }
        }
#pragma unroll
        for (int ks = 0; ks < kKt / 16; ++ks) {
            const bf16x8 pa = *reinterpret_cast<const bf16x8 *>(prow + (16 * ks + 8 * half) * 2);
#pragma unroll
            for (int c = 0; c < DT; ++c) {
                const uint8_t *vp = vt + (16 * ks + vrow) * Mt::v_pitch + vcol + 64 * c;
                typedef __attribute__((address_space(3))) bf16x4 *lds_v4;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)vp);
                const bf16x4 hi4 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4)(vp + 4 * Mt::v_pitch));
                const bf16x8 vbf = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vbf, o[c], 0, 0, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // done with the tiles and xw before the next park
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // normalise: l of query l32 = both key halves; hand 1/l to the O layout
    const float l_all = l_run + __shfl_xor(l_run, 32, 64);
    if (half == 0) xw[l32] = l_all > 0.0f ? 1.0f / l_all : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
        const int qr = qb * kQb + 8 * (rg >> 2) + 4 * half + (rg & 3);
        if (qr >= rows) continue;
        const float inv = xw[8 * (rg >> 2) + 4 * half + (rg & 3)];
        Tout *op = out + (((size_t)b * T + row0 + qr) * H + h) * D + l32;
#pragma unroll
        for (int c = 0; c < DT; ++c) mha_store(op + 32 * c, o[c][rg] * inv);
    }
    if (lse && half == 0 && my_live)
        lse[((size_t)b * T + row0 + my_r) * H + h] =
            l_all > 0.0f ? (m_run + log2f(l_all)) * 0.6931471805599453f : -INFINITY;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Masked-dense MFMA form: bf16 in, d_qk = d_v in {64, 128}, at least one full
// query block of rows, and a selection covering at least a quarter of the
// keys (then the dense area is at most ~4x the selected work).
bool mha_dense_path(const dsa_attn_desc_t &d, int rows, int S, int k) {
    return d.form == DSA_MHA && d.dtype == DSA_BF16 && d.d_qk == d.d_v &&
           (d.d_qk == 64 || d.d_qk == 128) && rows >= kQb && S <= kMaxS &&
           4LL * k >= (long long)S;
}

size_t mha_workspace_bytes(int B, int rows, int S) {
    const size_t words = (size_t)(S + 31) / 32;
    return align256((size_t)B * rows * words * 4) + align256((size_t)B * rows * 4);
}

hipError_t launch_mha_dense(const dsa_attn_desc_t &d, const void *q, const void *kv,
                            const void *v, const int32_t *idx, int B, int T, int S, int row0,
                            int rows, int k, void *out, float *lse, void *workspace,
                            hipStream_t stream) {
    const size_t words = (size_t)(S + 31) / 32;
    uint32_t *bits = static_cast<uint32_t *>(workspace);
    int32_t *row_hi = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                  align256((size_t)B * rows * words * 4));
    for (int r0 = 0; r0 < rows; r0 += kMaxGridY) {
        const int n = min(kMaxGridY, rows - r0);
        hipLaunchKernelGGL(mha_bitmap_kernel, dim3(n, B), dim3(256), 0, stream, idx, T, S,
                           row0 + r0, rows, k, bits + (size_t)r0 * words, row_hi + r0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nqb = (rows + kQb - 1) / kQb;
    const long long units = (long long)B * nqb * d.num_heads;
    const dim3 grid((unsigned)((units + 3) / 4));
    const uint16_t *qp = static_cast<const uint16_t *>(q);
    const uint16_t *kp = static_cast<const uint16_t *>(kv);
    const uint16_t *vp = static_cast<const uint16_t *>(v);
    if (d.d_qk == 128) {
        if (d.out_dtype == DSA_BF16)
            hipLaunchKernelGGL((mha_dense_kernel<128, uint16_t>), grid, dim3(256), 0, stream, qp,
                               kp, vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<uint16_t *>(out), lse);
        else
            hipLaunchKernelGGL((mha_dense_kernel<128, float>), grid, dim3(256), 0, stream, qp, kp,
                               vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<float *>(out), lse);
    } else {
        if (d.out_dtype == DSA_BF16)
            hipLaunchKernelGGL((mha_dense_kernel<64, uint16_t>), grid, dim3(256), 0, stream, qp,
                               kp, vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<uint16_t *>(out), lse);
        else
            hipLaunchKernelGGL((mha_dense_kernel<64, float>), grid, dim3(256), 0, stream, qp, kp,
                               vp, bits, row_hi, T, S, d.num_heads, d.scale, row0, rows, B,
                               static_cast<float *>(out), lse);
    }
    return hipGetLastError();
}

}  // namespace dsa
