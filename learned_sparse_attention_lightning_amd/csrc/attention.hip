// attention.hip -- softmax attention over the selected rows, on gfx950.
//
//   out[t,h] = sum_{s in S_t} softmax_s( scale * q[t,h] . key(s,h) ) value(s,h)
// ("DeepSeek Sparse Attention: Learned Token Selection from Scratch",
// sections 3.3 and 10.1).  One selected set per query serves every head
// (MQA mode of MLA, section 4.1 of the same page).  MHA form: per-head K and V
// rows.  MLA form: one latent row c_s per position; key = the whole row,
// value = its first d_v entries.
//
// This file holds the gather kernel that serves every supported shape: one
// wave per (query row, head) walks the selected positions in groups of 64
// (one per lane) with an online softmax in fp32.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxQk = 576;
constexpr int kMaxVPerLane = 8;  // d_v <= 512

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void st(T *p, size_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float *p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t *p, size_t i, float v) {
    p[i] = (uint16_t)f32_to_bf16_bits(v);
}

// One workgroup = 4 waves = 4 heads of one query row.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void attention_gather_kernel(
    int form, const Tin *__restrict__ q, const Tin *__restrict__ kv, const Tin *__restrict__ v,
    const int32_t *__restrict__ idx, int T, int S, int H, int dqk, int dv, int k, float scale,
    int row0, Tout *__restrict__ out, float *__restrict__ lse) {
    __shared__ float qs[4][kMaxQk];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + wave;
    const int i = row0 + blockIdx.y;
    const int b = blockIdx.z;
    const bool active = h < H;
    const size_t qoff = (((size_t)b * T + i) * H + h) * dqk;
    if (active)
        for (int d = lane; d < dqk; d += 64) qs[wave][d] = ld(q, qoff + d);
    __syncthreads();
    if (!active) return;

    const int32_t *sel = idx + ((size_t)b * T + i) * k;
    float m = -INFINITY, l = 0.0f;
    float acc[kMaxVPerLane];
#pragma unroll
    for (int e = 0; e < kMaxVPerLane; ++e) acc[e] = 0.0f;

    for (int c0 = 0; c0 < k; c0 += 64) {
        const int j = c0 + lane;
        // entries past the cache (outside the contract) count as unused, as in
        // the selection bitmap of the MHA kernel
        const int sj = j < k ? sel[j] : -1;
        const int s = sj < S ? sj : -1;
        float logit = -INFINITY;
        if (s >= 0) {
            const size_t koff = form == DSA_MHA ? (((size_t)b * S + s) * H + h) * dqk
                                                : ((size_t)b * S + s) * dqk;
            float dot = 0.0f;
            for (int d = 0; d < dqk; ++d) dot = fmaf(qs[wave][d], ld(kv, koff + d), dot);
            logit = dot * scale;
        }
        float cmax = logit;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));
        if (cmax == -INFINITY) continue;  // no valid entry in this group (uniform)
        const float m_new = fmaxf(m, cmax);
        const float corr = __expf(m - m_new);
        const float p = s >= 0 ? __expf(logit - m_new) : 0.0f;
        float psum = p;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) psum += __shfl_xor(psum, off, 64);
        l = l * corr + psum;
        m = m_new;
#pragma unroll
        for (int e = 0; e < kMaxVPerLane; ++e) acc[e] *= corr;
        const int cnt = min(64, k - c0);
        for (int e2 = 0; e2 < cnt; ++e2) {
            const int se = __shfl(s, e2, 64);
            if (se < 0) continue;  // uniform
            const float pe = __shfl(p, e2, 64);
            const size_t voff = form == DSA_MHA ? (((size_t)b * S + se) * H + h) * dv
                                                : ((size_t)b * S + se) * dqk;
            const Tin *vrow = form == DSA_MHA ? v : kv;
#pragma unroll
            for (int e = 0; e < kMaxVPerLane; ++e) {
                const int d = lane + 64 * e;
                if (d < dv) acc[e] = fmaf(pe, ld(vrow, voff + d), acc[e]);
            }
        }
    }
    const size_t ooff = (((size_t)b * T + i) * H + h) * dv;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int e = 0; e < kMaxVPerLane; ++e) {
        const int d = lane + 64 * e;
        if (d < dv) st(out, ooff + d, acc[e] * inv);
    }
    if (lse && lane == 0) lse[((size_t)b * T + i) * H + h] = l > 0.0f ? m + __logf(l) : -INFINITY;
}

template <typename Tin, typename Tout>
hipError_t launch_gather(const dsa_attn_desc_t &d, const void *q, const void *kv, const void *v,
                         const int32_t *idx, int B, int T, int S, int row0, int rows, int k,
                         void *out, float *lse, hipStream_t stream) {
    for (int r0 = 0; r0 < rows; r0 += kMaxGridY) {
        dim3 grid(ceil_div(d.num_heads, 4), min(kMaxGridY, rows - r0), B);
        hipLaunchKernelGGL((attention_gather_kernel<Tin, Tout>), grid, dim3(256), 0, stream,
                           d.form, static_cast<const Tin *>(q), static_cast<const Tin *>(kv),
                           static_cast<const Tin *>(v), idx, T, S, d.num_heads, d.d_qk, d.d_v,
                           k, d.scale, row0 + r0, static_cast<Tout *>(out), lse);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t attention_workspace_bytes(const dsa_attn_desc_t &d, int B, int T, int S, int k) {
    if (mla_fast_path(d)) return mla_workspace_bytes(d, B, T, k);
    // the masked-dense MHA form keeps a selection bitmap; a launch covers up
    // to T rows (dsa_forward passes its chunk)
    if (mha_dense_path(d, T, S, k)) return mha_workspace_bytes(B, T, S);
    return 0;
}

hipError_t launch_attention(const dsa_attn_desc_t &d, const void *q, const void *kv,
                            const void *v, const int32_t *idx, int B, int T, int S, int row0,
                            int rows, int k, void *out, float *lse, void *workspace,
                            hipStream_t stream, const int32_t *q_pos, bool causal_tail,
                            bool bitmap_ready) {
    if (mla_fast_path(d))
        return launch_mla(d, q, kv, idx, B, T, S, row0, rows, k, out, lse, workspace, stream,
                          q_pos, causal_tail);
    if (mha_dense_path(d, rows, S, k) && workspace)
        return launch_mha_dense(d, q, kv, v, idx, B, T, S, row0, rows, k, out, lse, workspace,
                                stream, bitmap_ready);
    const bool in_bf16 = d.dtype == DSA_BF16;
    const bool out_bf16 = d.out_dtype == DSA_BF16;
    if (in_bf16 && out_bf16)
        return launch_gather<uint16_t, uint16_t>(d, q, kv, v, idx, B, T, S, row0, rows, k, out,
                                                 lse, stream);
    if (in_bf16)
        return launch_gather<uint16_t, float>(d, q, kv, v, idx, B, T, S, row0, rows, k, out, lse,
                                              stream);
    if (out_bf16)
        return launch_gather<float, uint16_t>(d, q, kv, v, idx, B, T, S, row0, rows, k, out, lse,
                                              stream);
    return launch_gather<float, float>(d, q, kv, v, idx, B, T, S, row0, rows, k, out, lse,
                                       stream);
}

}  // namespace dsa
