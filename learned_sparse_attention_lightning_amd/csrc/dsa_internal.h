// dsa_internal.h -- device helpers and kernel launchers shared by the HIP
// translation units of the DSA library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// ----------------------------------------------------------- vector types --
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxGridY = 65535;  // launch limit of gridDim.y / gridDim.z

// ------------------------------------------------------------- barriers --
// Workgroup barrier for LDS traffic only.  __syncthreads() carries a
// workgroup release fence, which also waits for this wave's outstanding
// global loads -- including direct-to-LDS loads meant to stay in flight
// across the barrier.  Here only the wave's LDS operations are waited for
// (s_waitcnt lgkmcnt(0), vmcnt and expcnt left at their maxima), and the
// compiler-only fences keep memory accesses on their side of the barrier.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Reductions across the two 32-lane halves of a wave: v_permlane32_swap
// exchanges the halves in registers (no trip through the LDS crossbar that
// a generic shuffle takes), then both halves hold the combined value.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------ scalar conversions --
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (the hardware conversion).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// OCP fp8 e4m3fn -> fp32, exact (bias 7, no infinities, S.1111.111 = NaN).
__device__ __forceinline__ float fp8e4m3_to_f32(uint32_t v) {
    const uint32_t sign = (v & 0x80u) << 24;
    const uint32_t e = (v >> 3) & 0xfu;
    const uint32_t m = v & 0x7u;
    if (e == 0xfu && m == 0x7u) return __uint_as_float(0x7fc00000u | sign);
    if (e == 0) {  // subnormal: m * 2^-9
        const float mag = (float)m * 0.001953125f;
        return sign ? -mag : mag;
    }
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// Load element i of an index-tensor of dtype `dt` as fp32.
__device__ __forceinline__ float load_as_f32(const void *p, size_t i, int dt) {
    if (dt == DSA_F32) return static_cast<const float *>(p)[i];
    if (dt == DSA_BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    return fp8e4m3_to_f32(static_cast<const uint8_t *>(p)[i]);
}

// Order-preserving map fp32 -> uint32 (a < b  <=>  key(a) < key(b)), with
// -0.0 folded onto +0.0 so that signed zeros tie.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Absolute position of query row i (see dsa.h), clamped to S-1.
__device__ __forceinline__ int query_pos(const int32_t *q_pos, int b, int i, int T, int S) {
    int t = q_pos ? q_pos[(size_t)b * T + i] : (S - T + i);
    return t >= S ? S - 1 : t;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ launchers --
// Every launcher enqueues on `stream` and returns the launch status.

// Indexer scores for rows [row0, row0+rows) of every batch.  `scores` points
// at row row0 of batch 0 with row stride S and batch stride `batch_stride`
// (in floats).  write_masked: also write -inf for s in (t, S).
// clear_words > 0: the launch also zeroes clear[0..clear_words) (the counters
// of the top-k that follows), so no separate clearing kernel is needed.
hipError_t launch_indexer(const void *q_idx, const void *k_idx, int idx_dtype, const float *w,
                          const int32_t *q_pos, int B, int T, int S, int H, int D, int row0,
                          int rows, float *scores, size_t batch_stride, bool write_masked,
                          uint32_t *clear, size_t clear_words, hipStream_t stream);

bool indexer_shape_supported(int H, int D);

size_t topk_workspace_bytes(int B, int T, int S, int k);
size_t topk_clear_words(int B, int rows, int S, int k, bool include_current);
// include_current: the query's own position is always selected and the
// other k-1 slots are ranked among the earlier positions.
// bits / row_hi (optional, where topk_writes_bitmap holds): the selection
// also as the bitmap and per-row bound that launch_selection_bitmap writes
// (row_hi = n - 1, an upper bound of the last selected position).
bool topk_writes_bitmap(int B, int rows, int S, int k, bool include_current);
hipError_t launch_topk(const float *scores, size_t batch_stride, const int32_t *q_pos, int B,
                       int T, int S, int row0, int rows, int k, int32_t *idx, void *workspace,
                       bool workspace_cleared, hipStream_t stream, bool include_current,
                       uint32_t *bits = nullptr, int32_t *row_hi = nullptr);
// Selection of every candidate (for rows whose causal length is at most k).
hipError_t launch_select_all(const int32_t *q_pos, int B, int T, int S, int row0, int rows,
                             int k, int32_t *idx, hipStream_t stream);

bool indexer_kl_supported(const dsa_attn_desc_t &d);
// workspace: kl_workspace_bytes(...) bytes (or NULL: the per-entry form)
size_t kl_workspace_bytes(const dsa_attn_desc_t &d, int B, int T, int S, int k);
hipError_t launch_indexer_kl(const dsa_attn_desc_t &d, const void *q, const void *kv,
                             const int32_t *idx, const float *lse, const float *scores, int B,
                             int T, int S, int k, float *loss, void *workspace,
                             hipStream_t stream);
// One bit per (row, key) of the selection idx[b, row0 + r, :] (rows r of
// the launch, bits[(b * rows + r) * ceil(S/32) + s/32] bit s%32) and each
// row's largest selected position (-1: none).  S <= 65536.
hipError_t launch_selection_bitmap(const int32_t *idx, int B, int T, int S, int row0, int rows,
                                   int k, uint32_t *bits, int32_t *row_hi, hipStream_t stream);

bool mha_dense_path(const dsa_attn_desc_t &d, int rows, int S, int k);
size_t mha_workspace_bytes(int B, int rows, int S);
// Where launch_mha_dense keeps the selection bitmap and per-row bound in its
// workspace (for a launch of `rows` rows).
void mha_bitmap_of(void *workspace, int B, int rows, int S, uint32_t **bits, int32_t **row_hi);
// bitmap_ready: the workspace already holds them (written by the top-k)
hipError_t launch_mha_dense(const dsa_attn_desc_t &d, const void *q, const void *kv,
                            const void *v, const int32_t *idx, int B, int T, int S, int row0,
                            int rows, int k, void *out, float *lse, void *workspace,
                            hipStream_t stream, bool bitmap_ready = false);
bool mla_fast_path(const dsa_attn_desc_t &d);
size_t mla_workspace_bytes(const dsa_attn_desc_t &d, int B, int T, int k);
// causal_tail: every row's selection is min(k, t+1) positions followed by -1
// only (what the top-k writes), so the kernel stops at that count.
hipError_t launch_mla(const dsa_attn_desc_t &d, const void *q, const void *kv,
                      const int32_t *idx, int B, int T, int S, int row0, int rows, int k,
                      void *out, float *lse, void *workspace, hipStream_t stream,
                      const int32_t *q_pos = nullptr, bool causal_tail = false);

size_t attention_workspace_bytes(const dsa_attn_desc_t &d, int B, int T, int S, int k);
hipError_t launch_attention(const dsa_attn_desc_t &d, const void *q, const void *kv,
                            const void *v, const int32_t *idx, int B, int T, int S, int row0,
                            int rows, int k, void *out, float *lse, void *workspace,
                            hipStream_t stream, const int32_t *q_pos = nullptr,
                            bool causal_tail = false, bool bitmap_ready = false);

}  // namespace dsa
