// capi.hip -- the extern "C" entry points declared in dsa.h: argument
// checks, workspace carving, chunked orchestration of the three steps.
#include <limits.h>
#include <math.h>

#include <mutex>

#include "dsa_internal.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace dsa;

constexpr size_t kAlign = 256;  // workspace carve-out alignment
// The forward pass keeps one fp32 block of scores for a chunk of query rows;
// this bounds that block.  Larger chunks give the prefill indexer launches
// with more workgroups (less tail per launch); the per-row top-k that reads
// the block back runs at the same speed from 256 MiB to 1 GiB blocks.
constexpr size_t kScoreChunkBytes = 1ull << 30;

// Largest selection budget accepted (k may exceed S: the surplus slots hold -1).
constexpr int kMaxTopk = 1 << 20;

bool valid_topk(int k) { return k >= 1 && k <= kMaxTopk; }

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int dt) { return dt == DSA_F32 || dt == DSA_BF16 || dt == DSA_FP8_E4M3; }

dsa_status_t check_sizes(int B, int T, int S, bool have_pos) {
    if (B < 1 || T < 1 || S < 1) return DSA_ERR_SHAPE;
    if (B > 65535) return DSA_ERR_SHAPE;
    if (!have_pos && T > S) return DSA_ERR_SHAPE;
    return DSA_OK;
}

dsa_status_t check_indexer(const void *q_idx, const void *k_idx, int idx_dtype, const float *w,
                           int H, int D) {
    if (!q_idx || !k_idx || !w) return DSA_ERR_NULL;
    if (!valid_dtype(idx_dtype)) return DSA_ERR_DTYPE;
    if (H < 1 || H > 128 || D < 1 || D > 256) return DSA_ERR_SHAPE;
    if (!indexer_shape_supported(H, D)) return DSA_ERR_UNSUPPORTED;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

dsa_status_t check_attention(const dsa_attn_desc_t *d, const void *q, const void *kv,
                             const void *v, const void *out) {
    if (!d || !q || !kv || !out) return DSA_ERR_NULL;
    if (d->form != DSA_MHA && d->form != DSA_MLA) return DSA_ERR_SHAPE;
    if (!valid_dtype(d->dtype) || !valid_dtype(d->out_dtype)) return DSA_ERR_DTYPE;
    if (d->dtype == DSA_FP8_E4M3 || d->out_dtype == DSA_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    if (d->num_heads < 1 || d->num_heads > 4096) return DSA_ERR_SHAPE;
    if (d->d_qk < 1 || d->d_qk > 576 || d->d_v < 1 || d->d_v > 512) return DSA_ERR_SHAPE;
    if (!(d->scale > 0.0f) || isinf(d->scale)) return DSA_ERR_SHAPE;  // finite, positive
    if (d->form == DSA_MHA) {
        if (!v) return DSA_ERR_NULL;
        if (!aligned16(v)) return DSA_ERR_ALIGN;
    } else {
        if (v) return DSA_ERR_SHAPE;  // MLA values are the latent row itself
        if (d->d_v > d->d_qk) return DSA_ERR_SHAPE;
        if (d->dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
    }
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

// Query rows per forward chunk so that B * rows * S fp32 scores fit the bound.
int forward_chunk_rows(int B, int T, int S) {
    const size_t per_row = (size_t)B * (size_t)S * sizeof(float);
    size_t rows = kScoreChunkBytes / per_row;
    if (rows < 1) rows = 1;
    if (rows > (size_t)T) rows = (size_t)T;
    return (int)rows;
}

size_t forward_workspace(const dsa_attn_desc_t *d, int B, int T, int S, int k) {
    const int rows = forward_chunk_rows(B, T, S);
    size_t total = round_up((size_t)B * rows * S * sizeof(float));    // score block
    total += round_up((size_t)B * T * k * sizeof(int32_t));            // selection
    total += round_up(topk_workspace_bytes(B, rows, S, k));
    total += round_up(attention_workspace_bytes(*d, B, rows, S, k));
    return total;
}

dsa_status_t hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// ---- scratch of the allocation-free entry point (dsa_forward_ex_noalloc) --
// Each GPU the library runs on holds its own copy of this array, allocated
// with the code object and kept until the process ends.  Host code never uses
// the array's name as an address: the device address is resolved once per
// device with hipGetSymbolAddress and kept below.
constexpr size_t kScratchBytes = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's scratch array.
dsa_status_t scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

dsa_status_t check_forward(const dsa_attn_desc_t *desc, const void *q_idx, const void *k_idx,
                           int idx_dtype, const float *w, const void *q, const void *kv,
                           const void *v, const int32_t *q_pos, int B, int T, int S,
                           int index_n_heads, int index_head_dim, int index_topk, int flags,
                           const void *out, const int32_t *idx_out) {
    dsa_status_t st = check_sizes(B, T, S, q_pos != nullptr);
    if (st != DSA_OK) return st;
    st = check_indexer(q_idx, k_idx, idx_dtype, w, index_n_heads, index_head_dim);
    if (st != DSA_OK) return st;
    st = check_attention(desc, q, kv, v, out);
    if (st != DSA_OK) return st;
    if (!valid_topk(index_topk)) return DSA_ERR_SHAPE;
    if (flags & ~DSA_SEL_INCLUDE_CURRENT) return DSA_ERR_UNSUPPORTED;
    if (idx_out && !aligned16(idx_out)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

// The three steps over chunks of query rows, in `workspace` (checked by the
// caller to hold forward_workspace(...) bytes, 16-byte aligned).
dsa_status_t forward_run(const dsa_attn_desc_t *desc, const void *q_idx, const void *k_idx,
                         int idx_dtype, const float *w, const void *q, const void *kv,
                         const void *v, const int32_t *q_pos, int B, int T, int S,
                         int index_n_heads, int index_head_dim, int index_topk, int flags,
                         void *out, int32_t *idx_out, void *workspace, hipStream_t s) {
    const bool include_current = (flags & DSA_SEL_INCLUDE_CURRENT) != 0;
    const int rows = forward_chunk_rows(B, T, S);
    char *ws = static_cast<char *>(workspace);
    float *score_block = reinterpret_cast<float *>(ws);
    ws += round_up((size_t)B * rows * S * sizeof(float));
    int32_t *sel = reinterpret_cast<int32_t *>(ws);
    ws += round_up((size_t)B * T * index_topk * sizeof(int32_t));
    void *topk_ws = ws;
    ws += round_up(topk_workspace_bytes(B, rows, S, index_topk));
    void *attn_ws = ws;
    if (idx_out) sel = idx_out;

    // A context no longer than the budget selects every causal position in
    // every row (with or without the current-token flag): the indexer and
    // the top-k are skipped and the attention runs over the whole prefix.
    const bool dense = S <= index_topk;
    const size_t batch_stride = (size_t)rows * S;
    for (int row0 = 0; row0 < T; row0 += rows) {
        const int n = T - row0 < rows ? T - row0 : rows;
        hipError_t e;
        bool bitmap_ready = false;
        if (dense) {
            e = launch_select_all(q_pos, B, T, S, row0, n, index_topk, sel, s);
        } else {
            // the indexer launch also clears the top-k counters where the
            // top-k needs them (a kernel, not a memset, so the step can be
            // captured in a graph)
            const size_t clear_words = topk_clear_words(B, n, S, index_topk, include_current);
            e = launch_indexer(q_idx, k_idx, idx_dtype, w, q_pos, B, T, S, index_n_heads,
                               index_head_dim, row0, n, score_block, batch_stride, false,
                               static_cast<uint32_t *>(topk_ws), clear_words, s);
            if (e != hipSuccess) return DSA_ERR_HIP;
            // the masked-dense MHA attention takes the selection as a bitmap:
            // where the per-row top-k runs, it writes that bitmap too, in
            // place of a separate pass over the selection
            uint32_t *bits = nullptr;
            int32_t *row_hi = nullptr;
            if (mha_dense_path(*desc, n, S, index_topk) &&
                topk_writes_bitmap(B, n, S, index_topk, include_current))
                mha_bitmap_of(attn_ws, B, n, S, &bits, &row_hi);
            e = launch_topk(score_block, batch_stride, q_pos, B, T, S, row0, n, index_topk, sel,
                            topk_ws, clear_words > 0, s, include_current, bits, row_hi);
            bitmap_ready = bits != nullptr;
        }
        if (e != hipSuccess) return DSA_ERR_HIP;
        // the selection just written is min(k, t+1) positions then -1 per row
        e = launch_attention(*desc, q, kv, v, sel, B, T, S, row0, n, index_topk, out, nullptr,
                             attn_ws, s, q_pos, true, bitmap_ready);
        if (e != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

}  // namespace

DSA_EXPORT int dsa_abi_version(void) { return DSA_ABI_VERSION; }

DSA_EXPORT const char *dsa_status_string(int s) {
    switch (s) {
        case DSA_OK: return "ok";
        case DSA_ERR_NULL: return "a required pointer is NULL";
        case DSA_ERR_SHAPE: return "a size is out of range or sizes disagree";
        case DSA_ERR_DTYPE: return "unknown dtype code";
        case DSA_ERR_UNSUPPORTED: return "combination not supported";
        case DSA_ERR_WORKSPACE: return "workspace missing or too small";
        case DSA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case DSA_ERR_HIP: return "kernel launch failed";
        default: return "unknown status";
    }
}

DSA_EXPORT size_t dsa_workspace_bytes(int op, const dsa_attn_desc_t *desc, int B, int T, int S,
                                      int index_n_heads, int index_head_dim, int index_topk) {
    (void)index_n_heads;
    (void)index_head_dim;
    if (B < 1 || T < 1 || S < 1 || !valid_topk(index_topk)) return (size_t)-1;
    switch (op) {
        case DSA_OP_TOPK: return topk_workspace_bytes(B, T, S, index_topk);
        case DSA_OP_ATTENTION:
            if (!desc) return (size_t)-1;
            return attention_workspace_bytes(*desc, B, T, S, index_topk);
        case DSA_OP_FORWARD:
            if (!desc) return (size_t)-1;
            return forward_workspace(desc, B, T, S, index_topk);
        case DSA_OP_KL:
            if (!desc) return (size_t)-1;
            return kl_workspace_bytes(*desc, B, T, S, index_topk);
        default: return (size_t)-1;
    }
}

DSA_EXPORT dsa_status_t dsa_indexer_scores_ex(const void *q_idx, const void *k_idx,
                                              int idx_dtype, const float *w,
                                              const int32_t *q_pos, int B, int T, int S,
                                              int index_n_heads, int index_head_dim, int flags,
                                              float *scores, void *stream) {
    dsa_status_t st = check_sizes(B, T, S, q_pos != nullptr);
    if (st != DSA_OK) return st;
    if (!scores) return DSA_ERR_NULL;
    st = check_indexer(q_idx, k_idx, idx_dtype, w, index_n_heads, index_head_dim);
    if (st != DSA_OK) return st;
    if (flags & ~DSA_IDX_CAUSAL_ONLY) return DSA_ERR_UNSUPPORTED;
    if (!aligned16(scores)) return DSA_ERR_ALIGN;
    const bool write_masked = (flags & DSA_IDX_CAUSAL_ONLY) == 0;
    return hip_status(launch_indexer(q_idx, k_idx, idx_dtype, w, q_pos, B, T, S, index_n_heads,
                                     index_head_dim, 0, T, scores, (size_t)T * S, write_masked,
                                     nullptr, 0, (hipStream_t)stream));
}

DSA_EXPORT dsa_status_t dsa_indexer_scores(const void *q_idx, const void *k_idx, int idx_dtype,
                                           const float *w, const int32_t *q_pos, int B, int T,
                                           int S, int index_n_heads, int index_head_dim,
                                           float *scores, void *stream) {
    return dsa_indexer_scores_ex(q_idx, k_idx, idx_dtype, w, q_pos, B, T, S, index_n_heads,
                                 index_head_dim, 0, scores, stream);
}

DSA_EXPORT dsa_status_t dsa_topk_ex(const float *scores, const int32_t *q_pos, int B, int T,
                                    int S, int index_topk, int flags, int32_t *idx,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    dsa_status_t st = check_sizes(B, T, S, q_pos != nullptr);
    if (st != DSA_OK) return st;
    if (!scores || !idx) return DSA_ERR_NULL;
    if (!valid_topk(index_topk)) return DSA_ERR_SHAPE;
    if (flags & ~DSA_SEL_INCLUDE_CURRENT) return DSA_ERR_UNSUPPORTED;
    if (!aligned16(scores) || !aligned16(idx)) return DSA_ERR_ALIGN;
    const size_t need = topk_workspace_bytes(B, T, S, index_topk);
    if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
    return hip_status(launch_topk(scores, (size_t)T * S, q_pos, B, T, S, 0, T, index_topk, idx,
                                  workspace, false, (hipStream_t)stream,
                                  (flags & DSA_SEL_INCLUDE_CURRENT) != 0));
}

DSA_EXPORT dsa_status_t dsa_topk(const float *scores, const int32_t *q_pos, int B, int T, int S,
                                 int index_topk, int32_t *idx, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    return dsa_topk_ex(scores, q_pos, B, T, S, index_topk, 0, idx, workspace, workspace_bytes,
                       stream);
}

DSA_EXPORT dsa_status_t dsa_sparse_attention_ex(const dsa_attn_desc_t *desc, const void *q,
                                                const void *kv, const void *v,
                                                const int32_t *idx, const int32_t *q_pos,
                                                int flags, int B, int T, int S, int index_topk,
                                                void *out, float *lse, void *workspace,
                                                size_t workspace_bytes, void *stream) {
    dsa_status_t st = check_sizes(B, T, S, q_pos != nullptr || !(flags & DSA_ATTN_CAUSAL_PREFIX));
    if (st != DSA_OK) return st;
    st = check_attention(desc, q, kv, v, out);
    if (st != DSA_OK) return st;
    if (!idx) return DSA_ERR_NULL;
    if (!valid_topk(index_topk)) return DSA_ERR_SHAPE;
    if (flags & ~DSA_ATTN_CAUSAL_PREFIX) return DSA_ERR_UNSUPPORTED;
    if (!aligned16(idx) || (lse && !aligned16(lse))) return DSA_ERR_ALIGN;
    const size_t need = attention_workspace_bytes(*desc, B, T, S, index_topk);
    if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
    return hip_status(launch_attention(*desc, q, kv, v, idx, B, T, S, 0, T, index_topk, out, lse,
                                       workspace, (hipStream_t)stream, q_pos,
                                       (flags & DSA_ATTN_CAUSAL_PREFIX) != 0));
}

DSA_EXPORT dsa_status_t dsa_sparse_attention(const dsa_attn_desc_t *desc, const void *q,
                                             const void *kv, const void *v, const int32_t *idx,
                                             int B, int T, int S, int index_topk, void *out,
                                             float *lse, void *workspace,
                                             size_t workspace_bytes, void *stream) {
    return dsa_sparse_attention_ex(desc, q, kv, v, idx, nullptr, 0, B, T, S, index_topk, out,
                                   lse, workspace, workspace_bytes, stream);
}

DSA_EXPORT dsa_status_t dsa_indexer_kl_ex(const dsa_attn_desc_t *desc, const void *q,
                                          const void *kv, const int32_t *idx, const float *lse,
                                          const float *scores, int B, int T, int S,
                                          int index_topk, float *loss, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    dsa_status_t st = check_sizes(B, T, S, true);
    if (st != DSA_OK) return st;
    if (!desc) return DSA_ERR_NULL;
    if (!indexer_kl_supported(*desc)) return DSA_ERR_UNSUPPORTED;
    // the loss reads keys only (MHA: K in kv; the value tensor is not needed)
    st = check_attention(desc, q, kv, desc->form == DSA_MHA ? kv : nullptr, loss);
    if (st != DSA_OK) return st;
    if (!idx || !lse || !scores) return DSA_ERR_NULL;
    if (!valid_topk(index_topk)) return DSA_ERR_SHAPE;
    if (!aligned16(idx) || !aligned16(lse) || !aligned16(scores)) return DSA_ERR_ALIGN;
    const size_t need = kl_workspace_bytes(*desc, B, T, S, index_topk);
    if (workspace && (workspace_bytes < need || !aligned16(workspace))) return DSA_ERR_WORKSPACE;
    return hip_status(launch_indexer_kl(*desc, q, kv, idx, lse, scores, B, T, S, index_topk,
                                        loss, need > 0 ? workspace : nullptr,
                                        (hipStream_t)stream));
}

DSA_EXPORT dsa_status_t dsa_indexer_kl(const dsa_attn_desc_t *desc, const void *q,
                                       const void *kv, const int32_t *idx, const float *lse,
                                       const float *scores, int B, int T, int S,
                                       int index_topk, float *loss, void *stream) {
    return dsa_indexer_kl_ex(desc, q, kv, idx, lse, scores, B, T, S, index_topk, loss, nullptr,
                             0, stream);
}

DSA_EXPORT dsa_status_t dsa_forward_ex(const dsa_attn_desc_t *desc, const void *q_idx,
                                       const void *k_idx, int idx_dtype, const float *w,
                                       const void *q, const void *kv, const void *v,
                                       const int32_t *q_pos, int B, int T, int S,
                                       int index_n_heads, int index_head_dim, int index_topk,
                                       int flags, void *out, int32_t *idx_out, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    dsa_status_t st = check_forward(desc, q_idx, k_idx, idx_dtype, w, q, kv, v, q_pos, B, T, S,
                                    index_n_heads, index_head_dim, index_topk, flags, out,
                                    idx_out);
    if (st != DSA_OK) return st;
    const size_t need = forward_workspace(desc, B, T, S, index_topk);
    if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA_ERR_ALIGN;
    return forward_run(desc, q_idx, k_idx, idx_dtype, w, q, kv, v, q_pos, B, T, S,
                       index_n_heads, index_head_dim, index_topk, flags, out, idx_out, workspace,
                       (hipStream_t)stream);
}

DSA_EXPORT dsa_status_t dsa_forward_ex_noalloc(const dsa_attn_desc_t *desc, const void *q_idx,
                                               const void *k_idx, int idx_dtype, const float *w,
                                               const void *q, const void *kv, const void *v,
                                               const int32_t *q_pos, int B, int T, int S,
                                               int index_n_heads, int index_head_dim,
                                               int index_topk, int flags, void *out,
                                               int32_t *idx_out, void *stream) {
    dsa_status_t st = check_forward(desc, q_idx, k_idx, idx_dtype, w, q, kv, v, q_pos, B, T, S,
                                    index_n_heads, index_head_dim, index_topk, flags, out,
                                    idx_out);
    if (st != DSA_OK) return st;
    if (forward_workspace(desc, B, T, S, index_topk) > kScratchBytes) return DSA_ERR_WORKSPACE;
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != DSA_OK) return st;
    return forward_run(desc, q_idx, k_idx, idx_dtype, w, q, kv, v, q_pos, B, T, S,
                       index_n_heads, index_head_dim, index_topk, flags, out, idx_out, ws,
                       (hipStream_t)stream);
}

DSA_EXPORT dsa_status_t dsa_forward(const dsa_attn_desc_t *desc, const void *q_idx,
                                    const void *k_idx, int idx_dtype, const float *w,
                                    const void *q, const void *kv, const void *v,
                                    const int32_t *q_pos, int B, int T, int S,
                                    int index_n_heads, int index_head_dim, int index_topk,
                                    void *out, int32_t *idx_out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return dsa_forward_ex(desc, q_idx, k_idx, idx_dtype, w, q, kv, v, q_pos, B, T, S,
                          index_n_heads, index_head_dim, index_topk, 0, out, idx_out, workspace,
                          workspace_bytes, stream);
}
