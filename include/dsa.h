/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) forward path for
 * AMD Instinct MI355X (gfx950).
 *
 * The path has three steps, each one entry point, plus one call that runs
 * them back to back:
 *   1. lightning-indexer scores      dsa_indexer_scores
 *   2. per-query top-k selection     dsa_topk
 *   3. attention over the selection  dsa_sparse_attention (MHA or MLA latent)
 *   1+2+3                            dsa_forward
 * dsa_topk_ex and dsa_forward_ex take selection flags (the current-token
 * variant); dsa_indexer_kl gives the indexer's distillation loss (forward).
 *
 * Page references (titles as published):
 *   [P1] "DeepSeek Sparse Attention: Learned Token Selection from Scratch"
 *   [P3] "Sparse Attention LLM Design: Native Sparse Attention and DeepSeek
 *        Sparse Attention"
 *   [P4] "DeepSeek NSA and DSA: From Native Sparse Attention to Fine-Grained
 *        Token Selection"
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.  Every tensor argument is caller-owned DEVICE memory (for instance a
 *   torch tensor's data pointer), dense row-major in the layout given, and
 *   16-byte aligned.  The library allocates nothing and keeps no pointer
 *   after a call returns.  Its only mutable global state is the scratch
 *   array of dsa_forward_ex_noalloc (below) and the per-device address of
 *   that array.  Buffers must stay alive until the work queued on `stream`
 *   has finished.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Every call only enqueues work; none synchronises the host.
 * Positions.  q_pos [B,T] int32 gives the absolute position t of each query
 *   row; NULL means t = S - T + i for row i (prefill: T == S, t = i; decode:
 *   T == 1, t = S - 1, the new token being the last cache entry).  The
 *   candidates of row t are the cache positions s = 0..t ([P1] sections 2.1,
 *   7.1).  A position t >= S is treated as S-1; a negative position has no
 *   candidates (all-masked scores, an all -1 selection, zero output).
 * Errors.  Argument checks run on the host before anything is enqueued; on
 *   failure the call returns a status != DSA_OK and writes nothing.  A failed
 *   kernel launch returns DSA_ERR_HIP.  Faults inside kernels surface at the
 *   caller's next synchronisation.  Nothing throws or aborts across the ABI.
 *   Calls are safe from several host threads on distinct streams.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 4

typedef enum {
    DSA_F32 = 0,      /* IEEE binary32 */
    DSA_BF16 = 1,     /* bfloat16 */
    DSA_FP8_E4M3 = 2  /* OCP fp8 e4m3fn (no infinities; the format of gfx950) */
} dsa_dtype_t;

typedef enum {
    DSA_MHA = 0,  /* per-head keys and values ([P1] section 3.3) */
    DSA_MLA = 1   /* one latent row per token shared by all heads, MQA mode
                     of MLA ([P1] section 4.1, [P4] section 3.1) */
} dsa_form_t;

typedef enum {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,         /* a required pointer is NULL */
    DSA_ERR_SHAPE = 2,        /* a size is out of range or sizes disagree */
    DSA_ERR_DTYPE = 3,        /* unknown dtype code */
    DSA_ERR_UNSUPPORTED = 4,  /* valid but not implemented combination */
    DSA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required */
    DSA_ERR_ALIGN = 6,        /* a tensor pointer is not 16-byte aligned */
    DSA_ERR_HIP = 7           /* a kernel launch failed */
} dsa_status_t;

/* Attention description.  Fields are plain ints for a stable ABI. */
typedef struct {
    int form;       /* dsa_form_t */
    int num_heads;  /* attention heads H */
    int d_qk;       /* query/key width: MHA 64 or 128; MLA 576 */
    int d_v;        /* value width: MHA == d_qk; MLA 512 (first d_v entries
                       of the latent row) */
    float scale;    /* softmax scale, 1/sqrt(d_k) on [P1] section 3.3; finite and
                       > 0 (else DSA_ERR_SHAPE) */
    int dtype;      /* dtype of q, K/V or latent: DSA_F32 or DSA_BF16
                       (MLA: DSA_BF16 only) */
    int out_dtype;  /* dtype of out: DSA_F32 or DSA_BF16 */
} dsa_attn_desc_t;

/* Version of this ABI (DSA_ABI_VERSION of the built library). */
int dsa_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *dsa_status_string(int status);

/*
 * Lightning-indexer scores, [P1] section 2.1 and [P4] section 3.2:
 *   scores[b,i,s] = sum_j w[b,i,j] * ReLU( q_idx[b,i,j,:] . k_idx[b,s,:] )
 * for 0 <= s <= t, and -inf for s > t.  One key per position is shared by
 * all index heads ([P1] section 2.3).  Products and sums are fp32 (exact
 * whenever inputs are small integers, as in the shipped workloads).
 *   q_idx   [B,T,H_I,d_I]  idx_dtype (DSA_F32, DSA_BF16 or DSA_FP8_E4M3)
 *   k_idx   [B,S,d_I]      idx_dtype
 *   w       [B,T,H_I]      fp32 head weights (any sign)
 *   q_pos   [B,T] int32 or NULL
 *   scores  [B,T,S]        fp32 output, written in full
 * index_n_heads (H_I) in 1..128, index_head_dim (d_I) in 1..256.
 */
dsa_status_t dsa_indexer_scores(const void *q_idx, const void *k_idx, int idx_dtype,
                                const float *w, const int32_t *q_pos, int B, int T, int S,
                                int index_n_heads, int index_head_dim, float *scores,
                                void *stream);

/* Indexer flags of dsa_indexer_scores_ex. */
enum {
    /* Write only the candidates s <= t of each row; entries s > t are left
     * as they were (dsa_topk never reads them).  This is what dsa_forward
     * does with its score block. */
    DSA_IDX_CAUSAL_ONLY = 1
};

/*
 * dsa_indexer_scores with indexer flags (DSA_IDX_*; 0 is
 * dsa_indexer_scores).  Unknown flag bits return DSA_ERR_UNSUPPORTED.
 */
dsa_status_t dsa_indexer_scores_ex(const void *q_idx, const void *k_idx, int idx_dtype,
                                   const float *w, const int32_t *q_pos, int B, int T, int S,
                                   int index_n_heads, int index_head_dim, int flags,
                                   float *scores, void *stream);

/*
 * Top-k selection, [P1] section 3.1: row i keeps the n_sel = min(k, t+1)
 * candidates s in 0..t with the highest scores, ties broken by the lower
 * position s (the one exactly-defined selection).  -0.0 equals +0.0; NaN
 * scores are outside the contract.
 *   scores  [B,T,S] fp32 (entries s > t are never read)
 *   idx     [B,T,k] int32 output: the n_sel selected positions in ASCENDING
 *           order, then -1 in the remaining k - n_sel slots.
 * index_topk (k) in 1..2^20; k may exceed S (rows then keep every candidate
 * and the surplus slots hold -1).  Needs dsa_workspace_bytes(DSA_OP_TOPK, ...)
 * bytes of workspace (may be 0; then workspace may be NULL).
 */
dsa_status_t dsa_topk(const float *scores, const int32_t *q_pos, int B, int T, int S,
                      int index_topk, int32_t *idx, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Selection flags of the _ex calls. */
enum {
    /* Always keep the current token ([P1] section 3.4 names this variant):
     * row i selects its own position t, and the other k-1 slots go to the
     * best candidates among s in 0..t-1 by the order above.  n_sel is still
     * min(k, t+1); the output stays ascending, so t is the last valid entry. */
    DSA_SEL_INCLUDE_CURRENT = 1
};

/*
 * dsa_topk with selection flags (DSA_SEL_*; 0 is dsa_topk).  Unknown flag
 * bits return DSA_ERR_UNSUPPORTED.  Same workspace as dsa_topk.
 */
dsa_status_t dsa_topk_ex(const float *scores, const int32_t *q_pos, int B, int T, int S,
                         int index_topk, int flags, int32_t *idx, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Softmax attention restricted to the selected rows, [P1] sections 3.3 and
 * 10.1, with one selected set per query shared by every head ([P1] section
 * 4.1):
 *   out[b,i,h,:] = sum_{s in S} softmax_s( scale * q[b,i,h,:] . key(s,h) ) * value(s,h)
 * where S = the entries of idx[b,i,:] that are >= 0 (distinct, each < S).
 * Entries >= S are outside this contract; they count as unused slots (like
 * -1) and no kernel reads a row past the sequence's S rows for them.
 *   MHA: kv = K [B,S,H,d_qk], v = V [B,S,H,d_v]; key(s,h) = K[b,s,h],
 *        value(s,h) = V[b,s,h].
 *   MLA: kv = latent [B,S,d_qk], v = NULL; key(s,h) = latent[b,s,:] (all
 *        576 entries), value(s,h) = latent[b,s,0:d_v].
 *   q    [B,T,H,d_qk]  desc->dtype
 *   out  [B,T,H,d_v]   desc->out_dtype; a row with an empty set gets zeros
 *   lse  [B,T,H] fp32 natural-log sum of exp of the scaled logits, or NULL
 * Logits, softmax and accumulation are fp32.  Needs
 * dsa_workspace_bytes(DSA_OP_ATTENTION, ...) bytes of workspace.
 */
dsa_status_t dsa_sparse_attention(const dsa_attn_desc_t *desc, const void *q, const void *kv,
                                  const void *v, const int32_t *idx, int B, int T, int S,
                                  int index_topk, void *out, float *lse, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Attention flags of dsa_sparse_attention_ex. */
enum {
    /* Every row's idx holds its min(k, t+1) selected positions first and -1
     * in every later slot (what dsa_topk and dsa_topk_ex write); the kernel
     * then reads no slot past that count.  t comes from q_pos (or the
     * default positions, which need T <= S). */
    DSA_ATTN_CAUSAL_PREFIX = 1
};

/*
 * dsa_sparse_attention with the query positions and attention flags
 * (DSA_ATTN_*; 0 is dsa_sparse_attention, and q_pos is then unused).
 * Unknown flag bits return DSA_ERR_UNSUPPORTED.  Same workspace.
 */
dsa_status_t dsa_sparse_attention_ex(const dsa_attn_desc_t *desc, const void *q, const void *kv,
                                     const void *v, const int32_t *idx, const int32_t *q_pos,
                                     int flags, int B, int T, int S, int index_topk, void *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * The whole forward path ([P4] section 3.2, three steps): indexer scores,
 * top-k, then attention over the selection, on one stream.  Query rows are
 * processed in chunks so the fp32 score block stays bounded.  Arguments are
 * those of the three calls above.  idx_out [B,T,k] receives the selection
 * when non-NULL.  Needs dsa_workspace_bytes(DSA_OP_FORWARD, ...) bytes.
 */
dsa_status_t dsa_forward(const dsa_attn_desc_t *desc, const void *q_idx, const void *k_idx,
                         int idx_dtype, const float *w, const void *q, const void *kv,
                         const void *v, const int32_t *q_pos, int B, int T, int S,
                         int index_n_heads, int index_head_dim, int index_topk, void *out,
                         int32_t *idx_out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * dsa_forward with selection flags (DSA_SEL_*; 0 is dsa_forward).  When the
 * context is no longer than the budget (S <= k) every causal position is
 * selected in every row -- the dense limit ([P1] section 7.6, the entry-count
 * table; [P3] section "Trade-offs, Gotchas, and What Goes Wrong" on short
 * inputs) -- so the indexer and the top-k are skipped and
 * attention runs over the whole prefix; dsa_forward does the same.  Same
 * workspace as dsa_forward.
 */
dsa_status_t dsa_forward_ex(const dsa_attn_desc_t *desc, const void *q_idx, const void *k_idx,
                            int idx_dtype, const float *w, const void *q, const void *kv,
                            const void *v, const int32_t *q_pos, int B, int T, int S,
                            int index_n_heads, int index_head_dim, int index_topk, int flags,
                            void *out, int32_t *idx_out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * dsa_forward_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The intermediate buffers (the score
 * block, the selection when idx_out is NULL, the top-k counters and the
 * attention's split partials) live in a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES (128 MiB) that each GPU the library runs on holds
 * until the process ends; the call itself allocates nothing.  Sizes whose
 * dsa_workspace_bytes(DSA_OP_FORWARD, ...) exceed that return
 * DSA_ERR_WORKSPACE before anything is enqueued (the decode workloads fit:
 * 8 x 131072 and 64 x 32768 contexts at k = 2048, 128 heads).  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (several
 * streams, several host threads) race and must be serialised by the caller;
 * the array keeps the last call's contents (whatever must start at zero is
 * cleared by the call's own kernels).  Results equal dsa_forward_ex's.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (128u << 20)
dsa_status_t dsa_forward_ex_noalloc(const dsa_attn_desc_t *desc, const void *q_idx,
                                    const void *k_idx, int idx_dtype, const float *w,
                                    const void *q, const void *kv, const void *v,
                                    const int32_t *q_pos, int B, int T, int S,
                                    int index_n_heads, int index_head_dim, int index_topk,
                                    int flags, void *out, int32_t *idx_out, void *stream);

/*
 * Forward value of the indexer's distillation loss over a selected set,
 * [P1] sections 5.2-5.4 (target and loss) and 6.2 (restricted to S_t).  For
 * each query row, with S = the entries of idx[b,i,:] that are >= 0:
 *   p_s     = (1/H) sum_h softmax_{s in S}( scale * q[b,i,h,:] . key(s,h) )
 *             (the head mean of the attention weights over S; key(s,h) as in
 *             dsa_sparse_attention),
 *   loss[b,i] = KL( p || softmax_{s in S}( scores[b,i,s] ) )
 *             = sum_{s in S} p_s ( log p_s - log softmax(scores)_s ),
 * with p renormalised over S.  A row with an empty set gets 0.  The dense
 * warm-up loss of [P1] section 5.4 is the same call with every causal
 * position selected (k >= S; dsa_topk writes that selection).
 *   MLA: desc->form DSA_MLA, dtype DSA_BF16, d_qk 576, num_heads 32, 64 or
 *   128; MHA: DSA_MHA, dtype DSA_BF16 or DSA_F32, d_qk 64 or 128, num_heads
 *   <= 64 (else DSA_ERR_UNSUPPORTED).  desc->scale is the attention's scale.
 *   q      [B,T,H,d_qk] desc->dtype
 *   kv     MLA: [B,S,576] bf16 latent rows; MHA: K [B,S,H,d_qk]
 *   idx    [B,T,k] int32 distinct positions < S, -1 = unused slot
 *   lse    [B,T,H] fp32 natural-log sum of exp of the scaled logits over the
 *          same set, as dsa_sparse_attention writes it for q, kv, idx
 *   scores [B,T,S] fp32 indexer scores (read at the selected positions)
 *   loss   [B,T] fp32 output (the total is its sum)
 * Logits in fp32 (bf16 or fp32 inputs); p, the log-sum-exp of the scores and
 * the sums in fp32.  No workspace (dsa_indexer_kl_ex takes one).
 */
dsa_status_t dsa_indexer_kl(const dsa_attn_desc_t *desc, const void *q, const void *kv,
                            const int32_t *idx, const float *lse, const float *scores, int B,
                            int T, int S, int index_topk, float *loss, void *stream);

/*
 * dsa_indexer_kl with a workspace (same loss, [P1] sections 5.2-5.4 and
 * 6.2).  When dsa_workspace_bytes(DSA_OP_KL, ...) is non-zero -- MHA, bf16,
 * d_qk 64 or 128, 8 or 16 heads, S <= 65536 and k >= S/4, the prefill
 * regime where the selection covers much of every causal prefix -- and a
 * workspace of at least that many bytes (16-byte aligned, caller-owned,
 * contents not preserved) is given, the target p_s is computed for every key
 * of the causal area on the matrix cores and the selection, turned into one
 * bit per (row, key), decides which keys enter the loss; otherwise (NULL
 * workspace, or a shape outside that set) the call is dsa_indexer_kl.  A
 * workspace smaller than needed gives DSA_ERR_WORKSPACE.
 */
dsa_status_t dsa_indexer_kl_ex(const dsa_attn_desc_t *desc, const void *q, const void *kv,
                               const int32_t *idx, const float *lse, const float *scores, int B,
                               int T, int S, int index_topk, float *loss, void *workspace,
                               size_t workspace_bytes, void *stream);

enum { DSA_OP_TOPK = 0, DSA_OP_ATTENTION = 1, DSA_OP_FORWARD = 2, DSA_OP_KL = 3 };

/*
 * Workspace bytes needed by one call of `op` with these sizes (desc may be
 * NULL for DSA_OP_TOPK; DSA_OP_KL: the bytes dsa_indexer_kl_ex uses, 0 when
 * it runs without one).  Returns (size_t)-1 when the sizes are invalid.
 */
size_t dsa_workspace_bytes(int op, const dsa_attn_desc_t *desc, int B, int T, int S,
                           int index_n_heads, int index_head_dim, int index_topk);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
