/*
 * dsa_oracle.c -- plain, slow, CPU reference for the DeepSeek Sparse Attention
 * (DSA) forward path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it; the product library never does.
 *
 * Every quantity is computed in IEEE double from inputs that the caller has
 * converted exactly (bf16, fp8 e4m3 and fp32 all embed exactly in double).
 * No blocking, no fusion, no reordering beyond the definitions below.  Built
 * with plain `-O2` (never -ffast-math), OpenMP only over independent rows.
 *
 * Sources (page titles as published):
 *  [P1] "DeepSeek Sparse Attention: Learned Token Selection from Scratch"
 *       (prathamp.com), sections 2.1, 3.1-3.3, 4.1, 7.1-7.2, 10.1.
 *  [P4] "DeepSeek NSA and DSA: From Native Sparse Attention to Fine-Grained
 *       Token Selection" (luowle.tech), section 3.2.
 *
 * Readings where the pages leave a step open (listed again in the design notes):
 *  - candidates of query position t are s = 0..t (the token itself included);
 *  - ties in the top-k are broken by the lower position s;
 *  - rows with t+1 <= k keep every candidate; unused slots hold -1;
 *  - the selected set is shared by all attention heads (MQA mode of MLA);
 *  - MLA keys are the whole latent row c_s, values are its first d_v entries.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* Absolute position of query row i of batch b: q_pos[b*T+i] if given, else
 * the last T positions of a length-S sequence (prefill T==S, decode T==1).
 * The candidates of position t are the cached positions s <= t ([P1] section
 * 2.1); the cache holds 0..S-1, so a position t >= S has the same candidates
 * as t = S-1 and is taken as S-1 (the position convention of the library's
 * interface).  A negative position has no candidates. */
static int64_t query_position(const int64_t *q_pos, int64_t b, int64_t i,
                              int64_t T, int64_t S) {
    const int64_t t = q_pos ? q_pos[b * T + i] : (S - T + i);
    return t >= S ? S - 1 : t;
}

/*
 * Lightning-indexer score, [P1] section 2.1 (boxed formula), [P4] section 3.2:
 *   I[t,s] = sum_j w[t,j] * ReLU( q_I[t,j] . k_I[s] ),   0 <= s <= t,
 * with one key k_I[s] shared by all H indexer heads ([P1] section 2.3/4.4).
 * Positions s > t are not candidates and are written as -inf.
 * Layouts: q_idx [B,T,H,D], k_idx [B,S,D], w [B,T,H], scores [B,T,S].
 */
ORACLE_API void oracle_indexer_scores(const double *q_idx, const double *k_idx,
                                      const double *w, const int64_t *q_pos,
                                      int64_t B, int64_t T, int64_t S,
                                      int64_t H, int64_t D, double *scores) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            const int64_t t = query_position(q_pos, b, i, T, S);
            double *row = scores + (b * T + i) * S;
            for (int64_t s = 0; s < S; ++s) {
                if (s > t) {
                    row[s] = -INFINITY;
                    continue;
                }
                const double *key = k_idx + (b * S + s) * D;
                double total = 0.0;
                for (int64_t j = 0; j < H; ++j) {
                    const double *qv = q_idx + ((b * T + i) * H + j) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += qv[d] * key[d];
                    const double relu = dot > 0.0 ? dot : 0.0;
                    total += w[(b * T + i) * H + j] * relu;
                }
                row[s] = total;
            }
        }
    }
}

/*
 * The same score in exact integer arithmetic, for inputs that are integers and
 * head weights that are integer multiples of 1/den (w = w_num / den).  Returns
 * den * I[t,s] exactly; s > t is written as INT64_MIN.  Used to show that the
 * double path loses nothing on the integer-valued workloads.
 */
ORACLE_API void oracle_indexer_scores_exact(const int64_t *q_idx,
                                            const int64_t *k_idx,
                                            const int64_t *w_num,
                                            const int64_t *q_pos, int64_t B,
                                            int64_t T, int64_t S, int64_t H,
                                            int64_t D, int64_t *scores_num) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            const int64_t t = query_position(q_pos, b, i, T, S);
            int64_t *row = scores_num + (b * T + i) * S;
            for (int64_t s = 0; s < S; ++s) {
                if (s > t) {
                    row[s] = INT64_MIN;
                    continue;
                }
                const int64_t *key = k_idx + (b * S + s) * D;
                int64_t total = 0;
                for (int64_t j = 0; j < H; ++j) {
                    const int64_t *qv = q_idx + ((b * T + i) * H + j) * D;
                    int64_t dot = 0;
                    for (int64_t d = 0; d < D; ++d) dot += qv[d] * key[d];
                    total += w_num[(b * T + i) * H + j] * (dot > 0 ? dot : 0);
                }
                row[s] = total;
            }
        }
    }
}

/* Candidate ordering for the top-k: higher score first, then lower position. */
typedef struct {
    double score;
    int64_t pos;
} candidate_t;

static int candidate_rank_order(const void *pa, const void *pb) {
    const candidate_t *a = (const candidate_t *)pa;
    const candidate_t *b = (const candidate_t *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos);
}

/*
 * Top-k selection, [P1] section 3.1 (boxed set S_t) and section 3.2:
 *   S_t = the k candidates s in 0..t with the highest I[t,s];
 * ties broken by the lower s.  A row keeps n_sel = min(k, t+1) entries
 * ([P1] section 7.2), written in rank order; slots n_sel..k-1 hold -1.
 *
 * include_current != 0 is the variant [P1] section 3.4 mentions (the current
 * token always kept): the query's own position t takes the first slot and
 * the other k-1 slots go to the best candidates among s in 0..t-1, by the
 * same order; n_sel is still min(k, t+1).
 * Layouts: scores [B,T,S], idx [B,T,k].
 */
ORACLE_API void oracle_topk(const double *scores, const int64_t *q_pos,
                            int64_t B, int64_t T, int64_t S, int64_t k,
                            int64_t include_current, int32_t *idx) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            const int64_t t = query_position(q_pos, b, i, T, S);
            const double *row = scores + (b * T + i) * S;
            int32_t *out = idx + (b * T + i) * k;
            /* the forced slot, then the ranked candidates after it */
            const int64_t forced = (include_current && t >= 0) ? 1 : 0;
            const int64_t n_cand = t + 1 - forced;
            int64_t r = 0;
            if (forced) out[r++] = (int32_t)t;
            const size_t n_alloc = n_cand > 0 ? (size_t)n_cand : 1;
            candidate_t *cand = (candidate_t *)malloc(sizeof(candidate_t) * n_alloc);
            for (int64_t s = 0; s < n_cand; ++s) {
                cand[s].score = row[s];
                cand[s].pos = s;
            }
            if (n_cand > 1) qsort(cand, (size_t)n_cand, sizeof(candidate_t), candidate_rank_order);
            for (int64_t c = 0; r < k; ++r, ++c)
                out[r] = c < n_cand ? (int32_t)cand[c].pos : -1;
            free(cand);
        }
    }
}

/* Key row and value row of position s for head h.
 * MHA ([P1] section 3.3): kv = K [B,S,H,dqk], v = V [B,S,H,dv].
 * MLA in MQA mode ([P1] section 4.1, [P4] section 3.1): kv = latent [B,S,dqk]
 * shared by every head; the value is the first dv entries of the same row. */
static const double *key_row(int form, const double *kv, int64_t b, int64_t s,
                             int64_t h, int64_t S, int64_t H, int64_t dqk) {
    if (form == 0) return kv + ((b * S + s) * H + h) * dqk;
    return kv + (b * S + s) * dqk;
}

static const double *value_row(int form, const double *kv, const double *v,
                               int64_t b, int64_t s, int64_t h, int64_t S,
                               int64_t H, int64_t dqk, int64_t dv) {
    if (form == 0) return v + ((b * S + s) * H + h) * dv;
    return kv + (b * S + s) * dqk;
}

/*
 * Attention restricted to a selected set, [P1] sections 3.3 and 10.1:
 *   alpha_s = exp(scale * q.k_s) / sum_{s' in S_t} exp(scale * q.k_s'),
 *   u_t     = sum_{s in S_t} alpha_s v_s,
 * evaluated with the maximum logit subtracted before exp (exact in real
 * arithmetic).  The set is idx[b,i,0..k-1] minus the -1 entries; it is the
 * same for every head.  Also returns lse = max + log(sum exp(logit - max)).
 * form 0 = MHA, 1 = MLA latent.  q [B,T,H,dqk], out [B,T,H,dv], lse [B,T,H].
 */
ORACLE_API void oracle_sparse_attention(int form, const double *q,
                                        const double *kv, const double *v,
                                        const int32_t *idx, int64_t B,
                                        int64_t T, int64_t S, int64_t H,
                                        int64_t dqk, int64_t dv, int64_t k,
                                        double scale, double *out, double *lse) {
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                const int32_t *sel = idx + (b * T + i) * k;
                const double *qv = q + ((b * T + i) * H + h) * dqk;
                double *o = out + ((b * T + i) * H + h) * dv;
                double *logit = (double *)malloc(sizeof(double) * (size_t)k);
                double m = -INFINITY;
                for (int64_t r = 0; r < k; ++r) {
                    if (sel[r] < 0) continue;
                    const double *key = key_row(form, kv, b, sel[r], h, S, H, dqk);
                    double dot = 0.0;
                    for (int64_t d = 0; d < dqk; ++d) dot += qv[d] * key[d];
                    logit[r] = scale * dot;
                    if (logit[r] > m) m = logit[r];
                }
                double denom = 0.0;
                for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
                for (int64_t r = 0; r < k; ++r) {
                    if (sel[r] < 0) continue;
                    const double p = exp(logit[r] - m);
                    denom += p;
                    const double *val = value_row(form, kv, v, b, sel[r], h, S, H, dqk, dv);
                    for (int64_t d = 0; d < dv; ++d) o[d] += p * val[d];
                }
                for (int64_t d = 0; d < dv; ++d) o[d] /= denom;
                if (lse) lse[(b * T + i) * H + h] = m + log(denom);
                free(logit);
            }
        }
    }
}

/*
 * Textbook dense causal softmax attention ([P1] section 7.1: every s in 0..t),
 * written independently of the routine above: a full logit row is formed,
 * normalised, then contracted with the values.  Same layouts and forms.
 */
ORACLE_API void oracle_dense_causal_attention(int form, const double *q,
                                              const double *kv, const double *v,
                                              const int64_t *q_pos, int64_t B,
                                              int64_t T, int64_t S, int64_t H,
                                              int64_t dqk, int64_t dv,
                                              double scale, double *out) {
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                const int64_t t = query_position(q_pos, b, i, T, S);
                const double *qv = q + ((b * T + i) * H + h) * dqk;
                double *o = out + ((b * T + i) * H + h) * dv;
                double *prob = (double *)malloc(sizeof(double) * (size_t)(t + 1));
                double m = -INFINITY;
                for (int64_t s = 0; s <= t; ++s) {
                    const double *key = key_row(form, kv, b, s, h, S, H, dqk);
                    double dot = 0.0;
                    for (int64_t d = 0; d < dqk; ++d) dot += qv[d] * key[d];
                    prob[s] = scale * dot;
                    if (prob[s] > m) m = prob[s];
                }
                double z = 0.0;
                for (int64_t s = 0; s <= t; ++s) {
                    prob[s] = exp(prob[s] - m);
                    z += prob[s];
                }
                for (int64_t s = 0; s <= t; ++s) prob[s] /= z;
                for (int64_t d = 0; d < dv; ++d) {
                    double acc = 0.0;
                    for (int64_t s = 0; s <= t; ++s)
                        acc += prob[s] * value_row(form, kv, v, b, s, h, S, H, dqk, dv)[d];
                    o[d] = acc;
                }
                free(prob);
            }
        }
    }
}

/*
 * Masked dense attention, the "masked MHA mode" of [P1] section 9.3: logits
 * over every position 0..S-1, with -inf wherever s is not in the selected set,
 * then an ordinary softmax over the whole row.  Brute-force cross-check of the
 * gather form above.
 */
ORACLE_API void oracle_masked_dense_attention(int form, const double *q,
                                              const double *kv, const double *v,
                                              const int32_t *idx, int64_t B,
                                              int64_t T, int64_t S, int64_t H,
                                              int64_t dqk, int64_t dv, int64_t k,
                                              double scale, double *out) {
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                const int32_t *sel = idx + (b * T + i) * k;
                const double *qv = q + ((b * T + i) * H + h) * dqk;
                double *o = out + ((b * T + i) * H + h) * dv;
                char *keep = (char *)calloc((size_t)S, 1);
                double *row = (double *)malloc(sizeof(double) * (size_t)S);
                for (int64_t r = 0; r < k; ++r)
                    if (sel[r] >= 0) keep[sel[r]] = 1;
                double m = -INFINITY;
                for (int64_t s = 0; s < S; ++s) {
                    if (!keep[s]) {
                        row[s] = -INFINITY;
                        continue;
                    }
                    const double *key = key_row(form, kv, b, s, h, S, H, dqk);
                    double dot = 0.0;
                    for (int64_t d = 0; d < dqk; ++d) dot += qv[d] * key[d];
                    row[s] = scale * dot;
                    if (row[s] > m) m = row[s];
                }
                double z = 0.0;
                for (int64_t s = 0; s < S; ++s) {
                    row[s] = keep[s] ? exp(row[s] - m) : 0.0;
                    z += row[s];
                }
                for (int64_t d = 0; d < dv; ++d) {
                    double acc = 0.0;
                    for (int64_t s = 0; s < S; ++s)
                        if (keep[s])
                            acc += (row[s] / z) * value_row(form, kv, v, b, s, h, S, H, dqk, dv)[d];
                    o[d] = acc;
                }
                free(row);
                free(keep);
            }
        }
    }
}

/*
 * Dense warm-up target of the indexer, [P1] section 5.2: the main attention
 * weights alpha^(h)[t,s] over s in 0..t are summed over the H heads and
 * L1-normalised along s, which gives p[t,s] = (1/H) sum_h alpha^(h)[t,s].
 * MHA form only.  p [B,T,S], zero for s > t.
 */
ORACLE_API void oracle_warmup_target(const double *q, const double *K,
                                     const int64_t *q_pos, int64_t B, int64_t T,
                                     int64_t S, int64_t H, int64_t dqk,
                                     double scale, double *p) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            const int64_t t = query_position(q_pos, b, i, T, S);
            double *prow = p + (b * T + i) * S;
            double *alpha = (double *)malloc(sizeof(double) * (size_t)(t + 1));
            for (int64_t s = 0; s < S; ++s) prow[s] = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                const double *qv = q + ((b * T + i) * H + h) * dqk;
                double m = -INFINITY;
                for (int64_t s = 0; s <= t; ++s) {
                    const double *key = K + ((b * S + s) * H + h) * dqk;
                    double dot = 0.0;
                    for (int64_t d = 0; d < dqk; ++d) dot += qv[d] * key[d];
                    alpha[s] = scale * dot;
                    if (alpha[s] > m) m = alpha[s];
                }
                double z = 0.0;
                for (int64_t s = 0; s <= t; ++s) {
                    alpha[s] = exp(alpha[s] - m);
                    z += alpha[s];
                }
                for (int64_t s = 0; s <= t; ++s) prow[s] += alpha[s] / z;
            }
            double total = 0.0;
            for (int64_t s = 0; s <= t; ++s) total += prow[s];
            for (int64_t s = 0; s <= t; ++s) prow[s] /= total;
            free(alpha);
        }
    }
}

/*
 * Sparse-stage target of the indexer, [P1] sections 6.2-6.3 with the head
 * aggregation of section 5.2: the main attention runs over the selected set
 * only, so its weights alpha^(h)[t,s] exist for s in S_t (the entries of
 * idx[b,i,:] that are >= 0); they are averaged over the H heads,
 *   p[t,s] = (1/H) sum_h alpha^(h)[t,s]  for s in S_t,  0 elsewhere,
 * which sums to 1 over S_t.  Keys as in oracle_sparse_attention (MHA: K per
 * head; MLA: the shared latent row).  p [B,T,S]; a row with an empty set is
 * all zero.
 */
ORACLE_API void oracle_sparse_target(int form, const double *q, const double *kv,
                                     const int32_t *idx, int64_t B, int64_t T,
                                     int64_t S, int64_t H, int64_t dqk, int64_t k,
                                     double scale, double *p) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < T; ++i) {
            const int32_t *sel = idx + (b * T + i) * k;
            double *prow = p + (b * T + i) * S;
            double *alpha = (double *)malloc(sizeof(double) * (size_t)k);
            for (int64_t s = 0; s < S; ++s) prow[s] = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                const double *qv = q + ((b * T + i) * H + h) * dqk;
                double m = -INFINITY;
                for (int64_t r = 0; r < k; ++r) {
                    if (sel[r] < 0) continue;
                    const double *key = key_row(form, kv, b, sel[r], h, S, H, dqk);
                    double dot = 0.0;
                    for (int64_t d = 0; d < dqk; ++d) dot += qv[d] * key[d];
                    alpha[r] = scale * dot;
                    if (alpha[r] > m) m = alpha[r];
                }
                double z = 0.0;
                for (int64_t r = 0; r < k; ++r) {
                    if (sel[r] < 0) continue;
                    alpha[r] = exp(alpha[r] - m);
                    z += alpha[r];
                }
                for (int64_t r = 0; r < k; ++r)
                    if (sel[r] >= 0) prow[sel[r]] += alpha[r] / z / (double)H;
            }
            free(alpha);
        }
    }
}

/*
 * Indexer distillation loss of one query row, [P1] sections 5.4 and 6.2:
 *   KL( p || softmax(I) ) = sum_s p_s (log p_s - log q_s),  q = softmax of I,
 * taken over the positions where mask[s] != 0 (all s <= t in the dense
 * warm-up; the selected set S_t in the sparse stage, where p and I are both
 * restricted to, and renormalised over, S_t).  Terms with p_s == 0 add 0.
 * Returns the sum of the per-row divergences over B*T rows.
 */
ORACLE_API double oracle_indexer_kl(const double *p, const double *scores,
                                    const char *mask, int64_t rows, int64_t S) {
    double loss = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const double *prow = p + r * S;
        const double *irow = scores + r * S;
        const char *mrow = mask + r * S;
        double m = -INFINITY, psum = 0.0;
        for (int64_t s = 0; s < S; ++s) {
            if (!mrow[s]) continue;
            if (irow[s] > m) m = irow[s];
            psum += prow[s];
        }
        double z = 0.0;
        for (int64_t s = 0; s < S; ++s)
            if (mrow[s]) z += exp(irow[s] - m);
        const double log_z = m + log(z);
        for (int64_t s = 0; s < S; ++s) {
            if (!mrow[s]) continue;
            const double ps = prow[s] / psum;
            if (ps > 0.0) loss += ps * (log(ps) - (irow[s] - log_z));
        }
    }
    return loss;
}
