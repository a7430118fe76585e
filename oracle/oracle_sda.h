/*
 * oracle_sda.h -- plain fp64 CPU oracle for sparse decode attention with a
 * tail estimate.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; the two are written independently from the pages.
 *
 * Sources (web pages, cited by title and section):
 *   [RESA]  "RESA: Bringing Back What Sparse Attention Ignores with Residual
 *           Estimation" (papernotes.org summary), sections "Prior Estimator"
 *           and "Online Aggregator".
 *   [vATT]  "vAttention: Verified Sparse Attention via Sampling"
 *           (papernotes.org summary), method sections 1-3 (eq. 3, the CLT
 *           sample-size lemma, Lemma 4.2).
 *   [OPEN]  "OpenAttention: One Percent Is Enough with Tail Proxies"
 *           (ai-frontier-tracker summary), abstract and the four-stage
 *           method list (stage 04: count-aware mean proxy; stage 05: one
 *           online softmax over exact tokens and proxies).
 *
 * Conventions shared by every routine:
 *   - q   [B, Hq, d]     in `dtype` (bf16 bit patterns or fp32)
 *   - K,V [B, Hkv, n, d] in `dtype`, contiguous
 *   - query head h belongs to KV head g = h / (Hq / Hkv)
 *   - every input value is widened exactly to double; all arithmetic is fp64
 *   - the logit of query head h against row j is  scale * <q_h, k_j>,
 *     with `scale` taken as the fp32 value given (the GPU receives the same)
 *   - idx [B, Hkv, m] int32 row positions; idx_len [B, Hkv] (or NULL = m)
 *     gives the number of valid leading entries of each unit's list
 *   - logw [B, Hkv, m] fp32 log-weights added to exact logits (NULL = 0)
 *   - outputs: out [B, Hq, d] and lse [B, Hq] as double.  lse is the natural
 *     log of the (unshifted) softmax denominator.  A unit with nothing to
 *     attend to gets out = 0 and lse = -inf.
 *
 * Every routine returns 0 on success and a negative value on a malformed
 * argument (which the tests never pass on purpose except to check it).
 */
#ifndef ORACLE_SDA_H
#define ORACLE_SDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1 };

typedef struct {
  int B, Hq, Hkv, n, d;
  int dtype;     /* ORC_BF16 or ORC_F32 */
  float scale;   /* logit scale, normally 1/sqrt(d) */
} orc_dims;

/* Thread count for the unit loops (OpenMP); <= 0 leaves the default. */
void orc_set_threads(int nthreads);
int orc_get_threads(void);

/* ---- dense softmax attention (textbook definition) ---------------------- */
int orc_dense(const orc_dims* D, const void* q, const void* K, const void* V,
              double* out, double* lse);

/* ---- sparse attention over an index list with log-weights ---------------
 * [vATT] eq. 3: each listed row contributes exp(logit + w) to the
 * denominator and exp(logit + w) v to the numerator; duplicates count as
 * separate terms. */
int orc_sparse(const orc_dims* D, const void* q, const void* K, const void* V,
               const int32_t* idx, const int32_t* idx_len, const float* logw,
               int m, double* out, double* lse);

/* ---- (a) count-aware mean proxies [OPEN] --------------------------------
 * Cluster b of unit u holds the rows j with cid[j] == b (cid == -1: in no
 * cluster).  Build: count, sum of keys and sum of values per cluster. */
int orc_proxy_build(const orc_dims* D, const void* K, const void* V,
                    const int32_t* cid, int C,
                    int32_t* count, double* sumK, double* sumV);

/* Plain definition, O(n): the unread members U_b of each cluster (members
 * not in the index set) fold into one virtual token with key mean(U_b),
 * value mean(U_b) and logit scale*<q, mean key> + ln |U_b|.  Clusters with
 * no unread member add nothing. */
int orc_sparse_proxy_def(const orc_dims* D, const void* q, const void* K,
                         const void* V, const int32_t* idx,
                         const int32_t* idx_len, const float* logw, int m,
                         const int32_t* cid, int C, double* out, double* lse);

/* The same result in O(|I|) from the built per-cluster sums: the listed rows
 * are subtracted from their cluster's count and sums.  Requires each unit's
 * list to hold distinct positions. */
int orc_sparse_proxy(const orc_dims* D, const void* q, const void* K,
                     const void* V, const int32_t* idx, const int32_t* idx_len,
                     const float* logw, int m, const int32_t* cid, int C,
                     const int32_t* count, const double* sumK,
                     const double* sumV, double* out, double* lse);

/* ---- (c) rank-1 prior [RESA] --------------------------------------------
 * Build from the mean query mu_Q [B, Hq, d] (fp32):
 *   mu_K[g]  = mean of the unit's n keys                      [B, Hkv, d]
 *   P_hj     = scale * <mu_Q_h, k_j>
 *   maxP_h   = max_j P_hj,  sumP_h = sum_j exp(P_hj - maxP_h)  [B, Hq]
 *   O_est_h  = sum_j exp(P_hj - maxP_h) v_j / sumP_h          [B, Hq, d]  */
int orc_prior_build(const orc_dims* D, const void* K, const void* V,
                    const float* mu_Q, double* mu_K, double* O_est,
                    double* maxP, double* sumP);

/* Plain definition, O(n): the prior covers rows [0, prior_n) (the cache as
 * it was when the prior was built; prior_n <= 0 means all n).  With
 * c_h = scale * <q_h - mu_Q_h, mu_K> (mu_K the exact mean of the covered
 * keys), every listed row j weighs exp(logit_hj + w_j), every unlisted
 * covered row weighs lambda * exp(P_hj + c_h), and an unlisted row past
 * prior_n weighs nothing; O = sum w v / sum w. */
int orc_sparse_prior_def(const orc_dims* D, const void* q, const void* K,
                         const void* V, const int32_t* idx,
                         const int32_t* idx_len, const float* logw, int m,
                         const float* mu_Q, double lambda, int prior_n,
                         double* out, double* lse);

/* Delta form, O(|I|) [RESA, Online Aggregator]: from the state built over
 * rows [0, prior_n) (prior_n <= 0: all n), with I' = the listed rows below
 * prior_n,
 *   E  = lambda exp(c_h + maxP_h)
 *   A  = E (sumP O_est - sum_{j in I'} exp(P_j - maxP) v_j)
 *   Bt = max(0, E (sumP - sum_{j in I'} exp(P_j - maxP)))
 *   O  = (A + sum_I exp(s_j + w_j) v_j) / (Bt + sum_I exp(s_j + w_j)).
 * Requires distinct positions in each unit's list. */
int orc_sparse_prior(const orc_dims* D, const void* q, const void* K,
                     const void* V, const int32_t* idx, const int32_t* idx_len,
                     const float* logw, int m, const float* mu_Q,
                     double lambda, int prior_n, const double* mu_K, const double* O_est,
                     const double* maxP, const double* sumP,
                     double* out, double* lse);

/* ---- (b) sampled tail [vATT] ---------------------------------------------
 * SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): state advances by the
 * golden-ratio increment and each output is the state passed through the
 * published 64-bit finaliser. */
uint64_t orc_splitmix64_next(uint64_t* state);

/* Key of unit u = s*Hkv + g: output number u (0-based) of SplitMix64 seeded
 * with `seed`.  Draw k of the unit: output number k of SplitMix64 seeded with
 * the key, mapped to a tail rank floor(x * n_s / 2^64). */
uint64_t orc_unit_key(uint64_t seed, int64_t unit);
int64_t orc_draw_rank(uint64_t key, int64_t k, int64_t n_s);

/* Tail rank -> position: the u-th (0-based) position of [0, n) that is not
 * in the sorted, duplicate-free list If[0..mf). */
int64_t orc_tail_pos(const int32_t* If, int mf, int64_t u);

/* CLT budget from explicit statistics [vATT] (one head):
 *   rD[k], rN[k*d + i] for k < b0: the b0 base-sample terms exp(s - M) and
 *   exp(s - M) v; Df, Nf[d]: exact sums over the deterministic set.
 * Returns the real budget b* = max(b_D, b_N) (before ceiling/clamping). */
double orc_budget_from_terms(int d, int b0, const double* rD, const double* rN,
                             double Df, const double* Nf, int64_t n_s,
                             double eps, double z);

/* Verified budget [vATT, verified-SDPA: Lemma 4.2 and Theorem 4.3] for one
 * head from the same statistics: the output's relative error eps (< 1) at
 * confidence 1 - delta, the smallest over the nz given splits
 * delta = d_N + d_D of (2 (z_N a + z_D c) / eps)^2 with
 * z_split[2k] = Phi^-1(1 - d_N/2), z_split[2k+1] = Phi^-1(1 - d_D/2),
 * a = n_s sqrt(Tr Sigma_N) / |N_hat|, c = n_s sigma_D / D_hat (the eps split
 * that balances b_N and b_D for each delta split). Returns the real budget. */
double orc_budget_verified_from_terms(int d, int b0, const double* rD,
                                      const double* rN, double Df,
                                      const double* Nf, int64_t n_s, double eps,
                                      int nz, const double* z_split);

/* Full sampled estimator.  idx/idx_len carry the deterministic set I_f
 * (sorted ascending, distinct).  Per unit: b0 base draws give the budget
 * b = min(n_s, max(1, ceil(max over the group's heads of b*))); draws
 * b0 .. b0+b-1 form I_dyn with log-weight ln(n_s / b).  Outputs b [B,Hkv],
 * b* [B,Hkv] (real, before rounding), the sampled positions
 * [B, Hkv, b_cap] (first min(b, b_cap) written), and out/lse.
 * If n_s == 0 no draw is made and b = 0. */
int orc_sampled(const orc_dims* D, const void* q, const void* K, const void* V,
                const int32_t* idx, const int32_t* idx_len, int m,
                double eps, double z, int b0, uint64_t seed,
                int32_t* b_out, double* bstar_out, int32_t* samples_out,
                int b_cap, double* out, double* lse);

/* The same with the verified budget (orc_budget_verified_from_terms per
 * head; z_split holds nz >= 1 pairs, eps < 1). */
int orc_sampled_verified(const orc_dims* D, const void* q, const void* K,
                         const void* V, const int32_t* idx,
                         const int32_t* idx_len, int m, double eps, int nz,
                         const double* z_split, int b0, uint64_t seed,
                         int32_t* b_out, double* bstar_out,
                         int32_t* samples_out, int b_cap, double* out,
                         double* lse);

/* Estimator terms for a forced budget b (the unbiasedness study):
 * returns per query head the unnormalised, unshifted estimates
 * Dhat = D_f + (n_s/b) sum_{I_dyn} exp(s) and Nhat[d] likewise, where I_dyn
 * is draws b0 .. b0+b-1 of the unit's stream. */
int orc_sampled_fixed_b(const orc_dims* D, const void* q, const void* K,
                        const void* V, const int32_t* idx,
                        const int32_t* idx_len, int m, int b0, int b,
                        uint64_t seed, double* Dhat, double* Nhat);

#ifdef __cplusplus
}
#endif
#endif
