/*
 * sda.h -- C ABI of libsda: sparse decode attention with a tail estimate,
 * hand-written HIP kernels for MI355X (gfx950).
 *
 * One decode step of attention reads only a listed subset I of the KV cache
 * (attention sinks + local window + selected top-k rows) and adds back an
 * estimate of the unread tail in the same softmax, in one of three forms:
 *   PROXY   count-aware mean proxies, one virtual token per cluster
 *           ("OpenAttention: One Percent Is Enough with Tail Proxies",
 *           abstract and method stages 04-05);
 *   SAMPLED inverse-probability-weighted uniform samples of the unread rows
 *           with a CLT-sized budget ("vAttention: Verified Sparse Attention
 *           via Sampling", method sections 1-3, eq. 3);
 *   PRIOR   a rank-1 prior O_Est, Z built once from the mean query and merged
 *           in O(|I|) ("RESA: Bringing Back What Sparse Attention Ignores
 *           with Residual Estimation", sections Prior Estimator and Online
 *           Aggregator).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates device memory, keeps no state between calls
 *     and is reentrant.  Scratch memory comes in through (ws, ws_bytes); ask
 *     sda_workspace_bytes() for the size.  Workspace contents need not be
 *     initialised and are not preserved.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Nothing synchronises the host.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns an error status and launches nothing.  A failed launch returns
 *     SDA_EHIP.  Nothing aborts or throws across the ABI.
 *   - Data errors only the device can see (an index out of range, a list
 *     that is not strictly increasing where it must be, an inconsistent
 *     cluster count, samples beyond the caller's buffer) are reported per
 *     (sequence, KV head) unit in the optional `dev_flags` array as the
 *     SDA_FLAG_* bits, OR-ed into the word (clear the array before the
 *     call); the offending entry is skipped, so no access ever leaves the
 *     caller's buffers.  Read the flags after synchronising.
 *   - Layouts (row-major, innermost last):
 *       q        [B, Hq, d]       in dims.dtype
 *       K, V     [B, Hkv, n, d]   in dims.dtype, element strides in dims
 *                                 (stride along d is 1; K and V share the
 *                                 strides, so one interleaved KV buffer
 *                                 [B, Hkv, n, 2, d] works with V = K + d)
 *       idx      [B, Hkv, m] int32 row positions; idx_len [B, Hkv] (or NULL)
 *                 is the number of valid leading entries of each row
 *       logw     [B, Hkv, m] fp32 natural-log weight added to each listed
 *                 row's logit (NULL = 0)
 *       out      [B, Hq, d] fp32;  lse [B, Hq] fp32 = ln(softmax
 *                 denominator), or NULL
 *     Query head h attends with KV head h / (Hq / Hkv).
 *   - The logit of query head h and row j is scale * <q_h, k_j>.
 *   - Supported: d == 128; Hq / Hkv in {1, 2, 4, 8}; dtype bf16 or fp32.
 *   - Rows are read as 16-byte vectors: q, K, V and the fp32 tail state
 *     must be 16-byte aligned (else SDA_EINVAL) and the K/V strides in
 *     bytes multiples of 16 (else SDA_ESHAPE).
 */
#ifndef SDA_H
#define SDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDA_OK = 0,
  SDA_EINVAL = -1,        /* null pointer, bad scalar parameter, bad kind */
  SDA_ESHAPE = -2,        /* inconsistent or non-positive sizes/strides   */
  SDA_EDTYPE = -3,        /* unknown element type                          */
  SDA_EWORKSPACE = -4,    /* workspace missing or smaller than required    */
  SDA_EUNSUPPORTED = -5,  /* valid but not implemented (e.g. d != 128)     */
  SDA_EHIP = -6           /* a HIP call or kernel launch failed            */
} sda_status;

typedef enum { SDA_BF16 = 0, SDA_F32 = 1 } sda_dtype;

typedef enum {
  SDA_TAIL_NONE = 0,
  SDA_TAIL_PROXY = 1,
  SDA_TAIL_PRIOR = 2,
  SDA_TAIL_SAMPLED = 3
} sda_tail_kind;

/* Device-side data error bits, one int32 word per (sequence, KV head). */
enum {
  SDA_FLAG_IDX_RANGE = 1,    /* a listed position outside [0, n): skipped  */
  SDA_FLAG_IDX_ORDER = 2,    /* list not strictly increasing (PROXY, PRIOR,
                                SAMPLED need distinct sorted positions)     */
  SDA_FLAG_SAMPLE_CAP = 4,   /* budget b exceeded b_cap: samples_out holds
                                only the first b_cap draws (the result
                                itself uses all b)                           */
  SDA_FLAG_CLUSTER = 8,      /* cluster id outside [-1, C), or more listed
                                rows in a cluster than its count            */
  SDA_FLAG_LEN = 16          /* idx_len outside [0, m]: clamped            */
};

typedef struct {
  int32_t B, Hq, Hkv, n, d;
  int32_t dtype;                 /* sda_dtype of q, K and V                 */
  int64_t kv_stride_b;           /* element strides of K and V; all three   */
  int64_t kv_stride_h;           /* zero means contiguous [B, Hkv, n, d]    */
  int64_t kv_stride_n;
  float scale;                   /* logit scale; 0 means 1/sqrt(d)          */
} sda_dims;

/* Tail description for sda_sparse_decode_attn.  Fields of kinds other than
 * `kind` are ignored. */
typedef struct {
  int32_t kind;                  /* sda_tail_kind */

  /* PROXY (OpenAttention, method stage 04): per-cluster state from
   * sda_build_tail_proxies.  Every cluster b with n_b = count[b] - (listed
   * rows in b) > 0 adds one entry with key sumK_b' / n_b, value
   * sumV_b' / n_b and logit scale*<q, key> + ln n_b, where the primes
   * denote the sums without the listed rows.  The list must hold distinct
   * positions in increasing order.  Lists of up to 512 entries per unit
   * (384 when 8 query heads share a KV head) run in one workgroup per unit
   * with no workspace, and so do bf16 lists of up to 1024 entries (a
   * second kernel that streams the value rows behind the key rows).  Longer
   * bf16 lists are split across workgroups, each split writing per-cluster
   * listed counts, logit sums and value sums to the workspace
   * (sda_workspace_bytes gives the size).  Longer fp32 lists return
   * SDA_EUNSUPPORTED. */
  int32_t C;                     /* clusters per unit, 1 <= C <= 64         */
  const int32_t* idx_cluster;    /* [B,Hkv,m] cluster of each listed row (as
                                    a per-cluster selector emits it), or
                                    NULL to look it up in cluster_id        */
  const int32_t* cluster_id;     /* [B,Hkv,n] cluster of every row, -1 =
                                    none; used when idx_cluster is NULL      */
  const int32_t* count;          /* [B,Hkv,C]                               */
  const float* sumK;             /* [B,Hkv,C,d]                             */
  const float* sumV;             /* [B,Hkv,C,d]                             */

  /* PRIOR (RESA): state from sda_build_prior over the rows [0, prior_n)
   * the cache held then (the prefill; prior_n = 0 means all n rows).  With
   * c_h = scale*<q_h - mu_Q_h, mu_K> every unlisted row j < prior_n weighs
   * lambda*exp(scale*<mu_Q_h, k_j> + c_h); listed rows weigh exp(logit);
   * rows appended later (j >= prior_n) count only when listed.  Evaluated
   * in O(|I|) by the delta merge.  The list must hold distinct positions in
   * increasing order. */
  const float* mu_Q;             /* [B,Hq,d]  mean (prefill) query          */
  const float* mu_K;             /* [B,Hkv,d] key mean                      */
  const float* O_est;            /* [B,Hq,d]                                */
  const float* maxP;             /* [B,Hq]                                  */
  const float* sumP;             /* [B,Hq]                                  */
  float lambda;                  /* prior weight, >= 0 (0 = plain sparse)   */
  int32_t prior_n;               /* rows the prior covers, 0..n (0 = all)   */

  /* SAMPLED (vAttention): idx/idx_len carry the deterministic set I_f
   * (distinct, increasing).  b0 base draws from the unread rows estimate
   * the statistics; the budget is b = min(n_s, max(1, ceil(max over the
   * group's query heads of max(b_D, b_N)))), b_X = (z n_s sigma_X /
   * (eps |X_hat|))^2; b fresh draws are added with weight n_s / b.
   * Draw k of unit u = s*Hkv + g is the k-th output of SplitMix64 seeded
   * with the u-th output of SplitMix64 seeded with `seed`, mapped to the
   * unread rank floor(x * n_s / 2^64).  Statistics are fp64. */
  double eps;                    /* relative error target, > 0              */
  double z;                      /* Phi^-1(1 - delta/2), > 0                */
  int32_t b0;                    /* base draws, 2 <= b0 <= 1024             */
  uint64_t seed;
  int32_t b_cap;                 /* capacity of samples_out per unit        */
  int32_t* b_out;                /* [B,Hkv] budget b, or NULL               */
  double* bstar_out;             /* [B,Hkv] real budget before rounding, or
                                    NULL                                     */
  int32_t* samples_out;          /* [B,Hkv,b_cap] drawn positions, or NULL  */

  /* SAMPLED, verified budget ("vAttention: Verified Sparse Attention via
   * Sampling", method section 3, verified-SDPA: Lemma 4.2 turns the
   * numerator's (e_N, d_N) and the denominator's (e_D, d_D) guarantees into
   * an output error 2 (e_N + e_D) |N/D| at confidence 1 - (d_N + d_D), and
   * Theorem 4.3 minimises the budget over that allocation).  With nz > 0,
   * eps and delta bound the output itself: per head the budget is the
   * smallest over the nz given splits delta = d_N + d_D of
   * (2 (z_N a + z_D c) / eps)^2, a = n_s sqrt(Tr Sigma_N) / |N_hat|,
   * c = n_s sigma_D / D_hat (the split of eps / 2 that balances b_N and b_D),
   * with z_split[2k] = Phi^-1(1 - d_N/2) and z_split[2k+1] =
   * Phi^-1(1 - d_D/2) for the k-th split; eps < 1, every entry > 0, z is
   * ignored.  nz = 0 keeps the budget above. */
  int32_t nz;                    /* 0..SDA_MAX_Z_SPLITS                      */
  const double* z_split;         /* HOST array [nz][2], read during the call */
} sda_tail;
#define SDA_MAX_Z_SPLITS 64

typedef enum {
  SDA_OP_SPARSE = 0,
  SDA_OP_DENSE = 1,
  SDA_OP_BUILD_PROXIES = 2,
  SDA_OP_BUILD_PRIOR = 3,
  SDA_OP_BUILD_QGS = 4,
  SDA_OP_SELECT_QGS = 5,
  SDA_OP_BUILD_QGC = 6
} sda_op;

/* Workspace bytes an entry point needs for these sizes (m: entries per unit
 * of the index list, C: clusters; ignored where they do not apply).
 * Returns 0 for invalid dims. */
size_t sda_workspace_bytes(const sda_dims* dims, int32_t op, int32_t tail_kind,
                           int32_t m, int32_t C);

/* Count-aware mean proxy state (OpenAttention, method stage 01: the
 * per-cluster count and mean tokens cached once per request; here as sums,
 * and the diagonal-variance token as the sum of squared keys).
 * For each unit and cluster b: count[b] = #{j : cluster_id[j] == b},
 * sumK[b] = sum of those keys, sumV[b] = sum of those values, and, when
 * sumK2 is not NULL, sumK2[b] = sum of their elementwise squared keys (all
 * fp32, [B,Hkv,C,d]).  Sums are deterministic (no atomics): repeated builds
 * give the same bits.
 * cluster_id [B,Hkv,n] int32 in [-1, C); -1 = the row is in no cluster.
 * Ids outside [-1, C) are ignored and flagged in dev_flags.  The workspace
 * size (SDA_OP_BUILD_PROXIES) covers either form. */
sda_status sda_build_tail_proxies(const sda_dims* dims, const void* K, const void* V,
                                  const int32_t* cluster_id, int32_t C,
                                  int32_t* count, float* sumK, float* sumV, float* sumK2,
                                  int32_t* dev_flags, void* ws, size_t ws_bytes,
                                  void* stream);

/* Rank-1 prior state (RESA, Prior Estimator): one extra "typical query"
 * mu_Q [B,Hq,d] (fp32) attends over the whole cache.  Writes
 * mu_K [B,Hkv,d] = key mean, maxP [B,Hq] = max_j scale*<mu_Q_h, k_j>,
 * sumP [B,Hq] = sum_j exp(P_hj - maxP_h) and O_est [B,Hq,d] =
 * sum_j exp(P_hj - maxP_h) v_j / sumP_h (all fp32).  Requires n >= 1. */
sda_status sda_build_prior(const sda_dims* dims, const void* K, const void* V,
                           const float* mu_Q, float* mu_K, float* O_est,
                           float* maxP, float* sumP, void* ws, size_t ws_bytes,
                           void* stream);

/* One decode step of sparse attention over the listed rows plus the tail
 * estimate described by `tail` (NULL or kind NONE = no tail: plain sparse
 * attention with log-weights, duplicates counted as separate terms).
 * A unit whose softmax is empty gets out = 0 and lse = -inf. */
sda_status sda_sparse_decode_attn(const sda_dims* dims, const void* q,
                                  const void* K, const void* V,
                                  const int32_t* idx, const int32_t* idx_len,
                                  const float* logw, int32_t m,
                                  const sda_tail* tail, float* out, float* lse,
                                  int32_t* dev_flags, void* ws, size_t ws_bytes,
                                  void* stream);

/* The same decode step for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the scratch it needs comes from one array of
 * SDA_NOALLOC_SCRATCH_BYTES that the library keeps per GPU until the process
 * ends.  Calls that need more than that (sda_workspace_bytes with
 * SDA_OP_SPARSE) return SDA_EWORKSPACE before any launch.  The call itself
 * allocates nothing.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (other streams, other threads) race: order
 * them on one stream.  The array keeps the last call's contents; the decode
 * initialises what it reads.  A failure to look up the array's device
 * address returns SDA_EHIP. */
#define SDA_NOALLOC_SCRATCH_BYTES (64u << 20)
sda_status sda_sparse_decode_attn_noalloc(const sda_dims* dims, const void* q,
                                          const void* K, const void* V,
                                          const int32_t* idx, const int32_t* idx_len,
                                          const float* logw, int32_t m,
                                          const sda_tail* tail, float* out, float* lse,
                                          int32_t* dev_flags, void* stream);

/* Dense decode attention over all n rows (the speedup reference):
 * out = softmax(scale * q K^T) V per query head, lse = ln denominator. */
sda_status sda_dense_decode_attn(const sda_dims* dims, const void* q,
                                 const void* K, const void* V, float* out,
                                 float* lse, void* ws, size_t ws_bytes,
                                 void* stream);

/* Static description of a status code. */
const char* sda_status_str(int32_t status);

/* Library version, "major.minor.patch". */
const char* sda_version(void);

/* ---- Query-geometry clustering of the keys ------------------------------
 * (OpenAttention, method stage 01 and the settings list: the keys, projected
 * on the top 16 query eigenvectors, are clustered with k-means; C = 64.)
 * Once per request; the ids then feed sda_build_tail_proxies and
 * sda_select_qgs.  Per unit:
 *   - V [B,Hkv,d,16] fp32: the projection basis (orthonormal columns; the
 *     leading 16 columns of the selector's basis);
 *   - coordinates z_j = V^T k_j, the projection summed over d in order in
 *     fp64 (exact products), clamped to |z| <= 2048 (a clamp sets
 *     SDA_FLAG_CLUSTER);
 *   - Lloyd's k-means with C centroids: start at the points of rows
 *     floor((2k + 1) n / (2C)); T passes of "each row to its nearest
 *     centroid (squared distance, its 16 terms added in coordinate order in
 *     fp64, ties to the lower k), each centroid to its rows' mean (an empty
 *     one stays)"; the mean is formed from an exact integer sum of the
 *     coordinates rounded to 2^-32, so it is within 2^-33 of the exact mean
 *     and the same in any order of the rows;
 *   - cluster_id [B,Hkv,n] int32 = the centroid of each row after pass T.
 * The result is reproducible bit for bit.  C in [1, 64] (else
 * SDA_EUNSUPPORTED), T in [1, 1000] (else SDA_EINVAL), n <= 2^20 (else
 * SDA_EUNSUPPORTED); K and V 16-byte aligned.  Workspace: SDA_OP_BUILD_QGC
 * with this C (128 B per row of coordinates). */
sda_status sda_build_qgc_clusters(const sda_dims* dims, const void* K, const float* V, int32_t C,
                                  int32_t T, int32_t* cluster_id, int32_t* dev_flags, void* ws,
                                  size_t ws_bytes, void* stream);

/* ---- Selector in front of the proxy decode ------------------------------
 * (OpenAttention, method stages 02-03 and the settings list: keys coded in
 * int8 per KV head and coordinate and scored in an r = 32 query subspace;
 * an exact-read budget per cluster from the estimated weight error of its
 * mean proxy; each cluster reads its best-scoring rows.)  The page states
 * the stages, not their formulas; the readings taken here are spelled out
 * below. */
#define SDA_QGS_RANK 32

/* Key codes, once per request.  U [B,Hkv,d,32] fp32: the subspace basis of
 * each unit (orthonormal columns; the leading eigenvectors of the queries'
 * second moment).  For every row: y_j = U^T k_j, summed over d in order in
 * fp64 (each product is exact); kmax [B,Hkv,32] fp64 = max_j |y_ji|;
 * codes [B,Hkv,n,32] int8 = rint(127 y_ji / kmax_i), half to even, 0 where
 * kmax_i = 0.  K and codes 16-byte aligned.  Workspace: SDA_OP_BUILD_QGS
 * gives the size with room for the fp64 projections (B*Hkv*n*32*8 bytes
 * beyond the chunk maxima), which spares the quantizing pass recomputing
 * them; a workspace of only the chunk maxima's size (rounded up to 256 bytes)
 * is accepted and recomputes them (the same codes, bit for bit). */
sda_status sda_build_qgs_codes(const sda_dims* dims, const void* K, const float* U,
                               int8_t* codes, double* kmax, void* ws, size_t ws_bytes,
                               void* stream);

typedef struct {
  int32_t n_sink;                /* rows [0, n_sink) are always listed       */
  int32_t n_local;               /* rows [n - n_local, n) are always listed  */
  int32_t E;                     /* rows to pick in between, over clusters   */
  int32_t C;                     /* clusters, 1..64                          */
  const int32_t* cluster_id;     /* [B,Hkv,n] in [-1, C)                     */
  const int32_t* count;          /* [B,Hkv,C]    from sda_build_tail_proxies */
  const float* sumK;             /* [B,Hkv,C,d]  from sda_build_tail_proxies */
  const float* sumK2;            /* [B,Hkv,C,d]  from sda_build_tail_proxies */
  const float* U;                /* [B,Hkv,d,32] the basis given to the codes */
  const int8_t* codes;           /* [B,Hkv,n,32] from sda_build_qgs_codes    */
  const double* kmax;            /* [B,Hkv,32]   from sda_build_qgs_codes    */
} sda_selector;

/* The index set of one decode step, per unit:
 *   - query weights: qt_h = U^T q_h (fp64, in order), w_hi = qt_hi kmax_i,
 *     wq_hi = rint(127 w_hi / max|w|) over the KV group (int8);
 *   - score of row j: S_j = max over the group's heads of
 *     sum_i wq_hi code_ji (exact integer);
 *   - weight error of cluster b (Gaussian logit model, diagonal variance):
 *     zbar = scale <q_h, mu_b>, s2 = scale^2 sum_d q_hd^2 nu_bd
 *     (mu = sumK/N, nu = max(0, sumK2/N - mu^2)),
 *     eps_b = sum_h N_b e^{zbar} (e^{s2/2} - 1) / sum_b' N_b' e^{zbar' + s2'/2};
 *   - budgets: E split in proportion to eps_b by the largest remainder (ties
 *     to the lower b), capped at A_b = members of b in [n_sink, n - n_local);
 *     capped clusters are fixed and the rest split again; with no error left
 *     the remaining capacity weighs; sum q_b = min(E, sum A_b);
 *   - cluster b lists its q_b eligible rows with the largest S_j (ties to
 *     the lower position); rows with cluster id -1 are never picked.
 * Writes idx [B,Hkv,m] ascending (sink, local window and the picked rows),
 * idx_len [B,Hkv], idx_cluster [B,Hkv,m] (cluster of each listed row, -1 if
 * none; entries past idx_len are 0 and -1), and budget [B,Hkv,C] (or NULL).
 * The output feeds sda_sparse_decode_attn with a PROXY tail directly.
 * Requires n <= 2^20 (else SDA_EUNSUPPORTED) and
 * m >= min(n, n_sink + n_local + E) (else SDA_EINVAL).  Cluster ids outside
 * [-1, C) are treated as -1 and flagged.  Workspace: SDA_OP_SELECT_QGS
 * (with this C). */
sda_status sda_select_qgs(const sda_dims* dims, const void* q, const sda_selector* sel,
                          int32_t m, int32_t* idx, int32_t* idx_len, int32_t* idx_cluster,
                          int32_t* budget, int32_t* dev_flags, void* ws, size_t ws_bytes,
                          void* stream);

/* ---- Measurement aid ----------------------------------------------------
 * Not part of the method: reads the listed K and V rows of every unit (the
 * first m entries of idx per unit; positions outside [0, n) are skipped)
 * and, when state_bytes > 0, state_bytes bytes of per-unit state at
 * state + u * state_bytes, with `parts` workgroups of `waves` waves per unit
 * (waves in {4, 8, 16}, parts in [1, 16]), and writes the XOR of every
 * 32-bit word a wave loaded to checksum[(u * parts + part) * waves + wave]
 * ([B * Hkv * parts * waves] uint32).  It computes nothing else: timing it
 * beside sda_sparse_decode_attn gives the rate at which the memory system
 * delivers the same rows in that launch shape.
 * Partition: part p takes list entries [p*EP, (p+1)*EP) (EP = ceil(m /
 * parts)), its wave w the run [w*EW, (w+1)*EW) of those (EW = ceil(EP /
 * waves)); part p takes the state bytes [p*SP, (p+1)*SP) (SP = ceil(
 * state_bytes / parts) rounded up to 16), thread t of the part the 16-byte
 * chunks at offsets p*SP + 16 t + k*16*64*waves that end inside the share,
 * XOR-ed into the checksum of wave t / 64.
 * bf16 rows only (else SDA_EUNSUPPORTED); SDA_EUNSUPPORTED also when a row
 * group would hold more rows than the kernel keeps in registers (24 at 4 or
 * 8 waves, 12 at 16).  K, V and state 16-byte aligned. */
sda_status sda_gather_rows(const sda_dims* dims, const void* K, const void* V, const int32_t* idx,
                           int32_t m, const void* state, int64_t state_bytes, int32_t waves,
                           int32_t parts, uint32_t* checksum, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SDA_H */
