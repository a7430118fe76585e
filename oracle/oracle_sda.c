/*
 * oracle_sda.c -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY; see
 * oracle_sda.h for what may use it and for the page citations).
 *
 * Everything here is written to be checked by eye against the pages: one
 * loop per definition, no blocking, no fusion, doubles throughout.  The only
 * parallelism is an OpenMP loop over independent (sequence, KV head) units.
 */
#include "oracle_sda.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* element access                                                            */

static double elem(int dtype, const void* p, int64_t i) {
  if (dtype == ORC_BF16) {
    /* a bf16 value is the upper half of an fp32 bit pattern */
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

static int64_t kv_row(const orc_dims* D, int s, int g, int64_t j) {
  return (((int64_t)s * D->Hkv + g) * D->n + j) * D->d;
}

static int64_t q_row(const orc_dims* D, int s, int h) {
  return ((int64_t)s * D->Hq + h) * D->d;
}

/* scale * <q_h, k_j> */
static double logit(const orc_dims* D, const void* q, const void* K, int s,
                    int h, int g, int64_t j) {
  int64_t qo = q_row(D, s, h), ko = kv_row(D, s, g, j);
  double acc = 0.0;
  for (int i = 0; i < D->d; ++i)
    acc += elem(D->dtype, q, qo + i) * elem(D->dtype, K, ko + i);
  return (double)D->scale * acc;
}

static int check_dims(const orc_dims* D) {
  if (!D || D->B < 1 || D->Hkv < 1 || D->Hq < 1 || D->n < 0 || D->d < 1)
    return -1;
  if (D->Hq % D->Hkv != 0) return -1;
  if (D->dtype != ORC_BF16 && D->dtype != ORC_F32) return -1;
  return 0;
}

static int unit_len(const int32_t* idx_len, int u, int m) {
  return idx_len ? idx_len[u] : m;
}

void orc_set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* A weighted sum  sum_t exp(x_t) v_t / sum_t exp(x_t)  over a list of
 * (log-weight, row) terms, evaluated with the max shift.  `vrow[t]` is the
 * element offset of the value row of term t, or -1 for a term whose value
 * vector is given explicitly in `vexp[t*d ..]`.                             */

typedef struct {
  int64_t cap, cnt;
  double* x;      /* log-weights */
  int64_t* vrow;  /* offsets into V, or -1 */
  double* vexp;   /* explicit value vectors (d per term) */
} terms_t;

static int terms_init(terms_t* T, int64_t cap, int d) {
  T->cap = cap > 0 ? cap : 1;
  T->cnt = 0;
  T->x = (double*)malloc(sizeof(double) * T->cap);
  T->vrow = (int64_t*)malloc(sizeof(int64_t) * T->cap);
  T->vexp = (double*)malloc(sizeof(double) * T->cap * d);
  return (T->x && T->vrow && T->vexp) ? 0 : -1;
}

static void terms_free(terms_t* T) {
  free(T->x);
  free(T->vrow);
  free(T->vexp);
}

static void terms_add_row(terms_t* T, double x, int64_t vrow) {
  T->x[T->cnt] = x;
  T->vrow[T->cnt] = vrow;
  T->cnt++;
}

static void terms_add_vec(terms_t* T, double x, const double* v, int d) {
  T->x[T->cnt] = x;
  T->vrow[T->cnt] = -1;
  memcpy(T->vexp + T->cnt * d, v, sizeof(double) * d);
  T->cnt++;
}

/* out[d] and *lse for the softmax-weighted value sum over the terms. */
static void terms_softmax(const terms_t* T, const orc_dims* D, const void* V,
                          double* out, double* lse) {
  int d = D->d;
  double M = -INFINITY;
  for (int64_t t = 0; t < T->cnt; ++t)
    if (T->x[t] > M) M = T->x[t];
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  if (T->cnt == 0 || M == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double den = 0.0;
  for (int64_t t = 0; t < T->cnt; ++t) {
    double w = exp(T->x[t] - M);
    den += w;
    if (T->vrow[t] >= 0) {
      for (int i = 0; i < d; ++i) out[i] += w * elem(D->dtype, V, T->vrow[t] + i);
    } else {
      for (int i = 0; i < d; ++i) out[i] += w * T->vexp[t * d + i];
    }
  }
  for (int i = 0; i < d; ++i) out[i] /= den;
  *lse = M + log(den);
}

/* ------------------------------------------------------------------------ */
/* dense                                                                     */

int orc_dense(const orc_dims* D, const void* q, const void* K, const void* V,
              double* out, double* lse) {
  if (check_dims(D)) return -1;
  int G = D->Hq / D->Hkv;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    terms_t T;
    if (terms_init(&T, D->n, D->d)) { err |= 1; continue; }
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      T.cnt = 0;
      for (int64_t j = 0; j < D->n; ++j)
        terms_add_row(&T, logit(D, q, K, s, h, g, j), kv_row(D, s, g, j));
      terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
    }
    terms_free(&T);
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* sparse over an index list                                                  */

static int check_list(const orc_dims* D, const int32_t* idx, int len) {
  for (int t = 0; t < len; ++t)
    if (idx[t] < 0 || idx[t] >= D->n) return -1;
  return 0;
}

static int list_is_set(const orc_dims* D, const int32_t* idx, int len,
                       unsigned char* mark) {
  memset(mark, 0, (size_t)D->n);
  for (int t = 0; t < len; ++t) {
    if (mark[idx[t]]) return 0;
    mark[idx[t]] = 1;
  }
  return 1;
}

int orc_sparse(const orc_dims* D, const void* q, const void* K, const void* V,
               const int32_t* idx, const int32_t* idx_len, const float* logw,
               int m, double* out, double* lse) {
  if (check_dims(D) || m < 0) return -1;
  int G = D->Hq / D->Hkv;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int len = unit_len(idx_len, u, m);
    const int32_t* I = idx + (int64_t)u * m;
    const float* w = logw ? logw + (int64_t)u * m : NULL;
    if (len < 0 || len > m || check_list(D, I, len)) { err |= 1; continue; }
    terms_t T;
    if (terms_init(&T, len, D->d)) { err |= 2; continue; }
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      T.cnt = 0;
      for (int t = 0; t < len; ++t)
        terms_add_row(&T, logit(D, q, K, s, h, g, I[t]) + (w ? (double)w[t] : 0.0),
                      kv_row(D, s, g, I[t]));
      terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
    }
    terms_free(&T);
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* (a) count-aware mean proxies                                              */

int orc_proxy_build(const orc_dims* D, const void* K, const void* V,
                    const int32_t* cid, int C,
                    int32_t* count, double* sumK, double* sumV) {
  if (check_dims(D) || C < 1) return -1;
  int U = D->B * D->Hkv, d = D->d;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    const int32_t* c = cid + (int64_t)u * D->n;
    int32_t* cnt = count + (int64_t)u * C;
    double* sk = sumK + (int64_t)u * C * d;
    double* sv = sumV + (int64_t)u * C * d;
    for (int b = 0; b < C; ++b) cnt[b] = 0;
    for (int64_t i = 0; i < (int64_t)C * d; ++i) sk[i] = sv[i] = 0.0;
    for (int64_t j = 0; j < D->n; ++j) {
      int b = c[j];
      if (b == -1) continue;
      if (b < 0 || b >= C) { err |= 1; break; }
      cnt[b] += 1;
      int64_t r = kv_row(D, s, g, j);
      for (int i = 0; i < d; ++i) {
        sk[(int64_t)b * d + i] += elem(D->dtype, K, r + i);
        sv[(int64_t)b * d + i] += elem(D->dtype, V, r + i);
      }
    }
  }
  return err ? -2 : 0;
}

/* One proxy term: key mean km, value mean vm, n_b unread members. */
static void add_proxy(terms_t* T, const orc_dims* D, const void* q, int s,
                      int h, const double* km, const double* vm, int64_t nb) {
  double acc = 0.0;
  for (int i = 0; i < D->d; ++i) acc += elem(D->dtype, q, q_row(D, s, h) + i) * km[i];
  terms_add_vec(T, (double)D->scale * acc + log((double)nb), vm, D->d);
}

int orc_sparse_proxy_def(const orc_dims* D, const void* q, const void* K,
                         const void* V, const int32_t* idx,
                         const int32_t* idx_len, const float* logw, int m,
                         const int32_t* cid, int C, double* out, double* lse) {
  if (check_dims(D) || m < 0 || C < 1) return -1;
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int len = unit_len(idx_len, u, m);
    const int32_t* I = idx + (int64_t)u * m;
    const float* w = logw ? logw + (int64_t)u * m : NULL;
    const int32_t* c = cid + (int64_t)u * D->n;
    if (len < 0 || len > m || check_list(D, I, len)) { err |= 1; continue; }
    unsigned char* read = (unsigned char*)calloc((size_t)D->n + 1, 1);
    int64_t* nb = (int64_t*)calloc((size_t)C, sizeof(int64_t));
    double* km = (double*)calloc((size_t)C * d, sizeof(double));
    double* vm = (double*)calloc((size_t)C * d, sizeof(double));
    terms_t T;
    if (!read || !nb || !km || !vm || terms_init(&T, (int64_t)len + C, d)) {
      err |= 2;
      free(read); free(nb); free(km); free(vm);
      continue;
    }
    for (int t = 0; t < len; ++t) read[I[t]] = 1;
    /* unread members of each cluster: count, key mean, value mean */
    for (int64_t j = 0; j < D->n; ++j) {
      int b = c[j];
      if (b == -1 || read[j]) continue;
      if (b < 0 || b >= C) { err |= 1; break; }
      nb[b] += 1;
      int64_t r = kv_row(D, s, g, j);
      for (int i = 0; i < d; ++i) {
        km[(int64_t)b * d + i] += elem(D->dtype, K, r + i);
        vm[(int64_t)b * d + i] += elem(D->dtype, V, r + i);
      }
    }
    for (int b = 0; b < C; ++b)
      for (int i = 0; i < d && nb[b] > 0; ++i) {
        km[(int64_t)b * d + i] /= (double)nb[b];
        vm[(int64_t)b * d + i] /= (double)nb[b];
      }
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      T.cnt = 0;
      for (int t = 0; t < len; ++t)
        terms_add_row(&T, logit(D, q, K, s, h, g, I[t]) + (w ? (double)w[t] : 0.0),
                      kv_row(D, s, g, I[t]));
      for (int b = 0; b < C; ++b)
        if (nb[b] > 0) add_proxy(&T, D, q, s, h, km + (int64_t)b * d, vm + (int64_t)b * d, nb[b]);
      terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
    }
    terms_free(&T);
    free(read); free(nb); free(km); free(vm);
  }
  return err ? -2 : 0;
}

int orc_sparse_proxy(const orc_dims* D, const void* q, const void* K,
                     const void* V, const int32_t* idx, const int32_t* idx_len,
                     const float* logw, int m, const int32_t* cid, int C,
                     const int32_t* count, const double* sumK,
                     const double* sumV, double* out, double* lse) {
  if (check_dims(D) || m < 0 || C < 1) return -1;
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int len = unit_len(idx_len, u, m);
    const int32_t* I = idx + (int64_t)u * m;
    const float* w = logw ? logw + (int64_t)u * m : NULL;
    const int32_t* c = cid + (int64_t)u * D->n;
    if (len < 0 || len > m || check_list(D, I, len)) { err |= 1; continue; }
    unsigned char* mark = (unsigned char*)malloc((size_t)D->n + 1);
    int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * C);
    double* km = (double*)malloc(sizeof(double) * C * d);
    double* vm = (double*)malloc(sizeof(double) * C * d);
    terms_t T;
    if (!mark || !nb || !km || !vm || terms_init(&T, (int64_t)len + C, d)) {
      err |= 2;
      free(mark); free(nb); free(km); free(vm);
      continue;
    }
    if (!list_is_set(D, I, len, mark)) {
      err |= 4;
    } else {
      /* start from the whole cluster and take the listed rows away */
      for (int b = 0; b < C; ++b) nb[b] = count[(int64_t)u * C + b];
      memcpy(km, sumK + (int64_t)u * C * d, sizeof(double) * C * d);
      memcpy(vm, sumV + (int64_t)u * C * d, sizeof(double) * C * d);
      for (int t = 0; t < len; ++t) {
        int b = c[I[t]];
        if (b == -1) continue;
        nb[b] -= 1;
        int64_t r = kv_row(D, s, g, I[t]);
        for (int i = 0; i < d; ++i) {
          km[(int64_t)b * d + i] -= elem(D->dtype, K, r + i);
          vm[(int64_t)b * d + i] -= elem(D->dtype, V, r + i);
        }
      }
      for (int b = 0; b < C; ++b)
        for (int i = 0; i < d && nb[b] > 0; ++i) {
          km[(int64_t)b * d + i] /= (double)nb[b];
          vm[(int64_t)b * d + i] /= (double)nb[b];
        }
      for (int hh = 0; hh < G; ++hh) {
        int h = g * G + hh;
        T.cnt = 0;
        for (int t = 0; t < len; ++t)
          terms_add_row(&T, logit(D, q, K, s, h, g, I[t]) + (w ? (double)w[t] : 0.0),
                        kv_row(D, s, g, I[t]));
        for (int b = 0; b < C; ++b)
          if (nb[b] > 0) add_proxy(&T, D, q, s, h, km + (int64_t)b * d, vm + (int64_t)b * d, nb[b]);
        terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
      }
    }
    terms_free(&T);
    free(mark); free(nb); free(km); free(vm);
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* (c) rank-1 prior                                                          */

/* scale * <mu_Q_h, k_j> */
static double prior_logit(const orc_dims* D, const float* mu_Q, const void* K,
                          int s, int h, int g, int64_t j) {
  int64_t qo = q_row(D, s, h), ko = kv_row(D, s, g, j);
  double acc = 0.0;
  for (int i = 0; i < D->d; ++i) acc += (double)mu_Q[qo + i] * elem(D->dtype, K, ko + i);
  return (double)D->scale * acc;
}

/* c_h = scale * <q_h - mu_Q_h, mu_K> */
static double bias_shift(const orc_dims* D, const void* q, const float* mu_Q,
                         const double* muK, int s, int h) {
  int64_t qo = q_row(D, s, h);
  double acc = 0.0;
  for (int i = 0; i < D->d; ++i)
    acc += (elem(D->dtype, q, qo + i) - (double)mu_Q[qo + i]) * muK[i];
  return (double)D->scale * acc;
}

int orc_prior_build(const orc_dims* D, const void* K, const void* V,
                    const float* mu_Q, double* mu_K, double* O_est,
                    double* maxP, double* sumP) {
  if (check_dims(D) || D->n < 1) return -1;
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    double* mk = mu_K + (int64_t)u * d;
    for (int i = 0; i < d; ++i) mk[i] = 0.0;
    for (int64_t j = 0; j < D->n; ++j)
      for (int i = 0; i < d; ++i) mk[i] += elem(D->dtype, K, kv_row(D, s, g, j) + i);
    for (int i = 0; i < d; ++i) mk[i] /= (double)D->n;

    double* P = (double*)malloc(sizeof(double) * D->n);
    if (!P) { err |= 2; continue; }
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      double M = -INFINITY;
      for (int64_t j = 0; j < D->n; ++j) {
        P[j] = prior_logit(D, mu_Q, K, s, h, g, j);
        if (P[j] > M) M = P[j];
      }
      double Z = 0.0;
      double* o = O_est + q_row(D, s, h);
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      for (int64_t j = 0; j < D->n; ++j) {
        double e = exp(P[j] - M);
        Z += e;
        for (int i = 0; i < d; ++i) o[i] += e * elem(D->dtype, V, kv_row(D, s, g, j) + i);
      }
      for (int i = 0; i < d; ++i) o[i] /= Z;
      maxP[(int64_t)s * D->Hq + h] = M;
      sumP[(int64_t)s * D->Hq + h] = Z;
    }
    free(P);
  }
  return err ? -2 : 0;
}

int orc_sparse_prior_def(const orc_dims* D, const void* q, const void* K,
                         const void* V, const int32_t* idx,
                         const int32_t* idx_len, const float* logw, int m,
                         const float* mu_Q, double lambda, int prior_n,
                         double* out, double* lse) {
  if (check_dims(D) || m < 0 || lambda < 0.0 || prior_n > D->n) return -1;
  const int64_t n0 = prior_n > 0 ? prior_n : D->n;   /* rows the prior covers */
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int len = unit_len(idx_len, u, m);
    const int32_t* I = idx + (int64_t)u * m;
    const float* w = logw ? logw + (int64_t)u * m : NULL;
    if (len < 0 || len > m || check_list(D, I, len)) { err |= 1; continue; }
    unsigned char* mark = (unsigned char*)malloc((size_t)D->n + 1);
    double* muK = (double*)calloc((size_t)d, sizeof(double));
    terms_t T;
    if (!mark || !muK || terms_init(&T, (int64_t)D->n + len, d)) {
      err |= 2; free(mark); free(muK); continue;
    }
    if (!list_is_set(D, I, len, mark)) {
      err |= 4;
    } else {
      for (int64_t j = 0; j < n0; ++j)
        for (int i = 0; i < d; ++i) muK[i] += elem(D->dtype, K, kv_row(D, s, g, j) + i);
      for (int i = 0; i < d; ++i) muK[i] /= (double)n0;
      for (int hh = 0; hh < G; ++hh) {
        int h = g * G + hh;
        double c = bias_shift(D, q, mu_Q, muK, s, h);
        T.cnt = 0;
        for (int t = 0; t < len; ++t)
          terms_add_row(&T, logit(D, q, K, s, h, g, I[t]) + (w ? (double)w[t] : 0.0),
                        kv_row(D, s, g, I[t]));
        if (lambda > 0.0)
          for (int64_t j = 0; j < n0; ++j)
            if (!mark[j])
              terms_add_row(&T, log(lambda) + prior_logit(D, mu_Q, K, s, h, g, j) + c,
                            kv_row(D, s, g, j));
        terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
      }
    }
    terms_free(&T);
    free(mark); free(muK);
  }
  return err ? -2 : 0;
}

int orc_sparse_prior(const orc_dims* D, const void* q, const void* K,
                     const void* V, const int32_t* idx, const int32_t* idx_len,
                     const float* logw, int m, const float* mu_Q,
                     double lambda, int prior_n, const double* mu_K, const double* O_est,
                     const double* maxP, const double* sumP,
                     double* out, double* lse) {
  if (check_dims(D) || m < 0 || lambda < 0.0 || prior_n > D->n) return -1;
  const int64_t n0 = prior_n > 0 ? prior_n : D->n;   /* rows the prior covers */
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int len = unit_len(idx_len, u, m);
    const int32_t* I = idx + (int64_t)u * m;
    const float* w = logw ? logw + (int64_t)u * m : NULL;
    if (len < 0 || len > m || check_list(D, I, len)) { err |= 1; continue; }
    unsigned char* mark = (unsigned char*)malloc((size_t)D->n + 1);
    double* SPv = (double*)malloc(sizeof(double) * d);
    double* num = (double*)malloc(sizeof(double) * d);
    double* x = (double*)malloc(sizeof(double) * (len > 0 ? len : 1));
    if (!mark || !SPv || !num || !x) {
      err |= 2; free(mark); free(SPv); free(num); free(x); continue;
    }
    if (!list_is_set(D, I, len, mark)) {
      err |= 4;
    } else {
      for (int hh = 0; hh < G; ++hh) {
        int h = g * G + hh;
        int64_t hq = (int64_t)s * D->Hq + h;
        double c = bias_shift(D, q, mu_Q, mu_K + (int64_t)u * d, s, h);
        /* the listed rows' prior terms, shifted by maxP */
        double SP = 0.0;
        for (int i = 0; i < d; ++i) SPv[i] = 0.0;
        for (int t = 0; t < len; ++t) {
          if (I[t] >= n0) continue;   /* a row the prior does not cover */
          double e = exp(prior_logit(D, mu_Q, K, s, h, g, I[t]) - maxP[hq]);
          SP += e;
          for (int i = 0; i < d; ++i) SPv[i] += e * elem(D->dtype, V, kv_row(D, s, g, I[t]) + i);
        }
        /* exact logits of the listed rows */
        double Mx = -INFINITY;
        for (int t = 0; t < len; ++t) {
          x[t] = logit(D, q, K, s, h, g, I[t]) + (w ? (double)w[t] : 0.0);
          if (x[t] > Mx) Mx = x[t];
        }
        /* common shift: the larger of the exact part and the prior mass */
        double Ms = Mx;
        double logprior = -INFINITY;
        if (lambda > 0.0) {
          logprior = log(lambda) + c + maxP[hq];
          if (logprior + log(sumP[hq]) > Ms) Ms = logprior + log(sumP[hq]);
        }
        double E = (lambda > 0.0) ? exp(logprior - Ms) : 0.0;
        double Bt = E * (sumP[hq] - SP);
        double den = 0.0;
        for (int i = 0; i < d; ++i) num[i] = 0.0;
        if (Bt > 0.0) {
          den = Bt;
          for (int i = 0; i < d; ++i)
            num[i] = E * (sumP[hq] * O_est[q_row(D, s, h) + i] - SPv[i]);
        }
        for (int t = 0; t < len; ++t) {
          double e = exp(x[t] - Ms);
          den += e;
          for (int i = 0; i < d; ++i) num[i] += e * elem(D->dtype, V, kv_row(D, s, g, I[t]) + i);
        }
        double* o = out + q_row(D, s, h);
        if (den > 0.0) {
          for (int i = 0; i < d; ++i) o[i] = num[i] / den;
          lse[hq] = Ms + log(den);
        } else {
          for (int i = 0; i < d; ++i) o[i] = 0.0;
          lse[hq] = -INFINITY;
        }
      }
    }
    free(mark); free(SPv); free(num); free(x);
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* (b) sampled tail                                                          */

static const uint64_t GOLDEN_GAMMA = 0x9E3779B97F4A7C15ULL;

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t orc_splitmix64_next(uint64_t* state) {
  *state += GOLDEN_GAMMA;
  return mix64(*state);
}

/* output number k (0-based) of a generator seeded with `seed` */
static uint64_t splitmix64_at(uint64_t seed, uint64_t k) {
  uint64_t state = seed;
  /* stepping k+1 times is the definition; k*gamma is the same state */
  state += (k + 1) * GOLDEN_GAMMA;
  return mix64(state);
}

uint64_t orc_unit_key(uint64_t seed, int64_t unit) {
  return splitmix64_at(seed, (uint64_t)unit);
}

int64_t orc_draw_rank(uint64_t key, int64_t k, int64_t n_s) {
  uint64_t x = splitmix64_at(key, (uint64_t)k);
  /* floor(x * n_s / 2^64): the high half of the 128-bit product */
  unsigned __int128 p = (unsigned __int128)x * (unsigned __int128)(uint64_t)n_s;
  return (int64_t)(p >> 64);
}

int64_t orc_tail_pos(const int32_t* If, int mf, int64_t u) {
  /* walk the gaps between listed positions in order */
  int64_t prev = 0;  /* first position not yet accounted for */
  for (int i = 0; i < mf; ++i) {
    int64_t gap = (int64_t)If[i] - prev;  /* tail positions before If[i] */
    if (u < gap) return prev + u;
    u -= gap;
    prev = (int64_t)If[i] + 1;
  }
  return prev + u;
}

/* The base sample's statistics for one head: the denominator terms'
 * variance varD and estimate Dhat, the numerator terms' covariance trace trN
 * and the estimate's norm normN (unbiased sample moments over b0 draws). */
static void budget_stats(int d, int b0, const double* rD, const double* rN,
                         double Df, const double* Nf, int64_t n_s,
                         double* varD_out, double* Dhat_out, double* trN_out,
                         double* normN_out) {
  double mD = 0.0;
  for (int k = 0; k < b0; ++k) mD += rD[k];
  mD /= (double)b0;
  double varD = 0.0;
  for (int k = 0; k < b0; ++k) varD += (rD[k] - mD) * (rD[k] - mD);
  varD /= (double)(b0 - 1);

  double trN = 0.0, normN2 = 0.0;
  for (int i = 0; i < d; ++i) {
    double mNi = 0.0;
    for (int k = 0; k < b0; ++k) mNi += rN[(int64_t)k * d + i];
    mNi /= (double)b0;
    for (int k = 0; k < b0; ++k) {
      double e = rN[(int64_t)k * d + i] - mNi;
      trN += e * e;
    }
    double Nhat_i = Nf[i] + (double)n_s * mNi;
    normN2 += Nhat_i * Nhat_i;
  }
  trN /= (double)(b0 - 1);
  *varD_out = varD;
  *Dhat_out = Df + (double)n_s * mD;
  *trN_out = trN;
  *normN_out = sqrt(normN2);
}

double orc_budget_from_terms(int d, int b0, const double* rD, const double* rN,
                             double Df, const double* Nf, int64_t n_s,
                             double eps, double z) {
  double varD, Dhat, trN, normN;
  budget_stats(d, b0, rD, rN, Df, Nf, n_s, &varD, &Dhat, &trN, &normN);

  /* CLT lemma with tau = eps * |estimate|, for the denominator and the
   * numerator; the budget is the larger of the two (Lemma 4.2). */
  double bD = 0.0, bN = 0.0;
  if (varD > 0.0) {
    double t = z * (double)n_s * sqrt(varD) / (eps * Dhat);
    bD = t * t;
  }
  if (trN > 0.0) {
    if (normN > 0.0) {
      double t = z * (double)n_s * sqrt(trN) / (eps * normN);
      bN = t * t;
    } else {
      bN = INFINITY;
    }
  }
  return bD > bN ? bD : bN;
}

double orc_budget_verified_from_terms(int d, int b0, const double* rD,
                                      const double* rN, double Df,
                                      const double* Nf, int64_t n_s, double eps,
                                      int nz, const double* z_split) {
  double varD, Dhat, trN, normN;
  budget_stats(d, b0, rD, rN, Df, Nf, n_s, &varD, &Dhat, &trN, &normN);
  /* The CLT lemma's budget for a target tau_X = e_X |X| at confidence
   * 1 - d_X is (z_X n_s sigma_X / (e_X |X|))^2, z_X = Phi^-1(1 - d_X/2):
   * with a = n_s sqrt(Tr) / |N| and c = n_s sigma_D / D, b_N = (z_N a / e_N)^2
   * and b_D = (z_D c / e_D)^2.  Lemma 4.2 turns (e_N, d_N) and (e_D, d_D)
   * into a relative error 2 (e_N + e_D) of the output with probability at
   * least 1 - (d_N + d_D), so the output's (eps, delta) needs
   * e_N + e_D = eps / 2 and d_N + d_D = delta.  For one split of delta,
   * max(b_N, b_D) over e_N + e_D = eps / 2 is smallest where the two are
   * equal, e_N / e_D = z_N a / (z_D c), which gives
   * (2 (z_N a + z_D c) / eps)^2; the budget is the smallest of these over
   * the given splits of delta (Theorem 4.3: the budget minimised over the
   * allocation of (eps', delta')). */
  double a = 0.0, c = 0.0;
  if (trN > 0.0) a = normN > 0.0 ? (double)n_s * sqrt(trN) / normN : INFINITY;
  if (varD > 0.0) c = (double)n_s * sqrt(varD) / Dhat;
  double best = INFINITY;
  for (int k = 0; k < nz; ++k) {
    double t = 2.0 * (z_split[2 * k] * a + z_split[2 * k + 1] * c) / eps;
    double v = t * t;
    if (v < best) best = v;
  }
  if (a == 0.0 && c == 0.0) best = 0.0;
  return best;
}

static int64_t budget_round(double bstar, int64_t n_s) {
  if (!(bstar < (double)n_s)) return n_s;  /* also catches inf / nan */
  double c = ceil(bstar);
  int64_t b = (int64_t)c;
  if (b < 1) b = 1;
  if (b > n_s) b = n_s;
  return b;
}

static int check_sorted_set(const orc_dims* D, const int32_t* I, int len) {
  for (int t = 0; t < len; ++t) {
    if (I[t] < 0 || I[t] >= D->n) return -1;
    if (t > 0 && I[t] <= I[t - 1]) return -1;
  }
  return 0;
}

static int sampled_impl(const orc_dims* D, const void* q, const void* K,
                        const void* V, const int32_t* idx,
                        const int32_t* idx_len, int m, double eps, double z,
                        int nz, const double* z_split, int b0, uint64_t seed,
                        int32_t* b_out, double* bstar_out, int32_t* samples_out,
                        int b_cap, double* out, double* lse) {
  if (check_dims(D) || m < 0 || b0 < 2 || !(eps > 0.0) || b_cap < 0) return -1;
  if (nz == 0 && !(z > 0.0)) return -1;
  if (nz < 0 || (nz > 0 && (!z_split || !(eps < 1.0)))) return -1;
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int mf = unit_len(idx_len, u, m);
    const int32_t* If = idx + (int64_t)u * m;
    if (mf < 0 || mf > m || check_sorted_set(D, If, mf)) { err |= 1; continue; }
    int64_t n_s = (int64_t)D->n - mf;
    uint64_t key = orc_unit_key(seed, u);

    if (n_s == 0) {
      /* nothing unread: the deterministic set is exact */
      b_out[u] = 0;
      if (bstar_out) bstar_out[u] = 0.0;
      terms_t T;
      if (terms_init(&T, mf, d)) { err |= 2; continue; }
      for (int hh = 0; hh < G; ++hh) {
        int h = g * G + hh;
        T.cnt = 0;
        for (int t = 0; t < mf; ++t)
          terms_add_row(&T, logit(D, q, K, s, h, g, If[t]), kv_row(D, s, g, If[t]));
        terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
      }
      terms_free(&T);
      continue;
    }

    /* base sample: draws 0 .. b0-1 */
    int64_t* jb = (int64_t*)malloc(sizeof(int64_t) * b0);
    double* rD = (double*)malloc(sizeof(double) * b0);
    double* rN = (double*)malloc(sizeof(double) * (int64_t)b0 * d);
    double* Nf = (double*)malloc(sizeof(double) * d);
    if (!jb || !rD || !rN || !Nf) {
      err |= 2; free(jb); free(rD); free(rN); free(Nf); continue;
    }
    for (int k = 0; k < b0; ++k) jb[k] = orc_tail_pos(If, mf, orc_draw_rank(key, k, n_s));

    double bstar = 0.0;
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      /* shift: the largest logit over the deterministic set and base draws */
      double M = -INFINITY;
      for (int t = 0; t < mf; ++t) {
        double x = logit(D, q, K, s, h, g, If[t]);
        if (x > M) M = x;
      }
      for (int k = 0; k < b0; ++k) {
        double x = logit(D, q, K, s, h, g, jb[k]);
        if (x > M) M = x;
      }
      double Df = 0.0;
      for (int i = 0; i < d; ++i) Nf[i] = 0.0;
      for (int t = 0; t < mf; ++t) {
        double e = exp(logit(D, q, K, s, h, g, If[t]) - M);
        Df += e;
        for (int i = 0; i < d; ++i) Nf[i] += e * elem(D->dtype, V, kv_row(D, s, g, If[t]) + i);
      }
      for (int k = 0; k < b0; ++k) {
        double e = exp(logit(D, q, K, s, h, g, jb[k]) - M);
        rD[k] = e;
        for (int i = 0; i < d; ++i)
          rN[(int64_t)k * d + i] = e * elem(D->dtype, V, kv_row(D, s, g, jb[k]) + i);
      }
      double bh = nz > 0 ? orc_budget_verified_from_terms(d, b0, rD, rN, Df, Nf,
                                                          n_s, eps, nz, z_split)
                         : orc_budget_from_terms(d, b0, rD, rN, Df, Nf, n_s, eps, z);
      if (bh > bstar || bh != bh) bstar = bh;
    }
    int64_t b = budget_round(bstar, n_s);
    b_out[u] = (int32_t)b;
    if (bstar_out) bstar_out[u] = bstar;

    /* I_dyn: fresh draws b0 .. b0+b-1, each weighted n_s / b */
    terms_t T;
    if (terms_init(&T, (int64_t)mf + b, d)) {
      err |= 2; free(jb); free(rD); free(rN); free(Nf); continue;
    }
    double logw_dyn = log((double)n_s / (double)b);
    for (int64_t k = 0; k < b; ++k) {
      int64_t j = orc_tail_pos(If, mf, orc_draw_rank(key, b0 + k, n_s));
      if (samples_out && k < b_cap) samples_out[(int64_t)u * b_cap + k] = (int32_t)j;
    }
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      T.cnt = 0;
      for (int t = 0; t < mf; ++t)
        terms_add_row(&T, logit(D, q, K, s, h, g, If[t]), kv_row(D, s, g, If[t]));
      for (int64_t k = 0; k < b; ++k) {
        int64_t j = orc_tail_pos(If, mf, orc_draw_rank(key, b0 + k, n_s));
        terms_add_row(&T, logit(D, q, K, s, h, g, j) + logw_dyn, kv_row(D, s, g, j));
      }
      terms_softmax(&T, D, V, out + q_row(D, s, h), lse + (int64_t)s * D->Hq + h);
    }
    terms_free(&T);
    free(jb); free(rD); free(rN); free(Nf);
  }
  return err ? -2 : 0;
}

int orc_sampled(const orc_dims* D, const void* q, const void* K, const void* V,
                const int32_t* idx, const int32_t* idx_len, int m,
                double eps, double z, int b0, uint64_t seed,
                int32_t* b_out, double* bstar_out, int32_t* samples_out,
                int b_cap, double* out, double* lse) {
  return sampled_impl(D, q, K, V, idx, idx_len, m, eps, z, 0, NULL, b0, seed,
                      b_out, bstar_out, samples_out, b_cap, out, lse);
}

int orc_sampled_verified(const orc_dims* D, const void* q, const void* K,
                         const void* V, const int32_t* idx,
                         const int32_t* idx_len, int m, double eps, int nz,
                         const double* z_split, int b0, uint64_t seed,
                         int32_t* b_out, double* bstar_out,
                         int32_t* samples_out, int b_cap, double* out,
                         double* lse) {
  if (nz < 1) return -1;
  return sampled_impl(D, q, K, V, idx, idx_len, m, eps, 0.0, nz, z_split, b0,
                      seed, b_out, bstar_out, samples_out, b_cap, out, lse);
}

int orc_sampled_fixed_b(const orc_dims* D, const void* q, const void* K,
                        const void* V, const int32_t* idx,
                        const int32_t* idx_len, int m, int b0, int b,
                        uint64_t seed, double* Dhat, double* Nhat) {
  if (check_dims(D) || m < 0 || b0 < 0 || b < 1) return -1;
  int G = D->Hq / D->Hkv, d = D->d;
  int U = D->B * D->Hkv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int u = 0; u < U; ++u) {
    int s = u / D->Hkv, g = u % D->Hkv;
    int mf = unit_len(idx_len, u, m);
    const int32_t* If = idx + (int64_t)u * m;
    if (mf < 0 || mf > m || check_sorted_set(D, If, mf) || mf >= D->n) { err |= 1; continue; }
    int64_t n_s = (int64_t)D->n - mf;
    uint64_t key = orc_unit_key(seed, u);
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      int64_t hq = (int64_t)s * D->Hq + h;
      double Dv = 0.0;
      double* Nv = Nhat + q_row(D, s, h);
      for (int i = 0; i < d; ++i) Nv[i] = 0.0;
      for (int t = 0; t < mf; ++t) {
        double e = exp(logit(D, q, K, s, h, g, If[t]));
        Dv += e;
        for (int i = 0; i < d; ++i) Nv[i] += e * elem(D->dtype, V, kv_row(D, s, g, If[t]) + i);
      }
      double f = (double)n_s / (double)b;
      for (int k = 0; k < b; ++k) {
        int64_t j = orc_tail_pos(If, mf, orc_draw_rank(key, b0 + k, n_s));
        double e = f * exp(logit(D, q, K, s, h, g, j));
        Dv += e;
        for (int i = 0; i < d; ++i) Nv[i] += e * elem(D->dtype, V, kv_row(D, s, g, j) + i);
      }
      Dhat[hq] = Dv;
    }
  }
  return err ? -2 : 0;
}
