/*
 * oracle.c -- plain, slow CPU reference for InfLLM v2 block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes or
 * calls this file; it is loaded by the tests, by the benchmark's CPU-baseline
 * leg and by the smoke check, and it shares no code with the HIP library.
 *
 * Sources (the MiniCPM4 pages):
 *   [ARCH]  MiniCPM4 technical-report summary (QbitAI repost, gangyiku.com),
 *           section "Model architecture: InfLLM v2 native sparse attention":
 *           the context is split into blocks, each query scores the blocks and
 *           only the most relevant blocks enter attention; item 1) a block is
 *           made of several fine-grained semantic kernels and a query's
 *           relevance to the block is the maximum of its relevance to the
 *           kernels the block contains; item 2) the query heads of one GQA
 *           group share the same context blocks; dense attention is kept for
 *           short sequences.
 *   [LAUNCH] MiniCPM 4.0 launch article (senqingzn.com), section 1 "efficient
 *           architecture": the same three points, and the long/short switch
 *           between sparse and dense attention.
 *   [FUSE]  same QbitAI summary, section "Fusing speculative sampling,
 *           quantization and long-context algorithms": tree-draft verification
 *           runs on the sparse kernel with a local attention mask and bit
 *           packing.
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reason in the design notes of the repository):
 *   - kernels: window 32, stride 16, only the 3 windows contained in a 64-token
 *     block belong to it; a kernel is the mean of its 32 keys, rounded to bf16
 *     (round to nearest even); computed here as the exact mean (fp64 sum of
 *     bf16 values, exact for these magnitudes) so the value has one definition;
 *   - block score = sum over the group's query heads of (max over the block's
 *     kernels of the raw dot product q.kbar); no 1/sqrt(D), no softmax;
 *   - candidates of a query at position p are the complete blocks j < p/64;
 *     the query's own block floor(p/64) is always attended (causally) and is
 *     not counted in top-K; with at most K candidates all are taken;
 *   - top-K ranks by the score in fp32 (the precision the selection kernel
 *     decides in), higher first, lower block index first on equal scores;
 *     output ascending, padded with -1;
 *   - a query row with fewer than dense_threshold visible keys attends all of
 *     them (dense); 0 switches the dense rule off;
 *   - attention: softmax(q.k / sqrt(D)) v over the attended keys, in fp64;
 *     lse = natural log of the softmax denominator (including the max shift).
 *   - tree: nodes sit at cache slots P+i; every node scores with position P;
 *     node i attends its own selected blocks, the prefix keys of block
 *     floor(P/64) before P, and the tree slots whose bit is set in mask[i].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ bf16 */

/* bf16 bit pattern -> value (exact). */
double orc_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even; overflow -> inf.
 * bf16: 8 significant bits, exponent range of fp32 (normals down to 2^-126,
 * subnormals down to 2^-133). The quantum of the binade holding |x| is
 * 2^(e-7) (2^-133 below the normal range); |x| / quantum is exact in double,
 * rint() rounds it to nearest-even, and the product is again exact. */
uint16_t orc_bf16_from_double(double x) {
  if (isnan(x)) return 0x7FC0;
  int neg = signbit(x) ? 1 : 0;
  double a = fabs(x);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else if (isinf(a)) {
    r = INFINITY;
  } else {
    int E;
    frexp(a, &E);                 /* a = f * 2^E, f in [0.5, 1) -> binade exponent e = E-1 */
    int e = E - 1;
    if (e < -126) e = -126;       /* subnormal range shares the quantum of the lowest binade */
    double quantum = ldexp(1.0, e - 7);
    r = rint(a / quantum) * quantum;
    if (r >= ldexp(1.0, 128)) r = INFINITY;
  }
  float f = (float)r;             /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t h = (uint16_t)(u >> 16);
  return neg ? (uint16_t)(h | 0x8000) : h;
}

static double bf(const uint16_t* p) { return orc_bf16_to_double(*p); }

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------- 1. kernels
 * [ARCH] item 1, [LAUNCH] section 1: each block holds several semantic
 * kernels. Kernel m of block j is the mean of keys [j*bs + m*kst, +ks),
 * for the kpb = (bs-ks)/kst + 1 windows that lie inside the block.
 * Only complete blocks (j < kv_len / bs) get kernels.
 * Layouts: k [B][Hkv][kv_cap][D] bf16; kbar [B][Hkv][kv_cap/bs][kpb][D] bf16. */
int orc_pool(int B, int Hkv, int D, int bs, int ks, int kst,
             int64_t kv_cap, int64_t kv_len, const uint16_t* k, uint16_t* kbar) {
  if (bs <= 0 || ks <= 0 || kst <= 0 || ks > bs || (bs - ks) % kst) return -1;
  if (kv_len > kv_cap || kv_cap % bs) return -1;
  const int kpb = (bs - ks) / kst + 1;
  const int64_t nblk_cap = kv_cap / bs;
  const int64_t nfull = kv_len / bs;
  #pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int64_t j = 0; j < nfull; ++j)
        for (int m = 0; m < kpb; ++m)
          for (int e = 0; e < D; ++e) {
            double s = 0.0;
            for (int r = 0; r < ks; ++r) {
              int64_t t = j * bs + (int64_t)m * kst + r;
              s += bf(&k[(((int64_t)b * Hkv + g) * kv_cap + t) * D + e]);
            }
            kbar[((((int64_t)b * Hkv + g) * nblk_cap + j) * kpb + m) * D + e] =
                orc_bf16_from_double(s / ks);
          }
  return 0;
}

/* ------------------------------------------------------------ 2. scores
 * [ARCH] items 1 and 2: a query's relevance to block j is the max over the
 * block's kernels of its relevance to each kernel; the heads of one GQA group
 * share one block set, so the group's per-head relevances are summed.
 * Candidates of a query row at position p: complete blocks j < floor(p/bs).
 * rows[r] = (b, g, i): batch, KV group, query row; pos[i] = its position.
 * R[r][j] for j < C[r]; -inf elsewhere up to nblk_cap.
 * Layout q [B][Hq][n_q][D]; heads of group g are g*G .. g*G+G-1. */
int orc_scores(int B, int Hq, int Hkv, int D, int bs, int kpb,
               const uint16_t* q, int n_q, const int64_t* pos,
               const uint16_t* kbar, int64_t nblk_cap,
               int n_rows, const int32_t* rows, double* R, int64_t* C) {
  if (Hq % Hkv) return -1;
  const int G = Hq / Hkv;
  int bad = 0;
  #pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < n_rows; ++r) {
    const int b = rows[3 * r], g = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || g < 0 || g >= Hkv || i < 0 || i >= n_q) { bad = 1; continue; }
    int64_t c = pos[i] / bs;
    if (c > nblk_cap) c = nblk_cap;
    C[r] = c;
    for (int64_t j = 0; j < nblk_cap; ++j) {
      if (j >= c) { R[(int64_t)r * nblk_cap + j] = -INFINITY; continue; }
      double sum = 0.0;
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        const uint16_t* qv = &q[(((int64_t)b * Hq + h) * n_q + i) * D];
        double best = -INFINITY;
        for (int m = 0; m < kpb; ++m) {
          const uint16_t* kv = &kbar[((((int64_t)b * Hkv + g) * nblk_cap + j) * kpb + m) * D];
          double dot = 0.0;
          for (int e = 0; e < D; ++e) dot += bf(&qv[e]) * bf(&kv[e]);
          if (dot > best) best = dot;
        }
        sum += best;
      }
      R[(int64_t)r * nblk_cap + j] = sum;
    }
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------ 2b. LSE-normalized scores
 * [ARCH] "more efficient operators": a LogSumExp estimate lets the top-K
 * blocks be chosen cheaply. The pages describe no formula; the reading taken
 * here: per head h of the group, the kernel scores s = scale * q_h . kbar[j][m]
 * over every candidate kernel (j < C, m < kpb) are softmax-normalized by their
 * log-sum-exp LSE_h = log sum_{j,m} exp(s), a block's normalized relevance is
 * the max over its kernels (as in section 2), and the group sums the heads:
 *   R[j] = sum_h exp(max_m s_{h,j,m} - LSE_h),  j < C;  -inf elsewhere.
 * Same rows, layouts and candidate rule as orc_scores. */
int orc_scores_lse(int B, int Hq, int Hkv, int D, int bs, int kpb,
                   const uint16_t* q, int n_q, const int64_t* pos,
                   const uint16_t* kbar, int64_t nblk_cap, double scale,
                   int n_rows, const int32_t* rows, double* R, int64_t* C) {
  if (Hq % Hkv) return -1;
  const int G = Hq / Hkv;
  int bad = 0;
  #pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(nblk_cap * kpb + 1));
    #pragma omp for schedule(dynamic)
    for (int r = 0; r < n_rows; ++r) {
      const int b = rows[3 * r], g = rows[3 * r + 1], i = rows[3 * r + 2];
      if (b < 0 || b >= B || g < 0 || g >= Hkv || i < 0 || i >= n_q) { bad = 1; continue; }
      int64_t c = pos[i] / bs;
      if (c > nblk_cap) c = nblk_cap;
      C[r] = c;
      double* Rr = &R[(int64_t)r * nblk_cap];
      for (int64_t j = 0; j < nblk_cap; ++j) Rr[j] = j < c ? 0.0 : -INFINITY;
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        const uint16_t* qv = &q[(((int64_t)b * Hq + h) * n_q + i) * D];
        double mx = -INFINITY;
        for (int64_t j = 0; j < c; ++j)
          for (int m = 0; m < kpb; ++m) {
            const uint16_t* kv = &kbar[((((int64_t)b * Hkv + g) * nblk_cap + j) * kpb + m) * D];
            double dot = 0.0;
            for (int e = 0; e < D; ++e) dot += bf(&qv[e]) * bf(&kv[e]);
            s[j * kpb + m] = scale * dot;
            if (s[j * kpb + m] > mx) mx = s[j * kpb + m];
          }
        double l = 0.0;
        for (int64_t t = 0; t < c * kpb; ++t) l += exp(s[t] - mx);
        const double lse = mx + log(l);
        for (int64_t j = 0; j < c; ++j) {
          double best = -INFINITY;
          for (int m = 0; m < kpb; ++m)
            if (s[j * kpb + m] > best) best = s[j * kpb + m];
          Rr[j] += exp(best - lse);
        }
      }
    }
    free(s);
  }
  return bad ? -1 : 0;
}

/* --------------------------------------------------------- 3. selection
 * [ARCH] section text and [LAUNCH] section 1: only the few most relevant
 * blocks take part in attention. Top-K by score (compared as fp32, the
 * selection kernel's precision), lower block index first on equal scores.
 * C <= K: all candidates. Output ascending, -1 padded. */
typedef struct { float s; int64_t j; } cand_t;

static int cmp_cand(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int orc_select(int n_rows, const double* R, int64_t nblk_cap, const int64_t* C,
               int K, int32_t* idx) {
  if (K < 1) return -1;
  #pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < n_rows; ++r) {
    int32_t* out = &idx[(int64_t)r * K];
    const int64_t c = C[r];
    for (int t = 0; t < K; ++t) out[t] = -1;
    if (c <= K) {
      for (int64_t j = 0; j < c; ++j) out[j] = (int32_t)j;
      continue;
    }
    cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * (size_t)c);
    for (int64_t j = 0; j < c; ++j) {
      cs[j].s = (float)R[(int64_t)r * nblk_cap + j];
      cs[j].j = j;
    }
    qsort(cs, (size_t)c, sizeof(cand_t), cmp_cand);
    for (int t = 0; t < K; ++t) out[t] = (int32_t)cs[t].j;
    qsort(out, (size_t)K, sizeof(int32_t), cmp_i32);
    free(cs);
  }
  return 0;
}

/* ------------------------------------------------------ 4. attended keys
 * mode 0 (sparse prefill / decode): row at position p; n_ctx = p + 1 keys are
 *   visible. If dense_threshold > 0 and n_ctx < dense_threshold the row is
 *   dense ([ARCH]: short contexts keep dense attention): keys 0..p.
 *   Otherwise: the bs keys of every selected block, and the own block's keys
 *   bs*floor(p/bs) .. p.
 * mode 1 (tree, [FUSE]): node i, prefix length P = pos[i]; n_ctx = P +
 *   popcount(mask[i]). Dense: keys 0..P-1. Sparse: selected blocks' keys and
 *   keys bs*floor(P/bs) .. P-1. Both: tree slots P+j for every set bit j.
 * mode 2 (dense causal): keys 0..p.
 * mode 3 (dense, no mask): keys 0..kv_len-1.
 * mode 4 (sliding window, [FUSE]: the draft model's attention): the last
 *   `window` positions up to the row's own, keys max(0, p - window + 1)..p.
 * Writes ascending key positions to keys[], returns their count (or -1). */
int64_t orc_keyset(int mode, int bs, int64_t p, int64_t kv_len,
                   const int32_t* sel, int K, int dense_threshold,
                   uint64_t mask, int64_t window, int64_t* keys) {
  int64_t n = 0;
  if (mode == 4) {
    if (window < 1) return -1;
    for (int64_t t = p - window + 1 < 0 ? 0 : p - window + 1; t <= p && t < kv_len; ++t)
      keys[n++] = t;
    return n;
  }
  if (mode == 3) {
    for (int64_t t = 0; t < kv_len; ++t) keys[n++] = t;
    return n;
  }
  if (mode == 2) {
    for (int64_t t = 0; t <= p && t < kv_len; ++t) keys[n++] = t;
    return n;
  }
  if (mode == 0) {
    const int64_t n_ctx = p + 1;
    if (dense_threshold > 0 && n_ctx < dense_threshold) {
      for (int64_t t = 0; t <= p; ++t) keys[n++] = t;
      return n;
    }
    const int64_t own = p / bs;
    if (!sel) return -1;
    for (int t = 0; t < K; ++t) {           /* sel is ascending, all < own */
      if (sel[t] < 0) continue;
      if (sel[t] >= own) return -1;
      for (int64_t x = 0; x < bs; ++x) keys[n++] = (int64_t)sel[t] * bs + x;
    }
    for (int64_t t = own * bs; t <= p; ++t) keys[n++] = t;
    return n;
  }
  if (mode == 1) {
    const int64_t P = p;
    const int64_t n_ctx = P + __builtin_popcountll(mask);
    if (dense_threshold > 0 && n_ctx < dense_threshold) {
      for (int64_t t = 0; t < P; ++t) keys[n++] = t;
    } else {
      const int64_t own = P / bs;
      if (!sel) return -1;
      for (int t = 0; t < K; ++t) {
        if (sel[t] < 0) continue;
        if (sel[t] >= own) return -1;
        for (int64_t x = 0; x < bs; ++x) keys[n++] = (int64_t)sel[t] * bs + x;
      }
      for (int64_t t = own * bs; t < P; ++t) keys[n++] = t;
    }
    for (int j = 0; j < 64; ++j)
      if ((mask >> j) & 1ull) {
        if (P + j >= kv_len) return -1;
        keys[n++] = P + j;
      }
    return n;
  }
  return -1;
}

/* ------------------------------------------------------- 5. attention
 * Softmax attention of one query vector over the listed keys, in fp64:
 * s_t = scale * q.k_t; o = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m);
 * lse = m + log(sum_t exp(s_t - m)).
 * rows[r] = (b, h, i). idx [B][Hkv][n_q][K] (may be NULL for modes 2, 3);
 * tree_mask [B][n_q] (mode 1 only). out [n_rows][D], lse [n_rows],
 * nkeys [n_rows] (number of attended keys). */
int orc_attend(int mode, int B, int Hq, int Hkv, int D, int bs,
               const uint16_t* q, int n_q, const int64_t* pos,
               const uint16_t* k, const uint16_t* v, int64_t kv_cap, int64_t kv_len,
               const int32_t* idx, int K, int dense_threshold, int64_t window,
               const uint64_t* tree_mask, double scale,
               int n_rows, const int32_t* rows,
               double* out, double* lse, int64_t* nkeys) {
  if (Hq % Hkv || kv_len > kv_cap) return -1;
  const int G = Hq / Hkv;
  int bad = 0;
  #pragma omp parallel
  {
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(kv_len + 64));
    double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len + 64));
    #pragma omp for schedule(dynamic)
    for (int r = 0; r < n_rows; ++r) {
      const int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= n_q) { bad = 1; continue; }
      const int g = h / G;
      const int32_t* sel = idx ? &idx[(((int64_t)b * Hkv + g) * n_q + i) * K] : NULL;
      const uint64_t msk = tree_mask ? tree_mask[(int64_t)b * n_q + i] : 0ull;
      int64_t n = orc_keyset(mode, bs, pos[i], kv_len, sel, K, dense_threshold, msk, window, keys);
      if (n <= 0) { bad = 1; nkeys[r] = n; continue; }
      nkeys[r] = n;
      const uint16_t* qv = &q[(((int64_t)b * Hq + h) * n_q + i) * D];
      double mx = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        const uint16_t* kv = &k[(((int64_t)b * Hkv + g) * kv_cap + keys[t]) * D];
        double dot = 0.0;
        for (int e = 0; e < D; ++e) dot += bf(&qv[e]) * bf(&kv[e]);
        s[t] = scale * dot;
        if (s[t] > mx) mx = s[t];
      }
      double l = 0.0;
      double* o = &out[(int64_t)r * D];
      for (int e = 0; e < D; ++e) o[e] = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        const double p = exp(s[t] - mx);
        l += p;
        const uint16_t* vv = &v[(((int64_t)b * Hkv + g) * kv_cap + keys[t]) * D];
        for (int e = 0; e < D; ++e) o[e] += p * bf(&vv[e]);
      }
      for (int e = 0; e < D; ++e) o[e] /= l;
      lse[r] = mx + log(l);
    }
    free(keys);
    free(s);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------- 6. backward
 * Gradients of L = sum over rows of dO . o (the rows' attention outputs of
 * orc_attend, same key sets) with respect to q, k and v, in fp64. Per row,
 * with P_t the softmax weights over its keys:
 *   dP_t = dO . v_t;  D = sum_t P_t dP_t;  dS_t = P_t (dP_t - D);
 *   dq = scale sum_t dS_t k_t;  dk_t += scale dS_t q;  dv_t += P_t dO.
 * (The softmax Jacobian is diag(P) - P P^T, so dL/ds_t = P_t (dP_t - D).)
 * Every row (b, h, i) of the call contributes (all heads, all n_q rows).
 * dout [B][Hq][n_q][D] bf16; dq [B][Hq][n_q][D], dk and dv [B][Hkv][kv_cap][D]
 * fp64, fully written (zeros where no row attends). */
int orc_attend_backward(int mode, int B, int Hq, int Hkv, int D, int bs,
                        const uint16_t* q, int n_q, const int64_t* pos,
                        const uint16_t* k, const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                        const int32_t* idx, int K, int dense_threshold, int64_t window,
                        const uint64_t* tree_mask, double scale, const uint16_t* dout,
                        double* dq, double* dk, double* dv) {
  if (Hq % Hkv || kv_len > kv_cap) return -1;
  const int G = Hq / Hkv;
  memset(dq, 0, sizeof(double) * (size_t)B * Hq * n_q * D);
  memset(dk, 0, sizeof(double) * (size_t)B * Hkv * kv_cap * D);
  memset(dv, 0, sizeof(double) * (size_t)B * Hkv * kv_cap * D);
  int bad = 0;
  /* one (b, g) per task: its rows write only its dk, dv slices */
  #pragma omp parallel
  {
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(kv_len + 64));
    double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len + 64));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(kv_len + 64));
    #pragma omp for schedule(dynamic)
    for (int bg = 0; bg < B * Hkv; ++bg) {
      const int b = bg / Hkv, g = bg % Hkv;
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        for (int i = 0; i < n_q; ++i) {
          const int32_t* sel = idx ? &idx[(((int64_t)b * Hkv + g) * n_q + i) * K] : NULL;
          const uint64_t msk = tree_mask ? tree_mask[(int64_t)b * n_q + i] : 0ull;
          const int64_t n = orc_keyset(mode, bs, pos[i], kv_len, sel, K, dense_threshold, msk, window,
                                       keys);
          if (n <= 0) { bad = 1; continue; }
          const uint16_t* qv = &q[(((int64_t)b * Hq + h) * n_q + i) * D];
          const uint16_t* gv = &dout[(((int64_t)b * Hq + h) * n_q + i) * D];
          double mx = -INFINITY;
          for (int64_t t = 0; t < n; ++t) {
            const uint16_t* kr = &k[((int64_t)bg * kv_cap + keys[t]) * D];
            const uint16_t* vr = &v[((int64_t)bg * kv_cap + keys[t]) * D];
            double dot = 0.0, dd = 0.0;
            for (int e = 0; e < D; ++e) {
              dot += bf(&qv[e]) * bf(&kr[e]);
              dd += bf(&gv[e]) * bf(&vr[e]);
            }
            s[t] = scale * dot;
            dp[t] = dd;
            if (s[t] > mx) mx = s[t];
          }
          double l = 0.0;
          for (int64_t t = 0; t < n; ++t) {
            s[t] = exp(s[t] - mx);          /* unnormalized P */
            l += s[t];
          }
          double Dsum = 0.0;
          for (int64_t t = 0; t < n; ++t) {
            s[t] /= l;                      /* P_t */
            Dsum += s[t] * dp[t];
          }
          double* dqr = &dq[(((int64_t)b * Hq + h) * n_q + i) * D];
          for (int64_t t = 0; t < n; ++t) {
            const double ds = s[t] * (dp[t] - Dsum);
            const uint16_t* kr = &k[((int64_t)bg * kv_cap + keys[t]) * D];
            double* dkr = &dk[((int64_t)bg * kv_cap + keys[t]) * D];
            double* dvr = &dv[((int64_t)bg * kv_cap + keys[t]) * D];
            for (int e = 0; e < D; ++e) {
              dqr[e] += scale * ds * bf(&kr[e]);
              dkr[e] += scale * ds * bf(&qv[e]);
              dvr[e] += s[t] * bf(&gv[e]);
            }
          }
        }
      }
    }
    free(keys);
    free(s);
    free(dp);
  }
  return bad ? -1 : 0;
}
