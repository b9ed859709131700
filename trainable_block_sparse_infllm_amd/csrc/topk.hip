// Top-K block selection (MiniCPM4 technical-report summary, QbitAI repost,
// section "Model architecture: InfLLM v2": only the most relevant context
// blocks take part in attention; item 2: one block set per GQA group).
// The selection rule and the wavefront routine are in topk_select.hpp.
//
// Two producers feed it: a score tensor (decode, trees), or scores computed
// in the same workgroup with MFMA and kept in LDS (prefill; never stored).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "topk_select.hpp"

namespace infllmv2 {

// ---------------------------------------------------------------- from scores
template <int KPL>
__global__ __launch_bounds__(256) void topk_scores_kernel(const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, int64_t rows,
                                                          int n_q, int64_t q_pos0, int is_tree,
                                                          int64_t nblk, int K) {
  __shared__ uint32_t scratch[4][2 * kWave];
  const int l = lane_id();
  const int64_t row = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (row >= rows) return;
  const int node = int(row % n_q);
  const int64_t pos = is_tree ? q_pos0 : q_pos0 + node;
  int64_t C = pos / kBlock;
  if (C > nblk) C = nblk;
  const float* src = scores + row * nblk;
  float val[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int64_t j = int64_t(r) * kWave + l;
    val[r] = ldf_or_neginf(j < C, src + j);      // -inf keys rank below every score
  }
  __builtin_amdgcn_sched_barrier(0);             // all loads issue before the first use
  uint32_t key[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) key[r] = ordered_key(val[r]);
  wave_topk<KPL>(key, int(C), K, idx + row * K, scratch[threadIdx.x / kWave]);
}

// Few rows of many candidates (a draft tree's nodes): eight wavefronts share
// one row (wg_topk8 of topk_select.hpp), so the row's selection is not one
// wavefront's sort over 64*KPL keys. Only candidates j < C are read.
template <int KPL>
__global__ __launch_bounds__(512) void topk_scores_wg_kernel(const float* __restrict__ scores,
                                                             int32_t* __restrict__ idx, int n_q,
                                                             int64_t q_pos0, int is_tree,
                                                             int64_t nblk, int K) {
  __shared__ uint32_t scratch[2 * kWave];
  __shared__ WgTopkLds sh;
  const int64_t row = blockIdx.x;
  const int node = int(row % n_q);
  const int64_t pos = is_tree ? q_pos0 : q_pos0 + node;
  const int C = int(min<int64_t>(pos / kBlock, nblk));
  const float* src = scores + row * nblk;
  // 16-byte loads when the row starts 16-byte aligned and whole quads lie below C
  const bool vec = (C & 3) == 0 && (nblk & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  wg_topk8<KPL>(src, C, vec, C, K, idx + row * K, scratch, sh);
}

// ---------------------------------------------------------- fused prefill path
// Workgroup: 4 wavefronts, 16*NT query columns holding TQ <= 16*NT/G tokens of
// one (b, g) (TQ is smaller only when TQ score rows of 64*KPL candidates would
// not fit LDS; the columns of tokens >= TQ are idle). Waves split the 16-block
// chunks of the k̄ table (MFMA, max over the 3 kernel slots, head sum by
// shuffles) and park the scores in LDS sc[TQ][64*KPL]; then each wave selects
// the rows of TQ/4 tokens.
template <int D, int NT, int KPL>
__global__ __launch_bounds__(256) void topk_fused_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ kbar,
                                                         int32_t* __restrict__ idx, int Hq, int Hkv,
                                                         int G, int n_q, int64_t q_pos0,
                                                         int is_tree, int64_t nblk, int K,
                                                         int ntile, int TQ) {
  constexpr int KS = D / 32;
  constexpr int LDSC = KPL * kWave;
  extern __shared__ float sc[];
  __shared__ uint32_t scratch[4][2 * kWave];
  __shared__ float s_neginf;
  const int w = threadIdx.x / kWave;
  if (threadIdx.x == 0) s_neginf = -INFINITY;
  __syncthreads();
  const int l = lane_id();
  const int r16 = l % 16, kg = l / 16;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tok0 = tile * TQ;
  const int ntok = min(TQ, n_q - tok0);
  const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + tok0 + ntok - 1;
  int64_t Cmax = pos_last / kBlock;
  if (Cmax > nblk) Cmax = nblk;

  if (Cmax > K) {
    bf16x8 qf[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = nt * 16 + r16;
      const int t = c / G, hh = c % G;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint16_t* qrow = q + ((int64_t(b) * Hq + g * G + hh) * n_q + tok0 + (t < ntok ? t : 0)) * D;
        qf[nt][ks] = as_bf16x8(ldg16_if(t < ntok, qrow + ks * 32 + kg * 8));
      }
    }
    const int nchunk = int((Cmax + 15) / 16);
    for (int ch = w; ch < nchunk; ch += 4) {
      const int64_t j0 = int64_t(ch) * 16;
      const int64_t jrow = j0 + r16;
      const bool row_ok = jrow < Cmax;
      const int64_t jr = row_ok ? jrow : 0;     // A row: block jr; d step ks = piece 4*ks + kg
      f32x4 best[NT];
#pragma unroll
      for (int m = 0; m < kKpb; ++m) {
        bf16x8 af[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          af[ks] = as_bf16x8(ldg16_if(row_ok, kbar + kbar_off<D>(bg, m, 4 * ks + kg, jr, nblk)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16(af[ks], qf[nt][ks], acc);
          if (m == 0) {
            best[nt] = acc;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) best[nt][i] = fmaxf(best[nt][i], acc[i]);
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = best[nt][i];
          for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o);
          best[nt][i] = v;
        }
        const int c = nt * 16 + r16;
        if (c % G == 0 && c / G < TQ) {
          float* dst = sc + (c / G) * LDSC;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t j = j0 + kg * 4 + i;
            if (j < LDSC) dst[j] = best[nt][i];
          }
        }
      }
    }
    __syncthreads();
  }

  for (int t = w; t < ntok; t += 4) {
    const int64_t pos = is_tree ? q_pos0 : q_pos0 + tok0 + t;
    int64_t C = pos / kBlock;
    if (C > nblk) C = nblk;
    uint32_t key[KPL];
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int j = r * kWave + l;
      const float* src = (C > K && j < C) ? &sc[t * LDSC + j] : &s_neginf;
      key[r] = ordered_key(*src);
    }
    wave_topk<KPL>(key, int(C), K, idx + ((int64_t(bg) * n_q + tok0 + t) * K), scratch[w]);
  }
}

// Row count up to which the workgroup-per-row selection is used (beyond it,
// one wavefront per row already fills the chip).
constexpr int64_t kWgRowsMax = 1024;

static int pick_kpl(int64_t cmax) {
  int kpl = 1;
  while (int64_t(kpl) * kWave < cmax) kpl <<= 1;
  return kpl;
}

namespace {

constexpr int kTopkFusedLds = 152 * 1024;   // the score tile's LDS budget (160 KB per CU on gfx950, less the static arrays)

struct TopkFusedPlan {
  int kpl, nt, tq;
};

// Columns per workgroup: the largest of 64/32/16 whose score tile (TQ tokens
// x 64*KPL candidates, fp32) fits the LDS budget; when even 16 columns' tokens
// do not fit (one query head per group and more than 2048 candidates), fewer
// tokens, each with its full score row, leaving the other columns idle.
TopkFusedPlan topk_fused_plan(const Dims& d, int64_t cmax) {
  TopkFusedPlan p;
  p.kpl = pick_kpl(cmax);
  const int64_t row = int64_t(p.kpl) * kWave * 4;
  p.nt = 4;
  while (p.nt > 1 && int64_t(16 * p.nt / d.G) * row > kTopkFusedLds) p.nt >>= 1;
  p.tq = std::min<int>(16 * p.nt / d.G, int(kTopkFusedLds / row));
  if (16 * p.nt < d.G) p.tq = 0;
  return p;
}

}  // namespace

bool topk_fused_ok(const Dims& d, int64_t cmax) {
  if (cmax > 64 * 64) return false;
  return topk_fused_plan(d, cmax).tq >= 1;
}

hipError_t launch_topk_from_scores(const Dims& d, const float* scores, int n_q, int64_t q_pos0,
                                   int is_tree, int64_t nblk, int32_t* idx, hipStream_t s) {
  const int64_t rows = int64_t(d.B) * d.Hkv * n_q;
  const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + n_q - 1;
  int64_t cmax = pos_last / kBlock;
  if (cmax > nblk) cmax = nblk;
  const int kpl = pick_kpl(cmax);
  if (kpl >= 8 && rows <= kWgRowsMax) {
#define TOPK_WG_CASE(P)                                                                        \
    if (kpl == P) {                                                                            \
      topk_scores_wg_kernel<P><<<dim3(unsigned(rows)), 512, 0, s>>>(scores, idx, n_q, q_pos0,  \
                                                                   is_tree, nblk, d.K);        \
      return hipGetLastError();                                                                \
    }
    TOPK_WG_CASE(8) TOPK_WG_CASE(16) TOPK_WG_CASE(32) TOPK_WG_CASE(64)
#undef TOPK_WG_CASE
  }
  const dim3 grid(unsigned((rows + 3) / 4));
#define TOPK_CASE(P)                                                                           \
  if (kpl == P) {                                                                              \
    topk_scores_kernel<P><<<grid, 256, 0, s>>>(scores, idx, rows, n_q, q_pos0, is_tree, nblk, \
                                               d.K);                                           \
    return hipGetLastError();                                                                  \
  }
  TOPK_CASE(1) TOPK_CASE(2) TOPK_CASE(4) TOPK_CASE(8) TOPK_CASE(16) TOPK_CASE(32) TOPK_CASE(64)
#undef TOPK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_topk_fused(const Dims& d, const uint16_t* q, const uint16_t* kbar, int n_q,
                             int64_t q_pos0, int is_tree, int64_t nblk, int32_t* idx,
                             hipStream_t s) {
  const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + n_q - 1;
  int64_t cmax = pos_last / kBlock;
  if (cmax > nblk) cmax = nblk;
  if (topk_prefill128_ok(d, cmax))
    return launch_topk_prefill128(d, q, kbar, n_q, q_pos0, is_tree, nblk, cmax, idx, s);
  const TopkFusedPlan p = topk_fused_plan(d, cmax);
  if (p.tq < 1) return hipErrorInvalidValue;
  const int kpl = p.kpl, nt = p.nt, tq = p.tq;
  const int ntile = (n_q + tq - 1) / tq;
  const size_t lds = size_t(tq) * kpl * kWave * sizeof(float);
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile));
#define FUSED_CASE(DD, NN, P)                                                                   \
  if (d.D == DD && nt == NN && kpl == P) {                                                      \
    auto kern = topk_fused_kernel<DD, NN, P>;                                                   \
    static const hipError_t attr = hipFuncSetAttribute(                                         \
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,        \
        kTopkFusedLds);                                                                         \
    if (attr != hipSuccess) return attr;                                                        \
    kern<<<grid, 256, lds, s>>>(q, kbar, idx, d.Hq, d.Hkv, d.G, n_q, q_pos0, is_tree, nblk,    \
                                d.K, ntile, tq);                                                \
    return hipGetLastError();                                                                   \
  }
#define FUSED_D(DD, NN) \
  FUSED_CASE(DD, NN, 1) FUSED_CASE(DD, NN, 2) FUSED_CASE(DD, NN, 4) FUSED_CASE(DD, NN, 8) \
  FUSED_CASE(DD, NN, 16) FUSED_CASE(DD, NN, 32) FUSED_CASE(DD, NN, 64)
  FUSED_D(128, 4) FUSED_D(128, 2) FUSED_D(128, 1) FUSED_D(64, 4) FUSED_D(64, 2) FUSED_D(64, 1)
#undef FUSED_D
#undef FUSED_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllmv2
