// Block scoring and top-K selection for a prefill chunk, fused, head_dim 128
// (MiniCPM4 technical-report summary, QbitAI repost, section "Model
// architecture: InfLLM v2": a block's relevance is the largest similarity of
// the query with the block's semantic kernels, summed over the query heads of
// a GQA group; the K most relevant blocks are attended).
//
// Rule (as in the top-K over a score tensor): with at most K candidates all are
// taken; otherwise the K highest scores, compared as fp32, with the lower block
// index first on equal scores. Rows are written ascending, padded with -1.
//
// Workgroup: 4 wavefronts, 64 query rows = TQ = 64/G tokens of one (b, g).
//   1. scoring: the wavefronts split the table of candidate blocks into chunks
//      of 32 and each computes, for all 64 rows, S = Q kbar^T with the
//      32x32x16 bf16 MFMA (A = Q rows, B = kbar^T). An accumulator column is
//      one block, so the max over the 3 kernels of a block is elementwise and
//      the head sum of a token stays within a lane (G <= 4) or a lane pair.
//      The next chunk's kbar fragments are loaded while one is computed.
//      Scores go to LDS, sc[token][block];
//   2. selection: one wavefront per token, with the exact wavefront top-K of
//      topk_select.hpp over the scores in LDS.
#include "common.hpp"
#include "launch.hpp"
#include "topk_select.hpp"

namespace infllmv2 {

namespace {

constexpr int kDK = 128;

__device__ __forceinline__ f32x16 max16(const f32x16& a, const f32x16& b) {
  f32x16 r;
#pragma unroll
  for (int e = 0; e < 16; ++e) r[e] = fmaxf(a[e], b[e]);
  return r;
}

__device__ __forceinline__ float pair_sum(float x) {   // lanes l and l ^ 32
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

template <int G, int KPL>
__global__ __launch_bounds__(256, 2) void topk_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbar, int32_t* __restrict__ idx,
    int Hq, int Hkv, int n_q, int64_t q_pos0, int is_tree, int64_t nblk, int K, int ntile, int scs) {
  constexpr int TQ = 64 / G;     // tokens per workgroup
  constexpr int TPS = 32 / G;    // tokens per 32-row sub-tile
  constexpr int DS = kDK / 16;   // k-steps

  extern __shared__ __align__(16) char smem[];
  float* sc = reinterpret_cast<float*>(smem);    // [TQ][scs]
  __shared__ uint32_t scratch[4][2 * kWave];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tok0 = tile * TQ;
  const int ntok = min(TQ, n_q - tok0);
  const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + tok0 + ntok - 1;
  const int64_t Cmax = min(pos_last / kBlock, nblk);

  // ---------------------------------------------------------------- 1. scores
  if (Cmax > K) {
    // A operand: row 32*st + r32 of the tile (token row / G, head row % G),
    // k-slots 8*hl .. 8*hl+7 of each 16-wide d step.
    bf16x8 qa[2][DS];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = 32 * st + r32;
      const int t = row / G;
      const int h = g * G + row % G;
      const uint16_t* qrow = q + ((int64_t(b) * Hq + h) * n_q + tok0 + (t < ntok ? t : 0)) * kDK + 8 * hl;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qa[st][ds] = as_bf16x8(ldg16_if(t < ntok, qrow + 16 * ds));
    }
    const int nchunk = int((Cmax + 31) / 32);
    // This wavefront's chunks are w, w + 4, ...; step s is (chunk w + 4*(s/3),
    // kernel s%3). B operand of a step: block 32*chunk + r32, d = 16*ds + 8*hl ..,
    // i.e. piece 2*ds + hl: 32 consecutive blocks of one piece are contiguous.
    const int nsteps = kKpb * ((nchunk - w + 3) / 4);
    auto load_step = [&](int s, bf16x8 (&dst)[DS]) {
      const int64_t blk = int64_t(w + 4 * (s / kKpb)) * 32 + r32;
      const bool ok = blk < Cmax;
      const int64_t jb = ok ? blk : 0;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        dst[ds] = as_bf16x8(ldg16_if(ok, kbar + kbar_off<kDK>(bg, s % kKpb, 2 * ds + hl, jb, nblk)));
    };
    // Accumulator register r of lane l: tile row 32*st + 8*(r/4) + 4*hl + r%4,
    // block 32*chunk + r32. Max over the kernels; after the last, head sums
    // and the store.
    f32x16 best[2];
    auto compute_step = [&](int s, const bf16x8 (&kf)[DS]) {
      const int m = s % kKpb;
      const int blk = (w + 4 * (s / kKpb)) * 32 + r32;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) acc = mfma32(qa[st][ds], kf[ds], acc);
        best[st] = m == 0 ? acc : max16(best[st], acc);
      }
      if (m != kKpb - 1) return;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if constexpr (G <= 4) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int u = 0; u < 4 / G; ++u) {
              float sum = 0.f;
#pragma unroll
              for (int v = 0; v < G; ++v) sum += best[st][4 * a + G * u + v];
              const int tk = st * TPS + (8 * a + 4 * hl + G * u) / G;
              sc[tk * scs + blk] = sum;
            }
        } else {
          float s4[4];
#pragma unroll
          for (int a = 0; a < 4; ++a)
            s4[a] = pair_sum(best[st][4 * a] + best[st][4 * a + 1] + best[st][4 * a + 2] + best[st][4 * a + 3]);
          if (hl == 0) {
            if constexpr (G == 8) {
#pragma unroll
              for (int a = 0; a < 4; ++a) sc[(st * TPS + a) * scs + blk] = s4[a];
            } else {
#pragma unroll
              for (int a = 0; a < 2; ++a) sc[(st * TPS + a) * scs + blk] = s4[2 * a] + s4[2 * a + 1];
            }
          }
        }
      }
    };

    // The next step's fragments load while one step computes. The loads are
    // issued unconditionally (a step past the end maps to blocks >= Cmax and
    // reads zeros): behind a branch, the wait placed before the current
    // step's MFMAs would also cover the prefetch.
    bf16x8 kfa[DS], kfb[DS];
    load_step(0, kfa);
    for (int s = 0; s < nsteps; s += 2) {
      load_step(s + 1, kfb);
      compute_step(s, kfa);
      if (s + 1 >= nsteps) break;
      load_step(s + 2, kfa);
      compute_step(s + 1, kfb);
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 2. selection
  for (int t = w; t < ntok; t += 4) {
    const int64_t pos = is_tree ? q_pos0 : q_pos0 + tok0 + t;
    const int C = int(min(pos / kBlock, nblk));
    uint32_t key[KPL];
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int j = r * kWave + l;
      key[r] = (C > K && j < C) ? ordered_key(sc[t * scs + j]) : 0u;
    }
    wave_topk<KPL>(key, C, K, idx + (int64_t(bg) * n_q + tok0 + t) * K, scratch[w]);
  }
}

namespace {

int topk_prefill_tq(int G) { return 64 / G; }

struct TopkPrefillPlan {
  int scs, kpl;
  size_t lds;
};

TopkPrefillPlan topk_prefill_plan(const Dims& d, int64_t cmax) {
  TopkPrefillPlan p;
  p.scs = int((cmax + 63) / 64 * 64 + 32);       // +32: rows of a store land in other banks
  p.kpl = 1;
  while (int64_t(p.kpl) * kWave < cmax) p.kpl <<= 1;
  p.lds = size_t(topk_prefill_tq(d.G)) * p.scs * 4;
  return p;
}

}  // namespace

bool topk_prefill128_ok(const Dims& d, int64_t cmax) {
  if (d.D != kDK || cmax > 512) return false;
  if (d.G != 1 && d.G != 2 && d.G != 4 && d.G != 8 && d.G != 16) return false;
  return topk_prefill_plan(d, cmax).lds <= 64 * 1024;
}

template <int G, int KPL>
static hipError_t launch_topk_prefill_t(const Dims& d, const uint16_t* q, const uint16_t* kbar,
                                        int n_q, int64_t q_pos0, int is_tree, int64_t nblk,
                                        int scs, int32_t* idx, hipStream_t s) {
  constexpr int TQ = 64 / G;
  const int ntile = (n_q + TQ - 1) / TQ;
  auto kern = topk_prefill_kernel<G, KPL>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     64 * 1024);
  if (attr != hipSuccess) return attr;
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile));
  kern<<<grid, 256, size_t(TQ) * scs * 4, s>>>(q, kbar, idx, d.Hq, d.Hkv, n_q, q_pos0, is_tree,
                                               nblk, d.K, ntile, scs);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_topk_prefill_g(const Dims& d, const uint16_t* q, const uint16_t* kbar,
                                        int n_q, int64_t q_pos0, int is_tree, int64_t nblk,
                                        int64_t cmax, int32_t* idx, hipStream_t s) {
  const TopkPrefillPlan p = topk_prefill_plan(d, cmax);
  switch (p.kpl) {
    case 1: return launch_topk_prefill_t<G, 1>(d, q, kbar, n_q, q_pos0, is_tree, nblk, p.scs, idx, s);
    case 2: return launch_topk_prefill_t<G, 2>(d, q, kbar, n_q, q_pos0, is_tree, nblk, p.scs, idx, s);
    case 4: return launch_topk_prefill_t<G, 4>(d, q, kbar, n_q, q_pos0, is_tree, nblk, p.scs, idx, s);
    case 8: return launch_topk_prefill_t<G, 8>(d, q, kbar, n_q, q_pos0, is_tree, nblk, p.scs, idx, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_topk_prefill128(const Dims& d, const uint16_t* q, const uint16_t* kbar, int n_q,
                                  int64_t q_pos0, int is_tree, int64_t nblk, int64_t cmax,
                                  int32_t* idx, hipStream_t s) {
  switch (d.G) {
    case 1: return launch_topk_prefill_g<1>(d, q, kbar, n_q, q_pos0, is_tree, nblk, cmax, idx, s);
    case 2: return launch_topk_prefill_g<2>(d, q, kbar, n_q, q_pos0, is_tree, nblk, cmax, idx, s);
    case 4: return launch_topk_prefill_g<4>(d, q, kbar, n_q, q_pos0, is_tree, nblk, cmax, idx, s);
    case 8: return launch_topk_prefill_g<8>(d, q, kbar, n_q, q_pos0, is_tree, nblk, cmax, idx, s);
    case 16: return launch_topk_prefill_g<16>(d, q, kbar, n_q, q_pos0, is_tree, nblk, cmax, idx, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace infllmv2
