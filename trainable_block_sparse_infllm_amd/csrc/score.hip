// Block scoring for decode and draft trees (MiniCPM4 technical-report summary,
// QbitAI repost, section "Model architecture: InfLLM v2": item 1, a query's
// relevance to a block is its maximum relevance to the block's semantic
// kernels; item 2, the query heads of one GQA group share the block choice, so
// their relevances are summed).
//
//   R[b][g][i][j] = sum_{h in group g} max_{m<3} q[b][h][i] . (kernel m of block j)
//
// for j < floor(p_i / 64), -inf for every other j (p_i = q_pos0 + i, or q_pos0
// for all tree nodes).
//
// HBM-bound: every candidate's 3*D bf16 kernels are read once per (b, g) and
// shared by all n_q*G query columns of the group. One wavefront scores 16
// blocks with MFMA 16x16x32 (A = 16 kernel rows of one kernel slot m, B = the
// group's query columns); the max over m is elementwise across the three
// accumulator tiles and the head sum is a shuffle over G adjacent lanes.
#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

// NT: 16-column tiles of query columns (n_q * G <= 16 * NT).
template <int D, int NT>
__global__ __launch_bounds__(64) void score_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ kbar,
                                                   float* __restrict__ scores, int Hq, int Hkv,
                                                   int G, int n_q, int64_t q_pos0, int is_tree,
                                                   int64_t nblk, int ntile) {
  constexpr int KS = D / 32;
  const int l = lane_id();
  const int r16 = l % 16, kg = l / 16;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int64_t j0 = int64_t(tile) * 16;

  // B operand: query columns c = col0 + nt*16 + r16 -> (node c / G, head c % G).
  const int col0 = blockIdx.y * NT * 16;
  bf16x8 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = col0 + nt * 16 + r16;
    const int node = c / G, hh = c % G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint16_t* qrow = q + ((int64_t(b) * Hq + g * G + hh) * n_q + (node < n_q ? node : 0)) * D;
      qf[nt][ks] = as_bf16x8(ldg16_if(node < n_q, qrow + ks * 32 + kg * 8));
    }
  }

  const int64_t jrow = j0 + r16;  // block row this lane feeds into the A operand
  const bool row_ok = jrow < nblk;
  // A fragment row: block jrow; k-slots 8*kg .. of d step ks = piece 4*ks + kg
  const int64_t jr = row_ok ? jrow : 0;

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

  // Sum over the G heads of each node: G adjacent lanes (aligned groups).
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = best[nt][i];
      for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o);
      best[nt][i] = v;
    }
    const int c = col0 + nt * 16 + r16;
    const int node = c / G;
    if (c % G == 0 && node < n_q) {
      const int64_t pos = is_tree ? q_pos0 : q_pos0 + node;
      const int64_t C = pos / kBlock;
      float* dst = scores + ((int64_t(bg) * n_q + node) * nblk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t j = j0 + kg * 4 + i;
        if (j < nblk) dst[j] = j < C ? best[nt][i] : -INFINITY;
      }
    }
  }
}

hipError_t launch_scores(const Dims& d, const uint16_t* q, int n_q, int64_t q_pos0, int is_tree,
                         const uint16_t* kbar, int64_t nblk, float* scores, hipStream_t s) {
  const int cols = n_q * d.G;
  const int NT = (cols + 15) / 16;
  const int ntile = int((nblk + 15) / 16);
  const unsigned ycols = unsigned((NT + 3) / 4);  // column groups of 64 when NT > 4
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile), NT > 4 ? ycols : 1u);
  const int NTk = NT > 4 ? 4 : NT;
#define SCORE_CASE(DD, NN)                                                                       \
  if (d.D == DD && NTk <= NN) {                                                                   \
    score_kernel<DD, NN><<<grid, 64, 0, s>>>(q, kbar, scores, d.Hq, d.Hkv, d.G, n_q, q_pos0,    \
                                             is_tree, nblk, ntile);                              \
    return hipGetLastError();                                                                    \
  }
  SCORE_CASE(128, 1) SCORE_CASE(128, 2) SCORE_CASE(128, 4)
  SCORE_CASE(64, 1) SCORE_CASE(64, 2) SCORE_CASE(64, 4)
#undef SCORE_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllmv2
