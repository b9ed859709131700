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
// shared by all n_q*G query rows of the group. One wavefront scores one tile
// of 32 blocks (3*D*64 contiguous bytes of the k-bar table; each load
// instruction reads one contiguous kilobyte) with the 32x32x16 MFMA: operand A
// is 32 (node, head) rows of q, operand B the 32 blocks' kernels of one slot
// m. The max over m is elementwise across the three accumulators; the rows of
// one node sit in one lane's registers (G <= 4) or in a lane and its partner
// 32 lanes away (G >= 8), so the head sum needs at most one cross-lane step,
// and each node's 32 scores leave as one 128-byte store.
#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

// NR: 32-row tiles of (node, head) rows per wavefront; rows are node * G + head.
template <int D, int G, int NR>
__global__ __launch_bounds__(64) void score_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ kbar,
                                                   float* __restrict__ scores, int Hq, int Hkv,
                                                   int n_q, int64_t q_pos0, int is_tree,
                                                   int64_t nblk, int ntile,
                                                   const int64_t* __restrict__ kv_lens) {
  constexpr int DS = D / 16;
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  if (kv_lens) q_pos0 = kv_lens[b] - 1;              // per-sequence single-token position
  const int64_t j0 = int64_t(tile) * 32;
  const int row0 = blockIdx.y * NR * 32;
  const int node_hi = min(n_q - 1, (row0 + NR * 32 - 1) / G);
  const int64_t cmax = min((is_tree ? q_pos0 : q_pos0 + node_hi) / kBlock, nblk);

  f32x16 best[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr)
#pragma unroll
    for (int e = 0; e < 16; ++e) best[nr][e] = 0.f;

  if (j0 < cmax) {
    // B operand: block j0 + r32, d = 16*ds + 8*hl .. = piece 2*ds + hl. The
    // table is padded to whole tiles, so every load is in bounds.
    bf16x8 kf[kKpb][DS];
#pragma unroll
    for (int m = 0; m < kKpb; ++m)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kf[m][ds] = as_bf16x8(ldg16_nt(kbar + kbar_off<D>(bg, m, 2 * ds + hl, j0 + r32, nblk)));
    // A operand: row row0 + 32*nr + r32 -> (node, head), same k-slots.
    bf16x8 qa[NR][DS];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      const int row = row0 + 32 * nr + r32;
      const int node = row / G;
      const bool ok = node < n_q;
      const uint16_t* qrow =
          q + ((int64_t(b) * Hq + g * G + row % G) * n_q + (ok ? node : 0)) * D + 8 * hl;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qa[nr][ds] = as_bf16x8(ldg16_if(ok, qrow + 16 * ds));
    }
#pragma unroll
    for (int m = 0; m < kKpb; ++m)
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) acc = mfma32(qa[nr][ds], kf[m][ds], acc);
#pragma unroll
        for (int e = 0; e < 16; ++e) best[nr][e] = m == 0 ? acc[e] : fmaxf(best[nr][e], acc[e]);
      }
  }

  // Register r of lane l holds row row0 + 32*nr + 8*(r/4) + 4*hl + r%4 and
  // block j0 + r32.
  const int64_t j = j0 + r32;
  auto store = [&](int row, float v) {
    const int node = row / G;
    if (node >= n_q || j >= nblk) return;
    const int64_t C = (is_tree ? q_pos0 : q_pos0 + node) / kBlock;
    scores[(int64_t(bg) * n_q + node) * nblk + j] = j < C ? v : -INFINITY;
  };
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const int rbase = row0 + 32 * nr + 4 * hl;
    if constexpr (G <= 4) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int u = 0; u < 4 / G; ++u) {
          float v = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) v += best[nr][4 * a + G * u + h];
          store(rbase + 8 * a + G * u, v);
        }
    } else {
      constexpr int NQ = G / 8;  // register quads per node in each lane half
#pragma unroll
      for (int a0 = 0; a0 < 4 / NQ; ++a0) {
        float v = 0.f;
#pragma unroll
        for (int a = a0 * NQ; a < a0 * NQ + NQ; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) v += best[nr][4 * a + i];
        v += __shfl_xor(v, 32);
        if (hl == 0) store(rbase + 8 * a0 * NQ, v);
      }
    }
  }
}

hipError_t launch_scores(const Dims& d, const uint16_t* q, int n_q, int64_t q_pos0, int is_tree,
                         const uint16_t* kbar, int64_t nblk, float* scores, hipStream_t s,
                         const int64_t* kv_lens) {
  const int rows = n_q * d.G;
  // One 32-row tile per wavefront up to four tiles: more wavefronts in flight for a few
  // hundred rows (a 16-node tree's 64 rows: 11.5 -> 8.8 us), the k-bar tile re-read from
  // L2 by each; larger row counts take two tiles per wavefront.
  const int NR = rows > 128 ? 2 : 1;
  const int ntile = int((nblk + 31) / 32);
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile), unsigned((rows + 32 * NR - 1) / (32 * NR)));
#define SCORE_CASE(DD, GG, NN)                                                                   \
  if (d.D == DD && d.G == GG && NR == NN) {                                                      \
    score_kernel<DD, GG, NN><<<grid, 64, 0, s>>>(q, kbar, scores, d.Hq, d.Hkv, n_q, q_pos0,      \
                                                 is_tree, nblk, ntile, kv_lens);                 \
    return hipGetLastError();                                                                    \
  }
#define SCORE_G(DD, GG) SCORE_CASE(DD, GG, 1) SCORE_CASE(DD, GG, 2)
  SCORE_G(128, 1) SCORE_G(128, 2) SCORE_G(128, 4) SCORE_G(128, 8) SCORE_G(128, 16)
  SCORE_G(64, 1) SCORE_G(64, 2) SCORE_G(64, 4) SCORE_G(64, 8) SCORE_G(64, 16)
#undef SCORE_G
#undef SCORE_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllmv2
