// LSE-normalized block scores (MiniCPM4 technical-report summary, QbitAI
// repost, section "Model architecture: InfLLM v2", item on more efficient
// operators: top-K blocks are chosen with the help of a LogSumExp estimate).
// The pages give no formula; the reading implemented here: per head h of a
// GQA group, the kernel scores s = scale * q_h . kbar[j][m] over every
// candidate kernel (j < C, m < 3) are softmax-normalized by their log-sum-exp
// LSE_h; a block's normalized relevance is the max over its kernels; the
// group sums its heads:
//   R[j] = sum_h exp(max_m s_{h,j,m} - LSE_h)  for j < C,  -inf otherwise.
// R has the layout of the raw scores, so the same selection paths consume it.
//
// Two kernels. score_lse_kernel: one wavefront per (b, g, tile of 32 blocks,
// 32 query rows), the 32x32x16 MFMA with 32 (node, head) rows of q as A and
// the tile's kernels as B (as the raw scoring kernel); it stores each head's
// block maxima (log2 units) and the tile's partial log-sum-exp per head
// (max, sum of exp2 relative to it), reduced across the 32 block lanes.
// score_lse_combine_kernel: per (b, g, node) and chunk of 512 blocks, merges
// the tile partials into LSE_h (one wavefront per head) and writes R.
// Workspace: hs [B*Hkv][n_q][G][nblk] fp32 and part [B*Hkv][n_q][G][ntile]
// float2.
#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

template <int D, int G>
__global__ __launch_bounds__(64) void score_lse_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kbar,
                                                       float* __restrict__ hs,
                                                       float2* __restrict__ part, int Hq, int Hkv,
                                                       int n_q, int64_t q_pos0, int is_tree,
                                                       int64_t nblk, int ntile, float scale_log2) {
  constexpr int DS = D / 16;
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;
  const int tile = blockIdx.x % ntile;
  const int bg = blockIdx.x / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int64_t j0 = int64_t(tile) * 32;
  const int row0 = blockIdx.y * 32;
  const int rows = n_q * G;

  // B operand: block j0 + r32, d = 16*ds + 8*hl .. (piece 2*ds + hl); the
  // table is padded to whole tiles, so every load is in bounds.
  bf16x8 kf[kKpb][DS];
#pragma unroll
  for (int m = 0; m < kKpb; ++m)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      kf[m][ds] = as_bf16x8(ldg16_nt(kbar + kbar_off<D>(bg, m, 2 * ds + hl, j0 + r32, nblk)));
  // A operand: row row0 + r32 -> (node, head)
  bf16x8 qa[DS];
  {
    const int row = row0 + r32;
    const int node = row / G;
    const bool ok = node < n_q;
    const uint16_t* qrow = q + ((int64_t(b) * Hq + g * G + row % G) * n_q + (ok ? node : 0)) * D + 8 * hl;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qa[ds] = as_bf16x8(ldg16_if(ok, qrow + 16 * ds));
  }
  f32x16 acc[kKpb];
#pragma unroll
  for (int m = 0; m < kKpb; ++m) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[m][e] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) acc[m] = mfma32(qa[ds], kf[m][ds], acc[m]);
  }

  // register e of lane l: row row0 + 8*(e/4) + 4*hl + e%4, block j0 + r32;
  // register groups whose rows all lie past the last row are skipped (a
  // single-token decode row of G <= 4 heads uses only the first group)
  const int64_t j = j0 + r32;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (row0 + 8 * (e / 4) >= rows) break;
    const int row = row0 + 8 * (e / 4) + 4 * hl + e % 4;
    const int node = row / G, hh = row % G;
    const int64_t C = min((is_tree ? q_pos0 : q_pos0 + node) / kBlock, nblk);
    const bool cand = j < C;
    float s[kKpb];
    float bm = -INFINITY;
#pragma unroll
    for (int m = 0; m < kKpb; ++m) {
      s[m] = cand ? acc[m][e] * scale_log2 : -INFINITY;
      bm = fmaxf(bm, s[m]);
    }
    // the tile's partial log-sum-exp of this row, over its 32 blocks x 3 kernels
    float mx = bm;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float ps = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int m = 0; m < kKpb; ++m) ps += __builtin_amdgcn_exp2f(s[m] - mx);
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) ps += __shfl_xor(ps, o);
    if (row < rows) {
      const int64_t rr = (int64_t(bg) * n_q + node) * G + hh;     // (bg, node, head)
      if (j < nblk) hs[rr * nblk + j] = bm;
      if (r32 == 0) part[rr * ntile + tile] = make_float2(mx, ps);
    }
  }
}

// One workgroup of 256 threads per (b, g, node) and chunk of 512 blocks.
// Every thread first loads the per-head block values of its two blocks;
// meanwhile wavefront w merges the tile partials of heads w, w + 4, ... into
// LSE_h (lanes over tiles) and shares them through LDS; then every thread
// writes R for its two blocks.
constexpr int kLseChunk = 512;

template <int G>
__global__ __launch_bounds__(256) void score_lse_combine_kernel(const float* __restrict__ hs,
                                                                const float2* __restrict__ part,
                                                                float* __restrict__ scores,
                                                                int n_q, int64_t q_pos0,
                                                                int is_tree, int64_t nblk,
                                                                int ntile) {
  constexpr int PER = kLseChunk / 256;
  __shared__ float s_lse2[G];
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const int64_t rowid = blockIdx.x;                  // (bg, node)
  const int node = int(rowid % n_q);
  const int64_t C = min((is_tree ? q_pos0 : q_pos0 + node) / kBlock, nblk);
  const float* hrow = hs + rowid * G * nblk;
  float hv[PER][G];
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int64_t j = int64_t(blockIdx.y) * kLseChunk + x * 256 + threadIdx.x;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) hv[x][hh] = j < C ? hrow[hh * nblk + j] : -INFINITY;
  }
  for (int hh = w; hh < G; hh += 256 / kWave) {
    const float2* pr = part + (rowid * G + hh) * ntile;
    float M = -INFINITY;
    for (int t = l; t < ntile; t += kWave) M = fmaxf(M, pr[t].x);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    float S = 0.f;
    if (M != -INFINITY)
      for (int t = l; t < ntile; t += kWave) {
        const float2 p = pr[t];
        if (p.x != -INFINITY) S += p.y * __builtin_amdgcn_exp2f(p.x - M);
      }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) S += __shfl_xor(S, o);
    if (l == 0) s_lse2[hh] = M + log2f(S);           // S >= 1: the tile holding M adds >= 1
  }
  __syncthreads();
  float* out = scores + rowid * nblk;
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int64_t j = int64_t(blockIdx.y) * kLseChunk + x * 256 + threadIdx.x;
    if (j >= nblk) break;
    float r = -INFINITY;
    if (j < C) {
      r = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) r += __builtin_amdgcn_exp2f(hv[x][hh] - s_lse2[hh]);
    }
    out[j] = r;
  }
}

size_t score_lse_workspace_bytes(const Dims& d, int n_q, int64_t nblk) {
  const int64_t ntile = (nblk + 31) / 32;
  const int64_t rr = int64_t(d.B) * d.Hkv * n_q * d.G;
  const size_t a = (size_t(rr * nblk) * 4 + 255) / 256 * 256;
  return a + size_t(rr * ntile) * 8;
}

hipError_t launch_scores_lse(const Dims& d, const uint16_t* q, int n_q, int64_t q_pos0,
                             int is_tree, const uint16_t* kbar, int64_t nblk, float* scores,
                             void* ws, size_t ws_bytes, hipStream_t s) {
  if (ws_bytes < score_lse_workspace_bytes(d, n_q, nblk)) return hipErrorInvalidValue;
  const int ntile = int((nblk + 31) / 32);
  const int64_t rr = int64_t(d.B) * d.Hkv * n_q * d.G;
  float* hs = static_cast<float*>(ws);
  float2* part = reinterpret_cast<float2*>(static_cast<char*>(ws) + (size_t(rr * nblk) * 4 + 255) / 256 * 256);
  const int rows = n_q * d.G;
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile), unsigned((rows + 31) / 32));
  const dim3 cgrid(unsigned(int64_t(d.B) * d.Hkv * n_q), unsigned((nblk + kLseChunk - 1) / kLseChunk));
  const float sl2 = d.scale * 1.4426950408889634f;
#define LSE_CASE(DD, GG)                                                                         \
  if (d.D == DD && d.G == GG) {                                                                  \
    score_lse_kernel<DD, GG><<<grid, 64, 0, s>>>(q, kbar, hs, part, d.Hq, d.Hkv, n_q, q_pos0,    \
                                                 is_tree, nblk, ntile, sl2);                     \
    const hipError_t e = hipGetLastError();                                                      \
    if (e != hipSuccess) return e;                                                               \
    score_lse_combine_kernel<GG><<<cgrid, 256, 0, s>>>(hs, part, scores, n_q, q_pos0, is_tree,    \
                                                      nblk, ntile);                              \
    return hipGetLastError();                                                                    \
  }
  LSE_CASE(128, 1) LSE_CASE(128, 2) LSE_CASE(128, 4) LSE_CASE(128, 8) LSE_CASE(128, 16)
  LSE_CASE(64, 1) LSE_CASE(64, 2) LSE_CASE(64, 4) LSE_CASE(64, 8) LSE_CASE(64, 16)
#undef LSE_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllmv2
