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
//   0. the item's Q rows go to LDS once (16 KB, loaded straight from global
//      memory), and each wavefront reads its A fragments from there;
//   1. scoring: the wavefronts split the table of candidate blocks into chunks
//      of 32 and each computes, for all 64 rows, S = Q kbar^T with the
//      32x32x16 bf16 MFMA (A = Q rows, B = kbar^T). An accumulator column is
//      one block, so the max over the 3 kernels of a block is elementwise and
//      the head sum of a token stays within a lane (G <= 4) or a lane pair.
//      The next step's kbar fragments are loaded while one is computed.
//      Order-preserving keys of the scores go to LDS, sc[token][block];
//   2. selection: for K <= 16, four tokens per wavefront, one per 16-lane row
//      (rows16_topk of topk_select.hpp); a row it leaves unresolved (ties at
//      the threshold, many survivors) and every row for larger K take the
//      exact one-row routine over the whole wavefront (wave_topk).
#include "common.hpp"
#include "launch.hpp"
#include "prefill_tile.hpp"
#include "topk_select.hpp"

namespace infllmv2 {

namespace {

constexpr int kDK = 128;
constexpr int kQPrefetchAhead = 64;   // items ahead whose Q rows a workgroup loads into L2

__device__ __forceinline__ float pair_sum(float x) {   // lanes l and l ^ 32
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

template <int G, int KPL, bool ROWSEL>
__global__ __launch_bounds__(256, 2) void topk_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbar, int32_t* __restrict__ idx,
    int Hq, int Hkv, int n_q, int64_t q_pos0, int is_tree, int64_t nblk, int K, int ntile, int scs) {
  constexpr int TQ = 64 / G;     // tokens per work item
  constexpr int TPS = 32 / G;    // tokens per 32-row sub-tile
  constexpr int DS = kDK / 16;   // k-steps
  constexpr int SLAB = kKpb * kDK * 32;   // k-bar elements of one 32-block tile (3 kernels)

  extern __shared__ __align__(16) char smem[];
  // [TQ][scs] order-preserving keys of the scores (ordered_key_nz: every sum
  // starts from +0 or ends with + 0, so none is -0)
  uint32_t* sc = reinterpret_cast<uint32_t*>(smem);
  // then the item's Q rows, 64 x 256 bytes
  char* qt = smem + size_t(TQ) * scs * 4;
  __shared__ uint32_t scratch[4][2 * kWave];
  __shared__ uint2 rbuf[ROWSEL ? 4 : 1][4][32];
  __shared__ int32_t obuf[ROWSEL ? 4 : 1][4][16];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;

  const int it = xcd_remap(blockIdx.x, gridDim.x);

  struct Item {
    int bg, b, g, tok0, ntok;
    int64_t Cmax;
  };
  auto item_of = [&](int i) {
    Item c;
    const int tile = i % ntile;
    c.bg = i / ntile;
    c.b = c.bg / Hkv;
    c.g = c.bg % Hkv;
    c.tok0 = tile * TQ;
    c.ntok = min(TQ, n_q - c.tok0);
    const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + c.tok0 + c.ntok - 1;
    c.Cmax = min(pos_last / kBlock, nblk);
    return c;
  };
  // This wavefront's chunks of 32 blocks are w, w + 4, ...: its i-th is chunk
  // w + 4i; nmine of them.
  auto nmine_of = [&](const Item& c) { return (int((c.Cmax + 31) / 32) - w + 3) / 4; };

  // The item's 64 Q rows go to LDS once per workgroup, straight from global
  // memory (each wavefront loads four 1 KB chunks of four rows); row r
  // (token r / G, head r % G) keeps logical 16-byte piece p at physical piece
  // p ^ swz(r). Rows past the item's tokens repeat its first token (their
  // scores are never read).
  auto issue_q = [&](const Item& c) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int ch = 4 * x + w;
      const int row = 4 * ch + l / 16;
      const int t = row / G;
      const int h = c.g * G + row % G;
      const int piece = (l % 16) ^ tile::swz(row);
      const uint16_t* src = q + ((int64_t(c.b) * Hq + h) * n_q + c.tok0 + (t < c.ntok ? t : 0)) * kDK + 8 * piece;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (las_void*)(qt + ch * 1024), 16,
                                       0, 0);
    }
  };
  // A operand from the LDS tile: row 32*st + r32 of the item, k-slots
  // 8*hl .. 8*hl+7 of each 16-wide d step (piece 2*ds + hl).
  auto read_q = [&](bf16x8 (&qa)[2][DS]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = 32 * st + r32;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qa[st][ds] = as_bf16x8(*reinterpret_cast<const uint4*>(
            qt + row * (kDK * 2) + (((2 * ds + hl) ^ tile::swz(row)) << 4)));
    }
  };
  // A step is (chunk, kernel m); its B operand, lane l: block 32*chunk + r32,
  // d = 16*ds + 8*hl .., i.e. piece 2*ds + hl of the k-bar tile (layout
  // [bg][tile][m][piece][32][8]): a wave-uniform base plus a per-lane offset.
  // A prefetch past the last step is clamped to the last chunk; blocks past
  // Cmax in the last chunk are in the table (whole tiles of 32) and their
  // scores are never selected.
  auto load_step = [&](const Item& c, int nm, int i, int m, bf16x8 (&dst)[DS]) {
    const int ch = w + 4 * min(i, nm - 1);
    const uint16_t* p = kbar + int64_t(c.bg) * ((nblk + 31) >> 5) * SLAB +
                        (int64_t(ch) * kKpb + m) * (kDK * 32) + (hl * 32 + r32) * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) dst[ds] = as_bf16x8(ldg16(p + ds * 512));
  };

  bf16x8 qa[2][DS], kf0[DS], kf1[DS], kf2[DS];
  const Item cur = item_of(it);
  if (cur.Cmax > K) {
    issue_q(cur);
    if (nmine_of(cur) > 0) {
      load_step(cur, nmine_of(cur), 0, 0, kf0);
      load_step(cur, nmine_of(cur), 0, 1, kf1);
    }
    wait_vmem();      // this wavefront's Q chunks (and first k-bar steps) landed
    lds_barrier();    // ... and every wavefront's
    read_q(qa);
  }
  {
    // ------------------------------------------------------------ 1. scores
    // (the item's Q rows and its first k-bar step are already in flight)
    const int nmine = nmine_of(cur);
    if (cur.Cmax > K && nmine > 0) {
      // Accumulator register r of lane l: item row 32*st + 8*(r/4) + 4*hl +
      // r%4, block 32*chunk + r32. Max over the kernels; after the last, head
      // sums and the store.
      f32x16 best[2];
      auto compute_step = [&](int i, int m, const bf16x8 (&kf)[DS]) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          f32x16 acc;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) acc = mfma32(qa[st][ds], kf[ds], acc);
          if (m == 0) {
            best[st] = acc;
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) best[st][e] = fmax_nq(best[st][e], acc[e]);
          }
        }
        if (m != kKpb - 1) return;
        // Token row of register group a (and head pair u): st*TPS + 8a/G + u,
        // plus 4*hl/G for G <= 4; this lane's column 32*chunk + r32.
        const uint32_t srow = uint32_t(G <= 4 ? (4 * hl / G) * scs + r32 : r32) + uint32_t((w + 4 * i) * 32);
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
                sc[srow + (st * TPS + 8 * a / G + u) * scs] = ordered_key_nz(sum);
              }
          } else {
            float s4[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
              s4[a] = pair_sum(best[st][4 * a] + best[st][4 * a + 1] + best[st][4 * a + 2] + best[st][4 * a + 3]);
            if (hl == 0) {
              if constexpr (G == 8) {
#pragma unroll
                for (int a = 0; a < 4; ++a) sc[srow + (st * TPS + a) * scs] = ordered_key_nz(s4[a] + 0.f);
              } else {
#pragma unroll
                for (int a = 0; a < 2; ++a)
                  sc[srow + (st * TPS + a) * scs] = ordered_key_nz(s4[2 * a] + s4[2 * a + 1] + 0.f);
              }
            }
          }
        }
      };

      // Fragments load two steps ahead of their MFMAs; the three buffers
      // follow the three kernel slots of a chunk, so they stay in place.
      for (int i = 0; i < nmine; ++i) {
        load_step(cur, nmine, i, 2, kf2);
        compute_step(i, 0, kf0);
        load_step(cur, nmine, i + 1, 0, kf0);   // past the last chunk: clamped, unused
        compute_step(i, 1, kf1);
        load_step(cur, nmine, i + 1, 1, kf1);
        compute_step(i, 2, kf2);
      }
    }
    // Warm the L2 with the Q rows of the item that a workgroup of this XCD
    // starts about one wave of workgroups later (the grid numbering gives each
    // XCD a contiguous item range, and 256 CUs x 2 resident workgroups are 64
    // per XCD): the lines arrive during this item's selection, and that item's
    // own Q loads, otherwise a full HBM latency at its start, then hit. One
    // dword per 128-byte line: item row (64*w + l) / 2, half (64*w + l) % 2.
    uint32_t pf = 0u;
    if (w < 2) {
      const int pit = it + kQPrefetchAhead;
      const Item pc = item_of(pit < int(gridDim.x) ? pit : it);
      const int k = w * kWave + l;
      const int row = k / 2, t = row / G;
      pf = *reinterpret_cast<const uint32_t*>(
          q + ((int64_t(pc.b) * Hq + pc.g * G + row % G) * n_q + pc.tok0 + (t < pc.ntok ? t : 0)) * kDK + (k % 2) * 64);
    }
    lds_barrier();    // the item's scores are in LDS

    // ---------------------------------------------------------- 2. selection
    const int64_t Cmax = cur.Cmax;
    const int tok0 = cur.tok0, ntok = cur.ntok, bg = cur.bg;
    if constexpr (ROWSEL) {
      // Four tokens per wavefront and pass, one per 16-lane row
      // (rows16_topk); rows it leaves unresolved go to the exact one-row
      // routine with the whole wavefront.
      const int rq = l >> 4, rl = l & 15;
      const int ng = int((Cmax + 63) / 64);
      for (int tb = 4 * w; tb < ntok; tb += 16) {
        const int t = tb + rq;
        const bool act = t < ntok;
        const int64_t pos = is_tree ? q_pos0 : q_pos0 + tok0 + (act ? t : tb);
        const int C = act ? int(min(pos / kBlock, nblk)) : 0;
        uint32_t* row = sc + (act ? t : tb) * scs;
        // Entries C .. 64*ng - 1 (later blocks, or never written) read as
        // key 0. The tokens of one item are < 64 positions apart, so
        // C >= Cmax - 1 and there are at most 64 of them.
        if (act && Cmax > K) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = C + rl + 16 * u;
            if (j < 64 * ng) row[j] = 0u;
          }
        }
        int32_t* out = act ? idx + (int64_t(bg) * n_q + tok0 + t) * K : nullptr;
        const bool ok = rows16_topk<KPL>(row, ng, C, K, out, rbuf[w][rq], obuf[w][rq]);
        uint64_t bad = ballot64(!ok && rl == 0);
        while (bad) {
          const int qq = __builtin_ctzll(bad) / 16;
          bad &= bad - 1;
          const int tt = tb + qq;
          const int64_t pp = is_tree ? q_pos0 : q_pos0 + tok0 + tt;
          const int Ct = int(min(pp / kBlock, nblk));
          uint32_t key[KPL];
#pragma unroll
          for (int r = 0; r < KPL; ++r) {
            const int j = r * kWave + l;
            key[r] = j < Ct ? sc[tt * scs + j] : 0u;
          }
          wave_topk<KPL>(key, Ct, K, idx + (int64_t(bg) * n_q + tok0 + tt) * K, scratch[w]);
        }
      }
    } else {
      for (int t = w; t < ntok; t += 4) {
        const int64_t pos = is_tree ? q_pos0 : q_pos0 + tok0 + t;
        const int C = int(min(pos / kBlock, nblk));
        uint32_t key[KPL];
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const int j = r * kWave + l;
          key[r] = (C > K && j < C) ? sc[t * scs + j] : 0u;
        }
        wave_topk<KPL>(key, C, K, idx + (int64_t(bg) * n_q + tok0 + t) * K, scratch[w]);
      }
    }
    // The prefetched dword is not used; an empty asm consumes it so that the
    // load stays (the wave ends only after it has returned).
    asm volatile("" ::"v"(pf));
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

template <int G, int KPL, bool ROWSEL>
static hipError_t launch_topk_prefill_t(const Dims& d, const uint16_t* q, const uint16_t* kbar,
                                        int n_q, int64_t q_pos0, int is_tree, int64_t nblk,
                                        int scs, int32_t* idx, hipStream_t s) {
  constexpr int TQ = 64 / G;
  const int ntile = (n_q + TQ - 1) / TQ;
  auto kern = topk_prefill_kernel<G, KPL, ROWSEL>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     80 * 1024);
  if (attr != hipSuccess) return attr;
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile));
  kern<<<grid, 256, size_t(TQ) * scs * 4 + 64 * kDK * 2, s>>>(q, kbar, idx, d.Hq, d.Hkv, n_q, q_pos0, is_tree,
                                               nblk, d.K, ntile, scs);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_topk_prefill_g(const Dims& d, const uint16_t* q, const uint16_t* kbar,
                                        int n_q, int64_t q_pos0, int is_tree, int64_t nblk,
                                        int64_t cmax, int32_t* idx, hipStream_t s) {
  const TopkPrefillPlan p = topk_prefill_plan(d, cmax);
  const bool rowsel = d.K <= 16;
#define TP_CASE(P)                                                                                  \
  case P:                                                                                           \
    return rowsel ? launch_topk_prefill_t<G, P, true>(d, q, kbar, n_q, q_pos0, is_tree, nblk, p.scs, idx, s) \
                  : launch_topk_prefill_t<G, P, false>(d, q, kbar, n_q, q_pos0, is_tree, nblk, p.scs, idx, s);
  switch (p.kpl) {
    TP_CASE(1) TP_CASE(2) TP_CASE(4) TP_CASE(8)
#undef TP_CASE
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
