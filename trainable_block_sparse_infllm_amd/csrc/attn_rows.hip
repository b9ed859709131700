// Sparse (and dense) causal attention for a chunk of queries: the prefill path
// and the dense path. (MiniCPM4 technical-report summary, QbitAI repost,
// section "Model architecture: InfLLM v2": each query attends only its selected
// context blocks, and the query heads of one GQA group share those blocks;
// short contexts keep dense attention.)
//
// Row (b, h, i) sits at position p = kv_len - n_q + i and attends
//   mode 0 (sparse): the 64 keys of every block in idx[b][h/G][i] plus its own
//           block up to p; all keys 0..p if p + 1 < dense_threshold;
//   mode 1 (dense causal): keys 0..p;      mode 2 (dense): keys 0..kv_len-1;
//   mode 3 (sliding window): keys max(0, p - window + 1)..p.
//
// Layout of the work: a workgroup (4 wavefronts) owns 4*NST*16/G consecutive
// tokens of one (b, g); each wavefront owns NST sub-tiles of 16 MFMA rows =
// 16/G tokens x G heads (one token's heads share a block set, so a sub-tile is
// the smallest set of rows with a common key set per token). The workgroup
// walks the union of its tokens' blocks in ascending order. The union (a
// range holding the tokens' own blocks and dense tokens' whole visible range,
// plus a bitmap of the selected blocks below it) is built in LDS first, so
// the walk is known ahead: each block's K and V go from HBM to registers two
// or three blocks ahead, and are staged once in LDS (two buffers, one barrier
// per block). Each wavefront runs only the sub-tiles that contain at least one
// token needing the block; rows of tokens not needing it are masked to -inf.
//
// Per active sub-tile and block (MFMA 16x16x32 bf16, fp32 accumulate):
//   S^T = K Q^T   (A = K rows from LDS, B = Q held in registers)
//   online softmax in the exp2 domain, P rounded to bf16
//   O^T += V^T P^T (A = V^T from an LDS copy stored transposed, B = P^T taken
//                   straight from the S^T accumulator layout)
// The K fragments of a key tile and the V fragments of a d tile are read from
// LDS once per wavefront and reused across its active sub-tiles.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

constexpr int kEnd = 0x7FFFFFFF;

template <int D>
struct AttnSmem {
  static constexpr int KST = D + 8;    // K row stride (bf16): conflict-free 16-byte fragment reads
  static constexpr int VST = 64 + 4;   // V^T row stride (bf16): 8-byte aligned, conflict-free 8-byte reads
  static constexpr int KSZ = 64 * KST;
  static constexpr int VSZ = D * VST;
  static constexpr int BUF = KSZ + VSZ;
};

// Global -> registers staging of one 64-key block of K and V (256 threads).
template <int D>
struct KVStage {
  static constexpr int KPIECES = 64 * D / 8 / 256;          // 16-byte K pieces per thread
  static constexpr int VPAIRS = 32 * (D / 8) / 256;         // (2 keys x 8 d) V pieces per thread
  uint4 kr[KPIECES];
  uint4 vr[VPAIRS][2];

  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase, int64_t j,
                                       int64_t kv_len, int tid) {
    const int64_t key0 = j * kBlock;
#pragma unroll
    for (int x = 0; x < KPIECES; ++x) {
      const int p = tid + 256 * x;
      const int row = p / (D / 8), c8 = p % (D / 8);
      const int64_t key = key0 + row;
      kr[x] = ldg16_if(key < kv_len, kbase + key * D + c8 * 8);
    }
#pragma unroll
    for (int x = 0; x < VPAIRS; ++x) {
      const int p = tid + 256 * x;
      const int dg = p % (D / 8), rp = p / (D / 8);
      const int64_t key = key0 + 2 * rp;
      vr[x][0] = ldg16_if(key < kv_len, vbase + key * D + dg * 8);
      vr[x][1] = ldg16_if(key + 1 < kv_len, vbase + (key + 1) * D + dg * 8);
    }
  }

  __device__ __forceinline__ void store(uint16_t* buf, int tid) const {
    using S = AttnSmem<D>;
    uint16_t* ks = buf;
    uint32_t* vt = reinterpret_cast<uint32_t*>(buf + S::KSZ);
#pragma unroll
    for (int x = 0; x < KPIECES; ++x) {
      const int p = tid + 256 * x;
      const int row = p / (D / 8), c8 = p % (D / 8);
      *reinterpret_cast<uint4*>(ks + row * S::KST + c8 * 8) = kr[x];
    }
#pragma unroll
    for (int x = 0; x < VPAIRS; ++x) {
      const int p = tid + 256 * x;
      const int dg = p % (D / 8), rp = p / (D / 8);
      const uint32_t a[4] = {vr[x][0].x, vr[x][0].y, vr[x][0].z, vr[x][0].w};
      const uint32_t c[4] = {vr[x][1].x, vr[x][1].y, vr[x][1].z, vr[x][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // d = 8*dg + 2e and 8*dg + 2e + 1; keys 2rp (low half) and 2rp+1 (high half)
        const uint32_t lo = (a[e] & 0xFFFFu) | (c[e] << 16);
        const uint32_t hi = (a[e] >> 16) | (c[e] & 0xFFFF0000u);
        vt[((8 * dg + 2 * e) * S::VST) / 2 + rp] = lo;
        vt[((8 * dg + 2 * e + 1) * S::VST) / 2 + rp] = hi;
      }
    }
  }
};

template <int D, int G, int NST>
__global__ __launch_bounds__(256) void attn_rows_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int Hq,
    int Hkv, int n_q, int64_t kv_cap, int64_t kv_len, int K, int dense_thr, int mode,
    int64_t window, float scale_log2, int ntile) {
  using S = AttnSmem<D>;
  constexpr int KS = D / 32;        // k-steps over D for S
  constexpr int DT = D / 16;        // 16-wide d tiles of O
  constexpr int TPS = 16 / G;       // tokens per sub-tile
  constexpr int TPW = NST * TPS;    // tokens per wavefront (<= 64)
  constexpr int TQ = 4 * TPW;       // tokens per workgroup
  static_assert(TPW <= 64, "one lane per token of a wavefront");

  extern __shared__ __align__(16) uint16_t smem[];
  const int64_t last_blk = (kv_len - 1) / kBlock;
  const int nwords = int(last_blk >> 5) + 1;
  constexpr int NB = (NST == 1 && D == 64) ? 2 : 1;   // blocks per step of the walk
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(smem + 2 * NB * S::BUF);   // [nwords] selected blocks
  int* s_rng = reinterpret_cast<int*>(s_bits + nwords);                // [2][4] per-wave range bounds
  int32_t* s_idx = s_rng + 8;                                          // [TQ][K]

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int r16 = l % 16, kg = l / 16;

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tok0 = tile * TQ;
  const int64_t pos0 = kv_len - n_q;          // position of query row 0
  const uint16_t* kbase = k + int64_t(bg) * kv_cap * D;
  const uint16_t* vbase = v + int64_t(bg) * kv_cap * D;

  // ---- idx rows of the tile -> LDS
  if (mode == 0) {
    for (int e = tid; e < TQ * K; e += 256) {
      const int t = e / K;
      s_idx[e] = tok0 + t < n_q ? idx[(int64_t(bg) * n_q + tok0 + t) * K + e % K] : -1;
    }
  }
  for (int e = tid; e < nwords; e += 256) s_bits[e] = 0u;

  // ---- Q fragments (B operand of S^T = K Q^T): row r16 = (token r16/G, head r16%G)
  bf16x8 qf[NST][KS];
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int t = tok0 + w * TPW + s * TPS + r16 / G;
    const int h = g * G + r16 % G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint16_t* qrow = q + ((int64_t(b) * Hq + h) * n_q + (t < n_q ? t : 0)) * D;
      qf[s][ks] = as_bf16x8(ldg16_if(t < n_q, qrow + ks * 32 + kg * 8));
    }
  }
  __syncthreads();

  // ---- per-token walk state: lane l < TPW owns token w*TPW + l of the tile
  const int my_t = tok0 + w * TPW + l;
  const bool tok_ok = l < TPW && my_t < n_q;
  const int64_t my_p = pos0 + my_t;
  const int my_own = tok_ok ? int(mode == 2 ? last_blk : my_p / kBlock) : -1;
  const bool my_dense = mode != 0 || (dense_thr > 0 && my_p + 1 < dense_thr);
  // mode 3: the block holding the token's first visible key
  const int my_lo = mode == 3 && my_p - window + 1 > 0 ? int((my_p - window + 1) / kBlock) : 0;
  const int32_t* my_idx = s_idx + (w * TPW + l) * K;
  int my_ptr = 0;
  auto next_needed = [&](int cur) -> int {
    if (!tok_ok || cur >= my_own) return kEnd;
    if (my_dense) return max(cur + 1, my_lo);
    while (my_ptr < K && my_idx[my_ptr] >= 0 && my_idx[my_ptr] <= cur) ++my_ptr;
    if (my_ptr < K && my_idx[my_ptr] >= 0 && my_idx[my_ptr] < my_own) return my_idx[my_ptr];
    return my_own;                       // own block last (entries past it are ignored)
  };
  int my_nxt = next_needed(-1);

  // ---- the tile's union of blocks, in ascending order the sequence of
  // "smallest block some token still needs" of the per-token walks, known in
  // advance so that the loads run several blocks ahead: a range [rlo, rhi]
  // (every token's own block, and all of a dense token's visible blocks)
  // plus the selected blocks below it, kept as bits.
  if (tok_ok && mode == 0 && !my_dense) {
    for (int p = 0; p < K; ++p) {
      const int j = my_idx[p];
      if (j >= 0 && j < my_own) atomicOr(&s_bits[j >> 5], 1u << (j & 31));
    }
  }
  {
    const int lo = wave_min_i32(tok_ok ? (my_dense ? my_lo : my_own) : kEnd);
    const int hi = -wave_min_i32(tok_ok ? -my_own : 1);
    if (l == 0) {
      s_rng[w] = lo;
      s_rng[4 + w] = hi;
    }
  }
  __syncthreads();
  const int rlo = __builtin_amdgcn_readfirstlane(min(min(s_rng[0], s_rng[1]), min(s_rng[2], s_rng[3])));
  const int rhi = __builtin_amdgcn_readfirstlane(max(max(s_rng[4], s_rng[5]), max(s_rng[6], s_rng[7])));
  auto find_next = [&](int j) -> int {          // the union's first block after j
    const int c = j + 1;
    if (c > rhi) return kEnd;
    if (c >= rlo) return c;
    int wd = c >> 5;
    const int wl = (rlo - 1) >> 5;
    uint32_t m = uint32_t(__builtin_amdgcn_readfirstlane(int(s_bits[wd] & (~0u << (c & 31)))));
    while (m == 0u && wd < wl) {
      ++wd;
      m = uint32_t(__builtin_amdgcn_readfirstlane(int(s_bits[wd])));
    }
    if (m != 0u) {
      const int bj = (wd << 5) + __builtin_ctz(m);
      if (bj < rlo) return bj;
    }
    return rlo;
  };

  // ---- running softmax state per sub-tile (lane's row = r16)
  f32x4 oacc[NST][DT];
  float m_run[NST], l_run[NST];
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    m_run[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[s][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int64_t row_p[NST];
#pragma unroll
  for (int s = 0; s < NST; ++s) row_p[s] = pos0 + tok0 + w * TPW + s * TPS + r16 / G;

  // Each step takes the next NB union entries: their register stages are
  // stored to LDS (buffers parity * NB + b), the barrier makes them visible
  // (and, every wavefront having finished the previous step, frees the other
  // parity's buffers), the stages are refilled with the following NB entries
  // and the NB blocks are computed. The loads of a step have the compute of
  // NB blocks to arrive: one-sequence calls at head_dim 64, whose per-block
  // compute is short against a load's latency, take two blocks per step.
  KVStage<D> st[NB];
  int jq[NB];
  jq[0] = find_next(-1);
#pragma unroll
  for (int b2 = 1; b2 < NB; ++b2) jq[b2] = jq[b2 - 1] == kEnd ? kEnd : find_next(jq[b2 - 1]);
  // an entry past the end loads a valid block that is never computed
#pragma unroll
  for (int b2 = 0; b2 < NB; ++b2) st[b2].load(kbase, vbase, jq[b2] == kEnd ? 0 : jq[b2], kv_len, tid);

  // One block of the walk: S^T, masked online softmax, O^T += V^T P^T for the
  // wavefront's sub-tiles whose tokens need it.
  auto compute = [&](int j_cur, const uint16_t* buf, uint64_t act) __attribute__((always_inline)) {
    const uint16_t* ks_ = buf;
    const uint16_t* vt_ = buf + S::KSZ;
    bool sub_on[NST];
    bool row_on[NST];
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const uint64_t bits = (act >> (s * TPS)) & ((1ull << TPS) - 1ull);
      sub_on[s] = bits != 0;
      row_on[s] = (bits >> (r16 / G)) & 1ull;
    }

    // S^T = K Q^T for every active sub-tile, one key tile (16 keys) at a time
    f32x4 sacc[NST][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(ks_ + (kt * 16 + r16) * S::KST + ks * 32 + kg * 8));
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        if (!sub_on[s]) continue;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a = mfma16(kf[ks], qf[s][ks], a);
        sacc[s][kt] = a;
      }
    }

    // masked online softmax; P^T packed for the B operand of the PV product
    bf16x8 pf[NST][2];
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      if (!sub_on[s]) continue;
      const int64_t lim = mode == 2 ? kv_len - 1 : row_p[s];   // last visible key
      const int64_t lo = mode == 3 ? row_p[s] - window + 1 : 0;  // first visible key
      float mb = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t key = int64_t(j_cur) * kBlock + kt * 16 + kg * 4 + i;
          const float x = (row_on[s] && key <= lim && key >= lo) ? sacc[s][kt][i] * scale_log2 : -INFINITY;
          sacc[s][kt][i] = x;
          mb = fmaxf(mb, x);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float m_new = fmaxf(m_run[s], mb);
      const bool none = m_new == -INFINITY;
      const float alpha = none ? 1.f : exp2f(m_run[s] - m_new);
      float ps = 0.f;
      float pv[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = none ? 0.f : exp2f(sacc[s][kt][i] - m_new);
          pv[kt][i] = e;
          ps += e;
        }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run[s] = l_run[s] * alpha + ps;
      m_run[s] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[s][dt][i] *= alpha;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint4 u;
        u.x = pack_bf16x2(pv[2 * k2][0], pv[2 * k2][1]);
        u.y = pack_bf16x2(pv[2 * k2][2], pv[2 * k2][3]);
        u.z = pack_bf16x2(pv[2 * k2 + 1][0], pv[2 * k2 + 1][1]);
        u.w = pack_bf16x2(pv[2 * k2 + 1][2], pv[2 * k2 + 1][3]);
        pf[s][k2] = as_bf16x8(u);
      }
    }

    // O^T += V^T P^T: A = V^T rows (d) from LDS, key slots matching pf's packing
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint16_t* vr = vt_ + (dt * 16 + r16) * S::VST + k2 * 32 + kg * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        const bf16x8 vf = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int s = 0; s < NST; ++s) {
          if (!sub_on[s]) continue;
          oacc[s][dt] = mfma16(vf, pf[s][k2], oacc[s][dt]);
        }
      }
    }
  };

  int parity = 0;
  while (jq[0] != kEnd) {
    int jc[NB];
    uint64_t act[NB];
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2) {
      // tokens needing this block; advance their walk
      jc[b2] = jq[b2];
      const bool active = jc[b2] != kEnd && my_nxt == jc[b2];
      act[b2] = ballot64(active);
      if (active) my_nxt = next_needed(jc[b2]);
      st[b2].store(smem + (parity * NB + b2) * S::BUF, tid);
    }
    lds_barrier();                              // no global traffic between the wavefronts here
    int j_last = jc[NB - 1];
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2) {
      jq[b2] = j_last == kEnd ? kEnd : find_next(j_last);
      j_last = jq[b2];
      st[b2].load(kbase, vbase, jq[b2] == kEnd ? jc[0] : jq[b2], kv_len, tid);
    }
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
      if (jc[b2] != kEnd) compute(jc[b2], smem + (parity * NB + b2) * S::BUF, act[b2]);
    parity ^= 1;
  }

  // ---- epilogue: O / l -> bf16; lse in natural-log units
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int t = tok0 + w * TPW + s * TPS + r16 / G;
    if (t >= n_q) continue;
    const int h = g * G + r16 % G;
    const float inv = l_run[s] > 0.f ? 1.f / l_run[s] : 0.f;
    uint16_t* dst = out + ((int64_t(b) * Hq + h) * n_q + t) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint2 u;
      u.x = pack_bf16x2(oacc[s][dt][0] * inv, oacc[s][dt][1] * inv);
      u.y = pack_bf16x2(oacc[s][dt][2] * inv, oacc[s][dt][3] * inv);
      *reinterpret_cast<uint2*>(dst + dt * 16 + kg * 4) = u;
    }
    if (lse && kg == 0)
      lse[(int64_t(b) * Hq + h) * n_q + t] = (m_run[s] + log2f(l_run[s])) * 0.69314718055994531f;
  }
}

template <int D, int G, int NST>
static hipError_t launch_rows_t(const Dims& d, int mode, const uint16_t* q, int n_q,
                                const uint16_t* k, const uint16_t* v, int64_t kv_cap,
                                int64_t kv_len, const int32_t* idx, uint16_t* out, float* lse,
                                hipStream_t s, int64_t window) {
  using S = AttnSmem<D>;
  constexpr int TQ = 4 * NST * (16 / G);
  const int ntile = (n_q + TQ - 1) / TQ;
  const int64_t nwords = ((kv_len - 1) / kBlock >> 5) + 1;      // union bitmap
  constexpr int NB = (NST == 1 && D == 64) ? 2 : 1;                // blocks per step
  const size_t lds = size_t(2 * NB * S::BUF) * 2 + size_t(nwords) * 4 + 8 * sizeof(int) +
                     size_t(TQ) * (mode == 0 ? d.K : 0) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = attn_rows_kernel<D, G, NST>;
  // raise the dynamic-LDS limit of this instance once (the largest request any call can make)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     160 * 1024);
  if (attr != hipSuccess) return attr;
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile));
  kern<<<grid, 256, lds, s>>>(q, k, v, idx, out, lse, d.Hq, d.Hkv, n_q, kv_cap, kv_len, d.K,
                              d.dense_thr, mode, window, d.scale * 1.4426950408889634f, ntile);
  return hipGetLastError();
}

hipError_t launch_attn_rows(const Dims& d, int mode, const uint16_t* q, int n_q, const uint16_t* k,
                            const uint16_t* v, int64_t kv_cap, int64_t kv_len, const int32_t* idx,
                            uint16_t* out, float* lse, hipStream_t s, int64_t window) {
  if (prefill128_stages(d, mode, kv_len) > 0)
    return launch_prefill128(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s, window);
  // Sub-tiles per wavefront: the full count when the grid fills the chip,
  // one when it would leave most CUs idle (a short or single-group call),
  // which gives four times as many workgroups.
  auto workgroups = [&](int nst) {
    const int tq = 4 * nst * (16 / d.G);
    return int64_t(d.B) * d.Hkv * ((n_q + tq - 1) / tq);
  };
  const bool few = workgroups(d.D == 128 ? 2 : 4) < 512;
#define ROWS_CASE(DD, GG, NN)                                                                    \
  if (d.D == DD && d.G == GG) {                                                                  \
    if (few) return launch_rows_t<DD, GG, 1>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s, window); \
    return launch_rows_t<DD, GG, NN>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s, window); \
  }
  ROWS_CASE(128, 4, 2) ROWS_CASE(128, 1, 2) ROWS_CASE(128, 2, 2) ROWS_CASE(128, 8, 2)
  ROWS_CASE(128, 16, 2)
  ROWS_CASE(64, 4, 4) ROWS_CASE(64, 1, 4) ROWS_CASE(64, 2, 4) ROWS_CASE(64, 8, 4)
  ROWS_CASE(64, 16, 4)
#undef ROWS_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllmv2
