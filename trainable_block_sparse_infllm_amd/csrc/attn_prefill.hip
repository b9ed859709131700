// Sparse causal prefill attention and dense attention, head_dim 128
// (MiniCPM4 technical-report summary, QbitAI repost, section "Model
// architecture: InfLLM v2": each query attends only its selected context
// blocks, the query heads of one GQA group share those blocks, and short
// contexts keep dense attention).
//
// Row (b, h, i) sits at position p = kv_len - n_q + i and attends
//   mode 0 (sparse): the 64 keys of every block in idx[b][h/G][i] below its own
//           block, plus its own block up to p; all keys 0..p if
//           p + 1 < dense_threshold;
//   mode 1 (dense causal): keys 0..p;      mode 2 (dense): keys 0..kv_len-1;
//   mode 3 (sliding window, the draft model's attention): keys
//           max(0, p - window + 1)..p.
//
// Work layout. A workgroup of NW wavefronts (4; 2 for G = 1) owns TQ <= 64
// consecutive tokens of one (b, g); each wavefront owns one sub-tile of 32
// MFMA rows (32/G tokens x G heads; one token's heads share a key set). Two
// workgroups share a CU, so the wavefronts on a SIMD are not tied by
// barriers and one's MFMA work overlaps the other's softmax and waits. The products run on the
// 32x32x16 bf16 MFMA, which on gfx950 sustains twice the rate of the 16x16x32
// form. On the 32K workload 64 consecutive tokens need ~45 distinct blocks
// between them while each needs 17, so the tile walks that union once and
// every staged block serves all of the tile's tokens that need it:
//
//   1. union: the tile's blocks are listed in ascending order, each with a
//      64-bit mask of the tile's tokens that attend it. Own blocks and dense
//      prefixes are ranges, so their mask bits are computed; only selected
//      blocks go through an LDS bitmap. A tile whose tokens are all dense
//      needs no list: block u is entry u;
//   2. a ring of NSTAGE LDS stages holds K and V of upcoming blocks, filled
//      straight from HBM (global_load_lds, no staging registers), so
//      NSTAGE - 1 blocks are in flight while one is computed; one barrier per
//      block;
//   3. per block, a wavefront whose tokens need it computes S^T = K Q^T
//      (A = K fragments from LDS, B = Q in registers), the masked online
//      softmax in the exp2 domain, and O^T += V^T P^T (A = V^T fragments from
//      the transpose read ds_read_b64_tr_b16 of the row-major V tile, B = P^T
//      taken from the S^T accumulators without data movement).
//
// LDS tiles are row-major 64 x 128 bf16 whose 16-byte pieces are XOR-swizzled
// per row by swz(r) (prefill_tile.hpp), which keeps both the row reads of K
// and the transpose reads of V free of bank conflicts.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "prefill_tile.hpp"

namespace infllmv2 {

using namespace tile;

// The kernel body; WINDOW (mode 3) is a template flag so the sliding-window
// code is compiled out of modes 0-2 and the two run as separately named
// kernels.
template <int G, bool WINDOW>
__device__ __forceinline__ void prefill_attn_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int Hq,
    int Hkv, int n_q, int64_t kv_cap, int64_t kv_len, int K, int dense_thr, int mode,
    int64_t window, float scale_log2, int ntile, int umax) {
  if constexpr (WINDOW) mode = 3;
  using Sh = PrefillShape<G>;
  constexpr int TPS = Sh::TPS, NW = Sh::NW, TQ = Sh::TQ, NT = Sh::NT, LPS = Sh::LPS;
  constexpr int DS = kD / 16;                // k-steps of S^T = K Q^T
  constexpr int DT = kD / 32;                // 32-wide d tiles of O^T
  constexpr float kRescale = 8.f;            // log2 headroom before the running max is moved

  extern __shared__ __align__(16) char smem[];
  char* ring = smem;                                                            // [2 stages]
  uint64_t* u_mask = reinterpret_cast<uint64_t*>(smem + 2 * kStageBytes);      // [umax]
  int32_t* u_blk = reinterpret_cast<int32_t*>(u_mask + umax);                   // [umax]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(u_blk + umax);                 // [256]
  int32_t* wbase = reinterpret_cast<int32_t*>(bitmap + 256);                    // [256]
  int32_t* wtot = wbase + 256;                                                  // [NW]
  int32_t* jsel = wtot + 16;                                                    // [TQ * K]

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;        // MFMA column (row of the sub-tile), lane half
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  // tiles of a (b, g) from the last one down: the grid's last workgroups then
  // hold the prompt's first tokens, whose unions are the shortest
  const int tile = ntile - 1 - item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tok0 = tile * TQ;
  const int ntok = min(TQ, n_q - tok0);
  const int64_t base = kv_len - n_q + tok0;             // position of the tile's first token
  const int64_t last_blk = (kv_len - 1) / kBlock;
  const int64_t own_lo = mode == 2 ? last_blk : base / kBlock;
  const int64_t own_hi = mode == 2 ? last_blk : (base + ntok - 1) / kBlock;
  // tokens t < dend attend densely
  const int64_t dend = mode != 0 ? ntok : (dense_thr > 0 ? dense_thr - 1 - base : 0);
  const bool tile_dense = dend >= ntok;
  // a tile walking a contiguous range starts at block blk0 (mode 3: the block
  // holding its first token's window start)
  const int64_t blk0 = WINDOW ? (base - window + 1 > 0 ? (base - window + 1) / kBlock : 0) : 0;
  const uint16_t* kbase = k + int64_t(bg) * kv_cap * kD;
  const uint16_t* vbase = v + int64_t(bg) * kv_cap * kD;

  // This lane's query row: token tok0 + w*TPS + r32/G, head g*G + r32%G.
  const int my_t = tok0 + w * TPS + r32 / G;

  auto range_mask_t = [&](int64_t j) -> uint64_t {
    return range_mask(j, mode, base, dend, ntok, window);
  };

  // ---------------------------------------------------------------- 1. union
  int U;
  if (tile_dense)
    U = int(own_hi - blk0) + 1;
  else
    U = build_union<NT, NW>(idx, bg, n_q, tok0, ntok, base, own_lo, own_hi, dend, K, umax, mode,
                            u_mask, u_blk, bitmap, wbase, wtot, jsel);
  U = __builtin_amdgcn_readfirstlane(U);
  auto blk_of = [&](int u) -> int64_t {
    return tile_dense ? blk0 + u : int64_t(__builtin_amdgcn_readfirstlane(lds_read(u_blk + u)));
  };
  // Raw LDS reads of an entry's block / token mask, issued one iteration
  // ahead so that their latency overlaps the stage wait; made uniform at use.
  auto blk_raw = [&](int u) -> int32_t { return tile_dense ? int32_t(blk0) + u : lds_read(u_blk + u); };
  auto mask_raw = [&](int u) -> uint64_t {
    return tile_dense ? range_mask_t(blk0 + u) : lds_read(u_mask + u);
  };

  // ---------------------------------------------------------------- ring prologue
  const uint32_t nrec = uint32_t(kv_len) * uint32_t(kD * 2);   // bytes of rows < kv_len
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kbase), 0, int(nrec), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vbase), 0, int(nrec), 0x00020000);
  if (U > 0) issue_stage<NW>(ring, rk, rv, blk_of(0) * kBlock, w, l);
  // Q^T fragments (B operand, k-slots 8*hl .. 8*hl+7 of each 16-wide d step),
  // loaded after the union is built (waiting for its index loads would also
  // wait for these, the counter being in order) and together with the first
  // ring stage, whose wait covers them.
  bf16x8 qf[DS];
  {
    const int h = g * G + r32 % G;
    const uint16_t* qrow = q + ((int64_t(b) * Hq + h) * n_q + (my_t < n_q ? my_t : 0)) * kD;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = as_bf16x8(ldg16_if(my_t < n_q, qrow + ds * 16 + hl * 8));
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  // Row sums of P come from the MFMA as well: O^T's product with an all-ones
  // A operand puts every row's sum of the bf16 P in each accumulator register
  // (register 0 is read). It takes four MFMAs per block off the VALU, which
  // bounds this loop.
  f32x16 lacc;
#pragma unroll
  for (int e = 0; e < 16; ++e) lacc[e] = 0.f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = __bf16(1.0f);
  float m_run = -INFINITY;
  const int64_t row_p = base + w * TPS + r32 / G;      // this lane's row position
  const int64_t p_first = base + w * TPS;              // the wavefront's first token

  // Lane parts of the fragment offsets. K fragment (kt, ds): row 32*kt + r32,
  // piece 2*ds + hl; swz(row) = swz(r32), so the offset is
  // 8192*kt + (k_lane ^ (ds << 5)). V^T fragment (dt, ks), group q: lane k of
  // each 16-lane group reads V[16*ks + 8*q + 4*hl + k/4][32*dt + 16*((l/16)%2) + 4*(k%4)];
  // the row's swizzle depends on (q, lane) only, so the offset is
  // 4096*ks + (v_lane[q] ^ (dt << 6)).
  const int k_lane = r32 * (kD * 2) + ((hl ^ swz(r32)) << 4);
  int v_lane[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int j = l % 16;
    const int row = 8 * qq + 4 * hl + j / 4;
    const int piece = 2 * ((l / 16) % 2) + (j % 4) / 2;
    v_lane[qq] = row * (kD * 2) + ((piece ^ swz(row)) << 4) + 8 * (j & 1);
  }

  // ---------------------------------------------------------------- 2/3. ring + compute
  // Two ring slots: entry u sits in slot u % 2; entry u + 1 is issued into
  // the other slot once every wavefront has passed the barrier of entry u
  // (so nobody still reads entry u - 1 there).
  int32_t blk_nx = U > 0 ? blk_raw(0) : 0;         // entry u's block and mask
  uint64_t mask_nx = U > 0 ? mask_raw(0) : 0ull;
  // Per-lane parts of the fragment addresses; the ring slot, tile and k-step
  // parts are compile-time offsets (the loop below is unrolled by the two
  // ring slots), so every fragment read is a ds_read with an immediate offset.
  int kaddr[DS], vaddr[2][DT];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) kaddr[ds] = k_lane ^ (ds << 5);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    vaddr[0][dt] = v_lane[0] ^ (dt << 6);
    vaddr[1][dt] = v_lane[1] ^ (dt << 6);
  }

  auto step = [&](int u, auto slot_c) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;   // == u % 2
    const int32_t blk_cur = blk_nx;
    const uint64_t mask_cur = mask_nx;
    if (u + 1 < U) {
      blk_nx = blk_raw(u + 1);
      mask_nx = mask_raw(u + 1);
    }
    wait_vmem();                                  // this wave's loads of entry u landed
    wait_lds();
    ring_barrier();                               // ... and every wave's; the other slot is free
    if (u + 1 < U)
      issue_stage<NW>(ring + (1 - SLOT) * kStageBytes, rk, rv,
                      int64_t(__builtin_amdgcn_readfirstlane(blk_nx)) * kBlock, w, l);
    const char* kt_b = ring + SLOT * kStageBytes;
    const lds_char* vt_b = (const lds_char*)(ring + SLOT * kStageBytes + kTileBytes);
    const int64_t key0 = int64_t(__builtin_amdgcn_readfirstlane(blk_cur)) * kBlock;
    const uint64_t tmask = uniform_u64(mask_cur);
    const uint32_t bits = uint32_t(tmask >> (w * TPS)) & uint32_t((1ull << TPS) - 1ull);
    if (bits == 0) return;                        // no token of this wavefront needs the block

    // S^T = K Q^T: two 32-key tiles. Accumulator register r of lane l holds
    // key 32*kt + 8*(r/4) + 4*hl + r%4 of row r32.
    f32x16 sacc[2];
    {
      bf16x8 kf[2][DS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) kf[kt][ds] = lds_read_k(kt_b + kt * 8192, kaddr[ds]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) sacc[kt] = mfma32(kf[kt][ds], qf[ds], sacc[kt]);
      }
      // K fragment reads run four ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }

    // Masked online softmax in the exp2 domain. A row whose token does not
    // need the block gets P = 0 through a -inf bias; only a block reaching past
    // a row's position (its own block, or keys beyond kv_len) is masked key by
    // key. The running max (log2 units) moves only when a row's block max
    // exceeds it by more than kRescale, so O and l are rescaled rarely;
    // exponents stay <= kRescale and the final O / l is unchanged.
    const bool row_on = (bits >> (r32 / G)) & 1u;
    const bool causal = mode == 2 ? key0 + kBlock > kv_len : key0 + kBlock - 1 > p_first;
    if (causal) {
      const int64_t rel = (mode == 2 ? kv_len - 1 : row_p) - key0;   // last visible key
      const int lim = int(rel < 63 ? rel : 63);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sacc[kt][e] = (32 * kt + 8 * (e / 4) + 4 * hl + e % 4 <= lim) ? sacc[kt][e] : -INFINITY;
    }
    // sliding window: keys before a row's window start, in a block that some
    // row of the wavefront sees only in part
    if (WINDOW && key0 < p_first + TPS - window) {
      const int64_t rlo = row_p - window + 1 - key0;                  // first visible key
      const int lo = int(rlo > 0 ? (rlo < kBlock ? rlo : kBlock) : 0);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sacc[kt][e] = (32 * kt + 8 * (e / 4) + 4 * hl + e % 4 >= lo) ? sacc[kt][e] : -INFINITY;
    }
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mb = fmaxf(mb, sacc[kt][e]);
    mb = halves_max(row_on ? mb : -INFINITY);
    const bool grow = mb * scale_log2 > m_run + kRescale;
    if (ballot64(grow)) {
      const float m_new = mb * scale_log2;
      const float alpha = grow ? exp2f(m_run - m_new) : 1.f;   // 0 on a row's first block
      if (grow) m_run = m_new;
      lacc[0] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    }
    // exp2 argument <= kRescale; results below 2^-126 flush to zero
    const float bias = !row_on ? -INFINITY : (m_run == -INFINITY ? 0.f : -m_run);
    // P^T as the B operand of k-step ks (keys 16*ks ..): k-slot jj of lane
    // half hl holds key 16*ks + 8*(jj/4) + 4*hl + jj%4, i.e. accumulator
    // registers 8*(ks%2) .. 8*(ks%2)+7 of sacc[ks/2].
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        pv[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[ks / 2][8 * (ks % 2) + jj], scale_log2, bias));
      }
      uint4 uu;
      uu.x = cvt_pk_bf16(pv[0], pv[1]);
      uu.y = cvt_pk_bf16(pv[2], pv[3]);
      uu.z = cvt_pk_bf16(pv[4], pv[5]);
      uu.w = cvt_pk_bf16(pv[6], pv[7]);
      pf[ks] = as_bf16x8(uu);
    }

    // O^T += V^T P^T. In a transpose read each 16-lane group returns, to lane
    // j, element j%4 of the 8-byte chunks addressed by lanes j/4 + 4*i
    // (i = 0..3); with lane k pointing at V[kb + k/4][d0 + 4*(k%4)], lane j
    // receives V^T entries (d0 + j, keys kb .. kb+3), matching P^T's k-slots.
    {
      bf16x8 vfr[DT][4];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          vfr[dt][ks] = lds_read_vt(vt_b + ks * 4096, vaddr[0][dt], vaddr[1][dt]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) lacc = mfma32(ones, pf[ks], lacc);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) oacc[dt] = mfma32(vfr[dt][ks], pf[ks], oacc[dt]);
      // transpose reads run ahead of the MFMAs that use them
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };
  for (int u = 0; u < U; u += 2) {
    step(u, std::integral_constant<int, 0>());
    if (u + 1 < U) step(u + 1, std::integral_constant<int, 1>());
  }

  // ---------------------------------------------------------------- epilogue
  // oacc[dt] register r of lane l: d = 32*dt + 8*(r/4) + 4*hl + r%4 of row r32.
  const float l_run = lacc[0];
  if (my_t < n_q) {
    const int h = g * G + r32 % G;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* dst = out + ((int64_t(b) * Hq + h) * n_q + my_t) * kD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint2 uu;
        uu.x = cvt_pk_bf16(oacc[dt][4 * rb] * inv, oacc[dt][4 * rb + 1] * inv);
        uu.y = cvt_pk_bf16(oacc[dt][4 * rb + 2] * inv, oacc[dt][4 * rb + 3] * inv);
        *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * rb + 4 * hl) = uu;
      }
    if (lse && hl == 0)
      lse[(int64_t(b) * Hq + h) * n_q + my_t] = (m_run + log2f(l_run)) * 0.69314718055994531f;
  }
}

template <int G>
__global__ __launch_bounds__(PrefillShape<G>::NT, PrefillShape<G>::MINW) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int Hq,
    int Hkv, int n_q, int64_t kv_cap, int64_t kv_len, int K, int dense_thr, int mode,
    int64_t window, float scale_log2, int ntile, int umax) {
  prefill_attn_body<G, false>(q, k, v, idx, out, lse, Hq, Hkv, n_q, kv_cap, kv_len, K, dense_thr,
                              mode, window, scale_log2, ntile, umax);
}

template <int G>
__global__ __launch_bounds__(PrefillShape<G>::NT, PrefillShape<G>::MINW) void window_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int Hq,
    int Hkv, int n_q, int64_t kv_cap, int64_t kv_len, int K, int dense_thr, int mode,
    int64_t window, float scale_log2, int ntile, int umax) {
  prefill_attn_body<G, true>(q, k, v, idx, out, lse, Hq, Hkv, n_q, kv_cap, kv_len, K, dense_thr,
                             mode, window, scale_log2, ntile, umax);
}

int prefill128_stages(const Dims& d, int mode, int64_t kv_len) {
  if (d.D != 128) return 0;
  const int64_t nb = (kv_len - 1) / kBlock + 1;
  if (nb > 256 * 32) return 0;
  if (kv_len > int64_t(INT32_MAX) / (kD * 2)) return 0;   // 32-bit buffer offsets
  // a two-stage ring; two workgroups per CU (80 KB of LDS each) when the
  // union list fits, so the wavefronts sharing a SIMD are not tied by one
  // barrier and one's MFMA work overlaps the other's softmax and waits
  const int64_t umax = prefill_umax(d, mode, nb);
  return prefill_lds(umax, prefill_tq(d.G), d.K) <= 160 * 1024 ? 2 : 0;
}

template <int G>
static hipError_t launch_prefill_t(const Dims& d, int mode, const uint16_t* q, int n_q,
                                   const uint16_t* k, const uint16_t* v, int64_t kv_cap,
                                   int64_t kv_len, const int32_t* idx, uint16_t* out, float* lse,
                                   int64_t window, hipStream_t s) {
  using Sh = PrefillShape<G>;
  const int ntile = (n_q + Sh::TQ - 1) / Sh::TQ;
  const int64_t nb = (kv_len - 1) / kBlock + 1;
  if (prefill128_stages(d, mode, kv_len) == 0) return hipErrorInvalidValue;
  const int64_t umax = prefill_umax(d, mode, nb);
  auto kern = mode == 3 ? window_attn_kernel<G> : prefill_attn_kernel<G>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(prefill_attn_kernel<G>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  static const hipError_t attr_w = hipFuncSetAttribute(
      reinterpret_cast<const void*>(window_attn_kernel<G>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  if (attr_w != hipSuccess) return attr_w;
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile));
  kern<<<grid, Sh::NT, prefill_lds(umax, Sh::TQ, d.K), s>>>(
      q, k, v, idx, out, lse, d.Hq, d.Hkv, n_q, kv_cap, kv_len, d.K, d.dense_thr, mode, window,
      d.scale * 1.4426950408889634f, ntile, int(umax));
  return hipGetLastError();
}

hipError_t launch_prefill128(const Dims& d, int mode, const uint16_t* q, int n_q,
                             const uint16_t* k, const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                             const int32_t* idx, uint16_t* out, float* lse, hipStream_t s,
                             int64_t window) {
  switch (d.G) {
#define PREFILL_CASE(GG)                                                                    \
  case GG:                                                                                  \
    return launch_prefill_t<GG>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, window, s);
    PREFILL_CASE(1) PREFILL_CASE(2) PREFILL_CASE(4) PREFILL_CASE(8) PREFILL_CASE(16)
#undef PREFILL_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace infllmv2
