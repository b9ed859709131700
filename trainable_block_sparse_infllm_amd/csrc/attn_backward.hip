// Backward of the sparse prefill attention, head_dim 128: the gradients that
// make the block-sparse attention trainable (MiniCPM4 technical-report
// summary, QbitAI repost, section "Model architecture: InfLLM v2": the sparse
// attention is native and trainable; the block choice itself is a discrete
// selection and carries no gradient).
//
// For a row with weights P over its attended keys (the forward's key sets:
// selected blocks, the own block up to the row's position, or the dense
// prefix below the threshold), upstream gradient dO and forward output O:
//   dP_t = dO . v_t;  Delta = dO . O;  dS_t = P_t (dP_t - Delta);
//   dq = scale sum_t dS_t k_t;  dk_t += scale dS_t q;  dv_t += P_t dO.
// P_t = exp(scale q.k_t - lse) is recomputed from the forward's lse.
//
// Kernels:
//   dq    -- query-centric, the forward's tiling: a workgroup walks the union
//            of its tile's blocks through the LDS ring and keeps dQ^T in MFMA
//            accumulators (S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T with
//            K^T from transpose reads of the K tile); it also computes each
//            row's Delta and lse in log2 units, which it stores for dkv;
//   index -- for every key block, the list of query tokens that attend it
//            (per-tile LDS histograms, one global add per tile and block,
//            prefix sums, fill) and its even split into segments of at most
//            kSegRows query rows; the dk, dv rows of blocks that no row
//            attends, or that are split into several segments (atomic
//            adds), are zeroed, every other block's rows are stored once;
//   dkv   -- key-centric: a workgroup owns one segment of one block's list;
//            K and V of the block stay in registers, chunks of 64 query rows
//            (Q, dO and the rows' token, lse and Delta) stream through a
//            four-slot LDS ring, and dK^T, dV^T stay in MFMA accumulators (S = Q K^T,
//            dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS with Q^T and dO^T
//            from transpose reads). A block split into several segments adds
//            its partial sums atomically, so the fp32 summation order of dk
//            and dv (and the order of each block's token list) can differ
//            between runs.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "prefill_tile.hpp"

namespace infllmv2 {

using namespace tile;

namespace {

constexpr int kSegRows = 4096;      // query rows (token x head) per dK/dV segment, at most
constexpr int kChunkRows = 64;      // query rows per dK/dV chunk (two 32-row halves)
constexpr int kIdxTile = 1024;      // query tokens per index workgroup (4 per thread)
constexpr int kHistMax = 16384;     // blocks per LDS histogram pass of the index kernels

struct BwdLayout {
  int64_t rows, bgs, nblk, emax, smax;
  size_t off_lse2, off_delta, off_cnt, off_cur, off_off, off_nseg, off_list, off_seg, total;
};

BwdLayout bwd_layout(const Dims& d, int n_q, int64_t kv_len) {
  BwdLayout L{};
  L.rows = int64_t(d.B) * d.Hq * n_q;
  L.bgs = int64_t(d.B) * d.Hkv;
  L.nblk = (kv_len - 1) / kBlock + 1;
  // blocks one token attends: K selected + its own; a dense row (p + 1 <
  // threshold) every block up to its own
  const int64_t dense_blocks = d.dense_thr > 0 ? (int64_t(d.dense_thr) - 2) / kBlock + 1 : 0;
  L.emax = int64_t(n_q) * std::max<int64_t>(d.K + 1, dense_blocks);
  L.smax = (L.emax * d.G + kSegRows - 1) / kSegRows + L.nblk;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t o = 0;
  L.off_lse2 = o;  o = al(o + size_t(L.rows) * 4);
  L.off_delta = o; o = al(o + size_t(L.rows) * 4);
  L.off_cnt = o;   o = al(o + size_t(L.bgs * L.nblk) * 4);
  L.off_cur = o;   o = al(o + size_t(L.bgs * L.nblk) * 4);
  L.off_off = o;   o = al(o + size_t(L.bgs * L.nblk) * 4);
  L.off_nseg = o;  o = al(o + size_t(L.bgs) * 4);
  L.off_list = o;  o = al(o + size_t(L.bgs * L.emax) * 4);
  L.off_seg = o;   o = al(o + size_t(L.bgs * L.smax) * 16);
  L.total = o;
  return L;
}

}  // namespace

// ------------------------------------------------------------------ zero
// Plain fill (no memset node, so the sequence can be captured in a graph).
__global__ __launch_bounds__(256) void bwd_zero_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// dk, dv rows < kv_len of the blocks whose rows dkv does not simply store:
// blocks no query row attends (count 0) and blocks split into several
// segments (their partial sums are added atomically). One workgroup per
// (b, g) and block; rows past kv_len are not touched.
__global__ __launch_bounds__(256) void bwd_zero_rows_kernel(const int32_t* __restrict__ cnt,
                                                            float* __restrict__ dk,
                                                            float* __restrict__ dv, int64_t kv_cap,
                                                            int64_t kv_len, int64_t nblk, int G) {
  const int64_t bg = blockIdx.x / nblk, j = blockIdx.x % nblk;
  const int64_t n = cnt[blockIdx.x];
  if (n != 0 && n * G <= kSegRows) return;
  const int64_t r0 = j * kBlock;
  const int64_t nr = min<int64_t>(kBlock, kv_len - r0);
  float4* k4 = reinterpret_cast<float4*>(dk + (bg * kv_cap + r0) * kD);
  float4* v4 = reinterpret_cast<float4*>(dv + (bg * kv_cap + r0) * kD);
  for (int64_t i = threadIdx.x; i < nr * (kD / 4); i += 256) {
    k4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    v4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ------------------------------------------------------------------ dq
template <int G>
__global__ __launch_bounds__(PrefillShape<G>::NT, PrefillShape<G>::MINW) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ out,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ lse2,
    float* __restrict__ delta, float* __restrict__ dq,
    int Hq, int Hkv, int n_q, int64_t kv_cap, int64_t kv_len, int K, int dense_thr,
    float scale_log2, float scale, int ntile, int umax) {
  using Sh = PrefillShape<G>;
  constexpr int TPS = Sh::TPS, NW = Sh::NW, TQ = Sh::TQ, NT = Sh::NT;
  constexpr int DS = kD / 16;
  constexpr int DT = kD / 32;
  constexpr int mode = 0;

  extern __shared__ __align__(16) char smem[];
  char* ring = smem;
  uint64_t* u_mask = reinterpret_cast<uint64_t*>(smem + 2 * kStageBytes);
  int32_t* u_blk = reinterpret_cast<int32_t*>(u_mask + umax);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(u_blk + umax);
  int32_t* wbase = reinterpret_cast<int32_t*>(bitmap + 256);
  int32_t* wtot = wbase + 256;
  int32_t* jsel = wtot + 16;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
  const int bg = item / ntile;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tok0 = tile * TQ;
  const int ntok = min(TQ, n_q - tok0);
  const int64_t base = kv_len - n_q + tok0;
  const int64_t own_lo = base / kBlock;
  const int64_t own_hi = (base + ntok - 1) / kBlock;
  const int64_t dend = dense_thr > 0 ? dense_thr - 1 - base : 0;
  const bool tile_dense = dend >= ntok;
  const uint16_t* kbase = k + int64_t(bg) * kv_cap * kD;
  const uint16_t* vbase = v + int64_t(bg) * kv_cap * kD;

  // This lane's row: token tok0 + w*TPS + r32/G, head g*G + r32%G.
  const int my_t = tok0 + w * TPS + r32 / G;
  const int h = g * G + r32 % G;
  const int64_t rid = (int64_t(b) * Hq + h) * n_q + (my_t < n_q ? my_t : 0);

  int U;
  if (tile_dense)
    U = int(own_hi) + 1;
  else
    U = build_union<NT, NW>(idx, bg, n_q, tok0, ntok, base, own_lo, own_hi, dend, K, umax, mode,
                            u_mask, u_blk, bitmap, wbase, wtot, jsel);
  U = __builtin_amdgcn_readfirstlane(U);
  auto blk_of = [&](int u) -> int {
    return tile_dense ? u : __builtin_amdgcn_readfirstlane(lds_read(u_blk + u));
  };
  auto mask_of = [&](int u) -> uint64_t {
    return tile_dense ? range_mask(u, mode, base, dend, ntok) : uniform_u64(lds_read(u_mask + u));
  };

  const uint32_t nrec = uint32_t(kv_len) * uint32_t(kD * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kbase), 0, int(nrec), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vbase), 0, int(nrec), 0x00020000);
  if (U > 0) issue_stage<NW>(ring, rk, rv, int64_t(blk_of(0)) * kBlock, w, l);
  // Q^T and dO^T fragments (B operands, k-slots 8*hl .. of each 16-wide d
  // step) and the row's lse and Delta, loaded after the union is built
  // (waiting for its index loads would also wait for these, the counter being
  // in order) and together with the first ring stage.
  bf16x8 qf[DS], df[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    qf[ds] = as_bf16x8(ldg16_if(my_t < n_q, q + rid * kD + ds * 16 + hl * 8));
    df[ds] = as_bf16x8(ldg16_if(my_t < n_q, dout + rid * kD + ds * 16 + hl * 8));
  }
  // Delta = dO . O over the row (bf16 products summed in fp32; this lane's
  // 64 columns, then its partner's) and lse in log2 units; stored for dkv.
  float row_delta;
  {
    float part = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const uint4 o = ldg16_if(my_t < n_q, out + rid * kD + ds * 16 + hl * 8);
      uint4 g;
      __builtin_memcpy(&g, &df[ds], sizeof g);
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part = fmaf(bf2f(uint16_t(ow[i] & 0xFFFFu)), bf2f(uint16_t(gw[i] & 0xFFFFu)), part);
        part = fmaf(bf2f(uint16_t(ow[i] >> 16)), bf2f(uint16_t(gw[i] >> 16)), part);
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    row_delta = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float row_lse2 = my_t < n_q ? lse[rid] * 1.4426950408889634f : 0.f;
  if (my_t < n_q && hl == 0) {
    delta[rid] = row_delta;
    lse2[rid] = row_lse2;
  }

  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[dt][e] = 0.f;
  const int row_p = int(base) + w * TPS + r32 / G;
  const int p_first = int(base) + w * TPS;
  // fragment lane offsets (the forward's): K / V row fragment (kt, ds) at
  // 8192*kt + (k_lane ^ (ds << 5)); transpose fragment (dt, ks) at
  // 4096*ks + (t_lane[q] ^ (dt << 6)), q = 0, 1
  const int k_lane = r32 * (kD * 2) + ((hl ^ swz(r32)) << 4);
  int t_lane[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int j = l % 16;
    const int row = 8 * qq + 4 * hl + j / 4;
    const int piece = 2 * ((l / 16) % 2) + (j % 4) / 2;
    t_lane[qq] = row * (kD * 2) + ((piece ^ swz(row)) << 4) + 8 * (j & 1);
  }

  for (int u = 0; u < U; ++u) {
    wait_vmem();
    wait_lds();
    ring_barrier();                               // entry u landed; the other slot is free
    char* const slot = ring + (u & 1) * kStageBytes;
    if (u + 1 < U)
      issue_stage<NW>(ring + ((u + 1) & 1) * kStageBytes, rk, rv, int64_t(blk_of(u + 1)) * kBlock,
                      w, l);
    const int key0 = blk_of(u) * kBlock;
    const uint32_t bits = uint32_t(mask_of(u) >> (w * TPS)) & uint32_t((1ull << TPS) - 1ull);
    if (bits == 0) continue;
    const char* kt_b = slot;
    const char* vt_b = slot + kTileBytes;

    // S^T = K Q^T and dP^T = V dO^T: register r of lane l holds key
    // 32*kt + 8*(r/4) + 4*hl + r%4 of row r32.
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[kt][e] = 0.f;
        pacc[kt][e] = 0.f;
      }
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        sacc[kt] = mfma32(lds_read_k(kt_b + kt * 8192, k_lane ^ (ds << 5)), qf[ds], sacc[kt]);
        pacc[kt] = mfma32(lds_read_k(vt_b + kt * 8192, k_lane ^ (ds << 5)), df[ds], pacc[kt]);
      }
    }
    // P^T from the forward's lse; dS^T = P^T (dP^T - Delta). Rows that do not
    // attend the block, and keys past a row's position, get P = 0.
    const bool row_on = (bits >> (r32 / G)) & 1u;
    const int lim = key0 + kBlock - 1 > p_first ? row_p - key0 : 63;
    bf16x8 sf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float ds_[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int e = 8 * (ks % 2) + jj;
        const int key = 32 * (ks / 2) + 8 * (e / 4) + 4 * hl + e % 4;
        const float p = (row_on && key <= lim)
                            ? __builtin_amdgcn_exp2f(fmaf(sacc[ks / 2][e], scale_log2, -row_lse2))
                            : 0.f;
        ds_[jj] = p * (pacc[ks / 2][e] - row_delta);
      }
      uint4 uu;
      uu.x = cvt_pk_bf16(ds_[0], ds_[1]);
      uu.y = cvt_pk_bf16(ds_[2], ds_[3]);
      uu.z = cvt_pk_bf16(ds_[4], ds_[5]);
      uu.w = cvt_pk_bf16(ds_[6], ds_[7]);
      sf[ks] = as_bf16x8(uu);
    }
    // dQ^T += K^T dS^T: K^T fragments by transpose reads of the K tile, run
    // ahead of the MFMAs that use them (S and dP are dead by now, so their
    // registers hold the fragments).
    {
      const lds_char* kt_l = (const lds_char*)kt_b;
      bf16x8 kfr[DT][4];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kfr[dt][ks] = lds_read_vt(kt_l + ks * 4096, t_lane[0] ^ (dt << 6), t_lane[1] ^ (dt << 6));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) dqacc[dt] = mfma32(kfr[dt][ks], sf[ks], dqacc[dt]);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  }

  // dqacc[dt] register r of lane l: d = 32*dt + 8*(r/4) + 4*hl + r%4 of row r32.
  if (my_t < n_q) {
    float* dst = dq + rid * kD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * rb + 4 * hl) =
            make_float4(dqacc[dt][4 * rb] * scale, dqacc[dt][4 * rb + 1] * scale,
                        dqacc[dt][4 * rb + 2] * scale, dqacc[dt][4 * rb + 3] * scale);
  }
}

// ------------------------------------------------------------------ index
// Blocks attended by token t (position p = P0 + t): every block <= own for a
// dense row, else its selected blocks below own, plus own.
template <typename F>
__device__ __forceinline__ void for_each_block(const int32_t* __restrict__ idx_row, int K,
                                               int64_t p, int dense_thr, F f) {
  const int own = int(p / kBlock);
  if (dense_thr > 0 && p + 1 < dense_thr) {
    for (int j = 0; j <= own; ++j) f(j);
    return;
  }
  for (int x = 0; x < K; ++x) {
    const int j = idx_row[x];
    if (j >= 0 && j < own) f(j);
  }
  f(own);
}

// One workgroup per (b, g) and tile of kIdxTile tokens, one pass per window of
// kHistMax blocks: the tile's counts per block gather in an LDS histogram.
// count adds each nonzero bin to the global count (one atomic per tile and
// block instead of one per token); fill reserves the tile's run in each
// block's list with one atomic and hands out slots in it from LDS.
__device__ __forceinline__ void hist_tokens(const int32_t* __restrict__ idx, int32_t* hist, int bg,
                                            int t0, int n_q, int64_t P0, int K, int dense_thr,
                                            int j0, int nj, bool rank, int32_t* __restrict__ list) {
  for (int x = 0; x < kIdxTile / 256; ++x) {
    const int t = t0 + x * 256 + int(threadIdx.x);
    if (t >= n_q) break;
    for_each_block(idx + (int64_t(bg) * n_q + t) * K, K, P0 + t, dense_thr, [&](int j) {
      const int b = j - j0;
      if (b >= 0 && b < nj) {
        const int o = atomicAdd(&hist[b], 1);
        if (rank) list[o] = t;
      }
    });
  }
}

__global__ __launch_bounds__(256) void bwd_count_kernel(const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ cnt, int n_q,
                                                        int64_t kv_len, int K, int dense_thr,
                                                        int64_t nblk, int ttiles) {
  extern __shared__ int32_t hist[];
  const int bg = blockIdx.x / ttiles;
  const int t0 = (blockIdx.x % ttiles) * kIdxTile;
  const int64_t P0 = kv_len - n_q;
  int32_t* c = cnt + int64_t(bg) * nblk;
  for (int64_t j0 = 0; j0 < nblk; j0 += kHistMax) {
    const int nj = int(min<int64_t>(kHistMax, nblk - j0));
    for (int b = threadIdx.x; b < nj; b += 256) hist[b] = 0;
    __syncthreads();
    hist_tokens(idx, hist, bg, t0, n_q, P0, K, dense_thr, int(j0), nj, false, nullptr);
    __syncthreads();
    for (int b = threadIdx.x; b < nj; b += 256)
      if (hist[b] > 0) atomicAdd(&c[j0 + b], hist[b]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ off,
                                                       int32_t* __restrict__ cur,
                                                       int32_t* __restrict__ list, int n_q,
                                                       int64_t kv_len, int K, int dense_thr,
                                                       int64_t nblk, int64_t emax, int ttiles) {
  extern __shared__ int32_t hist[];
  const int bg = blockIdx.x / ttiles;
  const int t0 = (blockIdx.x % ttiles) * kIdxTile;
  const int64_t P0 = kv_len - n_q;
  const int32_t* o = off + int64_t(bg) * nblk;
  int32_t* c = cur + int64_t(bg) * nblk;
  int32_t* ls = list + int64_t(bg) * emax;
  for (int64_t j0 = 0; j0 < nblk; j0 += kHistMax) {
    const int nj = int(min<int64_t>(kHistMax, nblk - j0));
    for (int b = threadIdx.x; b < nj; b += 256) hist[b] = 0;
    __syncthreads();
    hist_tokens(idx, hist, bg, t0, n_q, P0, K, dense_thr, int(j0), nj, false, nullptr);
    __syncthreads();
    for (int b = threadIdx.x; b < nj; b += 256) {
      const int n = hist[b];
      if (n > 0) hist[b] = o[j0 + b] + atomicAdd(&c[j0 + b], n);
    }
    __syncthreads();
    hist_tokens(idx, hist, bg, t0, n_q, P0, K, dense_thr, int(j0), nj, true, ls);
    __syncthreads();
  }
}

// One workgroup per (b, g): exclusive prefix of the per-block counts (list
// offsets) and the segment table. Block j's n tokens (n*G rows) are cut into
// ceil(n*G / kSegRows) segments of near-equal length, each entry (j, start,
// length, split flag); a segment then holds at most kSegRows / G tokens.
__global__ __launch_bounds__(256) void bwd_scan_kernel(const int32_t* __restrict__ cnt,
                                                       int32_t* __restrict__ off,
                                                       int4* __restrict__ seg,
                                                       int32_t* __restrict__ nseg, int64_t nblk,
                                                       int64_t smax, int G) {
  __shared__ int s_a[256], s_b[256];
  const int bg = blockIdx.x;
  const int tid = threadIdx.x;
  const int per = int((nblk + 255) / 256);
  const int lo = min<int64_t>(nblk, int64_t(tid) * per), hi = min<int64_t>(nblk, lo + per);
  const int32_t* c = cnt + int64_t(bg) * nblk;
  auto nsplit = [&](int n) { return int((int64_t(n) * G + kSegRows - 1) / kSegRows); };
  int ca = 0, cs = 0;
  for (int j = lo; j < hi; ++j) {
    ca += c[j];
    cs += nsplit(c[j]);
  }
  s_a[tid] = ca;
  s_b[tid] = cs;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {             // inclusive scans
    const int xa = tid >= o ? s_a[tid - o] : 0;
    const int xb = tid >= o ? s_b[tid - o] : 0;
    __syncthreads();
    s_a[tid] += xa;
    s_b[tid] += xb;
    __syncthreads();
  }
  int pa = s_a[tid] - ca, ps = s_b[tid] - cs;
  int4* sg = seg + int64_t(bg) * smax;
  for (int j = lo; j < hi; ++j) {
    off[int64_t(bg) * nblk + j] = pa;
    const int n = c[j];
    const int ns = nsplit(n);
    for (int x = 0; x < ns; ++x) {
      const int s0 = int(int64_t(x) * n / ns), s1 = int(int64_t(x + 1) * n / ns);
      sg[ps + x] = make_int4(j, pa + s0, s1 - s0, ns > 1);
    }
    pa += n;
    ps += ns;
  }
  if (tid == 255) nseg[bg] = s_b[255];
}

// ------------------------------------------------------------------ dkv
// LDS: a four-slot ring of stages, each (Q tile, dO tile, row metadata) for
// 64 query rows, then the segment's tokens. Row metadata: token, lse2 and
// Delta of rows 0..63. K and V of the block live in registers as the B
// fragments of S = Q K^T and dP = dO V^T.
constexpr int kDkvSlots = 4;
constexpr int kDkvQTile = kChunkRows * kD * 2;                    // 16 KB
constexpr int kDkvMeta = 3 * kChunkRows * 4;
constexpr int kDkvStage = 2 * kDkvQTile + kDkvMeta;
static_assert(kDkvStage % 16 == 0, "stage alignment");

constexpr size_t dkv_lds(int G) {
  return size_t(kDkvSlots) * kDkvStage + size_t(kSegRows / G) * 4;
}

// Direct HBM -> LDS copy of 4 bytes per lane (lane l's word lands at
// lds_base + 4 l).
__device__ __forceinline__ void load_lds4(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gas_void*)gsrc, (las_void*)lds_base, 4, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// +inf lse for rows past a segment: their P (and dS) come out exactly 0.
static __device__ float kLsePad = INFINITY;

// Per-lane constants of the stage loads. Load x (0..3) of tensor Q (dO:
// x + 4) fills row 16x + 4w + l/16 of the tile; as G divides 64, that row's
// head and token slot within a chunk are fixed: head row % G, slot
// row0/G + row/G. Lane l also copies metadata row l (waves 0..2).
struct StageLanes {
  const char* qrow[4];     // q (bytes) at the row's head row, plus the lane's swizzled piece
  int rowq[4];             // row / G
  const char* mrow;        // wave 1: lse2, wave 2: Delta at the head row of metadata row l
  int mq;                  // l / G
  int mrr;                 // l
};

template <int G>
__device__ __forceinline__ StageLanes stage_lanes(const uint16_t* q, const float* lse2,
                                                  const float* delta, int64_t qb, int n_q, int w,
                                                  int l) {
  StageLanes s;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = 16 * x + 4 * w + l / 16;
    s.qrow[x] = reinterpret_cast<const char*>(q) +
                ((qb + row % G) * n_q * kD + (((l % 16) ^ swz(row)) << 3)) * 2;
    s.rowq[x] = row / G;
  }
  s.mrow = reinterpret_cast<const char*>(w == 1 ? lse2 : delta) + (qb + l % G) * n_q * 4;
  s.mq = l / G;
  s.mrr = l;
  return s;
}

// Rows row0..row0+63 of the segment -> one stage. Tiles: 16 pieces of 1 KB per
// tensor (rows 4c..4c+3); lane l's 16 bytes land in slot l % 16 of row
// 4c + l/16 and it fetches the global piece stored there. Metadata: waves
// 0, 1, 2 copy the token, lse2 and Delta of row l. Rows past the segment
// repeat its last row (finite data) with lse2 = +inf, which zeroes their P
// and dS. Per stage a wave issues 9 loads (waves 0..2) or 8 (wave 3).
__device__ __forceinline__ void issue_qd_stage(char* stage, const StageLanes& sl, int64_t dq_off,
                                               const int32_t* list_seg, const int32_t* s_tok,
                                               int lenm1, int nrows, int row0, int G, int w) {
  const int cq = row0 / G;
  // every token first, so the LDS reads are not held behind the direct loads
  int tok[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) tok[x] = lds_read(s_tok + min(cq + sl.rowq[x], lenm1));
  const int tslot_m = min(cq + sl.mq, lenm1);
  const int tok_m = lds_read(s_tok + tslot_m);
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const char* src = sl.qrow[x] + int64_t(uint32_t(tok[x])) * (kD * 2);
    load_lds16(src, stage + (4 * x + w) * 1024);
    load_lds16(src + dq_off, stage + (16 + 4 * x + w) * 1024);
  }
  if (w < 3) {
    char* meta = stage + 2 * kDkvQTile + w * (kChunkRows * 4);
    if (w == 0) {
      load_lds4(list_seg + tslot_m, meta);
    } else {
      const bool pad = w == 1 && row0 + sl.mrr >= nrows;
      const void* src = pad ? static_cast<const void*>(&kLsePad)
                            : static_cast<const void*>(sl.mrow + int64_t(uint32_t(tok_m)) * 4);
      load_lds4(src, meta);
    }
  }
}

// Waits of the ring, per wave: the loads of `after` later stages may stay in
// flight (0, 1 or 2 stages of 9 or 8 loads).
__device__ __forceinline__ void wait_stage(int after, int w) {
  if (w < 3) {
    if (after >= 2) wait_vmcnt<18>();
    else if (after == 1) wait_vmcnt<9>();
    else wait_vmcnt<0>();
  } else {
    if (after >= 2) wait_vmcnt<16>();
    else if (after == 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
  }
}

template <int G>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, const int32_t* __restrict__ list,
    const int4* __restrict__ seg, const int32_t* __restrict__ nseg, float* __restrict__ dk,
    float* __restrict__ dv, int Hq, int Hkv, int n_q, int64_t kv_cap, int64_t kv_len,
    int64_t emax, int64_t smax, int64_t total_items, float scale_log2, float scale) {
  constexpr int DS = kD / 16;
  constexpr int DT = kD / 32;
  extern __shared__ __align__(16) char smem[];
  char* ring = smem;                                  // kDkvSlots x (Q, dO, metadata)
  int32_t* s_tok = reinterpret_cast<int32_t*>(ring + kDkvSlots * kDkvStage);

  // Workgroups go to the XCDs round-robin by index; chunks of 8 consecutive
  // segments are dealt to the XCDs in turn, so the segments of one split
  // block (adjacent in the table) share an L2 for their atomic adds while the
  // workgroups running at once still cover consecutive segments.
  const int x = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const int64_t item = (int64_t(slot / 8) * kNumXcd + x) * 8 + slot % 8;
  if (item >= total_items) return;
  const int bg = int(item / smax);
  const int sidx = int(item % smax);
  if (sidx >= nseg[bg]) return;
  const int4 sg = seg[int64_t(bg) * smax + sidx];
  const int j = sg.x, start = sg.y, len = sg.z;
  const bool split = sg.w != 0;
  const int b = bg / Hkv, g = bg % Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int r32 = l % 32, hl = l / 32;
  const int kt = w & 1;             // keys 32*kt .. of the block
  const int rh = w >> 1;            // rows 32*rh .. of each chunk
  const int64_t P0 = kv_len - n_q;
  const int64_t qb = int64_t(b) * Hq + int64_t(g) * G;      // first head row of the group
  const int32_t* list_seg = list + int64_t(bg) * emax + start;
  const int nrows = len * G;
  const int key = j * kBlock + 32 * kt + r32;
  const int kp = int(key - P0);     // a row of token t sees this key when kp <= t

  // K and V B fragments: key `key`, piece 2*ds + hl (zeros past kv_len)
  bf16x8 kf[DS], vf[DS];
  {
    const bool ok = key < kv_len;
    const int64_t o = (int64_t(bg) * kv_cap + (ok ? key : 0)) * kD + 8 * hl;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      kf[ds] = as_bf16x8(ldg16_if(ok, k + o + 16 * ds));
      vf[ds] = as_bf16x8(ldg16_if(ok, v + o + 16 * ds));
    }
  }
  // the segment's tokens
  for (int i = threadIdx.x; i < len; i += 256) s_tok[i] = list_seg[i];
  __syncthreads();

  const int nch = (nrows + kChunkRows - 1) / kChunkRows;
  auto stage_of = [&](int c) { return ring + (c % kDkvSlots) * kDkvStage; };
  const StageLanes sl = stage_lanes<G>(q, lse2, delta, qb, n_q, w, l);
  const int64_t dq_off = reinterpret_cast<const char*>(dout) - reinterpret_cast<const char*>(q);
#pragma unroll
  for (int c = 0; c < 3; ++c)
    if (c < nch)
      issue_qd_stage(stage_of(c), sl, dq_off, list_seg, s_tok, len - 1, nrows, c * kChunkRows, G, w);

  f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dkacc[dt][e] = 0.f;
      dvacc[dt][e] = 0.f;
    }
  // A fragments of S = Q K^T and dP = dO V^T: row 32*rh + r32, piece 2*ds + hl
  // (offset r_lane ^ (ds << 5) within the half). Transpose fragments (dt, ks)
  // of the Q / dO half: 4096*ks + (t_lane[q] ^ (dt << 6)).
  const int r_lane = r32 * (kD * 2) + ((hl ^ swz(r32)) << 4);
  int t_lane[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int jj = l % 16;
    const int row = 8 * qq + 4 * hl + jj / 4;
    const int piece = 2 * ((l / 16) % 2) + (jj % 4) / 2;
    t_lane[qq] = row * (kD * 2) + ((piece ^ swz(row)) << 4) + 8 * (jj & 1);
  }

  // S and dP of one chunk (this wave's 32 rows x 32 keys)
  auto s_dp = [&](const char* st, f32x16& sacc, f32x16& pacc) __attribute__((always_inline)) {
    const char* qh = st + rh * (32 * kD * 2);
    const char* dh = st + kDkvQTile + rh * (32 * kD * 2);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sacc[e] = 0.f;
      pacc[e] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      sacc = mfma32(lds_read_k(qh, r_lane ^ (ds << 5)), kf[ds], sacc);
      pacc = mfma32(lds_read_k(dh, r_lane ^ (ds << 5)), vf[ds], pacc);
    }
  };

  f32x16 sacc, pacc;
  wait_stage(min(nch - 1, 2), w);                    // chunk 0 landed
  ring_barrier();
  s_dp(stage_of(0), sacc, pacc);

  for (int c = 0; c < nch; ++c) {
    // chunk c + 1 landed (chunk c + 2 may still be in flight); every wave is
    // done with chunk c - 1, whose slot takes chunk c + 3
    wait_stage(c + 2 < nch ? 1 : 0, w);
    wait_lds();
    ring_barrier();
    if (c + 3 < nch)
      issue_qd_stage(stage_of(c + 3), sl, dq_off, list_seg, s_tok, len - 1, nrows,
                     (c + 3) * kChunkRows, G, w);
    const char* st = stage_of(c);
    const char* sn = stage_of(c + 1);
    // Reads first: A fragments of chunk c + 1 (past the last chunk: stale
    // slot data, discarded), chunk c's row metadata and its Q^T, dO^T
    // transpose fragments.
    bf16x8 qa[DS], da[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qa[ds] = lds_read_k(sn + rh * (32 * kD * 2), r_lane ^ (ds << 5));
      da[ds] = lds_read_k(sn + kDkvQTile + rh * (32 * kD * 2), r_lane ^ (ds << 5));
    }
    // register e of lane l: chunk row 32*rh + 8*(e/4) + 4*hl + e%4, key
    // 32*kt + r32 of the block; rows 4m..4m+3 of the metadata are one read
    const char* meta = st + 2 * kDkvQTile;
    int4 tk[4];
    float4 ls[4], dl4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 32 * rh + 8 * m + 4 * hl;
      tk[m] = lds_read(reinterpret_cast<const int4*>(meta + row * 4));
      ls[m] = lds_read(reinterpret_cast<const float4*>(meta + kChunkRows * 4 + row * 4));
      dl4[m] = lds_read(reinterpret_cast<const float4*>(meta + 2 * kChunkRows * 4 + row * 4));
    }
    const lds_char* ql = (const lds_char*)(st + rh * (32 * kD * 2));
    const lds_char* dl = (const lds_char*)(st + kDkvQTile + rh * (32 * kD * 2));
    bf16x8 qt[DT][2], dtr[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dtr[dt][ks] = lds_read_vt(dl + ks * 4096, t_lane[0] ^ (dt << 6), t_lane[1] ^ (dt << 6));
        qt[dt][ks] = lds_read_vt(ql + ks * 4096, t_lane[0] ^ (dt << 6), t_lane[1] ^ (dt << 6));
      }

    // S, dP of chunk c + 1
    f32x16 sacc_n, pacc_n;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sacc_n[e] = 0.f;
      pacc_n[e] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      sacc_n = mfma32(qa[ds], kf[ds], sacc_n);
      pacc_n = mfma32(da[ds], vf[ds], pacc_n);
    }

    // P and dS of chunk c (bf16 B operands); rows past the segment have
    // lse2 = +inf and so P = 0
    bf16x8 pf[2], sf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv[8], dv_[8];
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        const int m = 2 * ks + gq;
        const int tt[4] = {tk[m].x, tk[m].y, tk[m].z, tk[m].w};
        const float lv[4] = {ls[m].x, ls[m].y, ls[m].z, ls[m].w};
        const float dd[4] = {dl4[m].x, dl4[m].y, dl4[m].z, dl4[m].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * m + i;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2, -lv[i]));
          const float pm = kp <= tt[i] ? p : 0.f;      // the key is past the row's position
          pv[4 * gq + i] = pm;
          dv_[4 * gq + i] = pm * (pacc[e] - dd[i]);
        }
      }
      uint4 a, d;
      a.x = cvt_pk_bf16(pv[0], pv[1]);   a.y = cvt_pk_bf16(pv[2], pv[3]);
      a.z = cvt_pk_bf16(pv[4], pv[5]);   a.w = cvt_pk_bf16(pv[6], pv[7]);
      d.x = cvt_pk_bf16(dv_[0], dv_[1]); d.y = cvt_pk_bf16(dv_[2], dv_[3]);
      d.z = cvt_pk_bf16(dv_[4], dv_[5]); d.w = cvt_pk_bf16(dv_[6], dv_[7]);
      pf[ks] = as_bf16x8(a);
      sf[ks] = as_bf16x8(d);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (rows of this half as the k dimension)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dvacc[dt] = mfma32(dtr[dt][ks], pf[ks], dvacc[dt]);
        dkacc[dt] = mfma32(qt[dt][ks], sf[ks], dkacc[dt]);
      }
    // A-fragment and metadata reads, then the S, dP MFMAs of chunk c + 1
    // interleaved with chunk c's softmax and the transpose reads, then the
    // dV, dK MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 28, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 60, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    sacc = sacc_n;
    pacc = pacc_n;
  }

  // The two row halves' partial sums meet in LDS (the ring is free now):
  // waves rh = 1 store, waves rh = 0 add and write out.
  wait_vmem();
  __syncthreads();
  float* red = reinterpret_cast<float*>(ring) + kt * (2 * DT * 16 * kWave);
  if (rh == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[(dt * 16 + e) * kWave + l] = dkacc[dt][e];
        red[((DT + dt) * 16 + e) * kWave + l] = dvacc[dt][e];
      }
  }
  __syncthreads();
  if (rh == 0 && key < kv_len) {
    // register e of lane l: d = 32*dt + 8*(e/4) + 4*hl + e%4, key 32*kt + r32
    float* dkr = dk + (int64_t(bg) * kv_cap + key) * kD;
    float* dvr = dv + (int64_t(bg) * kv_cap + key) * kD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        float a4[4], v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * rb + i;
          a4[i] = (dkacc[dt][e] + red[(dt * 16 + e) * kWave + l]) * scale;
          v4[i] = dvacc[dt][e] + red[((DT + dt) * 16 + e) * kWave + l];
        }
        const int d0 = 32 * dt + 8 * rb + 4 * hl;
        if (split) {
          // hardware fp32 add at L2 (the gradients live in ordinary
          // coarse-grained device memory), not a compare-and-swap loop
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            unsafeAtomicAdd(dkr + d0 + i, a4[i]);
            unsafeAtomicAdd(dvr + d0 + i, v4[i]);
          }
        } else {
          *reinterpret_cast<float4*>(dkr + d0) = make_float4(a4[0], a4[1], a4[2], a4[3]);
          *reinterpret_cast<float4*>(dvr + d0) = make_float4(v4[0], v4[1], v4[2], v4[3]);
        }
      }
  }
}

// ------------------------------------------------------------------ launch
// ------------------------------------------------------------------ head_dim 64
// A head_dim-64 call runs the kernels above on zero-padded copies: appending
// 64 zero columns to q, k, v, out and dO leaves every dot product (scores, dP,
// Delta) unchanged, and the first 64 columns of the padded dq, dk, dv are the
// gradients (the softmax scale stays the head_dim-64 one). The copies live in
// the workspace: q, out, dO [B*Hq][n_q][128] and k, v [B*Hkv][kv_len][128]
// bf16; dq [B*Hq][n_q][128] and dk, dv [B*Hkv][kv_len][128] fp32.
struct PadLayout {
  size_t off_q, off_out, off_dout, off_k, off_v, off_dq, off_dk, off_dv, off_bwd, total;
};

PadLayout pad_layout(const Dims& d, int n_q, int64_t kv_len) {
  PadLayout P{};
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rq = size_t(d.B) * d.Hq * n_q, rk = size_t(d.B) * d.Hkv * kv_len;
  size_t o = 0;
  P.off_q = o;    o = al(o + rq * kD * 2);
  P.off_out = o;  o = al(o + rq * kD * 2);
  P.off_dout = o; o = al(o + rq * kD * 2);
  P.off_k = o;    o = al(o + rk * kD * 2);
  P.off_v = o;    o = al(o + rk * kD * 2);
  P.off_dq = o;   o = al(o + rq * kD * 4);
  P.off_dk = o;   o = al(o + rk * kD * 4);
  P.off_dv = o;   o = al(o + rk * kD * 4);
  P.off_bwd = o;
  Dims d128 = d;
  d128.D = kD;
  P.total = o + bwd_layout(d128, n_q, kv_len).total;
  return P;
}

// Rows r < nrows of each of nb matrices: bf16 [src_cap][64] -> [dst_cap][128],
// columns 64..127 zero. One thread per 16-byte piece of a padded row.
__global__ __launch_bounds__(256) void pad64_kernel(const uint16_t* __restrict__ src,
                                                    uint16_t* __restrict__ dst, int64_t nb,
                                                    int64_t nrows, int64_t src_cap,
                                                    int64_t dst_cap) {
  const int64_t total = nb * nrows * 16;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * 256) {
    const int64_t piece = e % 16, r = (e / 16) % nrows, m = e / (16 * nrows);
    const uint4 val = piece < 8 ? ldg16(src + (m * src_cap + r) * 64 + piece * 8) : uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(dst + (m * dst_cap + r) * kD + piece * 8) = val;
  }
}

// Rows r < nrows: fp32 [src_cap][128] -> the first 64 columns, [dst_cap][64].
__global__ __launch_bounds__(256) void unpad64_kernel(const float* __restrict__ src,
                                                      float* __restrict__ dst, int64_t nb,
                                                      int64_t nrows, int64_t src_cap,
                                                      int64_t dst_cap) {
  const int64_t total = nb * nrows * 16;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * 256) {
    const int64_t piece = e % 16, r = (e / 16) % nrows, m = e / (16 * nrows);
    *reinterpret_cast<float4*>(dst + (m * dst_cap + r) * 64 + piece * 4) =
        *reinterpret_cast<const float4*>(src + (m * src_cap + r) * kD + piece * 4);
  }
}

size_t prefill_backward_workspace_bytes(const Dims& d, int n_q, int64_t kv_len) {
  return d.D == 64 ? pad_layout(d, n_q, kv_len).total : bwd_layout(d, n_q, kv_len).total;
}

bool prefill_backward_ok(const Dims& d, int64_t kv_len) {
  Dims d128 = d;
  d128.D = kD;
  return (d.D == kD || d.D == 64) && prefill128_stages(d128, 0, kv_len) > 0;
}

template <int G>
static hipError_t launch_bwd_t(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                               const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                               const int32_t* idx, const uint16_t* out, const float* lse,
                               const uint16_t* dout, float* dq, float* dk, float* dv, void* ws,
                               hipStream_t s) {
  const BwdLayout L = bwd_layout(d, n_q, kv_len);
  char* w8 = static_cast<char*>(ws);
  float* lse2 = reinterpret_cast<float*>(w8 + L.off_lse2);
  float* delta = reinterpret_cast<float*>(w8 + L.off_delta);
  int32_t* cnt = reinterpret_cast<int32_t*>(w8 + L.off_cnt);
  int32_t* cur = reinterpret_cast<int32_t*>(w8 + L.off_cur);
  int32_t* off = reinterpret_cast<int32_t*>(w8 + L.off_off);
  int32_t* nseg = reinterpret_cast<int32_t*>(w8 + L.off_nseg);
  int32_t* list = reinterpret_cast<int32_t*>(w8 + L.off_list);
  int4* seg = reinterpret_cast<int4*>(w8 + L.off_seg);
  const float sl2 = d.scale * 1.4426950408889634f;
  hipError_t e;

  // counters (cnt and cur are adjacent) -> 0
  const int64_t n16 = int64_t(L.off_off - L.off_cnt) / 16;
  bwd_zero_kernel<<<dim3(unsigned(std::min<int64_t>(1024, (n16 + 255) / 256))), 256, 0, s>>>(
      reinterpret_cast<uint4*>(cnt), n16);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // dq: the forward's tiling
  {
    using Sh = PrefillShape<G>;
    const int ntile = (n_q + Sh::TQ - 1) / Sh::TQ;
    const int64_t umax = prefill_umax(d, 0, L.nblk);
    auto kern = bwd_dq_kernel<G>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       160 * 1024);
    if (attr != hipSuccess) return attr;
    kern<<<dim3(unsigned(L.bgs * ntile)), Sh::NT, prefill_lds(umax, Sh::TQ, d.K), s>>>(
        q, k, v, idx, out, dout, lse, lse2, delta, dq, d.Hq, d.Hkv, n_q, kv_cap, kv_len, d.K, d.dense_thr,
        sl2, d.scale, ntile, int(umax));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // inverse index
  const int ttiles = (n_q + kIdxTile - 1) / kIdxTile;
  const size_t hist_lds = size_t(std::min<int64_t>(L.nblk, kHistMax)) * 4;
  bwd_count_kernel<<<dim3(unsigned(L.bgs * ttiles)), 256, hist_lds, s>>>(
      idx, cnt, n_q, kv_len, d.K, d.dense_thr, L.nblk, ttiles);
  bwd_scan_kernel<<<dim3(unsigned(L.bgs)), 256, 0, s>>>(cnt, off, seg, nseg, L.nblk, L.smax, G);
  bwd_zero_rows_kernel<<<dim3(unsigned(L.bgs * L.nblk)), 256, 0, s>>>(cnt, dk, dv, kv_cap, kv_len,
                                                                      L.nblk, G);
  bwd_fill_kernel<<<dim3(unsigned(L.bgs * ttiles)), 256, hist_lds, s>>>(
      idx, off, cur, list, n_q, kv_len, d.K, d.dense_thr, L.nblk, L.emax, ttiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // dk, dv
  {
    auto kern = bwd_dkv_kernel<G>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       160 * 1024);
    if (attr != hipSuccess) return attr;
    const int64_t items = L.bgs * L.smax;
    const int64_t grid = (items + 8 * kNumXcd - 1) / (8 * kNumXcd) * (8 * kNumXcd);
    kern<<<dim3(unsigned(grid)), 256, dkv_lds(G), s>>>(
        q, k, v, dout, lse2, delta, list, seg, nseg, dk, dv, d.Hq, d.Hkv, n_q, kv_cap, kv_len,
        L.emax, L.smax, items, sl2, d.scale);
  }
  return hipGetLastError();
}

static hipError_t launch_bwd_any(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                                 const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                                 const int32_t* idx, const uint16_t* out, const float* lse,
                                 const uint16_t* dout, float* dq, float* dk, float* dv, void* ws,
                                 hipStream_t s);

hipError_t launch_prefill_backward(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                                   const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                                   const int32_t* idx, const uint16_t* out, const float* lse,
                                   const uint16_t* dout, float* dq, float* dk, float* dv, void* ws,
                                   size_t ws_bytes, hipStream_t s) {
  if (ws_bytes < prefill_backward_workspace_bytes(d, n_q, kv_len)) return hipErrorInvalidValue;
  if (d.D == kD)
    return launch_bwd_any(d, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, dout, dq, dk, dv, ws, s);
  if (d.D != 64) return hipErrorInvalidValue;
  const PadLayout P = pad_layout(d, n_q, kv_len);
  char* w8 = static_cast<char*>(ws);
  uint16_t* qp = reinterpret_cast<uint16_t*>(w8 + P.off_q);
  uint16_t* op = reinterpret_cast<uint16_t*>(w8 + P.off_out);
  uint16_t* gp = reinterpret_cast<uint16_t*>(w8 + P.off_dout);
  uint16_t* kp = reinterpret_cast<uint16_t*>(w8 + P.off_k);
  uint16_t* vp = reinterpret_cast<uint16_t*>(w8 + P.off_v);
  float* dqp = reinterpret_cast<float*>(w8 + P.off_dq);
  float* dkp = reinterpret_cast<float*>(w8 + P.off_dk);
  float* dvp = reinterpret_cast<float*>(w8 + P.off_dv);
  const int64_t nbq = int64_t(d.B) * d.Hq, nbk = int64_t(d.B) * d.Hkv;
  auto grid_of = [](int64_t pieces) { return dim3(unsigned(std::min<int64_t>(4096, (pieces + 255) / 256))); };
  pad64_kernel<<<grid_of(nbq * n_q * 16), 256, 0, s>>>(q, qp, nbq, n_q, n_q, n_q);
  pad64_kernel<<<grid_of(nbq * n_q * 16), 256, 0, s>>>(out, op, nbq, n_q, n_q, n_q);
  pad64_kernel<<<grid_of(nbq * n_q * 16), 256, 0, s>>>(dout, gp, nbq, n_q, n_q, n_q);
  pad64_kernel<<<grid_of(nbk * kv_len * 16), 256, 0, s>>>(k, kp, nbk, kv_len, kv_cap, kv_len);
  pad64_kernel<<<grid_of(nbk * kv_len * 16), 256, 0, s>>>(v, vp, nbk, kv_len, kv_cap, kv_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Dims d128 = d;
  d128.D = kD;
  e = launch_bwd_any(d128, qp, n_q, kp, vp, kv_len, kv_len, idx, op, lse, gp, dqp, dkp, dvp,
                     w8 + P.off_bwd, s);
  if (e != hipSuccess) return e;
  unpad64_kernel<<<grid_of(nbq * n_q * 16), 256, 0, s>>>(dqp, dq, nbq, n_q, n_q, n_q);
  unpad64_kernel<<<grid_of(nbk * kv_len * 16), 256, 0, s>>>(dkp, dk, nbk, kv_len, kv_len, kv_cap);
  unpad64_kernel<<<grid_of(nbk * kv_len * 16), 256, 0, s>>>(dvp, dv, nbk, kv_len, kv_len, kv_cap);
  return hipGetLastError();
}

static hipError_t launch_bwd_any(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                                 const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                                 const int32_t* idx, const uint16_t* out, const float* lse,
                                 const uint16_t* dout, float* dq, float* dk, float* dv, void* ws,
                                 hipStream_t s) {
  switch (d.G) {
#define BWD_CASE(GG)                                                                              \
  case GG:                                                                                        \
    return launch_bwd_t<GG>(d, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, dout, dq, dk, dv, ws, \
                            s);
    BWD_CASE(1) BWD_CASE(2) BWD_CASE(4) BWD_CASE(8) BWD_CASE(16)
#undef BWD_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace infllmv2
