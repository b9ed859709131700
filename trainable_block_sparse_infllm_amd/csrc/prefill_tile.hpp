// Shared pieces of the head_dim-128 prefill kernels (forward attention and its
// backward): the per-tile block union, the K/V ring stages in LDS and the LDS
// fragment reads. Workloads: a workgroup owns a tile of consecutive query
// tokens of one (b, g) and walks the ascending union of the blocks its tokens
// attend (MiniCPM4 technical-report summary, QbitAI repost, section "Model
// architecture: InfLLM v2": the query heads of a group share their blocks, and
// short contexts attend densely).
#pragma once

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {
namespace tile {

constexpr int kD = 128;
constexpr int kTileBytes = kBlock * kD * 2;   // one K or V tile
constexpr int kStageBytes = 2 * kTileBytes;   // K then V

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// Tile rows are 256 bytes = 16 pieces of 16 bytes; row r stores logical piece
// p at physical piece p ^ swz(r). swz permutes the bits of r % 16 (so
// swz(r + 16) = swz(r)) such that both read patterns of a tile hit distinct
// LDS banks per phase, for 128- and 256-byte-per-clock LDS alike:
//   row reads (16 bytes of one piece from each of 16 consecutive rows):
//     swz is a bijection on 0..15 and on 0..7 modulo 8;
//   transpose reads (pieces 0..3 of four consecutive rows 4a..4a+3):
//     bits 2-3, and bits 1-2, of swz differ across the four rows.
__device__ __forceinline__ int swz(int r) {
  return ((r >> 2) & 1) | (r & 2) | ((r & 1) << 2) | ((((r >> 1) ^ (r >> 3)) & 1) << 3);
}

// Shape of one instance: TPS tokens per wavefront (32 MFMA rows), NW
// wavefronts, TQ tokens per workgroup, LPS direct loads per thread per stage.
template <int G>
struct PrefillShape {
  static constexpr int TPS = 32 / G;
  static constexpr int NW = TPS >= 16 ? 64 / TPS : 4;
  static constexpr int TQ = NW * TPS;
  static constexpr int NT = 64 * NW;
  static constexpr int LPS = 32 / NW;
  // wavefronts per SIMD the register budget must allow (two workgroups per CU)
  static constexpr int MINW = G == 1 ? 1 : 2;
  static_assert(TQ <= 64, "token masks are 64-bit");
};

// Keys key0 .. key0+63 of K and V -> one LDS stage. The stage is 32 chunks of
// 1 KB (chunk c < 16: K rows 4c..4c+3, else V rows 4(c-16)..); wavefront w
// loads chunks w, w + NW, ... Lane l's 16 bytes land in slot l % 16 of row
// 4c + l / 16, so it fetches the global piece stored in that slot.
//
// The loads are buffer loads straight into LDS: the resource holds the
// (b, g) base and bounds the rows at kv_len (rows past it read zeros: finite,
// and their scores are masked; nothing past the tensor is touched), and a
// load costs one 32-bit add (scalar block offset + per-lane offset). The lane
// part of chunk c depends on c % 4 only: row 4*(c%16) + l/16 has swizzle
// ((4*(c%2) + l/16) << 1) | ((c/2) % 2).
__device__ __forceinline__ uint32_t stage_lane_off(int c4, int l) {
  const int row = 4 * c4 + l / 16;
  return uint32_t((l / 16) * (kD * 2) + (((l % 16) ^ swz(row)) << 4));
}

template <int NW>
__device__ __forceinline__ void issue_stage(char* stage, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, int64_t key0, int w, int l) {
  constexpr int LPS = 32 / NW;
  const uint32_t blk_off = uint32_t(key0) * uint32_t(kD * 2);
#pragma unroll
  for (int x = 0; x < LPS; ++x) {
    const int c = x * NW + w;
    // the whole offset goes in the VGPR operand, which the range check covers
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c < 16 ? rk : rv, (las_void*)(stage + c * 1024), 16,
                                             stage_lane_off(c % 4, l) + blk_off + (c % 16) * 1024,
                                             0, 0, 0);
  }
}

// Bits lo .. hi-1 of a token mask, clamped to tokens 0 .. n-1 (n <= 64).
__device__ __forceinline__ uint64_t range_bits(int64_t lo, int64_t hi, int n) {
  lo = lo < 0 ? 0 : (lo > n ? n : lo);
  hi = hi < 0 ? 0 : (hi > n ? n : hi);
  if (hi <= lo) return 0ull;
  const int len = int(hi - lo);
  const uint64_t ones = len >= 64 ? ~0ull : ((1ull << len) - 1ull);
  return ones << int(lo);
}

// LDS reads inside the ring loop go through these helpers: the __restrict__
// parameter gives each inlined read an alias scope, which tells the compiler
// the read cannot overlap the ring stages still being filled by direct loads;
// without it the compiler waits for every outstanding direct load before any
// LDS read. Completion of the stage being read is established explicitly
// (vmcnt wait + barrier) at the top of each iteration.
template <typename T>
__device__ __forceinline__ T lds_read(const T* __restrict__ p) {
  return *p;
}

__device__ __forceinline__ bf16x8 lds_read_k(const char* __restrict__ tile, int off) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(tile + off));
}

// V^T fragment: two transpose reads (the key groups q = 0 and q = 1).
__device__ __forceinline__ bf16x8 lds_read_vt(const lds_char* __restrict__ tile, int off0, int off1) {
  v4i16 h[2];
  h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + off0));
  h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + off1));
  bf16x8 r;
  __builtin_memcpy(&r, h, sizeof r);
  return r;
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// semantics would also wait for every in-flight direct load). The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Max over lanes l and l ^ 32 (the two halves of a 32-row MFMA column).
__device__ __forceinline__ float halves_max(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}



// Tokens t of a tile (positions base + t) attending block j through their own
// block or a dense prefix (t < dend); mode 2 (dense, no mask): every token;
// mode 3 (sliding window of `window` keys): the tokens whose window
// [p - window + 1, p] meets the block, i.e. j*64 <= p < j*64 + 63 + window.
__device__ __forceinline__ uint64_t range_mask(int64_t j, int mode, int64_t base, int64_t dend,
                                               int ntok, int64_t window = 0) {
  if (mode == 2) return range_bits(0, ntok, ntok);
  const int64_t lo = j * kBlock - base;
  if (mode == 3) return range_bits(lo, lo + kBlock - 1 + window, ntok);
  return range_bits(lo, max(lo + kBlock, dend), ntok);
}

// The ascending union of the blocks a tile's tokens attend, each with a
// 64-bit mask of those tokens: own blocks and dense prefixes are ranges, so
// their bits are computed; selected blocks go through an LDS bitmap, then an
// ordered compaction. Every thread of the workgroup calls it (it holds
// barriers); returns the entry count (at most umax listed). LDS: u_mask,
// u_blk [umax], bitmap, wbase [256], wtot [NW], jsel [TQ*K].
template <int NT, int NW>
__device__ __forceinline__ int build_union(const int32_t* __restrict__ idx, int64_t bg, int n_q,
                                           int tok0, int ntok, int64_t base, int64_t own_lo,
                                           int64_t own_hi, int64_t dend, int K, int umax, int mode,
                                           uint64_t* u_mask, int32_t* u_blk, uint32_t* bitmap,
                                           int32_t* wbase, int32_t* wtot, int32_t* jsel) {
  constexpr int WPT = (256 + NT - 1) / NT;   // bitmap words per thread
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id();
  const int nwords = int(own_hi / 32) + 1;    // <= 256, checked on the host
  const int64_t rlo = dend > 0 ? 0 : own_lo;  // range part: [rlo, own_hi]
  // Four index loads per thread are issued before any of them is used, so
  // their latencies overlap; the first four go out before the bitmap is set
  // up, so their latency also covers that work and its barrier.
  const int nsel = ntok * K;
  auto load4 = [&](int e0, int (&jv)[4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = e0 + x * NT;
      const int t = e / K;
      jv[x] = (e < nsel && t >= dend) ? idx[(bg * n_q + tok0 + t) * K + e % K] : -1;
    }
  };
  int jv[4];
  load4(tid, jv);
  for (int i = tid; i < nwords; i += NT)
    bitmap[i] = uint32_t(range_bits(rlo - int64_t(i) * 32, own_hi + 1 - int64_t(i) * 32, 32));
  __syncthreads();
  for (int e0 = tid; e0 < nsel; e0 += 4 * NT) {
    if (e0 != tid) load4(e0, jv);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = e0 + x * NT;
      if (e < nsel) {
        const int t = e / K;
        int j = jv[x];
        if (j >= 0 && j < (base + t) / kBlock)
          atomicOr(&bitmap[j >> 5], 1u << (j & 31));
        else
          j = -1;
        jsel[e] = j;
      }
    }
  }
  __syncthreads();
  // exclusive prefix of the words' popcounts (thread t owns words t*WPT ..),
  // then each thread lists its words' blocks in order
  int c = 0;
#pragma unroll
  for (int x = 0; x < WPT; ++x) {
    const int i = tid * WPT + x;
    if (i < nwords) c += __popc(bitmap[i]);
  }
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (l >= o) incl += y;
  }
  if (l == kWave - 1) wtot[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int x = 0; x < NW; ++x) {
    before += x < w ? wtot[x] : 0;
    total += wtot[x];
  }
  int pos = before + incl - c;
#pragma unroll
  for (int x = 0; x < WPT; ++x) {
    const int i = tid * WPT + x;
    if (i >= nwords) break;
    wbase[i] = pos;
    uint32_t bits = bitmap[i];
    while (bits) {
      const int j = i * 32 + __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < umax) {
        u_blk[pos] = j;
        u_mask[pos] = range_mask(j, mode, base, dend, ntok);
      }
      ++pos;
    }
  }
  __syncthreads();
  for (int e = tid; e < ntok * K; e += NT) {
    const int t = e / K;
    const int j = jsel[e];
    if (j >= 0) {
      const int u = wbase[j >> 5] + __popc(bitmap[j >> 5] & ((1u << (j & 31)) - 1u));
      if (u < umax) atomicOr(reinterpret_cast<unsigned long long*>(&u_mask[u]), 1ull << t);
    }
  }
  __syncthreads();
  return min(total, umax);
}

// ---------------------------------------------------------------- host side
inline int prefill_tq(int G) {
  switch (G) {
    case 1: return PrefillShape<1>::TQ;
    case 2: return PrefillShape<2>::TQ;
    case 4: return PrefillShape<4>::TQ;
    case 8: return PrefillShape<8>::TQ;
    default: return PrefillShape<16>::TQ;
  }
}

// Largest number of union entries one tile can list (tiles whose tokens are
// all dense list none): the selected blocks of TQ tokens plus at most 2 own
// blocks; or, for the tile holding the dense threshold, every block up to its
// last own block.
inline int64_t prefill_umax(const Dims& d, int mode, int64_t nb) {
  if (mode != 0) return 0;
  const int tq = prefill_tq(d.G);
  const int64_t sparse = int64_t(tq) * d.K + 2;
  const int64_t mixed = d.dense_thr > 0 ? (int64_t(d.dense_thr) + tq) / kBlock + 2 : 0;
  return std::min(nb, std::max(sparse, mixed));
}

inline size_t prefill_lds(int64_t umax, int tq, int K) {
  return size_t(2) * kStageBytes + size_t(umax) * 12 + 512 * 4 + 64 + size_t(tq) * K * 4;
}


}  // namespace tile
}  // namespace infllmv2
