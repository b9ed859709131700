// Wavefront-level exact top-K over order-preserving score keys, shared by the
// selection kernels (MiniCPM4 technical-report summary, QbitAI repost, section
// "Model architecture: InfLLM v2": only the most relevant context blocks take
// part in attention).
//
// Rule: with at most K candidates all are taken; otherwise the K highest
// scores, compared as fp32, with the lower block index first on equal scores.
// Rows are written ascending and padded with -1.
//
// One wavefront selects one row whose n <= 64*KPL candidates sit in registers
// (candidate j in lane j % 64, slot j / 64). The K-th largest score key T is
// found bit by bit from the most significant end, each step counting the keys
// >= a trial value with ballots (after a prefilter that usually leaves one
// candidate per lane); the row is then emitted in index order with
// ballot/mbcnt compaction, taking every key > T and the first K - #(> T) keys
// equal to T. All decisions are integer comparisons on order-preserving score
// keys, so the choice is exact for the given scores.
#pragma once

#include "common.hpp"

namespace infllmv2 {

// Exact K-th largest key by a most-significant-bit-first search: T is the
// largest value with #(keys >= T) >= K. One ballot per register slot per bit.
template <int N>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[N], int K) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < N; ++r) cnt += popc64(ballot64(key[r] >= cand));
    if (cnt >= uint32_t(K)) T = cand;
  }
  return T;
}

// Value of lane l ^ J (J = 1, 2, ..., 32) without going through LDS: quad
// permutes for 1 and 2, row shifts for 4 and 8, the gfx950 row swaps for 16
// and 32 (permlane16_swap(x, x) leaves rows (0,0,2,2) / (1,1,3,3),
// permlane32_swap(x, x) rows (0,1,0,1) / (2,3,2,3)).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int l) {
  if constexpr (J == 1) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  } else if constexpr (J == 2) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  } else if constexpr (J == 4 || J == 8) {
    const uint32_t up = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x100 + J, 0xF, 0xF, false));  // row_shl
    const uint32_t dn = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x110 + J, 0xF, 0xF, false));  // row_shr
    return (l & J) ? dn : up;
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((l >> 4) & 1) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (l >= 32) ? r[0] : r[1];
  }
}

// One bitonic stage: lanes l and l ^ J exchange so that segments of 2K lanes
// (K = size of the merged run) end descending.
template <int KS, int J>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t v, int l) {
  const uint32_t p = xor_lane<J>(v, l);
  const bool lower = (l & J) == 0;
  const bool desc = (l & KS) == 0;
  return lower == desc ? max(v, p) : min(v, p);
}

// K-th largest (with multiplicity, 1 <= K <= 64) of one key per lane: sort the
// wavefront descending with a bitonic network and read lane K-1.
__device__ __forceinline__ uint32_t kth_largest_lanes(uint32_t v, int K) {
  const int l = lane_id();
  v = bitonic_step<2, 1>(v, l);
  v = bitonic_step<4, 2>(v, l);  v = bitonic_step<4, 1>(v, l);
  v = bitonic_step<8, 4>(v, l);  v = bitonic_step<8, 2>(v, l);  v = bitonic_step<8, 1>(v, l);
  v = bitonic_step<16, 8>(v, l); v = bitonic_step<16, 4>(v, l); v = bitonic_step<16, 2>(v, l);
  v = bitonic_step<16, 1>(v, l);
  v = bitonic_step<32, 16>(v, l); v = bitonic_step<32, 8>(v, l); v = bitonic_step<32, 4>(v, l);
  v = bitonic_step<32, 2>(v, l);  v = bitonic_step<32, 1>(v, l);
  v = bitonic_step<64, 32>(v, l); v = bitonic_step<64, 16>(v, l); v = bitonic_step<64, 8>(v, l);
  v = bitonic_step<64, 4>(v, l);  v = bitonic_step<64, 2>(v, l);  v = bitonic_step<64, 1>(v, l);
  return uint32_t(__builtin_amdgcn_readlane(int(v), K - 1));
}

// Emit, in ascending slot order (r*64 + lane), every key > T and the first
// K - #(> T) keys equal to T; `idx_of` maps a slot to the block index written.
template <int N, typename F>
__device__ __forceinline__ void emit_topk(const uint32_t (&key)[N], uint32_t T, int K,
                                          int32_t* __restrict__ out, F idx_of) {
  const int l = lane_id();
  uint32_t ngt = 0;
#pragma unroll
  for (int r = 0; r < N; ++r) ngt += popc64(ballot64(key[r] > T));
  const uint32_t take_eq = uint32_t(K) - ngt;
  uint32_t base = 0, eq_seen = 0;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const bool eq = key[r] == T;
    const uint64_t eqm = ballot64(eq);
    const bool take = key[r] > T || (eq && eq_seen + mbcnt64(eqm) < take_eq);
    const uint64_t tm = ballot64(take);
    if (take) out[base + mbcnt64(tm)] = idx_of(r, l);
    base += popc64(tm);
    eq_seen += popc64(eqm);
  }
}

// Top-K of one row held by one wavefront: candidate j sits in lane j % 64,
// slot j / 64; keys of slots past n are 0 (below every real key). `scratch`
// is 64 (key, index) pairs of LDS private to the wavefront.
//
// Prefilter: the K-th largest of the 64 per-lane maxima, T0, is a lower bound
// of the K-th largest key (at least K lanes hold a key >= T0), so the answer
// lies among the keys >= T0. When those fit one per lane (the usual case: a
// few dozen), the exact search runs over them alone; otherwise over all keys.
template <int KPL>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[KPL], int n, int K,
                                          int32_t* __restrict__ out, uint32_t* scratch) {
  const int l = lane_id();
  if (n <= K) {
    for (int t = l; t < K; t += kWave) out[t] = t < n ? t : -1;
    return;
  }
  if (K <= kWave) {
    uint32_t mx[1] = {0u};
#pragma unroll
    for (int r = 0; r < KPL; ++r) mx[0] = max(mx[0], key[r]);
    const uint32_t T0 = kth_largest_lanes(mx[0], K);
    uint32_t nc = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) nc += popc64(ballot64(key[r] >= T0));
    if (nc <= uint32_t(kWave)) {
      uint32_t base = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const bool c = key[r] >= T0;
        const uint64_t m = ballot64(c);
        if (c) {
          const uint32_t pos = base + mbcnt64(m);
          scratch[2 * pos] = key[r];
          scratch[2 * pos + 1] = uint32_t(r * kWave + l);
        }
        base += popc64(m);
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t ck[1] = {uint32_t(l) < nc ? scratch[2 * l] : 0u};
      const int32_t cj = uint32_t(l) < nc ? int32_t(scratch[2 * l + 1]) : -1;
      const uint32_t T = kth_largest_lanes(ck[0], K);
      emit_topk<1>(ck, T, K, out, [&](int, int) { return cj; });
      __builtin_amdgcn_wave_barrier();
      return;
    }
  }
  const uint32_t T = kth_largest<KPL>(key, K);
  emit_topk<KPL>(key, T, K, out, [](int r, int ln) { return r * kWave + ln; });
}

}  // namespace infllmv2
