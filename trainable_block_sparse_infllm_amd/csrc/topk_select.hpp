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
// (wave_topk: candidate j in lane j % 64, slot j / 64; wave_topk_lc: candidate
// j in lane j / KPL, slot j % KPL, so lane order is index order). A prefilter
// usually leaves one candidate per lane; the K-th largest key T among them is
// read off a bitonic sort (or, after heavy ties, found bit by bit from the
// most significant end over all keys), and the row is emitted in index order,
// taking every key > T and the first K - #(> T) keys equal to T. All decisions are integer comparisons on order-preserving score
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

// Inclusive prefix sum over the wavefront's lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int l) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = uint32_t(__shfl_up(int(v), o));
    if (l >= o) v += t;
  }
  return v;
}

// K-th largest (with multiplicity, 1 <= K <= 64) of one fp32 value per lane
// (no NaNs): the same bitonic network on floats, so -0 and +0 compare equal.
template <int KS, int J>
__device__ __forceinline__ float bitonic_step_f(float v, int l) {
  const float p = __uint_as_float(xor_lane<J>(__float_as_uint(v), l));
  const bool lower = (l & J) == 0;
  const bool desc = (l & KS) == 0;
  return lower == desc ? fmaxf(v, p) : fminf(v, p);
}

__device__ __forceinline__ float kth_largest_lanes_f(float v, int K) {
  const int l = lane_id();
  v = bitonic_step_f<2, 1>(v, l);
  v = bitonic_step_f<4, 2>(v, l);  v = bitonic_step_f<4, 1>(v, l);
  v = bitonic_step_f<8, 4>(v, l);  v = bitonic_step_f<8, 2>(v, l);  v = bitonic_step_f<8, 1>(v, l);
  v = bitonic_step_f<16, 8>(v, l); v = bitonic_step_f<16, 4>(v, l); v = bitonic_step_f<16, 2>(v, l);
  v = bitonic_step_f<16, 1>(v, l);
  v = bitonic_step_f<32, 16>(v, l); v = bitonic_step_f<32, 8>(v, l); v = bitonic_step_f<32, 4>(v, l);
  v = bitonic_step_f<32, 2>(v, l);  v = bitonic_step_f<32, 1>(v, l);
  v = bitonic_step_f<64, 32>(v, l); v = bitonic_step_f<64, 16>(v, l); v = bitonic_step_f<64, 8>(v, l);
  v = bitonic_step_f<64, 4>(v, l);  v = bitonic_step_f<64, 2>(v, l);  v = bitonic_step_f<64, 1>(v, l);
  return __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(v)), K - 1)));
}

// Top-K of one row of fp32 scores, lane-contiguous layout: candidate j in lane
// j / KPL, slot j % KPL. Slots j >= n may hold anything (they are never
// chosen); values must not be NaN. Same rule and output as wave_topk;
// `scratch` is 64 (value, index) pairs of LDS private to the wavefront.
//
// Prefilter: T0 = K-th largest of the per-lane maxima. If no slot past n took
// part, at least K candidates are >= T0, so the answer lies among the values
// >= T0 (usually a few dozen). They are counted per lane and written, in index
// order, at offsets from a prefix sum over lanes: one ballot-free pass over the
// slots. The survivors then sit one per lane; those with j >= n are dropped,
// and if K candidates remain, T is read off their bitonic sort. Otherwise
// (more than 64 survivors after heavy ties, or slots past n that raised T0)
// the exact search runs over all candidates.
template <int KPL>
__device__ __forceinline__ void wave_topk_lc(const float (&val)[KPL], int n, int K,
                                             int32_t* __restrict__ out, uint32_t* scratch) {
  const int l = lane_id();
  if (n <= K) {
    for (int t = l; t < K; t += kWave) out[t] = t < n ? t : -1;
    return;
  }
  if (K <= kWave) {
    float mx = val[0];
#pragma unroll
    for (int r = 1; r < KPL; ++r) mx = fmaxf(mx, val[r]);
    const float T0 = kth_largest_lanes_f(mx, K);
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) cnt += val[r] >= T0 ? 1u : 0u;
    const uint32_t incl = wave_incl_scan(cnt, l);
    const uint32_t total = uint32_t(__builtin_amdgcn_readlane(int(incl), kWave - 1));
    if (total <= uint32_t(kWave)) {
      uint32_t pos = incl - cnt;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        if (val[r] >= T0) {
          scratch[2 * pos] = __float_as_uint(val[r]);
          scratch[2 * pos + 1] = uint32_t(l * KPL + r);
          ++pos;
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int32_t cj = uint32_t(l) < total ? int32_t(scratch[2 * l + 1]) : -1;
      const bool ok = cj >= 0 && cj < n;
      const float cv = ok ? __uint_as_float(scratch[2 * l]) : -INFINITY;
      __builtin_amdgcn_wave_barrier();
      if (popc64(ballot64(ok)) >= uint32_t(K)) {
        const float T = kth_largest_lanes_f(cv, K);
        const uint32_t ngt = popc64(ballot64(ok && cv > T));
        const uint64_t eqm = ballot64(ok && cv == T);
        const bool take = ok && (cv > T || (cv == T && ngt + mbcnt64(eqm) < uint32_t(K)));
        const uint64_t tm = ballot64(take);
        if (take) out[mbcnt64(tm)] = cj;
        return;
      }
    }
  }
  // Exact search over all candidates on order-preserving keys: every key > T,
  // then the first K - #(> T) keys equal to T in index order (lower lanes
  // first, then lower slots).
  uint32_t key[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) key[r] = l * KPL + r < n ? ordered_key(val[r]) : 0u;
  const uint32_t T = kth_largest<KPL>(key, K);
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    ngt += key[r] > T ? 1u : 0u;
    neq += key[r] == T ? 1u : 0u;
  }
  const uint32_t ngt_all = uint32_t(__builtin_amdgcn_readlane(int(wave_incl_scan(ngt, l)), kWave - 1));
  const uint32_t take_eq = uint32_t(K) - ngt_all;
  const uint32_t eq_before = wave_incl_scan(neq, l) - neq;
  const uint32_t eq_here = eq_before >= take_eq ? 0u : min(neq, take_eq - eq_before);
  const uint32_t taken = ngt + eq_here;
  uint32_t pos = wave_incl_scan(taken, l) - taken, eq_used = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const bool eq = key[r] == T;
    if (key[r] > T || (eq && eq_used < eq_here)) out[pos++] = l * KPL + r;
    eq_used += eq ? 1u : 0u;
  }
}

// Inclusive prefix sum over the wavefront's lanes with DPP: row shifts build
// the sums inside each 16-lane row, then the row broadcasts carry row totals.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, true));   // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, true));   // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, true));   // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, true));   // row_shr:8
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// LDS of the workgroup selection below.
struct WgTopkLds {
  uint32_t gmax[kWave];     // maxima of the 64 candidate groups (keys)
  uint32_t wtot[8];         // survivors per wavefront
  uint32_t lk[kWave];       // survivors: key, candidate index (index order)
  int32_t lj[kWave];
};

// Top-K of one row of fp32 scores by the 8 first wavefronts of a workgroup;
// every wavefront of the workgroup must call it (it holds workgroup
// barriers). Candidate j = (64*w + l)*S + s sits in wavefront w, lane l, slot
// s, S = SKPL/8 (so a 64*SKPL-candidate row is spread over 8*64 lanes in index
// order). Same rule, prefilter and fallback as wave_topk_lc: the groups are
// the 64 runs of SKPL consecutive candidates (8 lanes of one wavefront), so
// the bound T0 and the survivors are those of the one-wavefront version; the
// slot work, the group maxima and the survivor counts are split 8 ways.
// `row` holds the scores (j < nblk readable; slots past n may hold anything);
// `vec`: rows are 16-byte aligned. Wavefront 0 writes out[0 .. K-1]; the
// caller synchronizes the workgroup before reading it.
template <int SKPL>
__device__ __forceinline__ void wg_topk8(const float* __restrict__ row, int64_t nblk, bool vec,
                                         int n, int K, int32_t* __restrict__ out,
                                         uint32_t* scratch, WgTopkLds& sh) {
  static_assert(SKPL >= 8, "eight wavefronts need at least one slot each");
  constexpr int S = SKPL / 8;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const bool part = w < 8;
  const int j0 = (w * kWave + l) * S;
  if (n <= K) {                          // every candidate is taken
    if (w == 0)
      for (int t = l; t < K; t += kWave) out[t] = t < n ? t : -1;
    return;
  }
  uint32_t key[S];
  if (part) {
    float val[S];
    bool done = false;
    if constexpr (S >= 4) {
      if (vec) {
#pragma unroll
        for (int s = 0; s < S; s += 4) {
          const int j = j0 + s;
          const uint4 u = ldg16_or_neginf(j < nblk, row + (j < nblk ? j : 0));
          val[s] = __uint_as_float(u.x);
          val[s + 1] = __uint_as_float(u.y);
          val[s + 2] = __uint_as_float(u.z);
          val[s + 3] = __uint_as_float(u.w);
        }
        done = true;
      }
    }
    if (!done) {
#pragma unroll
      for (int s = 0; s < S; ++s) val[s] = ldf_or_neginf(j0 + s < nblk, row + j0 + s);
    }
    uint32_t mx = 0u;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      key[s] = ordered_key(val[s]);
      mx = max(mx, key[s]);
    }
    mx = max(mx, xor_lane<1>(mx, l));
    mx = max(mx, xor_lane<2>(mx, l));
    mx = max(mx, xor_lane<4>(mx, l));
    if ((l & 7) == 0) sh.gmax[w * 8 + l / 8] = mx;
  }
  lds_barrier();
  uint32_t mask = 0u, excl = 0u;
  if (part && K <= kWave) {
    const uint32_t T0 = kth_largest_lanes(sh.gmax[l], K);
#pragma unroll
    for (int s = 0; s < S; ++s) mask |= (key[s] >= T0 ? 1u : 0u) << s;
    const uint32_t cnt = __popc(mask);
    const uint32_t incl = wave_incl_scan_dpp(cnt);
    excl = incl - cnt;
    if (l == kWave - 1) sh.wtot[w] = incl;
  }
  lds_barrier();
  uint32_t total = ~0u;
  if (part && K <= kWave) {
    uint32_t base = 0u;
    total = 0u;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint32_t t = sh.wtot[v];
      base += v < w ? t : 0u;
      total += t;
    }
    if (total <= uint32_t(kWave)) {
      uint32_t pos = base + excl;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if ((mask >> s) & 1u) {
          sh.lk[pos] = key[s];
          sh.lj[pos] = j0 + s;
          ++pos;
        }
      }
    }
  }
  lds_barrier();
  if (w != 0) return;
  if (total <= uint32_t(kWave)) {
    const int32_t cj = uint32_t(l) < total ? sh.lj[l] : -1;
    const bool ok = cj >= 0 && cj < n;
    const uint32_t ck = ok ? sh.lk[l] : 0u;
    if (popc64(ballot64(ok)) >= uint32_t(K)) {
      const uint32_t T = kth_largest_lanes(ck, K);
      const uint32_t ngt = popc64(ballot64(ok && ck > T));
      const uint64_t eqm = ballot64(ok && ck == T);
      const bool take = ok && (ck > T || (ck == T && ngt + mbcnt64(eqm) < uint32_t(K)));
      const uint64_t tm = ballot64(take);
      if (take) out[mbcnt64(tm)] = cj;
      return;
    }
  }
  // Heavy ties, or slots past n that raised T0: wavefront 0 takes the whole
  // row (lane-contiguous) and runs the one-wavefront selection.
  float all[SKPL];
#pragma unroll
  for (int r = 0; r < SKPL; ++r) all[r] = ldf_or_neginf(l * SKPL + r < nblk, row + l * SKPL + r);
  wave_topk_lc<SKPL>(all, n, K, out, scratch);
}

// ------------------------------------------------------- one row per 16 lanes
// Top-K (K <= 16) of four score rows at once, one per 16-lane row of the
// wavefront (row q = lanes 16q .. 16q+15). Every cross-lane step stays inside
// a 16-lane row (DPP), so the four rows share each instruction.
//
// The rows hold order-preserving score keys, 0 past the row's candidates.
// Lane r of a row holds candidates 64g + 4r + e (g < ng, e < 4): a 16-byte LDS
// read per group, and every lane holds candidates as soon as n >= 64.
//   1. bound: each lane keeps its two largest keys; the K-th largest T0 of
//      those 32 is a lower bound of the row's K-th largest key (K distinct
//      candidates are >= T0), so every chosen candidate, and every candidate
//      tied with the K-th, is >= T0. (With fewer than K candidates among them,
//      T0 is 0 and every candidate survives.)
//   2. survivors (usually 16-24): compacted into 32 LDS slots per row;
//   3. threshold: the K-th largest key T among the survivors (two 16-lane
//      bitonic sorts and their elementwise max = the 16 largest of 32);
//   4. emit: when exactly K survivors are >= T the row's choice is these,
//      written ascending after one more 16-lane sort of their indices.
// A row with more than 32 survivors, or with more survivors equal to T than
// the K-th place can take (ties that the lower index must break), is left
// unresolved for the exact one-row routine (wave_topk).
//
// Row of 16 lanes: the value of lane l ^ J (J < 16) of the same row.
template <int J>
__device__ __forceinline__ uint32_t row_xor(uint32_t v, int rl) {
  if constexpr (J == 8) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  } else {
    return xor_lane<J>(v, rl);
  }
}

// Bitonic stage inside a 16-lane row; runs of KS lanes end descending when
// `desc` (ascending otherwise) at KS = 16, alternating below.
template <int KS, int J>
__device__ __forceinline__ uint32_t row_cex(uint32_t v, int rl, bool desc) {
  const uint32_t p = row_xor<J>(v, rl);
  const bool lower = (rl & J) == 0;
  const bool d = ((rl & KS) == 0) == desc;
  return lower == d ? max(v, p) : min(v, p);
}

__device__ __forceinline__ uint32_t row_sort16(uint32_t v, int rl, bool desc) {
  v = row_cex<2, 1>(v, rl, desc);
  v = row_cex<4, 2>(v, rl, desc);   v = row_cex<4, 1>(v, rl, desc);
  v = row_cex<8, 4>(v, rl, desc);   v = row_cex<8, 2>(v, rl, desc);   v = row_cex<8, 1>(v, rl, desc);
  v = row_cex<16, 8>(v, rl, desc);  v = row_cex<16, 4>(v, rl, desc);  v = row_cex<16, 2>(v, rl, desc);
  v = row_cex<16, 1>(v, rl, desc);
  return v;
}

// A bitonic 16-lane row -> descending.
__device__ __forceinline__ uint32_t row_merge16_desc(uint32_t v, int rl) {
  v = row_cex<16, 8>(v, rl, true);  v = row_cex<16, 4>(v, rl, true);
  v = row_cex<16, 2>(v, rl, true);  v = row_cex<16, 1>(v, rl, true);
  return v;
}

__device__ __forceinline__ uint32_t row_min16(uint32_t v, int rl) {
  v = min(v, row_xor<1>(v, rl));
  v = min(v, row_xor<2>(v, rl));
  v = min(v, row_xor<4>(v, rl));
  return min(v, row_xor<8>(v, rl));
}

__device__ __forceinline__ uint32_t row_sum16(uint32_t v, int rl) {
  v += row_xor<1>(v, rl);
  v += row_xor<2>(v, rl);
  v += row_xor<4>(v, rl);
  return v + row_xor<8>(v, rl);
}

__device__ __forceinline__ uint32_t row_incl_scan16(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, true));   // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, true));   // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, true));   // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, true));   // row_shr:8
  return v;
}

// Lane rl = i of this lane's row.
__device__ __forceinline__ uint32_t row_lane(uint32_t v, int l, int i) {
  return uint32_t(__shfl(int(v), (l & 48) | i));
}

// max / median of fp32 without the NaN quieting fmaxf carries (scores are
// never NaN): v_max_f32.
__device__ __forceinline__ float fmax_nq(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

// Order-preserving key of a score that is not -0 (a sum that started from +0):
// larger float -> larger key, -inf -> 0x007FFFFF, so key 0 is below every score.
__device__ __forceinline__ uint32_t ordered_key_nz(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

// `row`: this lane's row of score keys (ordered_key) in LDS, 16-byte aligned,
// 64*ng entries, those j >= n holding 0. `n`: candidates of the row;
// 1 <= K <= 16 (wave-uniform). `out`: the row's K outputs, or null for a row
// that writes nothing. `buf` (32 pairs) and `obuf` (16 ints): LDS private to
// the row. Every lane of the wavefront calls it; returns whether this lane's
// row is resolved (rows with n <= K always are: all taken, -1 padded).
template <int NG>
__device__ __forceinline__ bool rows16_topk(const uint32_t* __restrict__ row, int ng, int n, int K,
                                            int32_t* __restrict__ out, uint2* buf, int32_t* obuf) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int l = lane_id();
  const int rl = l & 15;
  // 1. per-lane two largest, then the bound T0
  u32x4 v[NG];
  uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    v[g] = g < ng ? *reinterpret_cast<const u32x4*>(row + 64 * g + 4 * rl) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m2 = umed3(m1, m2, v[g][e]);
      m1 = max(m1, v[g][e]);
    }
  }
  const uint32_t a = row_sort16(m1, rl, true);
  const uint32_t b = row_sort16(m2, rl, false);
  const uint32_t c = max(a, b);                  // the 16 largest of the 32, bitonic
  uint32_t t0 = K < 16 ? row_lane(row_merge16_desc(c, rl), l, K - 1) : row_min16(c, rl);
  t0 = max(t0, 1u);                              // padding (key 0) never survives

  // 2. survivors
  uint32_t mask = 0u;
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) mask |= (v[g][e] >= t0 ? 1u : 0u) << (4 * g + e);
  const uint32_t cnt = __popc(mask);
  const uint32_t incl = row_incl_scan16(cnt);
  const uint32_t total = row_lane(incl, l, 15);
  const bool trivial = n <= K;
  if (trivial || total > 32u) mask = 0u;
  uint32_t pos = incl - cnt;
  while (ballot64(mask != 0u)) {
    if (mask != 0u) {
      const int bit = __builtin_ctz(mask);
      const int j = (bit >> 2) * 64 + 4 * rl + (bit & 3);
      buf[pos] = make_uint2(row[j], uint32_t(j));
      ++pos;
      mask &= mask - 1u;
    }
  }

  // 3. threshold among the survivors (keys of empty slots are 0, below all)
  const bool va = uint32_t(rl) < total, vb = uint32_t(rl) + 16u < total;
  const uint2 ea = va ? buf[rl] : make_uint2(0u, 0u);
  const uint2 eb = vb ? buf[rl + 16] : make_uint2(0u, 0u);
  const uint32_t sa = row_sort16(ea.x, rl, true);
  const uint32_t sb = row_sort16(eb.x, rl, false);
  const uint32_t c2 = max(sa, sb);
  const uint32_t T = K < 16 ? row_lane(row_merge16_desc(c2, rl), l, K - 1) : row_min16(c2, rl);
  const uint32_t ta = ea.x >= T ? 1u : 0u, tb = eb.x >= T ? 1u : 0u;
  const uint32_t nge = row_sum16(ta + tb, rl);
  const bool resolved = trivial || (total <= 32u && nge == uint32_t(K));

  // 4. emit ascending
  const uint32_t tin = row_incl_scan16(ta + tb);
  const uint32_t p = tin - ta - tb;
  if (resolved && !trivial) {
    if (ta) obuf[p] = int32_t(ea.y);
    if (tb) obuf[p + ta] = int32_t(eb.y);
  }
  const uint32_t o = row_sort16(rl < K ? uint32_t(obuf[rl]) : 0x7FFFFFFFu, rl, false);
  if (out != nullptr && rl < K) {
    if (trivial) out[rl] = rl < n ? rl : -1;
    else if (resolved) out[rl] = int32_t(o);
  }
  return resolved;
}

}  // namespace infllmv2
