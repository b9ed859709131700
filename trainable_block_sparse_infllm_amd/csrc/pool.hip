// Semantic-kernel pooling (MiniCPM4 technical-report summary, QbitAI repost,
// section "Model architecture: InfLLM v2", item 1: every context block is
// represented by several fine-grained semantic kernels).
//
// Kernel m of block j is the mean of the 32 keys 64j+16m .. 64j+16m+31
// (m = 0, 1, 2), rounded to bf16 (nearest even). The sums run in fp64: a sum
// of 32 bf16 values is exact there for any data whose nonzero magnitudes span
// fewer than 2^40, so the mean has a single value whatever the summation order
// and the rounded kernel is reproducible bit for bit.
//
// HBM-bound: one read of K (64*D*2 bytes per block), 3*D*2 bytes written
// (16-byte pieces, in the tiled k-bar layout of kbar_off).
// One wavefront per block; lane l owns D/64 adjacent columns, so each row is a
// single coalesced 2*D-byte wavefront load.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

// Kernels of block j of (b, g) from its 64 key rows, row r at row_of(r): one
// wavefront, lane l owns D/64 adjacent columns.
template <int D, typename RowOf>
__device__ __forceinline__ void pool_block(RowOf row_of, uint16_t* __restrict__ kbar, int64_t bg,
                                           int64_t j, int64_t nblk, int l) {
  constexpr int CPL = D / kWave;  // columns per lane: 1 or 2
  // lane l owns columns CPL*l ..: piece CPL*l/8, offset CPL*l%8 within it
  const int piece = CPL * l / 8, within = CPL * l % 8;
  double s[4][CPL];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int x = 0; x < CPL; ++x) s[c][x] = 0.0;
  if constexpr (CPL == 2) {
    uint32_t row[kBlock];
#pragma unroll
    for (int r = 0; r < kBlock; ++r) row[r] = *reinterpret_cast<const uint32_t*>(row_of(r) + CPL * l);
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
      s[r / 16][0] += double(bf2f(uint16_t(row[r] & 0xFFFFu)));
      s[r / 16][1] += double(bf2f(uint16_t(row[r] >> 16)));
    }
  } else {
    uint16_t row[kBlock];
#pragma unroll
    for (int r = 0; r < kBlock; ++r) row[r] = row_of(r)[CPL * l];
#pragma unroll
    for (int r = 0; r < kBlock; ++r) s[r / 16][0] += double(bf2f(row[r]));
  }
#pragma unroll
  for (int m = 0; m < kKpb; ++m) {
    if constexpr (CPL == 2) {
      const uint32_t lo = d2bf((s[m][0] + s[m + 1][0]) * 0.03125);
      const uint32_t hi = d2bf((s[m][1] + s[m + 1][1]) * 0.03125);
      *reinterpret_cast<uint32_t*>(kbar + kbar_off<D>(bg, m, piece, j, nblk) + within) = lo | (hi << 16);
    } else {
      kbar[kbar_off<D>(bg, m, piece, j, nblk) + within] = d2bf((s[m][0] + s[m + 1][0]) * 0.03125);
    }
  }
}

// Blocks first .. first+nb-1 of every (b, g), one wavefront each.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ k,
                                                   uint16_t* __restrict__ kbar, int64_t kv_cap,
                                                   int64_t nblk, int64_t first, int64_t nb,
                                                   int64_t total) {
  const int w = threadIdx.x / kWave;
  const int l = threadIdx.x % kWave;
  const int64_t item = int64_t(blockIdx.x) * 4 + w;
  if (item >= total) return;
  const int64_t bg = item / nb;
  const int64_t j = first + item % nb;
  const uint16_t* src = k + (bg * kv_cap + j * kBlock) * D;
  pool_block<D>([&](int r) { return src + r * D; }, kbar, bg, j, nblk, l);
}

hipError_t launch_pool(const Dims& d, const uint16_t* k, int64_t kv_cap, int64_t nblk,
                       int64_t first, int64_t last, uint16_t* kbar, hipStream_t s) {
  const int64_t nb = last - first;
  if (nb <= 0) return hipSuccess;
  const int64_t total = int64_t(d.B) * d.Hkv * nb;
  const dim3 grid(unsigned((total + 3) / 4));
  if (d.D == 128)
    pool_kernel<128><<<grid, 256, 0, s>>>(k, kbar, kv_cap, nblk, first, nb, total);
  else
    pool_kernel<64><<<grid, 256, 0, s>>>(k, kbar, kv_cap, nblk, first, nb, total);
  return hipGetLastError();
}

// ------------------------------------------------------------------ cache append
// The decode loop's cache maintenance (QbitAI summary, efficiency evaluation:
// the semantic-kernel representation is the part that grows with the
// context): n_new tokens' K and V rows [B][Hkv][n_new][D] go to rows
// len_b .. len_b+n_new-1 of the caches (len_b = lens[b], or kv_len for every
// sequence); rows that would land at or past kv_cap are not written. Every
// block the append completes is pooled in the same launch.
//
// One workgroup per (b, g) and block the append touches (block len_b/64 + t,
// t < nbt): it copies the appended rows that fall in the block (16-byte
// pieces, K then V) and, if they complete it, its first wavefront pools the
// block, taking rows before len_b from the cache and appended rows from the
// inputs, so no row this launch writes is read back.
template <int D>
__global__ __launch_bounds__(256) void append_kv_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, uint16_t* __restrict__ kbar,
    int64_t kv_cap, int64_t nblk, const int64_t* __restrict__ lens, int64_t kv_len, int64_t n_new,
    int Hkv, int nbt) {
  constexpr int64_t PPR = D / 8;                      // 16-byte pieces per row
  const int64_t bg = blockIdx.x / nbt;
  const int64_t len0 = lens ? lens[bg / Hkv] : kv_len;
  if (len0 < 0) return;
  const int64_t j = len0 / kBlock + blockIdx.x % nbt;
  const int64_t r_lo = max(len0, j * kBlock);
  const int64_t r_hi = min(min(len0 + n_new, (j + 1) * kBlock), kv_cap);
  if (r_lo >= r_hi) return;                           // no appended row lands in this block
  const int64_t np = (r_hi - r_lo) * PPR;
  for (int64_t e = threadIdx.x; e < 2 * np; e += 256) {
    const bool is_v = e >= np;
    const int64_t x = is_v ? e - np : e;
    const int64_t r = r_lo + x / PPR, piece = x % PPR;
    const uint4 val = ldg16((is_v ? v_new : k_new) + (bg * n_new + (r - len0)) * D + piece * 8);
    *reinterpret_cast<uint4*>((is_v ? v_cache : k_cache) + (bg * kv_cap + r) * D + piece * 8) = val;
  }
  if (!kbar || r_hi != (j + 1) * kBlock || threadIdx.x >= kWave) return;
  const uint16_t* old_rows = k_cache + (bg * kv_cap + j * kBlock) * D;
  const int64_t r_new = len0 - j * kBlock;            // first appended row within the block
  pool_block<D>([&](int r) {
    return r < r_new ? old_rows + r * D : k_new + (bg * n_new + (r - r_new)) * D;
  }, kbar, bg, j, nblk, int(threadIdx.x));
}

hipError_t launch_append(const Dims& d, const uint16_t* k_new, const uint16_t* v_new,
                         int64_t n_new, uint16_t* k_cache, uint16_t* v_cache, int64_t kv_cap,
                         const int64_t* lens, int64_t kv_len, uint16_t* kbar, hipStream_t s) {
  if (n_new <= 0) return hipSuccess;
  const int64_t nblk = (kv_cap + kBlock - 1) / kBlock;
  const int64_t nbt = (n_new + kBlock - 1) / kBlock + 1;   // blocks an append of n_new rows touches
  const int64_t grid = int64_t(d.B) * d.Hkv * nbt;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (d.D == 128)
    append_kv_kernel<128><<<dim3(unsigned(grid)), 256, 0, s>>>(k_new, v_new, k_cache, v_cache, kbar,
                                                               kv_cap, nblk, lens, kv_len, n_new,
                                                               d.Hkv, int(nbt));
  else
    append_kv_kernel<64><<<dim3(unsigned(grid)), 256, 0, s>>>(k_new, v_new, k_cache, v_cache, kbar,
                                                              kv_cap, nblk, lens, kv_len, n_new,
                                                              d.Hkv, int(nbt));
  return hipGetLastError();
}

}  // namespace infllmv2
