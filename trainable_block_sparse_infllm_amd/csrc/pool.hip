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

// Blocks first .. first+nb-1 of every (b, g); with lens (a cache append of
// n_new tokens to sequences of lengths lens[b]): the blocks of sequence b
// that the append completes, lens[b]/64 .. (lens[b]+n_new)/64 - 1, at most
// nb of them.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ k,
                                                   uint16_t* __restrict__ kbar, int64_t kv_cap,
                                                   int64_t nblk, int64_t first, int64_t nb,
                                                   int64_t total, const int64_t* __restrict__ lens,
                                                   int64_t n_new, int Hkv) {
  constexpr int CPL = D / kWave;  // columns per lane: 1 or 2
  const int w = threadIdx.x / kWave;
  const int l = threadIdx.x % kWave;
  const int64_t item = int64_t(blockIdx.x) * 4 + w;
  if (item >= total) return;
  const int64_t bg = item / nb;
  int64_t j = first + item % nb;
  if (lens) {
    const int64_t len0 = lens[bg / Hkv];
    j = len0 / kBlock + item % nb;
    if (len0 < 0 || j >= min((len0 + n_new) / kBlock, kv_cap / kBlock)) return;
  }
  const uint16_t* src = k + (bg * kv_cap + j * kBlock) * D + CPL * l;
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
    for (int r = 0; r < kBlock; ++r) row[r] = *reinterpret_cast<const uint32_t*>(src + r * D);
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
      s[r / 16][0] += double(bf2f(uint16_t(row[r] & 0xFFFFu)));
      s[r / 16][1] += double(bf2f(uint16_t(row[r] >> 16)));
    }
  } else {
    uint16_t row[kBlock];
#pragma unroll
    for (int r = 0; r < kBlock; ++r) row[r] = src[r * D];
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

hipError_t launch_pool(const Dims& d, const uint16_t* k, int64_t kv_cap, int64_t nblk,
                       int64_t first, int64_t last, uint16_t* kbar, hipStream_t s,
                       const int64_t* lens, int64_t n_new) {
  const int64_t nb = lens ? (n_new + kBlock - 1) / kBlock + 1 : last - first;
  if (nb <= 0) return hipSuccess;
  const int64_t total = int64_t(d.B) * d.Hkv * nb;
  const dim3 grid(unsigned((total + 3) / 4));
  if (d.D == 128)
    pool_kernel<128><<<grid, 256, 0, s>>>(k, kbar, kv_cap, nblk, first, nb, total, lens, n_new, d.Hkv);
  else
    pool_kernel<64><<<grid, 256, 0, s>>>(k, kbar, kv_cap, nblk, first, nb, total, lens, n_new, d.Hkv);
  return hipGetLastError();
}

// ------------------------------------------------------------------ cache append
// The decode loop's cache maintenance (QbitAI summary, efficiency evaluation:
// the semantic-kernel representation is the part that grows with the
// context): n_new tokens' K and V rows [B][Hkv][n_new][D] go to rows
// len_b .. len_b+n_new-1 of the caches (len_b = lens[b], or kv_len for every
// sequence); rows that would land at or past kv_cap are not written.
// Grid-stride over 16-byte pieces, K then V.
__global__ __launch_bounds__(256) void append_kv_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int64_t kv_cap,
    const int64_t* __restrict__ lens, int64_t kv_len, int64_t n_new, int D, int Hkv,
    int64_t total) {
  const int64_t ppr = D / 8;                          // pieces per row
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * 256) {
    const int64_t per_t = total / 2;                  // pieces per tensor
    const bool is_v = e >= per_t;
    const int64_t x = is_v ? e - per_t : e;
    const int64_t piece = x % ppr;
    const int64_t i = (x / ppr) % n_new;
    const int64_t bg = x / (ppr * n_new);
    const int64_t len0 = lens ? lens[bg / Hkv] : kv_len;
    const int64_t row = len0 + i;
    if (len0 < 0 || row >= kv_cap) continue;
    const uint4 val = ldg16((is_v ? v_new : k_new) + (bg * n_new + i) * D + piece * 8);
    *reinterpret_cast<uint4*>((is_v ? v_cache : k_cache) + (bg * kv_cap + row) * D + piece * 8) = val;
  }
}

hipError_t launch_append(const Dims& d, const uint16_t* k_new, const uint16_t* v_new,
                         int64_t n_new, uint16_t* k_cache, uint16_t* v_cache, int64_t kv_cap,
                         const int64_t* lens, int64_t kv_len, uint16_t* kbar, hipStream_t s) {
  if (n_new <= 0) return hipSuccess;
  const int64_t total = 2 * int64_t(d.B) * d.Hkv * n_new * (d.D / 8);
  const unsigned blocks = unsigned(std::min<int64_t>(4096, (total + 255) / 256));
  append_kv_kernel<<<dim3(blocks), 256, 0, s>>>(k_new, v_new, k_cache, v_cache, kv_cap, lens,
                                                kv_len, n_new, d.D, d.Hkv, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !kbar) return e;
  // the blocks the append completes, read back from the cache in stream order
  const int64_t nblk = (kv_cap + kBlock - 1) / kBlock;
  if (lens) return launch_pool(d, k_cache, kv_cap, nblk, 0, 0, kbar, s, lens, n_new);
  const int64_t first = kv_len / kBlock;
  const int64_t last = std::min(kv_len + n_new, kv_cap) / kBlock;
  return launch_pool(d, k_cache, kv_cap, nblk, first, last, kbar, s);
}

}  // namespace infllmv2
