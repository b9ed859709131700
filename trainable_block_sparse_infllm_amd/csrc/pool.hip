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
#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ k,
                                                   uint16_t* __restrict__ kbar, int64_t kv_cap,
                                                   int64_t nblk, int64_t first, int64_t nb,
                                                   int64_t total) {
  constexpr int CPL = D / kWave;  // columns per lane: 1 or 2
  const int w = threadIdx.x / kWave;
  const int l = threadIdx.x % kWave;
  const int64_t item = int64_t(blockIdx.x) * 4 + w;
  if (item >= total) return;
  const int64_t bg = item / nb;
  const int64_t j = first + item % nb;
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

}  // namespace infllmv2
