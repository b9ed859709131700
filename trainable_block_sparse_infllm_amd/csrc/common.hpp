// Device-side helpers shared by the gfx950 kernels: bf16 conversion, MFMA
// fragment types, wavefront reductions, and the XCD-aware grid remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infllmv2 {

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kBlock = 64;    // tokens per context block
constexpr int kKpb = 3;       // semantic kernels per block (window 32, stride 16)
constexpr int kNumXcd = 8;    // MI355X: 8 accelerator complex dies, one L2 each

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}

// Offset (in elements) of the 16-byte piece p (elements 8p .. 8p+7) of kernel
// m of block j in the k-bar table of group bg:
//   [bg][ceil(nblk/32)][3][D/8][32][8]
// Blocks are grouped in tiles of 32; inside a tile the 32 blocks' copies of
// one piece are adjacent. A wavefront reading pieces 2s and 2s+1 of one tile
// (lanes 0-31 and 32-63, the k-slot halves of a 16-wide MFMA step) touches
// one contiguous kilobyte, and a whole tile is 3*D*64 contiguous bytes.
template <int D>
__device__ __forceinline__ int64_t kbar_off(int64_t bg, int m, int p, int64_t j, int64_t nblk) {
  const int64_t ntile = (nblk + 31) >> 5;
  return (((bg * ntile + (j >> 5)) * kKpb + m) * (D / 8) + p) * 256 + (j & 31) * 8;
}

// 32x32x16 bf16 MFMA. Operand A: lane l holds row l%32, k-slots 8*(l/32) ..
// +7; operand B: lane l holds column l%32, the same k-slots. Accumulator
// register r of lane l: row 8*(r/4) + 4*(l/32) + r%4, column l%32.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (lo in the low half) with the hardware
// round-to-nearest-even conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2_t b = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, sizeof u);
  return u;
}

// Exact double (a mean of bf16 values) -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t d2bf(double x) {
  uint64_t u = __double_as_longlong(x);
  const uint16_t sign = uint16_t((u >> 48) & 0x8000u);
  u &= 0x7FFFFFFFFFFFFFFFull;
  if (u > 0x7FF0000000000000ull) return 0x7FC0;                 // NaN
  if (u < 0x3810000000000000ull) {                              // |x| < 2^-126: quantum 2^-133
    const double a = __longlong_as_double(u);
    return sign | uint16_t(rint(a * 0x1p133));                  // 0..128 (128 = smallest normal)
  }
  u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);              // RNE: half of 2^45, minus 1, plus lsb
  const int e = int(u >> 52) - 1023;
  if (e > 127) return sign | 0x7F80;                            // overflow -> inf
  return sign | uint16_t(((e + 127) << 7) | int((u >> 45) & 0x7Fu));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof r);
  return r;
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load marked nontemporal: for data read once per kernel (the k-bar
// table in decode scoring), so it does not displace reusable lines in the
// caches.
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{x[0], x[1], x[2], x[3]};
}

// Guarded loads without branches. A guarded load reads either the real
// location or a device-global constant holding the neutral value (zeros, -inf)
// and uses the result unconditionally: the choice is made on the address, so a
// run of guarded loads issues back to back instead of one round trip each (a
// select on the loaded value would be turned back into a conditional load).
// The constant's address goes through an empty asm, which hides what it points
// to: otherwise the compiler folds the load of the constant and recreates the
// value select. (The asm holds no instruction and no load.)
// (Declared without const so they live in the global address space, like the
// tensors they stand in for: the load then stays a global load, not a flat one.)
static __device__ __align__(16) uint32_t kZeroPiece[4] = {0u, 0u, 0u, 0u};
static __device__ float kNegInf = -INFINITY;
static __device__ __align__(16) float kNegInf4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
static __device__ float kZeroF = 0.f;

typedef __attribute__((address_space(1))) const uint32_t g_u32;   // global-space views
typedef __attribute__((address_space(1))) const float g_float;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t g_u32x4;

__device__ __forceinline__ uint64_t opaque_addr(const void* p) {
  uint64_t a = reinterpret_cast<uint64_t>(p);
  asm("" : "+v"(a));
  return a;
}

__device__ __forceinline__ uint4 ldg16_if(bool ok, const void* p) {
  const g_u32x4* z = (const g_u32x4*)opaque_addr(kZeroPiece);
  const u32x4_t v = *(ok ? (const g_u32x4*)p : z);
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint4 ldg16_or_neginf(bool ok, const void* p) {   // four fp32 -inf
  const g_u32x4* z = (const g_u32x4*)opaque_addr(kNegInf4);
  const u32x4_t v = *(ok ? (const g_u32x4*)p : z);
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ float ldf_or_neginf(bool ok, const float* p) {
  const g_float* z = (const g_float*)opaque_addr(&kNegInf);
  return *(ok ? (const g_float*)p : z);
}

__device__ __forceinline__ float ldf_or_zero(bool ok, const float* p) {
  const g_float* z = (const g_float*)opaque_addr(&kZeroF);
  return *(ok ? (const g_float*)p : z);
}

typedef __attribute__((address_space(1))) void gas_void;   // global address space
typedef __attribute__((address_space(3))) void las_void;   // LDS address space

// Direct HBM -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_base + 16*l; lds_base must be wave-uniform.
// Completion is tracked by the vector-memory counter only (see wait_vmem).
__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gas_void*)gsrc, (las_void*)lds_base, 16, 0, 0);
}

// The same copy marked nontemporal (cache policy NT): for data read once per
// kernel, so it does not displace reusable lines.
__device__ __forceinline__ void load_lds16_nt(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gas_void*)gsrc, (las_void*)lds_base, 16, 0, 2);
}

// s_waitcnt vmcnt(0): every vector-memory load of this wave, including the
// direct-to-LDS ones the compiler does not track, has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier for LDS traffic only: the wavefront's LDS operations have
// completed, then s_barrier. Unlike __syncthreads it does not wait for the
// wavefront's outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  wait_lds();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int W>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int W>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Reductions over the four 16-lane rows of a wavefront (lanes l, l^16, l^32,
// l^48), with the gfx950 row-swap instructions instead of LDS-routed shuffles:
// permlane16_swap(x, x) leaves rows (0,0,2,2) in one result and (1,1,3,3) in
// the other, permlane32_swap(x, x) rows (0,1,0,1) and (2,3,2,3).
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lane 0's value of a 64-bit quantity, as a wave-uniform (scalar) value.
// (readfirstlane works on 32-bit ints; each half is zero-extended.)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(x))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(x >> 32))));
  return uint64_t(lo) | (uint64_t(hi) << 32);
}

__device__ __forceinline__ uint32_t popc64(uint64_t x) { return __popcll(x); }

// Lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Order-preserving map fp32 -> uint32 (larger float -> larger key; -inf lowest
// among non-NaN values).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = u == 0x80000000u ? 0u : u;   // -0 and +0 are equal scores
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8). Renumber them so that each XCD receives one contiguous range of
// work items: neighbouring items (same KV group) then share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / kNumXcd;
  const int rem = nblocks % kNumXcd;
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  // XCDs 0..rem-1 own per+1 items, the rest own per.
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + slot;
}

}  // namespace infllmv2
