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
//   mode 1 (dense causal): keys 0..p;      mode 2 (dense): keys 0..kv_len-1.
//
// Work layout. A workgroup (4 wavefronts) owns TQ <= 64 consecutive tokens of
// one (b, g); a wavefront owns NST sub-tiles of 16 MFMA rows (16/G tokens x G
// heads: one token's heads share a key set). On the 32K workload 64
// consecutive tokens need ~45 distinct blocks between them while each needs
// 17, so the tile walks that union once and reuses every staged block for all
// of its tokens that need it:
//
//   1. union: the tile's blocks are listed in ascending order, each with a
//      64-bit mask of the tile's tokens that attend it. Own blocks and dense
//      prefixes are ranges, so their mask bits are computed; only selected
//      blocks go through an LDS bitmap. A tile whose tokens are all dense
//      needs no list at all: block u is entry u;
//   2. a ring of NSTAGE LDS stages holds K and V of upcoming blocks, filled
//      straight from HBM (global_load_lds, no staging registers), so
//      NSTAGE - 1 blocks are in flight while one is computed; one barrier per
//      block;
//   3. per block, each wavefront runs its sub-tiles that hold a token needing
//      it: S^T = K Q^T (MFMA 16x16x32 bf16; A = K fragments from LDS, B = Q
//      in registers), online softmax in the exp2 domain with the rows of other
//      tokens masked, O^T += V^T P^T (A = V^T fragments from the transpose
//      read ds_read_b64_tr_b16 of the row-major V tile, B = P^T taken from
//      the S^T accumulators).
//
// LDS tiles are row-major 64 x 128 bf16 whose 16-byte pieces are XOR-swizzled
// per row by swz(r) = ((r & 7) << 1) | ((r >> 3) & 1): the 16 rows of a K
// fragment read land in 16 distinct piece slots, and the 4 rows x 2 pieces of
// each 16-lane transpose read in 8.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace infllmv2 {

namespace {

constexpr int kD = 128;
constexpr int kTileBytes = kBlock * kD * 2;   // one K or V tile
constexpr int kStageBytes = 2 * kTileBytes;   // K then V

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Keys key0 .. key0+63 of K and V -> one LDS stage (8 direct loads per
// thread). Chunk c (1 KB, rows 4c..4c+3) is loaded by wavefront c % 4; lane
// l's 16 bytes land in slot l % 16 of row 4c + l / 16, so it fetches the global
// piece stored in that slot. Rows past kv_len repeat row kv_len - 1 (finite
// data; their scores are masked).
__device__ __forceinline__ void issue_stage(char* stage, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t key0, int64_t kv_len,
                                           int w, int l) {
  if (key0 + kBlock <= kv_len) {
    const uint16_t* kb = kbase + key0 * kD;
    const uint16_t* vb = vbase + key0 * kD;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int c = x * 4 + w;
      const int row = 4 * c + l / 16;
      const int off = row * kD + ((l % 16) ^ swz(row)) * 8;
      load_lds16(kb + off, stage + c * 1024);
      load_lds16(vb + off, stage + kTileBytes + c * 1024);
    }
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int c = x * 4 + w;
      const int row = 4 * c + l / 16;
      const int64_t key = min(key0 + row, kv_len - 1);
      const int64_t off = key * kD + ((l % 16) ^ swz(row)) * 8;
      load_lds16(kbase + off, stage + c * 1024);
      load_lds16(vbase + off, stage + kTileBytes + c * 1024);
    }
  }
}

// s_waitcnt vmcnt(8 * stages): stages complete in issue order, so an entry has
// landed once only the stages issued after it (8 loads each) are pending.
__device__ __forceinline__ void wait_stages_pending(int stages) {
  switch (stages) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;                   // vmcnt(0)
    case 1: __builtin_amdgcn_s_waitcnt(0x0F70 | 8); break;               // vmcnt(8)
    case 2: __builtin_amdgcn_s_waitcnt(0x0F70 | (1 << 14)); break;       // vmcnt(16)
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | 8 | (1 << 14)); break;  // vmcnt(24)
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

}  // namespace

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

// V^T fragment: two transpose reads (keys +0 and +16 of the fragment's row).
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

template <int G, int NST>
__global__ __launch_bounds__(256) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int Hq,
    int Hkv, int n_q, int64_t kv_cap, int64_t kv_len, int K, int dense_thr, int mode,
    float scale_log2, int ntile, int umax, int nstage) {
  constexpr int KS = kD / 32;          // k-steps over D for S
  constexpr int DT = kD / 16;          // 16-wide d tiles of O
  constexpr int TPS = 16 / G;          // tokens per sub-tile
  constexpr int TPW = NST * TPS;       // tokens per wavefront
  constexpr int TQ = 4 * TPW;          // tokens per workgroup
  static_assert(TQ <= 64, "token masks are 64-bit");
  constexpr float kRescale = 8.f;      // log2 headroom before the running max is moved

  extern __shared__ __align__(16) char smem[];
  char* ring = smem;                                                            // [nstage]
  uint64_t* u_mask = reinterpret_cast<uint64_t*>(smem + nstage * kStageBytes);  // [umax]
  int32_t* u_blk = reinterpret_cast<int32_t*>(u_mask + umax);                   // [umax]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(u_blk + umax);                 // [256]
  int32_t* wbase = reinterpret_cast<int32_t*>(bitmap + 256);                    // [256]
  int32_t* wtot = wbase + 256;                                                  // [4]

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id();
  const int r16 = l % 16, kg = l / 16;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = item % ntile;
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
  const uint16_t* kbase = k + int64_t(bg) * kv_cap * kD;
  const uint16_t* vbase = v + int64_t(bg) * kv_cap * kD;

  // Q fragments (B operand of S^T = K Q^T), loaded first so their latency
  // overlaps the union construction.
  bf16x8 qf[NST][KS];
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int t = tok0 + w * TPW + s * TPS + r16 / G;
    const int h = g * G + r16 % G;
    const uint16_t* qrow = q + ((int64_t(b) * Hq + h) * n_q + (t < n_q ? t : 0)) * kD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[s][ks] = as_bf16x8(ldg16_if(t < n_q, qrow + ks * 32 + kg * 8));
  }

  // Tokens of this tile attending block j through their own block or a dense prefix.
  auto range_mask = [&](int64_t j) -> uint64_t {
    if (mode == 2) return range_bits(0, ntok, ntok);
    const int64_t lo = j * kBlock - base;
    return range_bits(lo, max(lo + kBlock, dend), ntok);
  };

  // ---------------------------------------------------------------- 1. union
  int U;
  if (tile_dense) {
    U = int(own_hi) + 1;
  } else {
    const int nwords = int(own_hi / 32) + 1;    // <= 256, checked on the host
    const int64_t rlo = dend > 0 ? 0 : own_lo;  // range part: [rlo, own_hi]
    if (tid < nwords) {
      const int64_t w0 = int64_t(tid) * 32;
      bitmap[tid] = uint32_t(range_bits(rlo - w0, own_hi + 1 - w0, 32));
    }
    __syncthreads();
    for (int e = tid; e < ntok * K; e += 256) {
      const int t = e / K;
      if (t < dend) continue;
      const int j = idx[(int64_t(bg) * n_q + tok0 + t) * K + e % K];
      if (j >= 0 && j < (base + t) / kBlock) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    // exclusive prefix of the words' popcounts, then compaction
    const int c = tid < nwords ? __popc(bitmap[tid]) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (l >= o) incl += y;
    }
    if (l == kWave - 1) wtot[w] = incl;
    __syncthreads();
    int before = 0;
    for (int x = 0; x < w; ++x) before += wtot[x];
    U = min(wtot[0] + wtot[1] + wtot[2] + wtot[3], umax);
    if (tid < nwords) {
      const int ex = before + incl - c;
      wbase[tid] = ex;
      uint32_t bits = bitmap[tid];
      int pos = ex;
      while (bits) {
        const int j = tid * 32 + __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < umax) {
          u_blk[pos] = j;
          u_mask[pos] = range_mask(j);
        }
        ++pos;
      }
    }
    __syncthreads();
    for (int e = tid; e < ntok * K; e += 256) {
      const int t = e / K;
      if (t < dend) continue;
      const int j = idx[(int64_t(bg) * n_q + tok0 + t) * K + e % K];
      if (j >= 0 && j < (base + t) / kBlock) {
        const int u = wbase[j >> 5] + __popc(bitmap[j >> 5] & ((1u << (j & 31)) - 1u));
        if (u < umax) atomicOr(reinterpret_cast<unsigned long long*>(&u_mask[u]), 1ull << t);
      }
    }
    __syncthreads();
  }
  U = __builtin_amdgcn_readfirstlane(U);
  auto blk_of = [&](int u) -> int64_t {
    return tile_dense ? int64_t(u) : int64_t(__builtin_amdgcn_readfirstlane(lds_read(u_blk + u)));
  };

  // ---------------------------------------------------------------- ring prologue
  for (int p = 0; p < nstage - 1 && p < U; ++p)
    issue_stage(ring + p * kStageBytes, kbase, vbase, blk_of(p) * kBlock, kv_len, w, l);

  f32x4 oacc[NST][DT];
  float m_run[NST], l_run[NST];
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    m_run[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[s][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // position of this lane's row in sub-tile s: base + w*TPW + s*TPS + r16/G
  const int64_t row_p0 = base + w * TPW + r16 / G;

  // lane parts of the fragment offsets (see the reads in the loop)
  const int k_lane = r16 * (kD * 2) + ((kg ^ swz(r16)) << 4);
  const int v_row = 4 * kg + r16 / 4;
  const int v_lane = v_row * (kD * 2) + ((((r16 % 4) >> 1) ^ swz(v_row)) << 4) + 8 * (r16 & 1);

  // ---------------------------------------------------------------- 2/3. ring + compute
  int cur = 0;                                    // ring slot of entry u
  int nxt = nstage - 1;                           // ring slot of entry u + nstage - 1
  for (int u = 0; u < U; ++u) {
    wait_stages_pending(min(nstage - 2, U - 1 - u));
    wait_lds();
    ring_barrier();                               // entry u landed for every wave; slot nxt is free
    if (u + nstage - 1 < U)
      issue_stage(ring + nxt * kStageBytes, kbase, vbase, blk_of(u + nstage - 1) * kBlock, kv_len,
                  w, l);
    const char* kt_b = ring + cur * kStageBytes;
    const lds_char* vt_b = (const lds_char*)(ring + cur * kStageBytes + kTileBytes);
    cur = cur + 1 == nstage ? 0 : cur + 1;
    nxt = nxt + 1 == nstage ? 0 : nxt + 1;
    const int64_t key0 = blk_of(u) * kBlock;
    uint64_t tmask;
    if (tile_dense) {
      tmask = range_mask(key0 / kBlock);
    } else {
      tmask = uniform_u64(lds_read(u_mask + u));
    }
    tmask >>= w * TPW;
    uint32_t son = 0;                             // sub-tiles holding a token that needs the block
#pragma unroll
    for (int s = 0; s < NST; ++s)
      if ((tmask >> (s * TPS)) & ((1ull << TPS) - 1ull)) son |= 1u << s;
    if (son == 0) continue;

    // S^T = K Q^T, 16 keys at a time: K fragment (kt, ks) of lane (r16, kg)
    // is row 16*kt + r16, piece 4*ks + kg; swz(row) = swz(r16), so its offset
    // is 4096*kt + (k_lane ^ (ks << 6)). Each fragment serves every active
    // sub-tile.
    f32x4 sacc[NST][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = lds_read_k(kt_b + kt * 4096, k_lane ^ (ks << 6));
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (son & (1u << s)) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = mfma16(kf[ks], qf[s][ks], a);
        }
        sacc[s][kt] = a;
      }
    }

    // Masked online softmax in the exp2 domain. A row whose token does not
    // need the block gets P = 0 through a -inf bias; only a block reaching past
    // a row's position (its own block, or keys beyond kv_len) is masked key by
    // key. The running max (log2 units) moves only when a row's block max
    // exceeds it by more than kRescale, so O and l are rescaled rarely;
    // exponents stay <= kRescale and the final O / l is unchanged.
    // P^T is packed as the B operand of the PV product: key slot (kg, jj)
    // holds key 32*k2 + 16*(jj/4) + 4*kg + jj%4.
    bf16x8 pf[NST][2];
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      if (!(son & (1u << s))) continue;
      const uint32_t bits = uint32_t(tmask >> (s * TPS)) & ((1u << TPS) - 1u);
      const bool row_on = (bits >> (r16 / G)) & 1u;
      const int64_t p_first = base + w * TPW + s * TPS;  // first token of the sub-tile
      const bool causal = mode == 2 ? key0 + kBlock > kv_len : key0 + kBlock - 1 > p_first;
      if (causal) {
        // last visible key of this row, block-relative
        const int64_t rel = (mode == 2 ? kv_len - 1 : row_p0 + s * TPS) - key0;
        const int lim = int(rel < 63 ? rel : 63);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sacc[s][kt][i] = (kt * 16 + kg * 4 + i <= lim) ? sacc[s][kt][i] : -INFINITY;
      }
      float mb = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mb = fmaxf(mb, sacc[s][kt][i]);
      mb = rows4_max(row_on ? mb : -INFINITY);
      const bool grow = mb * scale_log2 > m_run[s] + kRescale;
      if (ballot64(grow)) {
        const float m_new = mb * scale_log2;
        const float alpha = grow ? exp2f(m_run[s] - m_new) : 1.f;   // 0 on a row's first block
        if (grow) m_run[s] = m_new;
        l_run[s] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[s][dt][i] *= alpha;
      }
      // exp2 argument <= kRescale; results below 2^-126 flush to zero
      const float bias = !row_on ? -INFINITY : (m_run[s] == -INFINITY ? 0.f : -m_run[s]);
      float ps = 0.f;
      float pv[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[s][kt][i], scale_log2, bias));
          pv[kt][i] = e;
          ps += e;
        }
      l_run[s] += rows4_sum(ps);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint4 uu;
        uu.x = cvt_pk_bf16(pv[2 * k2][0], pv[2 * k2][1]);
        uu.y = cvt_pk_bf16(pv[2 * k2][2], pv[2 * k2][3]);
        uu.z = cvt_pk_bf16(pv[2 * k2 + 1][0], pv[2 * k2 + 1][1]);
        uu.w = cvt_pk_bf16(pv[2 * k2 + 1][2], pv[2 * k2 + 1][3]);
        pf[s][k2] = as_bf16x8(uu);
      }
    }

    // O^T += V^T P^T. In a transpose read each 16-lane group returns, to lane
    // j, element j%4 of the 8-byte chunks addressed by lanes j/4 + 4*i
    // (i = 0..3); pointing lane k of group kg at
    // V[32*k2 + 16*hh + 4*kg + k/4][16*dt + 4*(k%4)] thus hands lane j the V^T
    // entries (d = 16*dt + j, keys 32*k2 + 16*hh + 4*kg + i), matching P^T's key
    // slots. The swizzle of those rows depends on the lane only, so the offset
    // is 8192*k2 + 4096*hh + (v_lane ^ (dt << 5)).
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 vf = lds_read_vt(vt_b + k2 * 8192, v_lane ^ (dt << 5), (v_lane ^ (dt << 5)) + 4096);
#pragma unroll
        for (int s = 0; s < NST; ++s)
          if (son & (1u << s)) oacc[s][dt] = mfma16(vf, pf[s][k2], oacc[s][dt]);
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int t = tok0 + w * TPW + s * TPS + r16 / G;
    if (t >= n_q) continue;
    const int h = g * G + r16 % G;
    const float inv = l_run[s] > 0.f ? 1.f / l_run[s] : 0.f;
    uint16_t* dst = out + ((int64_t(b) * Hq + h) * n_q + t) * kD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint2 uu;
      uu.x = cvt_pk_bf16(oacc[s][dt][0] * inv, oacc[s][dt][1] * inv);
      uu.y = cvt_pk_bf16(oacc[s][dt][2] * inv, oacc[s][dt][3] * inv);
      *reinterpret_cast<uint2*>(dst + dt * 16 + kg * 4) = uu;
    }
    if (lse && kg == 0)
      lse[(int64_t(b) * Hq + h) * n_q + t] = (m_run[s] + log2f(l_run[s])) * 0.69314718055994531f;
  }
}

namespace {

int prefill_nst(int G) { return G == 1 ? 1 : 2; }

int prefill_tq(int G) { return 4 * prefill_nst(G) * (16 / G); }

// Largest number of union entries one tile can list (tiles whose tokens are
// all dense list none): the selected blocks of TQ tokens plus at most 2 own
// blocks; or, for the tile holding the dense threshold, every block up to its
// last own block.
int64_t prefill_umax(const Dims& d, int mode, int64_t nb) {
  if (mode != 0) return 0;
  const int tq = prefill_tq(d.G);
  const int64_t sparse = int64_t(tq) * d.K + 2;
  const int64_t mixed = d.dense_thr > 0 ? (int64_t(d.dense_thr) + tq) / kBlock + 2 : 0;
  return std::min(nb, std::max(sparse, mixed));
}

size_t prefill_lds(int nstage, int64_t umax) {
  return size_t(nstage) * kStageBytes + size_t(umax) * 12 + 512 * 4 + 16;
}

}  // namespace

int prefill128_stages(const Dims& d, int mode, int64_t kv_len) {
  if (d.D != 128) return 0;
  const int64_t nb = (kv_len - 1) / kBlock + 1;
  if (nb > 256 * 32) return 0;
  const int64_t umax = prefill_umax(d, mode, nb);
  for (int ns = 4; ns >= 2; --ns)
    if (prefill_lds(ns, umax) <= 160 * 1024) return ns;
  return 0;
}

template <int G, int NST>
static hipError_t launch_prefill_t(const Dims& d, int mode, const uint16_t* q, int n_q,
                                   const uint16_t* k, const uint16_t* v, int64_t kv_cap,
                                   int64_t kv_len, const int32_t* idx, uint16_t* out, float* lse,
                                   hipStream_t s) {
  constexpr int TQ = 4 * NST * (16 / G);
  const int ntile = (n_q + TQ - 1) / TQ;
  const int64_t nb = (kv_len - 1) / kBlock + 1;
  const int nstage = prefill128_stages(d, mode, kv_len);
  if (nstage == 0) return hipErrorInvalidValue;
  const int64_t umax = prefill_umax(d, mode, nb);
  auto kern = prefill_attn_kernel<G, NST>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     160 * 1024);
  if (attr != hipSuccess) return attr;
  const dim3 grid(unsigned(int64_t(d.B) * d.Hkv * ntile));
  kern<<<grid, 256, prefill_lds(nstage, umax), s>>>(
      q, k, v, idx, out, lse, d.Hq, d.Hkv, n_q, kv_cap, kv_len, d.K, d.dense_thr, mode,
      d.scale * 1.4426950408889634f, ntile, int(umax), nstage);
  return hipGetLastError();
}

hipError_t launch_prefill128(const Dims& d, int mode, const uint16_t* q, int n_q,
                             const uint16_t* k, const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                             const int32_t* idx, uint16_t* out, float* lse, hipStream_t s) {
  switch (d.G) {
    case 1: return launch_prefill_t<1, 1>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s);
    case 2: return launch_prefill_t<2, 2>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s);
    case 4: return launch_prefill_t<4, 2>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s);
    case 8: return launch_prefill_t<8, 2>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s);
    case 16: return launch_prefill_t<16, 2>(d, mode, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace infllmv2
