// Sparse attention of a few new tokens against a long KV cache: decode steps
// and draft-tree verification. (MiniCPM4 technical-report summary, QbitAI
// repost, section "Model architecture: InfLLM v2": sparse attention speeds up
// decoding too, and the blocks read per token stay constant as the context
// grows; section on fusing speculative sampling with long-context algorithms:
// the sparse kernel verifies tree drafts through a local mask kept as bits.)
//
// HBM-bound: per (b, g) the kernel reads each needed 64-key block of K and V
// once (64*D*2*2 bytes) and serves all n_q*G query rows of the group with it.
// The blocks of the union are split across workgroups (flash-decoding style);
// each writes an unnormalized partial (m, l, O) per row, and a combine kernel
// merges the partials by log-sum-exp.
//
//   union (n_q > 1 only): per (b, g), the ascending list of blocks any row
//     needs, each with a bitmask of the rows (tokens) that need it;
//   split: one workgroup per (b, g, split of SB union entries), one wavefront
//     per entry, so every entry's loads are in flight together. K fragments go
//     from HBM straight into MFMA registers (A operand of S^T = K Q^T); V goes
//     through LDS (A operand of O^T = V^T P^T). The wavefronts' partials merge
//     in LDS; a workgroup covering all of a group's entries writes the output
//     itself, otherwise one partial per split is stored;
//   combine (more than one split): one wavefront per (b, h, row).
//
// Single-token decode can also take the block scores instead of the block
// list (SKPL > 0): wavefront 0 of every split workgroup selects the group's
// top-K from the score row (the wavefront top-K of topk_select.hpp; the other
// splits of the group repeat the same selection) and the entries follow. This
// saves the separate selection kernel and its round trip.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "topk_select.hpp"

namespace infllmv2 {

namespace {

constexpr int kMaxWaves = 9;    // one 16-row sub-tile per wavefront (<= 170 registers)
constexpr int kMaxWaves2 = 4;   // two sub-tiles per wavefront

struct DecodeLayout {
  int64_t bgs, max_e, nsplit, rows, sb;
  size_t off_union, off_mask, off_count, off_ml, off_o, total;
};

// varlen: single-token rows of sequences with lengths up to kv_len, any of
// which may be below the dense threshold.
DecodeLayout decode_layout(const Dims& d, int n_q, int64_t kv_len, bool varlen = false) {
  DecodeLayout L{};
  L.bgs = int64_t(d.B) * d.Hkv;
  const int64_t P = kv_len - n_q;
  const int64_t last_blk = (kv_len - 1) / kBlock;
  const bool maybe_dense = d.dense_thr > 0 && P + 1 < d.dense_thr;
  if (n_q == 1 && varlen) {
    const int64_t dense_e = d.dense_thr > 1 ? (int64_t(d.dense_thr) - 2) / kBlock + 1 : 0;
    L.max_e = std::max<int64_t>(int64_t(d.K) + 1, std::min(last_blk + 1, dense_e));
  } else if (n_q == 1) {
    L.max_e = maybe_dense ? last_blk + 1 : int64_t(d.K) + 1;
  } else {
    const int64_t local = last_blk - P / kBlock + 1;
    L.max_e = maybe_dense ? last_blk + 1 : std::min(last_blk + 1, int64_t(n_q) * d.K + local);
  }
  // entries per split (= wavefronts per workgroup): about one workgroup per CU
  // for the whole step, at most kMaxWaves (their V tiles share 160 KB of LDS),
  // at least 3: a small step (one sequence) is latency-bound, and fewer, wider
  // splits shorten the selection each split repeats and the merge (32K, one
  // sequence: 21.9 -> 18.9 us per step)
  L.rows = int64_t(n_q) * d.G;
  const int maxw = L.rows > 16 ? kMaxWaves2 : kMaxWaves;
  L.sb = std::min<int64_t>(maxw, std::max<int64_t>(3, (L.bgs * L.max_e + 255) / 256));
  L.nsplit = (L.max_e + L.sb - 1) / L.sb;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  L.off_union = off;
  off = al(off + (n_q > 1 ? size_t(L.bgs * L.max_e) * 4 : 0));
  L.off_mask = off;
  off = al(off + (n_q > 1 ? size_t(L.bgs * L.max_e) * 8 : 0));
  L.off_count = off;
  off = al(off + size_t(L.bgs) * 4);
  L.off_ml = off;
  off = al(off + size_t(L.bgs * L.nsplit * L.rows) * 2 * 4);
  L.off_o = off;
  off = al(off + size_t(L.bgs * L.nsplit * L.rows) * d.D * 4);
  L.total = off;
  return L;
}

}  // namespace

// ------------------------------------------------------------------ union
__global__ __launch_bounds__(256) void decode_union_kernel(
    const int32_t* __restrict__ idx, const uint64_t* __restrict__ tree_mask,
    int32_t* __restrict__ u_blk, uint64_t* __restrict__ u_mask, int32_t* __restrict__ u_count,
    int Hkv, int n_q, int K, int64_t kv_len, int is_tree, int dense_thr, int64_t max_e) {
  extern __shared__ uint64_t nm[];          // [last_blk + 1] row masks per block
  __shared__ int s_cnt[4];
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int tid = threadIdx.x;
  const int64_t P = kv_len - n_q;
  const int nb = int((kv_len - 1) / kBlock) + 1;
  // the first index entries are loaded before the row masks are cleared, so
  // their latency overlaps the clearing and its barrier
  constexpr int kPre = 4;
  const int ne = n_q * K;
  int jpre[kPre];
#pragma unroll
  for (int x = 0; x < kPre; ++x) {
    const int e = tid + x * 256;
    jpre[x] = e < ne ? idx[int64_t(bg) * ne + e] : -1;
  }
  for (int j = tid; j < nb; j += 256) nm[j] = 0ull;
  __syncthreads();
  for (int e = tid; e < ne; e += 256) {
    const int i = e / K;
    const int64_t own = (is_tree ? P : P + i) / kBlock;
    const int x = (e - tid) / 256;
    const int j = x < kPre ? jpre[x < kPre ? x : 0] : idx[int64_t(bg) * ne + e];
    if (j >= 0 && j < own) atomicOr(reinterpret_cast<unsigned long long*>(&nm[j]), 1ull << i);
  }
  for (int i = tid; i < n_q; i += 256) {
    const int64_t own = (is_tree ? P : P + i) / kBlock;
    bool dense;
    if (is_tree) {
      dense = dense_thr > 0 && P + __popcll(tree_mask[int64_t(b) * n_q + i]) < dense_thr;
    } else {
      dense = dense_thr > 0 && P + i + 1 < dense_thr;
      atomicOr(reinterpret_cast<unsigned long long*>(&nm[own]), 1ull << i);
    }
    if (dense)
      for (int64_t j = 0; j < own; ++j) atomicOr(reinterpret_cast<unsigned long long*>(&nm[j]), 1ull << i);
  }
  if (is_tree) {
    const uint64_t all = n_q >= 64 ? ~0ull : ((1ull << n_q) - 1ull);
    for (int64_t j = P / kBlock + tid; j < nb; j += 256)
      atomicOr(reinterpret_cast<unsigned long long*>(&nm[j]), all);
  }
  __syncthreads();
  // ascending compaction: thread t scans blocks [t*per, (t+1)*per); offsets
  // from a DPP scan within each wavefront and the four wavefront totals
  const int per = (nb + 255) / 256;
  const int lo = min(nb, tid * per), hi = min(nb, lo + per);
  int c = 0;
  for (int j = lo; j < hi; ++j) c += nm[j] != 0ull;
  const int incl = int(wave_incl_scan_dpp(uint32_t(c)));
  const int wv = tid / kWave;
  if (lane_id() == kWave - 1) s_cnt[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    before += x < wv ? s_cnt[x] : 0;
    total += s_cnt[x];
  }
  int pos = before + incl - c;
  for (int j = lo; j < hi; ++j) {
    if (nm[j] != 0ull && pos < max_e) {
      u_blk[int64_t(bg) * max_e + pos] = j;
      u_mask[int64_t(bg) * max_e + pos] = nm[j];
      ++pos;
    }
  }
  if (tid == 255) u_count[bg] = min<int64_t>(total, max_e);
}

// ------------------------------------------------------------------ split
// V tile in LDS, row-major (64 keys x D), 16-byte pieces XOR-swizzled by key
// and filled straight from HBM (global_load_lds, 1 KB per wavefront
// instruction); rows past kv_len read zeros.
//   D = 128: piece p of row r holds V[r][8*(p ^ swz(r)) ..], swz(r) =
//     ((r & 7) << 1) | ((r >> 3) & 1). V^T fragments come from transpose reads
//     (ds_read_b64_tr_b16): each 16-lane group reads 4 consecutive rows x 2
//     adjacent pieces, which the swizzle spreads over distinct banks.
//   D = 64: piece p of row r holds V[r][8*(p ^ sw(r)) ..], sw(r) =
//     2*((r >> 2) & 3); a V^T element is one 2-byte read, and the four 16-lane
//     groups of a fragment read use keys 4 apart, which the swizzle sends to
//     distinct pieces.
__device__ __forceinline__ int vswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <int D>
__device__ __forceinline__ void load_v_tile(__amdgpu_buffer_rsrc_t rv, uint16_t* vt) {
  constexpr int PPR = D / 8;                 // 16-byte pieces per row
  constexpr int RPI = kWave / PPR;           // rows per 1 KB instruction
  const int l = lane_id();
#pragma unroll
  for (int x = 0; x < kBlock / RPI; ++x) {
    const int r = x * RPI + l / PPR;
    const int piece = l % PPR;
    const int sw = D == 128 ? vswz(r) : ((r >> 2) & 3) << 1;
    // nontemporal (cache policy 2): each selected block is read once per step
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (las_void*)(vt + x * RPI * D), 16,
                                             uint32_t(r * D * 2 + ((piece ^ sw) << 4)), 0, 0, 2);
  }
}

// The rows of block j (keys 64j .. 64j+63) below kv_len as a buffer resource:
// loads through it take 32-bit offsets below 16 KB whatever the context
// length, and rows past kv_len read zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* base, int64_t key0,
                                                             int64_t kv_len) {
  const int64_t live = kv_len - key0;
  const int rows = int(live < 0 ? 0 : (live > kBlock ? kBlock : live));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + key0 * D), 0, rows * D * 2,
                                           0x00020000);
}

typedef short dv4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dv4i16 lds_dv4i16;
typedef __attribute__((address_space(3))) char lds_dchar;

// V^T fragment of the 16x16x32 product (D = 128): two transpose reads, keys
// +0 and +16 of the fragment's row group. Each 16-lane group returns, to lane
// j, element j%4 of the 8-byte chunks addressed by lanes j/4 + 4*i; lane k of
// group kg points at V[32*k2 + 16*hh + 4*kg + k/4][16*dt + 4*(k%4)], so lane j
// receives V^T(d = 16*dt + j, keys 32*k2 + 16*hh + 4*kg + i), the P^T key slots.
__device__ __forceinline__ bf16x8 read_vt_tr(const uint16_t* vt, int off0, int off1) {
  const lds_dchar* base = (const lds_dchar*)vt;
  dv4i16 h[2];
  h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_dv4i16*)(base + off0));
  h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_dv4i16*)(base + off1));
  bf16x8 r;
  __builtin_memcpy(&r, h, sizeof r);
  return r;
}

template <int D, int NSTD, int SKPL>
__global__ __launch_bounds__(64 * (NSTD == 1 ? kMaxWaves : kMaxWaves2)) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const uint64_t* __restrict__ tree_mask,
    const int32_t* __restrict__ u_blk, const uint64_t* __restrict__ u_mask,
    const int32_t* __restrict__ u_count, float* __restrict__ part_ml, float* __restrict__ part_o,
    uint16_t* __restrict__ out, float* __restrict__ lse, int Hq, int Hkv, int G, int n_q,
    int64_t kv_cap, int64_t kv_len, int K, int dense_thr, int is_tree, int sb, int nsplit,
    int nsg, int max_e, int rows, float scale_log2, const float* __restrict__ scores, int64_t nblk,
    int32_t* __restrict__ idx_out, const int64_t* __restrict__ kv_lens) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int WR = 16 * NSTD;                       // rows of a workgroup
  extern __shared__ __align__(16) uint16_t dsm[];     // [waves][64*D]: V tile, then O partial
  __shared__ float2 s_ml[kMaxWaves][WR];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nwv = blockDim.x / kWave;
  // Waves past the split's entries (helpers of a wide selection) hold no
  // entry, no V tile and no partial.
  const int nwe = min(nwv, sb);
  uint16_t* vt = dsm + w * kBlock * D;
  const int l = lane_id();
  const int r16 = l % 16, kg = l / 16;
  // The grid holds nsg splits per (b, g) (nsg < nsplit only for multi-row
  // calls, whose union size is known on the device alone); a workgroup takes
  // splits split0, split0 + nsg, ... while they hold union entries.
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int split0 = item % nsg;
  const int bg = item / nsg;
  const int b = bg / Hkv, g = bg % Hkv;
  const int row0 = blockIdx.y * 16 * NSTD;
  // per-sequence length (single-token rows), kept within 1 .. the bound the
  // grid and workspace were sized for
  if (kv_lens) kv_len = min(max(kv_lens[b], int64_t(1)), kv_len);
  const int64_t P = kv_len - n_q;
  const uint16_t* kbase = k + int64_t(bg) * kv_cap * D;
  const uint16_t* vbase = v + int64_t(bg) * kv_cap * D;

  int n_e = 0;
  bool dense1 = false;
  int64_t own1 = 0;
  if (n_q == 1) {
    own1 = (kv_len - 1) / kBlock;
    dense1 = dense_thr > 0 && kv_len < dense_thr;
    n_e = dense1 ? int(own1) + 1 : K + 1;
  }
  // A multi-row call reads its union size and this wavefront's first entry
  // together (the entry, then its K and V, would otherwise be a third
  // dependent round trip). Vector loads (a lane offset the compiler cannot
  // see through): as scalar loads, the kernel's scalar register pressure had
  // them issued one after another, each waited for. The entry is clamped
  // into the union table's row.
  // (Two-sub-tile instances only: the single-sub-tile ones, at 168 registers,
  // spill with the entry held across the selection.)
  int32_t pre_j = 0;
  uint64_t pre_m = 0;
  const int u_pre = NSTD > 1 ? split0 * sb + w : -1;
  if (n_q > 1) {
    if constexpr (NSTD > 1) {
      int zo = 0;
      asm volatile("" : "+v"(zo));
      const int64_t e = int64_t(bg) * max_e + min(u_pre, max_e - 1) + zo;
      const int32_t cnt = u_count[bg + zo];
      pre_j = u_blk[e];
      pre_m = u_mask[e];
      n_e = __builtin_amdgcn_readfirstlane(cnt);
    } else {
      n_e = u_count[bg];
    }
  }
  // A multi-row call sizes its splits for the largest possible union, and its
  // combine reads only the splits that hold entries (u_count): a split past
  // the union has nothing to write. (Single-token rows keep every split: their
  // combine reads all of them.)
  if (n_q > 1 && nsplit > 1 && split0 * sb >= n_e) return;

  // block list of a single-token row selected here from its scores
  __shared__ int32_t s_sel[SKPL > 0 ? 64 : 1];
  if constexpr (SKPL > 0) {
    __shared__ uint32_t s_scr[2 * kWave];
    const int C = int(min(own1, nblk));           // (dense rows ignore the list; idx_out gets it)
    const float* row = scores + int64_t(bg) * nblk;
    const bool vec = (nblk & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    // Over more than 512 candidates the selection always runs on eight
    // wavefronts (the launch adds helpers): one wavefront holding 16+ keys
    // per lane next to the attention state spilled registers.
    bool many = false;
    if constexpr (SKPL >= 16) many = true;
    else if constexpr (SKPL >= 8) many = nwv >= 8;
    if constexpr (SKPL >= 8) {
      if (many) {                                 // eight wavefronts share the selection
        __shared__ WgTopkLds s_tk;
        wg_topk8<SKPL>(row, nblk, vec, C, K, s_sel, s_scr, s_tk);
      }
    }
    if (SKPL < 16 && !many && w == 0) {
      // lane l holds candidates SKPL*l .. SKPL*l + SKPL-1 (lane order = index order)
      const int jl = l * SKPL;
      float val[SKPL];
      bool done = false;
      if constexpr (SKPL >= 4) {
        if (vec) {
#pragma unroll
          for (int r = 0; r < SKPL; r += 4) {
            const int j = jl + r;
            const uint4 u = ldg16_or_neginf(j < nblk, row + (j < nblk ? j : 0));
            val[r] = __uint_as_float(u.x);
            val[r + 1] = __uint_as_float(u.y);
            val[r + 2] = __uint_as_float(u.z);
            val[r + 3] = __uint_as_float(u.w);
          }
          done = true;
        }
      }
      if (!done) {
#pragma unroll
        for (int r = 0; r < SKPL; ++r) val[r] = ldf_or_neginf(jl + r < nblk, row + jl + r);
      }
      wave_topk_lc<SKPL>(val, C, K, s_sel, s_scr);
    }
    lds_barrier();
    if (w == 0 && split0 == 0 && idx_out)
      for (int t = l; t < K; t += kWave) idx_out[int64_t(bg) * K + t] = s_sel[t];
  }

  // rows of this lane: sub-tile s, row r16 -> (node, head)
  int node_of[NSTD];
  uint64_t tmask[NSTD];
  bf16x8 qf[NSTD][KS];
#pragma unroll
  for (int s = 0; s < NSTD; ++s) {
    const int row = row0 + s * 16 + r16;
    const int node = row / G, hh = row % G;
    node_of[s] = node < n_q ? node : -1;
    tmask[s] = (is_tree && node < n_q) ? tree_mask[int64_t(b) * n_q + node] : 0ull;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint16_t* qrow = q + ((int64_t(b) * Hq + g * G + hh) * n_q + (node < n_q ? node : 0)) * D;
      qf[s][ks] = as_bf16x8(ldg16_if(node < n_q, qrow + ks * 32 + kg * 8));
    }
  }

  // (Only two-sub-tile instances loop: a loop around the single-sub-tile
  // kernels, which run nine wavefronts at 168 registers, makes them spill.)
  constexpr bool kLoop = NSTD > 1;
  for (int split = split0;; split += nsg) {
    const int u0 = split * sb;
    const int u1 = min(u0 + sb, n_e);
    f32x4 oacc[NSTD][DT];
    float m_run[NSTD], l_run[NSTD];
#pragma unroll
    for (int s = 0; s < NSTD; ++s) {
      m_run[s] = -INFINITY;
      l_run[s] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[s][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int u = u0 + w; u < u1; u += nwv) {
      int64_t j;
      uint64_t nmask;
      if (n_q == 1) {
        j = dense1 ? u : (u < K ? (SKPL > 0 ? s_sel[u] : idx[int64_t(bg) * K + u]) : own1);
        if (!dense1 && u < K && (j < 0 || j >= own1)) continue;
        nmask = 1ull;
      } else {
        if (u == u_pre) {
          j = pre_j;
          nmask = pre_m;
        } else {
          j = u_blk[int64_t(bg) * max_e + u];
          nmask = u_mask[int64_t(bg) * max_e + u];
        }
      }
      const int64_t key0 = int64_t(uniform_u64(uint64_t(j))) * kBlock;

      // K fragments straight from HBM (lane feeds key 16*kt + r16, d = 32*ks +
      // 8*kg .. +7; nontemporal), issued before the V tile: the products with
      // K wait for the K loads alone (the vector-memory counter is in order),
      // while V still arrives. A wave-uniform base at the block and 32-bit
      // lane offsets; rows are clamped into the cache (scores of keys past
      // kv_len are replaced by -inf in the softmax, whatever K holds there).
      bf16x8 kf[4][KS];
      {
        const uint16_t* kblk = kbase + key0 * D;
        const int rmax = int(min<int64_t>(kBlock - 1, kv_cap - 1 - key0));
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int row = min(kt * 16 + r16, rmax);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kf[kt][ks] = as_bf16x8(ldg16_nt(kblk + row * D + ks * 32 + kg * 8));
        }
      }
      // Every K load issues before the V tile's and before any product (left
      // free, the scheduler sinks them to their uses, one round trip each).
      __builtin_amdgcn_sched_barrier(0);
      wait_lds();                                    // previous block's V reads are done
      load_v_tile<D>(block_rsrc<D>(vbase, key0, kv_len), vt);   // V -> LDS, no registers
      __builtin_amdgcn_sched_barrier(0);

      bool sub_on[NSTD], row_on[NSTD];
#pragma unroll
      for (int s = 0; s < NSTD; ++s) {
        row_on[s] = node_of[s] >= 0 && ((nmask >> node_of[s]) & 1ull);
        sub_on[s] = ballot64(row_on[s]) != 0ull;
      }
      // S for every sub-tile, needed or not: with the products behind the
      // sub-tile test, the compiler moves the K loads into that branch and
      // issues them one at a time next to their uses.
      f32x4 sacc[NSTD][4];
#pragma unroll
      for (int s = 0; s < NSTD; ++s) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = mfma16(kf[kt][ks], qf[s][ks], a);
          sacc[s][kt] = a;
        }
      }
      bf16x8 pf[NSTD][2];
#pragma unroll
      for (int s = 0; s < NSTD; ++s) {
        if (!sub_on[s]) continue;
        const int node = node_of[s];
        const int64_t p_row = P + (node < 0 ? 0 : node);
        float mb = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t key = key0 + kt * 16 + kg * 4 + i;
            bool ok;
            if (is_tree)
              ok = key < P || (key < kv_len && ((tmask[s] >> (key - P)) & 1ull));
            else
              ok = key <= p_row;
            const float x = (row_on[s] && ok) ? sacc[s][kt][i] * scale_log2 : -INFINITY;
            sacc[s][kt][i] = x;
            mb = fmaxf(mb, x);
          }
        mb = rows4_max(mb);
        const float m_new = fmaxf(m_run[s], mb);
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.f : exp2f(m_run[s] - m_new);
        const float neg_m = none ? 0.f : -m_new;    // masked keys: exp2(-inf) = 0
        float ps = 0.f;
        float pv[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = __builtin_amdgcn_exp2f(sacc[s][kt][i] + neg_m);
            pv[kt][i] = e;
            ps += e;
          }
        ps = rows4_sum(ps);
        l_run[s] = l_run[s] * alpha + ps;
        m_run[s] = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[s][dt][i] *= alpha;
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
      wait_vmem();                                   // the V tile has landed in LDS
      if constexpr (D == 128) {
        // byte offset of lane (r16, kg)'s chunk for d tile 0, rows 4*kg + r16/4
        const int v_row = 4 * kg + r16 / 4;
        const int v_lane = v_row * (D * 2) + ((((r16 % 4) >> 1) ^ vswz(v_row)) << 4) + 8 * (r16 & 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int off = k2 * 32 * D * 2 + (v_lane ^ (dt << 5));
            const bf16x8 vf = read_vt_tr(vt, off, off + 16 * D * 2);
#pragma unroll
            for (int s = 0; s < NSTD; ++s) {
              if (!sub_on[s]) continue;
              oacc[s][dt] = mfma16(vf, pf[s][k2], oacc[s][dt]);
            }
          }
        }
      } else {
        const uint16_t* vlane = vt + 4 * kg * D + r16;  // key 4*kg, column r16 (swizzle applied per dt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* vcol = vlane + ((dt ^ kg) << 4);
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            // key slots (kg, jj): key = 32*k2 + 16*(jj/4) + 4*kg + jj%4, matching pf's packing
            uint32_t w4[4];
#pragma unroll
            for (int hp = 0; hp < 4; ++hp) {
              const int koff = 32 * k2 + 16 * (hp / 2) + 2 * (hp % 2);   // jj = 2*hp
              const uint32_t lo = vcol[koff * D];
              const uint32_t hi = vcol[(koff + 1) * D];
              w4[hp] = lo | (hi << 16);
            }
            const bf16x8 vf = as_bf16x8(uint4{w4[0], w4[1], w4[2], w4[3]});
#pragma unroll
            for (int s = 0; s < NSTD; ++s) {
              if (!sub_on[s]) continue;
              oacc[s][dt] = mfma16(vf, pf[s][k2], oacc[s][dt]);
            }
          }
        }
      }
    }

    // This wavefront's partial -> LDS: (m, l) per row, O (unnormalized, zeros
    // for rows that saw no key) in the wavefront's V tile, [row][D] fp32.
    wait_lds();
    float* o_s = reinterpret_cast<float*>(vt);
    if (w < nwe) {
#pragma unroll
      for (int s = 0; s < NSTD; ++s) {
        const int wr = s * 16 + r16;
        if (row0 + wr >= rows) continue;          // (the merge reads only the call's rows)
        if (kg == 0) s_ml[w][wr] = make_float2(m_run[s], l_run[s]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<float4*>(o_s + wr * D + dt * 16 + kg * 4) =
              make_float4(oacc[s][dt][0], oacc[s][dt][1], oacc[s][dt][2], oacc[s][dt][3]);
      }
    }
    __syncthreads();
    // Merge the wavefronts by log-sum-exp. A thread takes 4-column units (row
    // wr, columns c .. c+3) and issues all of a unit's LDS reads (every
    // wavefront's (m, l) and O values) before it uses any of them; the sums run
    // over the wavefronts in order.
    constexpr int MAXW = NSTD == 1 ? kMaxWaves : kMaxWaves2;
    constexpr int U4 = D / 4;
    const bool final = nsplit == 1;
    for (int unit = threadIdx.x; unit < WR * U4; unit += blockDim.x) {
      const int wr = unit / U4, c = (unit % U4) * 4;
      const int row = row0 + wr;
      if (row >= rows) continue;
      float2 ml[MAXW];
      f32x4 ov[MAXW];
#pragma unroll
      for (int x = 0; x < MAXW; ++x) {
        if (x < nwe) {
          ml[x] = s_ml[x][wr];
          ov[x] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(dsm + x * kBlock * D) + wr * D + c);
        }
      }
      float M = -INFINITY;
#pragma unroll
      for (int x = 0; x < MAXW; ++x)
        if (x < nwe) M = fmaxf(M, ml[x].x);
      float Lsum = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < MAXW; ++x) {
        if (x < nwe) {
          const float wgt = ml[x].x == -INFINITY ? 0.f : exp2f(ml[x].x - M);
          Lsum += wgt * ml[x].y;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += wgt * ov[x][i];
        }
      }
      if (final) {
        const int node = row / G, hh = row % G;
        const int64_t rid = (int64_t(b) * Hq + g * G + hh) * n_q + node;
        uint2 uu;
        uu.x = uint32_t(f2bf(Lsum > 0.f ? acc[0] / Lsum : 0.f)) | (uint32_t(f2bf(Lsum > 0.f ? acc[1] / Lsum : 0.f)) << 16);
        uu.y = uint32_t(f2bf(Lsum > 0.f ? acc[2] / Lsum : 0.f)) | (uint32_t(f2bf(Lsum > 0.f ? acc[3] / Lsum : 0.f)) << 16);
        *reinterpret_cast<uint2*>(out + rid * D + c) = uu;
        if (lse && c == 0) lse[rid] = (M + log2f(Lsum)) * 0.69314718055994531f;
      } else {
        // partials: ml[bg][split][row] = (m, l); o[bg][split][row][d] (unnormalized)
        const int64_t pr = (int64_t(bg) * nsplit + split) * rows + row;
        *reinterpret_cast<f32x4*>(part_o + pr * D + c) = acc;
        if (c == 0) {
          part_ml[pr * 2 + 0] = M;
          part_ml[pr * 2 + 1] = Lsum;
        }
      }
    }
    if (!kLoop || split + nsg >= nsplit || (split + nsg) * sb >= n_e) break;
    __syncthreads();                              // the next split reuses the LDS
  }
}

// ------------------------------------------------------------------ combine
// One wavefront per output row (b, h, i), in two round trips: lanes over splits
// read every split's (m, l), then every lane issues the loads of its D/64
// columns for all splits of the chunk before using any of them.
template <int D, int CH>
__device__ __forceinline__ void combine_chunks(const float* __restrict__ part_ml,
                                               const float* __restrict__ part_o, int64_t pr0,
                                               int rows, int ns, float& M, float& L,
                                               float (&acc)[D / kWave]) {
  constexpr int CPL = D / kWave;
  const int l = lane_id();
  for (int s0 = 0; s0 < ns; s0 += CH) {
    const int s = s0 + (l % CH);
    const float* ml = part_ml + (pr0 + int64_t(s) * rows) * 2;
    const float ms = l < CH ? ldf_or_neginf(s < ns, ml) : -INFINITY;
    const float ls = l < CH ? ldf_or_zero(s < ns, ml + 1) : 0.f;
    float o[CH][CPL];                          // this lane's columns of every split in the chunk
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const bool ok = s0 + t < ns;
      const float* src = part_o + (pr0 + int64_t(s0 + t) * rows) * D + CPL * l;
#pragma unroll
      for (int x = 0; x < CPL; ++x) o[t][x] = ldf_or_zero(ok, src + x);
    }
    __builtin_amdgcn_sched_barrier(0);         // all loads of the chunk are in flight
    const float m_new = fmaxf(M, xor_max<kWave>(ms));
    const float a = M == -INFINITY ? 0.f : exp2f(M - m_new);
    const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - m_new);   // 0 where the row saw no key
    L = L * a + xor_sum<kWave>(wgt * ls);
#pragma unroll
    for (int x = 0; x < CPL; ++x) acc[x] *= a;
    M = m_new;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const float wt = __shfl(wgt, t);
#pragma unroll
      for (int x = 0; x < CPL; ++x) acc[x] += wt * o[t][x];
    }
  }
}

// CH = 8: every row has at most 8 splits. CH = 64: a row's splits go in chunks
// of 16 while it has at most 16 (a multi-row call's union usually fills a few
// of the splits the grid was sized for; loads of empty slots still cost an
// instruction each), else in chunks of 64.
template <int D, int CH>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const int32_t* __restrict__ u_count, uint16_t* __restrict__ out, float* __restrict__ lse,
    int Hq, int Hkv, int G, int n_q, int nsplit, int sb, int n_e1, int rows, int64_t nrows) {
  constexpr int CPL = D / kWave;
  const int l = lane_id();
  // (b, h, i); workgroups numbered like the split kernel's, so a row's partials
  // are read on the XCD that wrote them (they still arrive at last-level-cache
  // latency across the kernel boundary)
  const int64_t rid = int64_t(xcd_remap(blockIdx.x, gridDim.x)) * 4 + threadIdx.x / kWave;
  if (rid >= nrows) return;
  const int i = int(rid % n_q);
  const int h = int((rid / n_q) % Hq);
  const int b = int(rid / (int64_t(n_q) * Hq));
  const int g = h / G;
  const int bg = b * Hkv + g;
  const int row = i * G + h % G;
  const int n_e = n_q == 1 ? n_e1 : u_count[bg];
  const int ns = min(nsplit, (n_e + sb - 1) / sb);
  const int64_t pr0 = int64_t(bg) * nsplit * rows + row;   // split s at pr0 + s * rows
  float M = -INFINITY, L = 0.f;
  float acc[CPL];
#pragma unroll
  for (int x = 0; x < CPL; ++x) acc[x] = 0.f;
  if (CH > 16 && ns <= 16)
    combine_chunks<D, 16>(part_ml, part_o, pr0, rows, ns, M, L, acc);
  else
    combine_chunks<D, CH>(part_ml, part_o, pr0, rows, ns, M, L, acc);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = out + rid * D + CPL * l;
#pragma unroll
  for (int x = 0; x < CPL; ++x) dst[x] = f2bf(acc[x] * inv);
  if (lse && l == 0) lse[rid] = (M + log2f(L)) * 0.69314718055994531f;
}

size_t decode_workspace_bytes(const Dims& d, int n_q, int64_t kv_len) {
  return decode_layout(d, n_q, kv_len).total;
}

// Scratch memory of the allocation-free single-token decode entry point: the
// split partials it would otherwise keep in a caller's workspace. One copy per
// GPU, allocated by the loader with the code object and held until the
// process ends. Host code never passes this array's name to a kernel (on the
// host it only stands for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kDecodeNoAllocScratchBytes];

hipError_t decode_noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_varlen_workspace_bytes(const Dims& d, int64_t kv_len_max) {
  return decode_layout(d, 1, kv_len_max, true).total;
}

hipError_t launch_decode(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                         const uint16_t* v, int64_t kv_cap, int64_t kv_len, const int32_t* idx,
                         const uint64_t* tree_mask, uint16_t* out, float* lse, void* ws,
                         size_t ws_bytes, hipStream_t s, const float* scores, int32_t* idx_out,
                         const int64_t* kv_lens) {
  if (kv_lens && n_q != 1) return hipErrorInvalidValue;
  const DecodeLayout L = decode_layout(d, n_q, kv_len, kv_lens != nullptr);
  if (ws_bytes < L.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  int32_t* u_blk = reinterpret_cast<int32_t*>(base + L.off_union);
  uint64_t* u_mask = reinterpret_cast<uint64_t*>(base + L.off_mask);
  int32_t* u_count = reinterpret_cast<int32_t*>(base + L.off_count);
  float* part_ml = reinterpret_cast<float*>(base + L.off_ml);
  float* part_o = reinterpret_cast<float*>(base + L.off_o);
  const int is_tree = tree_mask != nullptr;
  const int sb = int(L.sb);
  if (n_q > 1) {
    const int nb = int((kv_len - 1) / kBlock) + 1;
    const size_t lds = size_t(nb) * 8;
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    decode_union_kernel<<<dim3(unsigned(L.bgs)), 256, lds, s>>>(
        idx, tree_mask, u_blk, u_mask, u_count, d.Hkv, n_q, d.K, kv_len, is_tree, d.dense_thr,
        L.max_e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rows = n_q * d.G;
  const int nstd_total = (rows + 15) / 16;
  const int nstd = nstd_total >= 2 ? 2 : nstd_total;
  const unsigned ygroups = unsigned((nstd_total + nstd - 1) / nstd);
  // Multi-row calls of two sub-tiles: splits for a union of about 2(K+1)
  // blocks plus the rows' own blocks (a tree's nodes mostly agree) or, for
  // dense rows, the whole range; a larger union is walked by the same
  // workgroups in turn. (Single-token calls keep every split: their combine
  // reads all of them, entries or not.)
  int nsg = int(L.nsplit);
  if (n_q > 1 && nstd > 1 && !(d.dense_thr > 0 && kv_len - n_q + 1 < d.dense_thr)) {
    const int64_t e_typ = 2 * (int64_t(d.K) + 1) + (n_q + kBlock - 1) / kBlock + 1;
    nsg = int(std::min<int64_t>(L.nsplit, (e_typ + sb - 1) / sb));
  }
  const dim3 grid(unsigned(L.bgs * nsg), ygroups);
  const float sl2 = d.scale * 1.4426950408889634f;
  const int n_e1 = int(L.max_e);
  const int64_t nblk = (kv_cap + kBlock - 1) / kBlock;
  int skpl = 0;                                   // keys per lane of the in-kernel selection
  if (scores) {
    const int64_t c = std::min((kv_len - 1) / kBlock, nblk);
    skpl = 1;
    while (int64_t(skpl) * kWave < c) skpl <<= 1;
  }
  // Wavefronts per workgroup: one per entry, and at least eight when the
  // in-kernel selection needs them (more than 512 candidates); helpers take
  // no entry and no LDS tile.
  const int nwv = skpl >= 16 ? std::max(sb, 8) : sb;
#define SPLIT_CASE(DD, NN, SK)                                                                    \
  if (d.D == DD && nstd == NN && skpl == SK) {                                                    \
    auto kern = decode_split_kernel<DD, NN, SK>;                                                  \
    static const hipError_t attr = hipFuncSetAttribute(                                           \
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,          \
        (NN == 1 ? kMaxWaves : kMaxWaves2) * kBlock * DD * 2);                                    \
    if (attr != hipSuccess) return attr;                                                          \
    kern<<<grid, 64 * nwv, size_t(sb) * kBlock * DD * 2, s>>>(                                    \
        q, k, v, idx, tree_mask, u_blk, u_mask, u_count, part_ml, part_o, out, lse, d.Hq, d.Hkv,  \
        d.G, n_q, kv_cap, kv_len, d.K, d.dense_thr, is_tree, sb, int(L.nsplit), nsg, int(L.max_e), \
        int(L.rows), sl2, scores, nblk, idx_out, kv_lens);                                        \
  } else
#define SPLIT_SEL(DD)                                                                             \
  SPLIT_CASE(DD, 1, 1) SPLIT_CASE(DD, 1, 2) SPLIT_CASE(DD, 1, 4) SPLIT_CASE(DD, 1, 8)            \
  SPLIT_CASE(DD, 1, 16) SPLIT_CASE(DD, 1, 32) SPLIT_CASE(DD, 1, 64)
  SPLIT_CASE(128, 1, 0) SPLIT_CASE(128, 2, 0) SPLIT_CASE(64, 1, 0) SPLIT_CASE(64, 2, 0)
  SPLIT_SEL(128) SPLIT_SEL(64)
  { return hipErrorInvalidValue; }
#undef SPLIT_SEL
#undef SPLIT_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (L.nsplit == 1) return hipSuccess;        // the split kernel wrote the output
  const int64_t nrows = int64_t(d.B) * d.Hq * n_q;
  const dim3 cgrid(unsigned((nrows + 3) / 4));
#define COMBINE_CASE(DD, CC)                                                                      \
  decode_combine_kernel<DD, CC><<<cgrid, 256, 0, s>>>(part_ml, part_o, u_count, out, lse, d.Hq,    \
                                                      d.Hkv, d.G, n_q, int(L.nsplit), sb, n_e1,  \
                                                      int(L.rows), nrows)
  const bool few = L.nsplit <= 8;
  if (d.D == 128) {
    if (few) COMBINE_CASE(128, 8); else COMBINE_CASE(128, 64);
  } else {
    if (few) COMBINE_CASE(64, 8); else COMBINE_CASE(64, 64);
  }
#undef COMBINE_CASE
  return hipGetLastError();
}

}  // namespace infllmv2
