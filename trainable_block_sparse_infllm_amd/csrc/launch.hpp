// Internal launchers: one per kernel family. The C ABI layer (api.cpp) checks
// arguments and picks template instances; these functions only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infllmv2 {

struct Dims {
  int B, Hq, Hkv, G, D, K, dense_thr;
  float scale;
};

// Blocks first..last-1 of every sequence.
hipError_t launch_pool(const Dims& d, const uint16_t* k, int64_t kv_cap, int64_t nblk,
                       int64_t first, int64_t last, uint16_t* kbar, hipStream_t s);

// Cache append of n_new tokens at each sequence's length (lens[b], or kv_len
// when lens is null), and pooling of the blocks it completes (kbar != null),
// in one launch.
hipError_t launch_append(const Dims& d, const uint16_t* k_new, const uint16_t* v_new,
                         int64_t n_new, uint16_t* k_cache, uint16_t* v_cache, int64_t kv_cap,
                         const int64_t* lens, int64_t kv_len, uint16_t* kbar, hipStream_t s);

// kv_lens (device, [B], single-token non-tree rows only): sequence b's new
// token sits at kv_lens[b] - 1 instead of q_pos0.
hipError_t launch_scores(const Dims& d, const uint16_t* q, int n_q, int64_t q_pos0, int is_tree,
                         const uint16_t* kbar, int64_t nblk, float* scores, hipStream_t s,
                         const int64_t* kv_lens = nullptr);

// LSE-normalized block scores (same layout as launch_scores), through a
// workspace of score_lse_workspace_bytes().
size_t score_lse_workspace_bytes(const Dims& d, int n_q, int64_t nblk);
hipError_t launch_scores_lse(const Dims& d, const uint16_t* q, int n_q, int64_t q_pos0,
                             int is_tree, const uint16_t* kbar, int64_t nblk, float* scores,
                             void* ws, size_t ws_bytes, hipStream_t s);

hipError_t launch_topk_from_scores(const Dims& d, const float* scores, int n_q, int64_t q_pos0,
                                   int is_tree, int64_t nblk, int32_t* idx, hipStream_t s);

// Whether the fused score + top-K path runs rows with cmax candidates.
bool topk_fused_ok(const Dims& d, int64_t cmax);
hipError_t launch_topk_fused(const Dims& d, const uint16_t* q, const uint16_t* kbar, int n_q,
                             int64_t q_pos0, int is_tree, int64_t nblk, int32_t* idx, hipStream_t s);

// mode: 0 sparse (idx + dense threshold), 1 dense causal, 2 dense without mask,
// 3 sliding window (keys max(0, p - window + 1)..p).
hipError_t launch_attn_rows(const Dims& d, int mode, const uint16_t* q, int n_q, const uint16_t* k,
                            const uint16_t* v, int64_t kv_cap, int64_t kv_len, const int32_t* idx,
                            uint16_t* out, float* lse, hipStream_t s, int64_t window = 0);

// head_dim 128 fused scoring + top-K for prefill chunks (at most 512
// candidate blocks); topk_prefill128_ok() says whether it takes the shape.
bool topk_prefill128_ok(const Dims& d, int64_t cmax);
hipError_t launch_topk_prefill128(const Dims& d, const uint16_t* q, const uint16_t* kbar, int n_q,
                                  int64_t q_pos0, int is_tree, int64_t nblk, int64_t cmax,
                                  int32_t* idx, hipStream_t s);

// head_dim 128 prefill / dense / sliding-window attention over a per-tile
// block union staged through an LDS ring (mode 3: keys max(0, p-window+1)..p).
// prefill128_stages() returns the ring depth for the shape, or 0 if it does
// not fit (then launch_attn_rows runs the rows kernel).
int prefill128_stages(const Dims& d, int mode, int64_t kv_len);
hipError_t launch_prefill128(const Dims& d, int mode, const uint16_t* q, int n_q,
                             const uint16_t* k, const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                             const int32_t* idx, uint16_t* out, float* lse, hipStream_t s,
                             int64_t window = 0);

size_t decode_workspace_bytes(const Dims& d, int n_q, int64_t kv_len);

// scores != nullptr (single-token rows only): the block lists are selected in
// the kernel from scores [B][Hkv][1][nblk] (written to idx_out when given).
// kv_lens (device, [B], single-token rows only): per-sequence cache lengths,
// kv_len then bounds them (it sizes the grid and the workspace).
hipError_t launch_decode(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                         const uint16_t* v, int64_t kv_cap, int64_t kv_len, const int32_t* idx,
                         const uint64_t* tree_mask, uint16_t* out, float* lse, void* ws,
                         size_t ws_bytes, hipStream_t s, const float* scores = nullptr,
                         int32_t* idx_out = nullptr, const int64_t* kv_lens = nullptr);
size_t decode_varlen_workspace_bytes(const Dims& d, int64_t kv_len_max);

// The allocation-free single-token decode keeps its workspace in a static
// device array of this size (one per GPU); decode_noalloc_scratch() gives the
// current device's address of it (looked up once per device).
constexpr size_t kDecodeNoAllocScratchBytes = size_t(16) << 20;
hipError_t decode_noalloc_scratch(void** ptr);

// Backward of the head_dim-128 sparse prefill (mode 0): dq, dk, dv (fp32).
bool prefill_backward_ok(const Dims& d, int64_t kv_len);
size_t prefill_backward_workspace_bytes(const Dims& d, int n_q, int64_t kv_len);
hipError_t launch_prefill_backward(const Dims& d, const uint16_t* q, int n_q, const uint16_t* k,
                                   const uint16_t* v, int64_t kv_cap, int64_t kv_len,
                                   const int32_t* idx, const uint16_t* out, const float* lse,
                                   const uint16_t* dout, float* dq, float* dk, float* dv, void* ws,
                                   size_t ws_bytes, hipStream_t s);

}  // namespace infllmv2
