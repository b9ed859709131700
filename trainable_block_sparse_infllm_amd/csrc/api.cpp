// C ABI of the InfLLM v2 block-sparse attention library (declared in
// include/infllmv2.h): argument checks, device check, dispatch to launchers.
// Every check that can reject a call runs before the first HIP API call, so a
// rejected call enqueues nothing and is testable without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/infllmv2.h"
#include "launch.hpp"

using infllmv2::Dims;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fn, const char* msg) {
  g_last_error = std::string(fn) + ": " + msg;
  return status;
}

int fail_hip(const char* fn, hipError_t e) {
  g_last_error = std::string(fn) + ": HIP error: " + hipGetErrorString(e);
  return INFLLMV2_HIP_ERROR;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and support checks on the configuration; fills dims on success.
int check_cfg(const char* fn, const infllmv2_cfg* c, bool need_topk, Dims* d) {
  if (!c) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "cfg is NULL");
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1)
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "batch and head counts must be >= 1");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "n_q_heads must be a multiple of n_kv_heads");
  if (c->head_dim < 1) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "head_dim must be >= 1");
  if (c->block_size < 1 || c->kernel_size < 1 || c->kernel_stride < 1 ||
      c->kernel_size > c->block_size || (c->block_size - c->kernel_size) % c->kernel_stride)
    return fail(INFLLMV2_INVALID_ARGUMENT, fn,
                "block/kernel geometry: need 1 <= kernel_size <= block_size and "
                "(block_size - kernel_size) % kernel_stride == 0");
  if (need_topk && c->top_k < 1) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "top_k must be >= 1");
  if (c->dense_threshold < 0) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "dense_threshold must be >= 0");
  if (!(c->softmax_scale == c->softmax_scale) || std::isinf(c->softmax_scale))
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "softmax_scale must be finite");
  const int G = c->n_q_heads / c->n_kv_heads;
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(INFLLMV2_UNSUPPORTED, fn, "head_dim must be 64 or 128");
  if (c->block_size != 64 || c->kernel_size != 32 || c->kernel_stride != 16)
    return fail(INFLLMV2_UNSUPPORTED, fn, "only block 64 with kernels of 32 at stride 16");
  if (G > 16 || (16 % G))
    return fail(INFLLMV2_UNSUPPORTED, fn, "the GQA group size must divide 16");
  if (need_topk && c->top_k > 4096) return fail(INFLLMV2_UNSUPPORTED, fn, "top_k above 4096");
  d->B = c->batch;
  d->Hq = c->n_q_heads;
  d->Hkv = c->n_kv_heads;
  d->G = G;
  d->D = c->head_dim;
  d->K = c->top_k;
  d->dense_thr = c->dense_threshold;
  d->scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt(float(c->head_dim));
  return INFLLMV2_OK;
}

int check_ptr(const char* fn, const void* p, const char* name, uintptr_t align) {
  if (!p) return fail(INFLLMV2_INVALID_ARGUMENT, fn, (std::string(name) + " is NULL").c_str());
  if (!aligned(p, align))
    return fail(INFLLMV2_INVALID_ARGUMENT, fn,
                (std::string(name) + " is not " + std::to_string(align) + "-byte aligned").c_str());
  return INFLLMV2_OK;
}

int check_kv(const char* fn, int64_t kv_cap, int64_t kv_len) {
  if (kv_len < 1) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "kv_len must be >= 1");
  if (kv_cap < kv_len) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "kv_len exceeds kv_cap");
  if (kv_cap > (int64_t(1) << 31)) return fail(INFLLMV2_UNSUPPORTED, fn, "kv_cap above 2^31");
  return INFLLMV2_OK;
}

// Device check (first HIP call of an accepted request): gfx950 only.
int check_device(const char* fn) {
  static std::mutex mu;
  static int arch_ok[64] = {0};   // 0 unknown, 1 gfx950, -1 another device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(fn, e);
  if (dev < 0 || dev >= 64) return fail(INFLLMV2_UNSUPPORTED, fn, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(mu);
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail_hip(fn, e);
    arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (arch_ok[dev] < 0) return fail(INFLLMV2_UNSUPPORTED, fn, "device is not gfx950 (MI355X)");
  return INFLLMV2_OK;
}

#define TRY(x)                         \
  do {                                 \
    const int rc_ = (x);               \
    if (rc_ != INFLLMV2_OK) return rc_; \
  } while (0)

#define LAUNCH(fn, call)                       \
  do {                                         \
    const hipError_t e_ = (call);              \
    if (e_ != hipSuccess) return fail_hip(fn, e_); \
  } while (0)

int64_t nblk_of(int64_t kv_cap) { return (kv_cap + 63) / 64; }

}  // namespace

extern "C" {

int infllmv2_pool_kernels(const infllmv2_cfg* cfg, const void* k, int64_t kv_cap, int64_t kv_len,
                          int64_t first_block, void* kbar, void* stream) {
  const char* fn = "infllmv2_pool_kernels";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_ptr(fn, k, "k", 16));
  TRY(check_ptr(fn, kbar, "kbar", 16));
  TRY(check_kv(fn, kv_cap, kv_len));
  const int64_t last = kv_len / 64;
  if (first_block < 0 || first_block > last)
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "first_block must lie in [0, kv_len/64]");
  if (int64_t(d.B) * d.Hkv * (last - first_block) / 4 > INT32_MAX)
    return fail(INFLLMV2_UNSUPPORTED, fn, "too many blocks for one launch");
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_pool(d, static_cast<const uint16_t*>(k), kv_cap, nblk_of(kv_cap),
                                   first_block, last, static_cast<uint16_t*>(kbar),
                                   static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

static int check_rows(const char* fn, const Dims& d, int32_t n_q, int64_t q_pos0, int32_t is_tree,
                      int64_t kv_cap) {
  if (n_q < 1) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "n_q must be >= 1");
  if (q_pos0 < 0) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "q_pos0 must be >= 0");
  if (kv_cap < 1) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "kv_cap must be >= 1");
  if (kv_cap > (int64_t(1) << 31)) return fail(INFLLMV2_UNSUPPORTED, fn, "kv_cap above 2^31");
  const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + n_q - 1;
  if (pos_last / 64 > nblk_of(kv_cap))
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "query positions lie beyond kv_cap");
  if (is_tree && n_q > 64) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "a tree has at most 64 nodes");
  if (int64_t(d.B) * d.Hkv * n_q > INT32_MAX / 64)
    return fail(INFLLMV2_UNSUPPORTED, fn, "too many rows for one launch");
  return INFLLMV2_OK;
}

int infllmv2_score_blocks(const infllmv2_cfg* cfg, const void* q, int32_t n_q, int64_t q_pos0,
                          int32_t is_tree, const void* kbar, int64_t kv_cap, float* scores,
                          void* stream) {
  const char* fn = "infllmv2_score_blocks";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_ptr(fn, q, "q", 16));
  TRY(check_ptr(fn, kbar, "kbar", 16));
  TRY(check_ptr(fn, scores, "scores", 4));
  TRY(check_rows(fn, d, n_q, q_pos0, is_tree, kv_cap));
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_scores(d, static_cast<const uint16_t*>(q), n_q, q_pos0, is_tree != 0,
                                     static_cast<const uint16_t*>(kbar), nblk_of(kv_cap), scores,
                                     static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

size_t infllmv2_score_lse_workspace_bytes(const infllmv2_cfg* cfg, int32_t n_q, int64_t kv_cap) {
  Dims d;
  if (check_cfg("infllmv2_score_lse_workspace_bytes", cfg, false, &d) != INFLLMV2_OK) return 0;
  if (n_q < 1 || kv_cap < 1) return 0;
  return infllmv2::score_lse_workspace_bytes(d, n_q, nblk_of(kv_cap));
}

int infllmv2_score_blocks_lse(const infllmv2_cfg* cfg, const void* q, int32_t n_q, int64_t q_pos0,
                              int32_t is_tree, const void* kbar, int64_t kv_cap, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "infllmv2_score_blocks_lse";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_ptr(fn, q, "q", 16));
  TRY(check_ptr(fn, kbar, "kbar", 16));
  TRY(check_ptr(fn, scores, "scores", 4));
  TRY(check_rows(fn, d, n_q, q_pos0, is_tree, kv_cap));
  TRY(check_ptr(fn, workspace, "workspace", 256));
  const size_t need = infllmv2::score_lse_workspace_bytes(d, n_q, nblk_of(kv_cap));
  if (workspace_bytes < need) {
    char msg[128];
    std::snprintf(msg, sizeof msg, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return fail(INFLLMV2_WORKSPACE_TOO_SMALL, fn, msg);
  }
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_scores_lse(d, static_cast<const uint16_t*>(q), n_q, q_pos0, is_tree != 0,
                                         static_cast<const uint16_t*>(kbar), nblk_of(kv_cap), scores,
                                         workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

int infllmv2_topk_blocks(const infllmv2_cfg* cfg, const float* scores, const void* q,
                         const void* kbar, int32_t n_q, int64_t q_pos0, int32_t is_tree,
                         int64_t kv_cap, int32_t* idx, void* stream) {
  const char* fn = "infllmv2_topk_blocks";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_ptr(fn, idx, "idx", 4));
  if (scores) {
    TRY(check_ptr(fn, scores, "scores", 4));
  } else {
    TRY(check_ptr(fn, q, "q", 16));
    TRY(check_ptr(fn, kbar, "kbar", 16));
  }
  TRY(check_rows(fn, d, n_q, q_pos0, is_tree, kv_cap));
  const int64_t pos_last = is_tree ? q_pos0 : q_pos0 + n_q - 1;
  if (std::min(pos_last / 64, nblk_of(kv_cap)) > 4096)
    return fail(INFLLMV2_UNSUPPORTED, fn, "more than 4096 candidate blocks per row");
  if (!scores && !infllmv2::topk_fused_ok(d, std::min(pos_last / 64, nblk_of(kv_cap))))
    return fail(INFLLMV2_UNSUPPORTED, fn, "fused scoring: the score rows do not fit LDS");
  TRY(check_device(fn));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (scores)
    LAUNCH(fn, infllmv2::launch_topk_from_scores(d, scores, n_q, q_pos0, is_tree != 0,
                                                 nblk_of(kv_cap), idx, s));
  else
    LAUNCH(fn, infllmv2::launch_topk_fused(d, static_cast<const uint16_t*>(q),
                                           static_cast<const uint16_t*>(kbar), n_q, q_pos0,
                                           is_tree != 0, nblk_of(kv_cap), idx, s));
  return INFLLMV2_OK;
}

static int check_attn(const char* fn, const Dims& d, const void* q, int32_t n_q, const void* k,
                      const void* v, int64_t kv_cap, int64_t kv_len, const void* out,
                      const float* lse) {
  TRY(check_ptr(fn, q, "q", 16));
  TRY(check_ptr(fn, k, "k", 16));
  TRY(check_ptr(fn, v, "v", 16));
  TRY(check_ptr(fn, out, "out", 16));
  if (lse) TRY(check_ptr(fn, lse, "lse", 4));
  TRY(check_kv(fn, kv_cap, kv_len));
  if (n_q < 1 || n_q > kv_len) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "need 1 <= n_q <= kv_len");
  if (int64_t(d.B) * d.Hkv * n_q > INT32_MAX / 64)
    return fail(INFLLMV2_UNSUPPORTED, fn, "too many rows for one launch");
  return INFLLMV2_OK;
}

int infllmv2_sparse_attn_prefill(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                 const void* k, const void* v, int64_t kv_cap, int64_t kv_len,
                                 const int32_t* idx, void* out, float* lse, void* stream) {
  const char* fn = "infllmv2_sparse_attn_prefill";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_attn(fn, d, q, n_q, k, v, kv_cap, kv_len, out, lse));
  TRY(check_ptr(fn, idx, "idx", 4));
  // the idx rows of a workgroup's 4*NST*16/G tokens (NST <= 4) are staged in 64 KB of LDS
  if (int64_t(256 / d.G) * d.K * 4 > 65536)
    return fail(INFLLMV2_UNSUPPORTED, fn, "top_k too large for the prefill tile (top_k * 1024 / G > 64 KB)");
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_attn_rows(d, 0, static_cast<const uint16_t*>(q), n_q,
                                        static_cast<const uint16_t*>(k),
                                        static_cast<const uint16_t*>(v), kv_cap, kv_len, idx,
                                        static_cast<uint16_t*>(out), lse,
                                        static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

size_t infllmv2_prefill_backward_workspace_bytes(const infllmv2_cfg* cfg, int32_t n_q,
                                                int64_t kv_len) {
  Dims d;
  if (check_cfg("infllmv2_prefill_backward_workspace_bytes", cfg, true, &d) != INFLLMV2_OK) return 0;
  if (n_q < 1 || kv_len < n_q) return 0;
  return infllmv2::prefill_backward_workspace_bytes(d, n_q, kv_len);
}

int infllmv2_sparse_attn_prefill_backward(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                          const void* k, const void* v, int64_t kv_cap,
                                          int64_t kv_len, const int32_t* idx, const void* out,
                                          const float* lse, const void* dout, float* dq, float* dk,
                                          float* dv, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  const char* fn = "infllmv2_sparse_attn_prefill_backward";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_attn(fn, d, q, n_q, k, v, kv_cap, kv_len, out, lse));
  TRY(check_ptr(fn, idx, "idx", 4));
  TRY(check_ptr(fn, lse, "lse", 4));
  TRY(check_ptr(fn, dout, "dout", 16));
  TRY(check_ptr(fn, dq, "dq", 16));
  TRY(check_ptr(fn, dk, "dk", 16));
  TRY(check_ptr(fn, dv, "dv", 16));
  if (!infllmv2::prefill_backward_ok(d, kv_len))
    return fail(INFLLMV2_UNSUPPORTED, fn, "backward needs head_dim 64 or 128 and a tile that fits LDS");
  TRY(check_ptr(fn, workspace, "workspace", 256));
  const size_t need = infllmv2::prefill_backward_workspace_bytes(d, n_q, kv_len);
  if (workspace_bytes < need) {
    char msg[128];
    std::snprintf(msg, sizeof msg, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return fail(INFLLMV2_WORKSPACE_TOO_SMALL, fn, msg);
  }
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_prefill_backward(
                 d, static_cast<const uint16_t*>(q), n_q, static_cast<const uint16_t*>(k),
                 static_cast<const uint16_t*>(v), kv_cap, kv_len, idx,
                 static_cast<const uint16_t*>(out), lse, static_cast<const uint16_t*>(dout), dq, dk,
                 dv, workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

size_t infllmv2_decode_workspace_bytes(const infllmv2_cfg* cfg, int32_t n_q, int64_t kv_len) {
  Dims d;
  if (check_cfg("infllmv2_decode_workspace_bytes", cfg, true, &d) != INFLLMV2_OK) return 0;
  if (n_q < 1 || kv_len < n_q) return 0;
  return infllmv2::decode_workspace_bytes(d, n_q, kv_len);
}

int infllmv2_sparse_attn_decode(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                const void* k_cache, const void* v_cache, int64_t kv_cap,
                                int64_t kv_len, const int32_t* idx, const uint64_t* tree_mask,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const char* fn = "infllmv2_sparse_attn_decode";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_attn(fn, d, q, n_q, k_cache, v_cache, kv_cap, kv_len, out, lse));
  TRY(check_ptr(fn, idx, "idx", 4));
  if (tree_mask) TRY(check_ptr(fn, tree_mask, "tree_mask", 8));
  if (n_q > 64) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "at most 64 query rows per call");
  if (n_q > 1 && (kv_len - 1) / 64 + 1 > 8192)
    return fail(INFLLMV2_UNSUPPORTED, fn, "multi-row decode beyond 8192 blocks");
  TRY(check_ptr(fn, workspace, "workspace", 256));
  const size_t need = infllmv2::decode_workspace_bytes(d, n_q, kv_len);
  if (workspace_bytes < need) {
    char msg[128];
    std::snprintf(msg, sizeof msg, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return fail(INFLLMV2_WORKSPACE_TOO_SMALL, fn, msg);
  }
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_decode(d, static_cast<const uint16_t*>(q), n_q,
                                     static_cast<const uint16_t*>(k_cache),
                                     static_cast<const uint16_t*>(v_cache), kv_cap, kv_len, idx,
                                     tree_mask, static_cast<uint16_t*>(out), lse, workspace,
                                     workspace_bytes, static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

int infllmv2_sparse_attn_decode_scores(const infllmv2_cfg* cfg, const void* q, const void* k_cache,
                                       const void* v_cache, int64_t kv_cap, int64_t kv_len,
                                       const float* scores, int32_t* idx_out, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const char* fn = "infllmv2_sparse_attn_decode_scores";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_attn(fn, d, q, 1, k_cache, v_cache, kv_cap, kv_len, out, lse));
  TRY(check_ptr(fn, scores, "scores", 4));
  if (idx_out) TRY(check_ptr(fn, idx_out, "idx_out", 4));
  if (d.K > 64) return fail(INFLLMV2_UNSUPPORTED, fn, "top_k above 64");
  if ((kv_len - 1) / 64 > 4096) return fail(INFLLMV2_UNSUPPORTED, fn, "more than 4096 candidate blocks");
  TRY(check_ptr(fn, workspace, "workspace", 256));
  const size_t need = infllmv2::decode_workspace_bytes(d, 1, kv_len);
  if (workspace_bytes < need) {
    char msg[128];
    std::snprintf(msg, sizeof msg, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return fail(INFLLMV2_WORKSPACE_TOO_SMALL, fn, msg);
  }
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_decode(d, static_cast<const uint16_t*>(q), 1,
                                     static_cast<const uint16_t*>(k_cache),
                                     static_cast<const uint16_t*>(v_cache), kv_cap, kv_len, nullptr,
                                     nullptr, static_cast<uint16_t*>(out), lse, workspace,
                                     workspace_bytes, static_cast<hipStream_t>(stream), scores,
                                     idx_out));
  return INFLLMV2_OK;
}

int infllmv2_sparse_attn_decode_scores_noalloc(const infllmv2_cfg* cfg, const void* q,
                                               const void* k_cache, const void* v_cache,
                                               int64_t kv_cap, int64_t kv_len, const float* scores,
                                               int32_t* idx_out, void* out, float* lse,
                                               void* stream) {
  const char* fn = "infllmv2_sparse_attn_decode_scores_noalloc";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_attn(fn, d, q, 1, k_cache, v_cache, kv_cap, kv_len, out, lse));
  TRY(check_ptr(fn, scores, "scores", 4));
  if (idx_out) TRY(check_ptr(fn, idx_out, "idx_out", 4));
  if (d.K > 64) return fail(INFLLMV2_UNSUPPORTED, fn, "top_k above 64");
  if ((kv_len - 1) / 64 > 4096) return fail(INFLLMV2_UNSUPPORTED, fn, "more than 4096 candidate blocks");
  const size_t need = infllmv2::decode_workspace_bytes(d, 1, kv_len);
  if (need > infllmv2::kDecodeNoAllocScratchBytes) {
    char msg[160];
    std::snprintf(msg, sizeof msg, "the call needs %zu bytes of scratch; the static scratch holds %zu",
                  need, infllmv2::kDecodeNoAllocScratchBytes);
    return fail(INFLLMV2_UNSUPPORTED, fn, msg);
  }
  TRY(check_device(fn));
  void* ws = nullptr;
  LAUNCH(fn, infllmv2::decode_noalloc_scratch(&ws));
  LAUNCH(fn, infllmv2::launch_decode(d, static_cast<const uint16_t*>(q), 1,
                                     static_cast<const uint16_t*>(k_cache),
                                     static_cast<const uint16_t*>(v_cache), kv_cap, kv_len, nullptr,
                                     nullptr, static_cast<uint16_t*>(out), lse, ws,
                                     infllmv2::kDecodeNoAllocScratchBytes,
                                     static_cast<hipStream_t>(stream), scores, idx_out));
  return INFLLMV2_OK;
}

int infllmv2_dense_attn(const infllmv2_cfg* cfg, const void* q, int32_t n_q, const void* k,
                        const void* v, int64_t kv_cap, int64_t kv_len, int32_t causal, void* out,
                        float* lse, void* stream) {
  const char* fn = "infllmv2_dense_attn";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_attn(fn, d, q, n_q, k, v, kv_cap, kv_len, out, lse));
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_attn_rows(d, causal ? 1 : 2, static_cast<const uint16_t*>(q), n_q,
                                        static_cast<const uint16_t*>(k),
                                        static_cast<const uint16_t*>(v), kv_cap, kv_len, nullptr,
                                        static_cast<uint16_t*>(out), lse,
                                        static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

int infllmv2_append_kv(const infllmv2_cfg* cfg, const void* k_new, const void* v_new, int32_t n_new,
                       void* k_cache, void* v_cache, int64_t kv_cap, const int64_t* kv_lens,
                       int64_t kv_len, void* kbar, void* stream) {
  const char* fn = "infllmv2_append_kv";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_ptr(fn, k_new, "k_new", 16));
  TRY(check_ptr(fn, v_new, "v_new", 16));
  TRY(check_ptr(fn, k_cache, "k_cache", 16));
  TRY(check_ptr(fn, v_cache, "v_cache", 16));
  if (kbar) TRY(check_ptr(fn, kbar, "kbar", 16));
  if (n_new < 0) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "n_new must be >= 0");
  if (kv_cap < 1 || kv_cap > (int64_t(1) << 31))
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "kv_cap must lie in [1, 2^31]");
  if (kv_lens) {
    TRY(check_ptr(fn, kv_lens, "kv_lens", 8));
  } else if (kv_len < 0 || kv_len + n_new > kv_cap) {
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "kv_len + n_new exceeds kv_cap");
  }
  if (n_new == 0) return INFLLMV2_OK;
  if (int64_t(d.B) * d.Hkv * ((int64_t(n_new) + 63) / 64 + 1) > INT32_MAX)
    return fail(INFLLMV2_UNSUPPORTED, fn, "too many blocks for one launch");
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_append(d, static_cast<const uint16_t*>(k_new),
                                     static_cast<const uint16_t*>(v_new), n_new,
                                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                                     kv_cap, kv_lens, kv_len, static_cast<uint16_t*>(kbar),
                                     static_cast<hipStream_t>(stream)));
  return INFLLMV2_OK;
}

int infllmv2_score_blocks_varlen(const infllmv2_cfg* cfg, const void* q, const int64_t* kv_lens,
                                 const void* kbar, int64_t kv_cap, float* scores, void* stream) {
  const char* fn = "infllmv2_score_blocks_varlen";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_ptr(fn, q, "q", 16));
  TRY(check_ptr(fn, kv_lens, "kv_lens", 8));
  TRY(check_ptr(fn, kbar, "kbar", 16));
  TRY(check_ptr(fn, scores, "scores", 4));
  if (kv_cap < 1 || kv_cap > (int64_t(1) << 31))
    return fail(INFLLMV2_INVALID_ARGUMENT, fn, "kv_cap must lie in [1, 2^31]");
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_scores(d, static_cast<const uint16_t*>(q), 1, 0, 0,
                                     static_cast<const uint16_t*>(kbar), nblk_of(kv_cap), scores,
                                     static_cast<hipStream_t>(stream), kv_lens));
  return INFLLMV2_OK;
}

size_t infllmv2_decode_varlen_workspace_bytes(const infllmv2_cfg* cfg, int64_t kv_len_max) {
  Dims d;
  if (check_cfg("infllmv2_decode_varlen_workspace_bytes", cfg, true, &d) != INFLLMV2_OK) return 0;
  if (kv_len_max < 1) return 0;
  return infllmv2::decode_varlen_workspace_bytes(d, kv_len_max);
}

int infllmv2_sparse_attn_decode_varlen(const infllmv2_cfg* cfg, const void* q, const void* k_cache,
                                       const void* v_cache, int64_t kv_cap, const int64_t* kv_lens,
                                       int64_t kv_len_max, const float* scores, int32_t* idx_out,
                                       void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const char* fn = "infllmv2_sparse_attn_decode_varlen";
  Dims d;
  TRY(check_cfg(fn, cfg, true, &d));
  TRY(check_attn(fn, d, q, 1, k_cache, v_cache, kv_cap, kv_len_max, out, lse));
  TRY(check_ptr(fn, kv_lens, "kv_lens", 8));
  TRY(check_ptr(fn, scores, "scores", 4));
  if (idx_out) TRY(check_ptr(fn, idx_out, "idx_out", 4));
  if (d.K > 64) return fail(INFLLMV2_UNSUPPORTED, fn, "top_k above 64");
  if ((kv_len_max - 1) / 64 > 4096)
    return fail(INFLLMV2_UNSUPPORTED, fn, "more than 4096 candidate blocks");
  TRY(check_ptr(fn, workspace, "workspace", 256));
  const size_t need = infllmv2::decode_varlen_workspace_bytes(d, kv_len_max);
  if (workspace_bytes < need) {
    char msg[128];
    std::snprintf(msg, sizeof msg, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return fail(INFLLMV2_WORKSPACE_TOO_SMALL, fn, msg);
  }
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_decode(d, static_cast<const uint16_t*>(q), 1,
                                     static_cast<const uint16_t*>(k_cache),
                                     static_cast<const uint16_t*>(v_cache), kv_cap, kv_len_max,
                                     nullptr, nullptr, static_cast<uint16_t*>(out), lse, workspace,
                                     workspace_bytes, static_cast<hipStream_t>(stream), scores,
                                     idx_out, kv_lens));
  return INFLLMV2_OK;
}

int infllmv2_sliding_window_attn(const infllmv2_cfg* cfg, const void* q, int32_t n_q,
                                 const void* k, const void* v, int64_t kv_cap, int64_t kv_len,
                                 int64_t window, void* out, float* lse, void* stream) {
  const char* fn = "infllmv2_sliding_window_attn";
  Dims d;
  TRY(check_cfg(fn, cfg, false, &d));
  TRY(check_attn(fn, d, q, n_q, k, v, kv_cap, kv_len, out, lse));
  if (window < 1) return fail(INFLLMV2_INVALID_ARGUMENT, fn, "window must be >= 1");
  TRY(check_device(fn));
  LAUNCH(fn, infllmv2::launch_attn_rows(d, 3, static_cast<const uint16_t*>(q), n_q,
                                        static_cast<const uint16_t*>(k),
                                        static_cast<const uint16_t*>(v), kv_cap, kv_len, nullptr,
                                        static_cast<uint16_t*>(out), lse,
                                        static_cast<hipStream_t>(stream),
                                        std::min<int64_t>(window, kv_len)));
  return INFLLMV2_OK;
}

const char* infllmv2_strerror(int status) {
  switch (status) {
    case INFLLMV2_OK: return "ok";
    case INFLLMV2_INVALID_ARGUMENT: return "invalid argument";
    case INFLLMV2_UNSUPPORTED: return "unsupported";
    case INFLLMV2_WORKSPACE_TOO_SMALL: return "workspace too small";
    case INFLLMV2_HIP_ERROR: return "HIP error";
    default: return "unknown status";
  }
}

const char* infllmv2_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
