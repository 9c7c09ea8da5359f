// abi.cpp -- the exported C entry points: argument checks, launch plans, dispatch.
//
// Every check here runs on the host before any HIP call, so a bad argument
// returns a status without touching the device (and can be exercised on a
// machine without a GPU).

#include <math.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "spec_internal.hpp"
#include "spec_verify.h"

using namespace specv;

namespace {

bool aligned(const void* p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool aligned_or_null(const void* p, size_t a) { return !p || aligned(p, a); }

float resolve_scale(float scale, int32_t D) {
  const float s = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf((float)D);
  return s * 1.4426950408889634f;  // log2(e): the kernels run their softmax in base 2
}

// Launch size of an attention plan: at most 2^22 work-groups (of up to 512
// threads), which keeps every grid and tile index in 32 bits.
bool grid_fits(int32_t B, int32_t Hkv, const AttnPlan& p) {
  return (long long)B * Hkv * p.n_splits * p.n_qs <= (1ll << 22);
}

spec_status_t check_attn_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, spec_dtype_t dtype,
                               int32_t num_splits) {
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SPEC_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > 65536) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

spec_status_t verify_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D,
                           int32_t L_cap, spec_dtype_t dtype, int32_t num_splits) {
  spec_status_t st = check_attn_shape(B, Hq, Hkv, D, dtype, num_splits);
  if (st != SPEC_OK) return st;
  if (n_q < 1) return SPEC_ERR_INVALID_ARG;
  if (n_q > SPEC_MAX_NQ) return SPEC_ERR_UNSUPPORTED;
  if (L_cap < n_q || L_cap > (1 << 30)) return SPEC_ERR_INVALID_ARG;
  if ((long long)(Hq / Hkv) * n_q > (1 << 20)) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

spec_status_t window_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t W, int32_t S,
                           spec_dtype_t dtype, int32_t num_splits) {
  spec_status_t st = check_attn_shape(B, Hq, Hkv, D, dtype, num_splits);
  if (st != SPEC_OK) return st;
  if (W < 1 || S < 0 || (long long)W + S > (1 << 30)) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

spec_status_t sample_shape(int32_t B, int32_t N, int32_t V) {
  if (B < 0 || N < 1 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (N > SPEC_MAX_SAMPLE_NODES) return SPEC_ERR_UNSUPPORTED;
  if (V > (1 << 27) || B > 65535) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

}  // namespace

extern "C" {

const char* spec_status_str(spec_status_t status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG: return "SPEC_ERR_INVALID_ARG";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_BAD_TREE: return "SPEC_ERR_BAD_TREE";
    case SPEC_ERR_MISALIGNED: return "SPEC_ERR_MISALIGNED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
    default: break;
  }
  return "SPEC_ERR_UNKNOWN";
}

spec_status_t spec_validate_tree(const int32_t* parent_host, int32_t n, int32_t require_single_root) {
  if (!parent_host || n < 1) return SPEC_ERR_INVALID_ARG;
  for (int32_t c = 0; c < n; ++c) {
    const int32_t p = parent_host[c];
    if (p < -1 || p >= c) return SPEC_ERR_BAD_TREE;
    if (require_single_root && ((c == 0) != (p == -1))) return SPEC_ERR_BAD_TREE;
  }
  return SPEC_OK;
}

int32_t spec_verify_attention_auto_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q,
                                          int32_t D, int32_t L_cap, spec_dtype_t dtype) {
  if (verify_shape(B, Hq, Hkv, n_q, D, L_cap, dtype, 0) != SPEC_OK || B == 0) return 0;
  return plan_attention(B, Hkv, (Hq / Hkv) * n_q, D, L_cap, dtype, 0, false).n_splits;
}

size_t spec_verify_attention_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D,
                                       int32_t L_cap, spec_dtype_t dtype, int32_t num_splits) {
  if (verify_shape(B, Hq, Hkv, n_q, D, L_cap, dtype, num_splits) != SPEC_OK) return 0;
  if (B == 0) return 0;
  const AttnPlan p = plan_attention(B, Hkv, (Hq / Hkv) * n_q, D, L_cap, dtype, num_splits, false);
  return grid_fits(B, Hkv, p) ? p.ws_bytes : 0;
}

}  // extern "C"

namespace {

// Paging parameters of a verify call (all zero for a contiguous cache).
struct Paging {
  const int32_t* block_table;
  int32_t bt_stride, num_pages, page_size;
};

int32_t log2_exact(int32_t x) {
  int32_t s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

spec_status_t paging_check(const Paging& pg, int32_t L_max, const int32_t* kv_len) {
  if (pg.page_size > (1 << 20) || log2_exact(pg.page_size) < 6) return SPEC_ERR_UNSUPPORTED;
  if (pg.num_pages < 1) return SPEC_ERR_INVALID_ARG;
  if (pg.bt_stride < (L_max + pg.page_size - 1) / pg.page_size) return SPEC_ERR_INVALID_ARG;
  if (!aligned(pg.block_table, 4) || !aligned(kv_len, 4)) return SPEC_ERR_MISALIGNED;
  return SPEC_OK;
}

// Workspace layout of an attention call: split-arrival counters (used when
// the plan merges the splits in the last work-group of each unit), then the
// O and (max, sum) partials.
void set_workspace(AttnArgs& a, const AttnPlan& p, void* workspace) {
  char* w = static_cast<char*>(workspace);
  a.arrive = p.fuse_merge ? reinterpret_cast<uint32_t*>(w) : nullptr;
  a.ws_o = reinterpret_cast<float*>(w + p.ws_sync_bytes);
  a.ws_ml = reinterpret_cast<float*>(w + p.ws_sync_bytes + p.ws_o_bytes);
}

spec_status_t verify_call(const void* q, const void* k_cache, const void* v_cache, void* out,
                          float* lse, const int32_t* kv_len, const int32_t* parent,
                          int32_t parent_batch_stride, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t n_q, int32_t D, int32_t L_cap, spec_dtype_t dtype, float scale,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          int32_t* dev_err, hipStream_t stream, const Paging& pg) {
  spec_status_t st = verify_shape(B, Hq, Hkv, n_q, D, L_cap, dtype, num_splits);
  if (st != SPEC_OK) return st;
  if (parent && parent_batch_stride != 0 && parent_batch_stride != n_q) return SPEC_ERR_INVALID_ARG;
  if (pg.page_size && (st = paging_check(pg, L_cap, kv_len)) != SPEC_OK) return st;
  if (B == 0) return SPEC_OK;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned_or_null(lse, 4) || !aligned_or_null(kv_len, 4) || !aligned_or_null(parent, 4) ||
      !aligned_or_null(dev_err, 4))
    return SPEC_ERR_MISALIGNED;
  const int32_t g = Hq / Hkv;
  const AttnPlan p =
      plan_attention(B, Hkv, g * n_q, D, L_cap, dtype, num_splits, false, pg.page_size);
  if (!grid_fits(B, Hkv, p)) return SPEC_ERR_UNSUPPORTED;
  if (!aligned(workspace, 256) || workspace_bytes < p.ws_bytes) return SPEC_ERR_WORKSPACE;

  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.lens = kv_len;
  a.parent = parent;
  a.parent_stride = parent ? parent_batch_stride : 0;
  if (pg.page_size) {
    a.block_table = pg.block_table;
    a.bt_stride = pg.bt_stride;
    a.page_shift = log2_exact(pg.page_size);
    a.num_pages = pg.num_pages;
  }
  set_workspace(a, p, workspace);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = g;
  a.n_q = n_q;
  a.D = D;
  a.L_cap = L_cap;
  a.M = g * n_q;
  a.tree_waves = p.tree_waves;
  a.slice_rows = p.slice_rows;
  a.n_qs = p.n_qs;
  a.n_splits = p.n_splits;
  a.n_tiles = B * Hkv * p.n_splits;
  a.grid = p.grid;
  a.scale_log2 = resolve_scale(scale, D);
  a.dev_err = dev_err;
  a.out = out;
  a.lse = lse;
  return launch_attention(a, false, dtype, out, lse, stream) == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace

extern "C" {

spec_status_t spec_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                                    void* out, float* lse, const int32_t* kv_len,
                                    const int32_t* parent, int32_t parent_batch_stride,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D,
                                    int32_t L_cap, spec_dtype_t dtype, float scale,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    int32_t* dev_err, hipStream_t stream) {
  return verify_call(q, k_cache, v_cache, out, lse, kv_len, parent, parent_batch_stride, B, Hq,
                     Hkv, n_q, D, L_cap, dtype, scale, num_splits, workspace, workspace_bytes,
                     dev_err, stream, Paging{nullptr, 0, 0, 0});
}

size_t spec_verify_attention_paged_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q,
                                             int32_t D, int32_t L_max, int32_t page_size,
                                             spec_dtype_t dtype, int32_t num_splits) {
  if (verify_shape(B, Hq, Hkv, n_q, D, L_max, dtype, num_splits) != SPEC_OK || B == 0) return 0;
  if (page_size > (1 << 20) || log2_exact(page_size) < 6) return 0;
  const AttnPlan p =
      plan_attention(B, Hkv, (Hq / Hkv) * n_q, D, L_max, dtype, num_splits, false, page_size);
  return grid_fits(B, Hkv, p) ? p.ws_bytes : 0;
}

spec_status_t spec_verify_attention_paged(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
    int32_t block_table_stride, int32_t num_pages, int32_t page_size, void* out, float* lse,
    const int32_t* kv_len, const int32_t* parent, int32_t parent_batch_stride, int32_t B,
    int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D, int32_t L_max, spec_dtype_t dtype,
    float scale, int32_t num_splits, void* workspace, size_t workspace_bytes, int32_t* dev_err,
    hipStream_t stream) {
  if (page_size < 1) return SPEC_ERR_INVALID_ARG;
  return verify_call(q, k_pages, v_pages, out, lse, kv_len, parent, parent_batch_stride, B, Hq,
                     Hkv, n_q, D, L_max, dtype, scale, num_splits, workspace, workspace_bytes,
                     dev_err, stream, Paging{block_table, block_table_stride, num_pages, page_size});
}

size_t spec_window_attention_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t W,
                                       int32_t S, spec_dtype_t dtype, int32_t num_splits) {
  if (window_shape(B, Hq, Hkv, D, W, S, dtype, num_splits) != SPEC_OK || B == 0) return 0;
  const AttnPlan p = plan_attention(B, Hkv, Hq / Hkv, D, W + S, dtype, num_splits, true);
  return grid_fits(B, Hkv, p) ? p.ws_bytes : 0;
}

spec_status_t spec_window_attention(const void* q, void* k_ring, void* v_ring, void* k_sink,
                                    void* v_sink, const void* k_new, const void* v_new,
                                    const int32_t* total_len, void* out, float* lse, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t D, int32_t W, int32_t S,
                                    spec_dtype_t dtype, float scale, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes, int32_t* dev_err,
                                    hipStream_t stream) {
  spec_status_t st = window_shape(B, Hq, Hkv, D, W, S, dtype, num_splits);
  if (st != SPEC_OK) return st;
  if (B == 0) return SPEC_OK;
  if ((k_new == nullptr) != (v_new == nullptr)) return SPEC_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_ring, 16) || !aligned(v_ring, 16) || !aligned(out, 16) ||
      !aligned(total_len, 4) || !aligned_or_null(lse, 4) || !aligned_or_null(k_new, 16) ||
      !aligned_or_null(v_new, 16) || !aligned_or_null(dev_err, 4))
    return SPEC_ERR_MISALIGNED;
  if (S > 0 && (!aligned(k_sink, 16) || !aligned(v_sink, 16))) return SPEC_ERR_MISALIGNED;
  const int32_t g = Hq / Hkv;
  const AttnPlan p = plan_attention(B, Hkv, g, D, W + S, dtype, num_splits, true);
  if (!grid_fits(B, Hkv, p)) return SPEC_ERR_UNSUPPORTED;
  if (!aligned(workspace, 256) || workspace_bytes < p.ws_bytes) return SPEC_ERR_WORKSPACE;

  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k_ring;
  a.v = v_ring;
  a.k_sink = k_sink;
  a.v_sink = v_sink;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_ring_w = k_ring;
  a.v_ring_w = v_ring;
  a.k_sink_w = k_sink;
  a.v_sink_w = v_sink;
  a.lens = total_len;
  set_workspace(a, p, workspace);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = g;
  a.n_q = 1;
  a.D = D;
  a.L_cap = W + S;
  a.M = g;
  a.W = W;
  a.S = S;
  a.slice_rows = p.slice_rows;
  a.n_qs = p.n_qs;
  a.n_splits = p.n_splits;
  a.n_tiles = B * Hkv * p.n_splits;
  a.grid = p.grid;
  a.scale_log2 = resolve_scale(scale, D);
  a.dev_err = dev_err;
  a.out = out;
  a.lse = lse;
  return launch_attention(a, true, dtype, out, lse, stream) == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_sample_workspace(int32_t B, int32_t N, int32_t V) {
  if (sample_shape(B, N, V) != SPEC_OK || B == 0) return 0;
  return plan_sample(B, N, V).bytes;
}

}  // extern "C"

namespace {

spec_status_t sample_call(const void* target_logits, const void* draft_logits,
                          const int32_t* tokens, const int32_t* parent,
                          int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                          uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_count,
                          int32_t* out_path, uint8_t* out_accept, void* workspace,
                          size_t workspace_bytes, int32_t* dev_err, hipStream_t stream,
                          bool bf16, bool lossless, bool noalloc = false) {
  spec_status_t st = sample_shape(B, N, V);
  if (st != SPEC_OK) return st;
  if (offset >= (1ull << 30)) return SPEC_ERR_INVALID_ARG;
  if (parent && parent_batch_stride != 0 && parent_batch_stride != N) return SPEC_ERR_INVALID_ARG;
  if (B == 0) return SPEC_OK;
  if (!aligned(target_logits, 16) || !aligned(draft_logits, 16) || !aligned(tokens, 4) ||
      !aligned(out_tokens, 4) || !aligned(out_count, 4) || !aligned_or_null(out_path, 4) ||
      !aligned_or_null(parent, 4) || !aligned_or_null(dev_err, 4))
    return SPEC_ERR_MISALIGNED;
  const SamplePlan p = plan_sample(B, N, V);
  if (noalloc) {
    // The library-owned array replaces the workspace; its arrival counters
    // (the workspace's first off_m bytes) are cleared before the kernels run.
    if (p.bytes > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ERR_UNSUPPORTED;
    if (noalloc_scratch(&workspace) != hipSuccess) return SPEC_ERR_HIP;
    workspace_bytes = SPEC_NOALLOC_SCRATCH_BYTES;
    if (launch_zero_words(workspace, p.off_m, stream) != hipSuccess) return SPEC_ERR_HIP;
  }
  if (!aligned(workspace, 256) || workspace_bytes < p.bytes) return SPEC_ERR_WORKSPACE;

  SampleArgs a;
  memset(&a, 0, sizeof(a));
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = tokens;
  a.parent = parent;
  a.parent_stride = parent ? parent_batch_stride : 0;
  a.B = B;
  a.N = N;
  a.V = V;
  a.key0 = (uint32_t)(seed & 0xffffffffu);
  a.key1 = (uint32_t)(seed >> 32);
  a.ctr3_base = (uint32_t)(4 * offset);
  a.out_tokens = out_tokens;
  a.out_count = out_count;
  a.out_path = out_path;
  a.out_accept = out_accept;
  char* ws = static_cast<char*>(workspace);
  a.arrive = reinterpret_cast<uint32_t*>(ws);
  a.part_m = reinterpret_cast<float*>(ws + p.off_m);
  a.part_s = reinterpret_cast<double*>(ws + p.off_s);
  a.tok_logit = reinterpret_cast<float*>(ws + p.off_g);
  a.race_w = reinterpret_cast<double*>(ws + p.off_w);
  a.decision = reinterpret_cast<int32_t*>(ws + p.off_dec);
  a.decision_lz = reinterpret_cast<double*>(ws + p.off_lz);
  a.dec_stride = p.dec_stride;
  a.n_vchunks = p.n_vchunks;
  a.vchunk = p.vchunk;
  a.n_race = p.n_race;
  a.n_groups = p.n_groups;
  a.logits_bf16 = bf16 ? 1 : 0;
  a.lossless = lossless ? 1 : 0;
  // The lossless walk may stop at any node with its rows cached; the
  // first-accepted rule reads a leaf's target row only if the walk ends there.
  a.leaf_rows = lossless ? 1 : 0;
  a.dev_err = dev_err;
  return launch_sample(a, stream) == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace

extern "C" {

spec_status_t spec_sample(const float* target_logits, const float* draft_logits,
                          const int32_t* tokens, const int32_t* parent,
                          int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                          uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_count,
                          int32_t* out_path, uint8_t* out_accept, void* workspace,
                          size_t workspace_bytes, int32_t* dev_err, hipStream_t stream) {
  return sample_call(target_logits, draft_logits, tokens, parent, parent_batch_stride, B, N, V,
                     seed, offset, out_tokens, out_count, out_path, out_accept, workspace,
                     workspace_bytes, dev_err, stream, false, false);
}

spec_status_t spec_sample_bf16(const void* target_logits, const void* draft_logits,
                               const int32_t* tokens, const int32_t* parent,
                               int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                               uint64_t seed, uint64_t offset, int32_t* out_tokens,
                               int32_t* out_count, int32_t* out_path, uint8_t* out_accept,
                               void* workspace, size_t workspace_bytes, int32_t* dev_err,
                               hipStream_t stream) {
  return sample_call(target_logits, draft_logits, tokens, parent, parent_batch_stride, B, N, V,
                     seed, offset, out_tokens, out_count, out_path, out_accept, workspace,
                     workspace_bytes, dev_err, stream, true, false);
}

spec_status_t spec_sample_ex(const void* target_logits, const void* draft_logits,
                             spec_dtype_t logits_dtype, spec_sibling_rule_t siblings,
                             const int32_t* tokens, const int32_t* parent,
                             int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                             uint64_t seed, uint64_t offset, int32_t* out_tokens,
                             int32_t* out_count, int32_t* out_path, uint8_t* out_accept,
                             void* workspace, size_t workspace_bytes, int32_t* dev_err,
                             hipStream_t stream) {
  if (logits_dtype != SPEC_F32 && logits_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
  if (siblings != SPEC_SIBLINGS_FIRST && siblings != SPEC_SIBLINGS_LOSSLESS)
    return SPEC_ERR_INVALID_ARG;
  return sample_call(target_logits, draft_logits, tokens, parent, parent_batch_stride, B, N, V,
                     seed, offset, out_tokens, out_count, out_path, out_accept, workspace,
                     workspace_bytes, dev_err, stream, logits_dtype == SPEC_BF16,
                     siblings == SPEC_SIBLINGS_LOSSLESS);
}

spec_status_t spec_sample_noalloc(const void* target_logits, const void* draft_logits,
                                  spec_dtype_t logits_dtype, spec_sibling_rule_t siblings,
                                  const int32_t* tokens, const int32_t* parent,
                                  int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                                  uint64_t seed, uint64_t offset, int32_t* out_tokens,
                                  int32_t* out_count, int32_t* out_path, uint8_t* out_accept,
                                  int32_t* dev_err, hipStream_t stream) {
  if (logits_dtype != SPEC_F32 && logits_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
  if (siblings != SPEC_SIBLINGS_FIRST && siblings != SPEC_SIBLINGS_LOSSLESS)
    return SPEC_ERR_INVALID_ARG;
  return sample_call(target_logits, draft_logits, tokens, parent, parent_batch_stride, B, N, V,
                     seed, offset, out_tokens, out_count, out_path, out_accept, nullptr, 0,
                     dev_err, stream, logits_dtype == SPEC_BF16,
                     siblings == SPEC_SIBLINGS_LOSSLESS, true);
}

size_t spec_draft_sample_workspace(int32_t B, int32_t V) {
  if (B < 1 || V < 1 || V > (1 << 27) || B > 65535) return 0;
  return plan_draft(B, V).bytes;
}

spec_status_t spec_draft_sample(const void* draft_logits, spec_dtype_t dtype, int64_t row_stride,
                                int32_t B, int32_t V, uint64_t seed, uint64_t offset, int32_t node,
                                int32_t* out_token, int32_t token_stride, float* out_logprob,
                                void* workspace, size_t workspace_bytes, int32_t* dev_err,
                                hipStream_t stream) {
  if (B < 0 || V < 1 || node < 0 || token_stride < 0) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
  if (V > (1 << 27) || B > 65535) return SPEC_ERR_UNSUPPORTED;
  if (offset >= (1ull << 30)) return SPEC_ERR_INVALID_ARG;
  if (row_stride == 0) row_stride = V;
  if (row_stride < V) return SPEC_ERR_INVALID_ARG;
  if (B == 0) return SPEC_OK;
  const size_t elt = dtype == SPEC_BF16 ? 2 : 4;
  if (!aligned(draft_logits, elt) || !aligned(out_token, 4) || !aligned_or_null(out_logprob, 4) ||
      !aligned_or_null(dev_err, 4))
    return SPEC_ERR_MISALIGNED;
  const DraftPlan p = plan_draft(B, V);
  if (!aligned(workspace, 256) || workspace_bytes < p.bytes) return SPEC_ERR_WORKSPACE;
  DraftArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = draft_logits;
  a.row_stride = row_stride;
  a.B = B;
  a.V = V;
  a.key0 = (uint32_t)(seed & 0xffffffffu);
  a.key1 = (uint32_t)(seed >> 32);
  a.ctr3 = (uint32_t)(4 * offset + 1);
  a.node = node;
  a.out_token = out_token;
  a.token_stride = token_stride ? token_stride : 1;
  a.out_logprob = out_logprob;
  char* ws = static_cast<char*>(workspace);
  a.arrive = reinterpret_cast<uint32_t*>(ws);
  a.part_best = reinterpret_cast<double*>(ws + p.off_best);
  a.part_idx = reinterpret_cast<int32_t*>(ws + p.off_idx);
  a.part_x = reinterpret_cast<float*>(ws + p.off_x);
  a.part_m = reinterpret_cast<float*>(ws + p.off_m);
  a.part_s = reinterpret_cast<double*>(ws + p.off_s);
  a.n_chunks = p.n_chunks;
  a.chunk = p.chunk;
  a.logits_bf16 = dtype == SPEC_BF16 ? 1 : 0;
  a.dev_err = dev_err;
  // Vector loads (4 ids) when every row starts aligned and holds whole vectors.
  const bool vec4 = aligned(draft_logits, 4 * elt) && V % 4 == 0 && row_stride % 4 == 0;
  return launch_draft(a, vec4, stream) == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status_t spec_kv_commit(void* k_cache, void* v_cache, int32_t* kv_len, const int32_t* path,
                             const int32_t* count, int32_t B, int32_t Hkv, int32_t n_q, int32_t D,
                             int32_t L_cap, spec_dtype_t dtype, int32_t* draft_total_len,
                             int32_t draft_appended, int32_t* dev_err, hipStream_t stream) {
  spec_status_t st = verify_shape(B, Hkv, Hkv, n_q, D, L_cap, dtype, 0);
  if (st != SPEC_OK) return st;
  if (draft_total_len && (draft_appended < 0 || draft_appended > n_q)) return SPEC_ERR_INVALID_ARG;
  if ((long long)B * Hkv > (1ll << 31) - 1) return SPEC_ERR_UNSUPPORTED;
  if (B == 0) return SPEC_OK;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(kv_len, 4) ||
      !aligned(count, 4) || !aligned_or_null(path, 4) || !aligned_or_null(draft_total_len, 4) ||
      !aligned_or_null(dev_err, 4))
    return SPEC_ERR_MISALIGNED;
  CommitArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k_cache;
  a.v = v_cache;
  a.kv_len = kv_len;
  a.path = path;
  a.count = count;
  a.draft_total_len = draft_total_len;
  a.draft_appended = draft_total_len ? draft_appended : 0;
  a.B = B;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.L_cap = L_cap;
  a.row_bytes = D * (dtype == SPEC_BF16 ? 2 : 4);
  a.dev_err = dev_err;
  return launch_commit(a, stream) == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // extern "C"
