// spec_internal.hpp -- host-side launch plans shared by the C ABI and the kernel files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "spec_verify.h"

namespace specv {

// Everything one split-K attention launch needs.  Built and checked on the
// host by the ABI layer; the kernels only read it.
struct AttnArgs {
  const void* q;          // [B, Hq, n_q, D]
  const void* k;          // verify: K cache [B, Hkv, L_cap, D]; window: ring [B, Hkv, W, D]
  const void* v;
  const void* k_sink;     // window only: [B, Hkv, S, D]
  const void* v_sink;
  const void* k_new;      // window only, nullable: [B, Hkv, 1, D]
  const void* v_new;
  void* k_ring_w;         // window fused append destinations (same buffers as k/v, k_sink/v_sink)
  void* v_ring_w;
  void* k_sink_w;
  void* v_sink_w;
  const int32_t* lens;    // verify: kv_len (nullable); window: total_len
  const int32_t* parent;  // verify: nullable parent array
  int32_t parent_stride;
  const int32_t* block_table;  // paged verify: [B, bt_stride] page ids; NULL = contiguous cache
  int32_t bt_stride;
  int32_t page_shift;     // log2 of the page size (keys per page)
  int32_t num_pages;      // pages in the pool (bounds check of block_table entries)
  float* ws_o;            // [n_partials][slice_rows][D]
  float* ws_ml;           // [n_partials][slice_rows][2]  (running max in log2 units, sum)
  uint32_t* arrive;       // [units * n_qs] split arrival counters; NULL: merge kernel
  void* out;              // [B, Hq, n_q, D]: written directly when n_splits == 1
  float* lse;             // nullable
  int32_t B, Hq, Hkv, g, n_q, D, L_cap, M;
  int32_t W, S;           // window geometry
  int32_t tree_waves;     // 0: streaming kernel; 4 or 8: LDS-shared wide-block kernel
  int32_t slice_rows;     // query rows per work-group slice
  int32_t n_qs;           // slices per (sequence, kv head)
  int32_t n_splits;       // key-range splits per (sequence, kv head)
  int32_t n_tiles;        // B * Hkv * n_splits
  int32_t grid;           // work-groups launched
  float scale_log2;       // softmax scale * log2(e)
  int32_t* dev_err;
};

struct MergeArgs {
  const float* ws_o;
  const float* ws_ml;
  void* out;
  float* lse;
  int32_t B, Hq, Hkv, g, n_q, D, M;
  int32_t slice_rows, n_qs, n_splits;
};

struct AttnPlan {
  int32_t tree_waves, slice_rows, n_qs, n_splits, grid;
  bool fuse_merge;        // splits merged by the last work-group of each unit
  // Workspace layout: arrival counters, then the O and (max, sum) partials.
  size_t ws_sync_bytes, ws_o_bytes, ws_ml_bytes, ws_bytes;
};

// page_size: keys per page of a paged verify cache (0: contiguous).
AttnPlan plan_attention(int32_t B, int32_t Hkv, int32_t M, int32_t D, int32_t n_keys_max,
                        spec_dtype_t dtype, int32_t num_splits, bool window,
                        int32_t page_size = 0);

hipError_t launch_attention(const AttnArgs& a, bool window, spec_dtype_t dtype, void* out,
                            float* lse, hipStream_t stream);

struct SampleArgs {
  const void* target;      // [B][N][V] logits, fp32 or bf16 (logits_bf16)
  const void* draft;
  const int32_t* tokens;
  const int32_t* parent;
  int32_t parent_stride;
  int32_t B, N, V;
  uint32_t key0, key1;
  uint32_t ctr3_base;      // 4 * offset
  int32_t* out_tokens;
  int32_t* out_count;
  int32_t* out_path;
  uint8_t* out_accept;
  // workspace views
  uint32_t* arrive;        // [B][..] arrival counters of the residual work-groups
  float* part_m;           // [B][2N][n_vchunks]
  double* part_s;          // [B][2N][n_vchunks]
  float* tok_logit;        // [B][2][N]: logit of node c's drafted token in its parent's
                           // target (0) and draft (1) row, gathered by the stats kernel
  double* race_w;          // [B][n_race][2]  (residual mass, target mass) per race chunk
  int32_t* decision;       // [B][dec_stride]: len, error, residual flag, -, path[N], accept[N]
  double* decision_lz;     // [B][kDecisionDoubles]: stop row's log normalisers (target,
                           // draft), residual shift, and (max, 1/sum) of both rows
  int32_t dec_stride;
  int32_t n_vchunks;       // stats chunks per row
  int32_t vchunk;          // ids per stats chunk
  int32_t n_race;          // race chunks per row (1024 ids each)
  int32_t n_groups;        // resample work-groups per sequence
  int32_t logits_bf16;
  int32_t lossless;        // siblings tested against successively updated residuals
  int32_t leaf_rows;       // 1: the statistics kernel also streams the target rows of
                           // leaves; 0: a leaf's target row is read only when the walk
                           // stops there (its statistics then come from the residual pass)
  int32_t* dev_err;
};

constexpr int kDecisionDoubles = 8;

struct SamplePlan {
  int32_t n_vchunks, vchunk, n_race, n_groups, dec_stride;
  // The arrival counters fill [0, off_m); then the row partials, gathered
  // token logits, race-chunk masses and the decision records.
  size_t off_m, off_s, off_g, off_w, off_dec, off_lz, bytes;
};

SamplePlan plan_sample(int32_t B, int32_t N, int32_t V);
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);

// The library-owned scratch array of spec_sample_noalloc on the current
// device (SPEC_NOALLOC_SCRATCH_BYTES bytes): its device address, looked up
// once per device.
hipError_t noalloc_scratch(void** ptr);
// Zero `bytes` (a multiple of 4) at device pointer p with a fill kernel.
hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t stream);

// Keeping the accepted path's K/V after a verification round.
struct CommitArgs {
  void* k;                  // [B, Hkv, L_cap, row_bytes]
  void* v;
  int32_t* kv_len;          // [B], updated in place
  const int32_t* path;      // [B, n_q] accepted node ids, nullable (chain: identity)
  const int32_t* count;     // [B] accepted path length
  int32_t* draft_total_len; // [B] nullable, rewound in place
  int32_t draft_appended;
  int32_t B, Hkv, n_q, L_cap, row_bytes;
  int32_t* dev_err;
};

hipError_t launch_commit(const CommitArgs& a, hipStream_t stream);

// One draft-step token draw per sequence.
struct DraftArgs {
  const void* logits;       // row b at logits + b * row_stride, V entries (fp32 or bf16)
  int64_t row_stride;
  int32_t B, V;
  uint32_t key0, key1;
  uint32_t ctr3;            // 4 * offset + 1
  int32_t node;
  int32_t* out_token;       // out_token[b * token_stride]
  int32_t token_stride;
  float* out_logprob;       // nullable, [B]
  uint32_t* arrive;         // [B][..] arrival counters of the chunk work-groups
  double* part_best;        // [B][n_chunks] best race score (natural log units)
  int32_t* part_idx;        // [B][n_chunks] its id
  float* part_x;            // [B][n_chunks] its logit * log2(e)
  float* part_m;            // [B][n_chunks] max of logit * log2(e)
  double* part_s;           // [B][n_chunks] sum of exp2(x - max)
  int32_t n_chunks;
  int32_t chunk;            // ids per work-group: 2048, or 4096 at large batch
  int32_t logits_bf16;
  int32_t* dev_err;
};

struct DraftPlan {
  int32_t n_chunks, chunk;
  size_t off_best, off_idx, off_x, off_m, off_s, bytes;
};

DraftPlan plan_draft(int32_t B, int32_t V);
hipError_t launch_draft(const DraftArgs& a, bool vec4, hipStream_t stream);

}  // namespace specv
