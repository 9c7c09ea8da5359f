/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-verification kernels.
 *
 * Three operations make up the data-parallel hot path of one speculative
 * decoding round:
 *
 *   spec_verify_attention  attention of a block of n_q query tokens (a
 *                          gamma+1 causal chain, or an N-node candidate tree
 *                          under an ancestor-only mask) against the full KV
 *                          cache of every sequence;
 *   spec_window_attention  the draft model's bounded attention: one query per
 *                          sequence against S sink tokens plus a W-slot FIFO
 *                          ring of the most recent tokens;
 *   spec_sample            softmax over the vocabulary, acceptance of each
 *                          drafted token with probability min(1, target/draft),
 *                          and one draw from the normalised max(target-draft, 0)
 *                          at the first rejection (or from the target row after
 *                          the last accepted token when nothing is rejected).
 *
 * Conventions shared by every entry point:
 *
 *   Ownership   The caller allocates and frees every buffer (inputs, outputs,
 *               workspace).  The library allocates nothing and keeps no
 *               mutable global state; calls on different streams with
 *               different buffers may run concurrently.
 *   Pointers    Device pointers unless marked "host".  Tensor pointers must
 *               be 16-byte aligned; workspaces 256-byte aligned.  All tensors
 *               are dense, row-major, in the layouts given per argument.
 *   Workspace   Scratch the caller owns, sized by the matching *_workspace
 *               function.  Zero-fill it once before its first use: the window
 *               attention, sampling and draft-draw calls keep work-group
 *               arrival counters in it, and every call leaves them at zero again, so the same
 *               workspace serves any later call (of any entry point) ordered
 *               after it on the device.  Calls that overlap in time need
 *               workspaces of their own.  Counters found non-zero set
 *               SPEC_DEVERR_WORKSPACE.
 *   Streams     All work is enqueued on `stream` (0 = the null stream); no
 *               call synchronises the host.  Outputs are valid once the
 *               stream reaches the end of the call.
 *   Errors      Scalar and pointer arguments are checked on the host before
 *               any HIP call: a bad argument returns a status and launches
 *               nothing.  Problems that can only be seen in device-resident
 *               data (a kv_len out of range, a bad parent entry, a token out
 *               of the vocabulary) set bits of *dev_err (if dev_err is not
 *               NULL) with an atomic OR; the affected sequence then gets a
 *               defined result (zero attention output, out_count = 0) and
 *               no memory outside the given buffers is touched.
 *   Empty work  B == 0 returns SPEC_OK and launches nothing.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below also lists a least and a greatest int32 value (not
 * meaningful codes): the enum's range is then all of int32, so any integer a
 * caller passes is a valid value of the type, and the library can refuse the
 * unlisted ones with SPEC_ERR_INVALID_ARG. */
typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = 1, /* a size, count or enum is out of range */
  SPEC_ERR_UNSUPPORTED = 2, /* a valid shape this build does not handle */
  SPEC_ERR_BAD_TREE = 3,    /* host-side parent array is not a valid tree */
  SPEC_ERR_MISALIGNED = 4,  /* a required pointer is NULL or misaligned */
  SPEC_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  SPEC_ERR_HIP = 6,         /* a HIP launch failed (hipGetLastError) */
  SPEC_STATUS_RANGE_MIN = -2147483647 - 1,
  SPEC_STATUS_RANGE_MAX = 2147483647
} spec_status_t;

typedef enum {
  SPEC_F32 = 0,
  SPEC_BF16 = 1,
  SPEC_DTYPE_RANGE_MIN = -2147483647 - 1,
  SPEC_DTYPE_RANGE_MAX = 2147483647
} spec_dtype_t;

/* How siblings of a candidate tree are tested (spec_sample_ex). */
typedef enum {
  SPEC_SIBLINGS_FIRST = 0,    /* every node against the target row; first passing child */
  SPEC_SIBLINGS_LOSSLESS = 1, /* in order, against residuals updated after each rejection */
  SPEC_SIBLINGS_RANGE_MIN = -2147483647 - 1,
  SPEC_SIBLINGS_RANGE_MAX = 2147483647
} spec_sibling_rule_t;

/* Bits OR-ed into *dev_err by the kernels. */
#define SPEC_DEVERR_KV_LEN 0x1    /* kv_len[b] outside [n_q, L_cap] */
#define SPEC_DEVERR_PARENT 0x2    /* parent[c] outside [-1, c) (sampling: a root other than 0) */
#define SPEC_DEVERR_TOTAL_LEN 0x4 /* total_len[b] < 1 */
#define SPEC_DEVERR_TOKEN 0x8     /* drafted token outside [0, V) */
#define SPEC_DEVERR_PATH 0x10     /* commit: count or path entries not a valid accepted path */
#define SPEC_DEVERR_LOGITS 0x20   /* draft draw: a row with no finite logit */
#define SPEC_DEVERR_PAGE 0x40     /* paged verify: a block_table entry outside [0, num_pages) */
#define SPEC_DEVERR_WORKSPACE 0x80 /* a workspace whose arrival counters were not zero-filled */

/* Largest supported query block (one 64-bit ancestor mask per node). */
#define SPEC_MAX_NQ 64
/* Largest supported number of nodes per sequence in spec_sample. */
#define SPEC_MAX_SAMPLE_NODES 256
/* Size of the library-owned device scratch array that spec_sample_noalloc
   uses on each GPU (one array per device, held until the process ends). */
#define SPEC_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * spec_verify_attention -- verification attention of the drafted block.
 *
 * Defines: "Guide to MagicDec" (aifetchly blog), section 2 "Lossless Target
 * Model Verification Across Full Context" (the target verifies the drafts with
 * attention over the full cache); "Speculative Decoding in LLM Serving
 * Systems" (elimelt notes), section "The algorithm", step 2 (one pass over
 * prefix + drafts gives every drafted position its distribution) and section
 * "Tree-based variants" (each tree token attends only to its ancestors);
 * "Speculative Decoding & Medusa Architecture" (zyekh blog), section 4 (tree
 * attention under a 2-D boolean mask).
 *
 * For sequence b, query head h and block node i:
 *   hk = h / (Hq/Hkv);  L = kv_len[b];  p0 = L - n_q;
 *   allowed keys: positions [0, p0) and p0 + t for every ancestor t of i
 *   (i itself included);  out = softmax(scale * q K^T) V over the allowed
 *   keys, lse = log(sum exp(scale * q K^T)) over the same keys (natural log).
 *
 *   q        [B, Hq, n_q, D]     dtype            query block (post-RoPE)
 *   k_cache  [B, Hkv, L_cap, D]  dtype            keys; the block's own K sits at
 *   v_cache  [B, Hkv, L_cap, D]  dtype            positions kv_len-n_q .. kv_len-1
 *   out      [B, Hq, n_q, D]     dtype            output
 *   lse      [B, Hq, n_q]        f32, nullable    log-sum-exp per row
 *   kv_len   [B] int32, nullable (NULL: every sequence holds L_cap tokens)
 *   parent   int32, nullable: NULL = chain (parent[i] = i-1); otherwise
 *            [n_q] (parent_batch_stride 0, shared) or [B, n_q]
 *            (parent_batch_stride n_q); parent[i] in [-1, i), -1 = root;
 *            forests are allowed.
 *   n_q      1 .. SPEC_MAX_NQ;  D in {64, 128};  Hq % Hkv == 0;  L_cap >= n_q.
 *   scale    softmax scale; <= 0 selects 1/sqrt(D).
 *   num_splits  key-range splits per (sequence, kv head); 0 = automatic.  A
 *               launch of more than 2^22 work-groups (B * Hkv * splits * row
 *               slices) returns SPEC_ERR_UNSUPPORTED.
 *   workspace   at least spec_verify_attention_workspace(...) bytes,
 *               zero-filled before its first use (see Workspace above).
 * Returns SPEC_OK or an error status (nothing launched on error).
 */
spec_status_t spec_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                                    void* out, float* lse, const int32_t* kv_len,
                                    const int32_t* parent, int32_t parent_batch_stride,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D,
                                    int32_t L_cap, spec_dtype_t dtype, float scale,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    int32_t* dev_err, hipStream_t stream);

/* Workspace bytes spec_verify_attention needs for these sizes (0 on invalid sizes). */
size_t spec_verify_attention_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D,
                                       int32_t L_cap, spec_dtype_t dtype, int32_t num_splits);

/* Split count spec_verify_attention uses when num_splits == 0 (0 on invalid sizes). */
int32_t spec_verify_attention_auto_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q,
                                          int32_t D, int32_t L_cap, spec_dtype_t dtype);

/*
 * spec_verify_attention_paged -- spec_verify_attention over a paged KV cache.
 *
 * Defines: the same attention as spec_verify_attention.  "Guide to MagicDec"
 * places the target's verification in serving engines under continuous
 * batching (sections "High-Concurrency Serving Throughput and VRAM Footprint"
 * and 4, "High-Concurrency Memory Scheduling in Serving Engines": vLLM /
 * TensorRT-LLM schedulers), whose KV caches are lists of fixed-size blocks.
 * Here:
 *
 *   k_pages, v_pages  [num_pages, Hkv, P, D] dtype, one page = P consecutive
 *                     keys of every kv head of one sequence (heads outermost,
 *                     so one page-head is P*D contiguous elements);
 *   block_table       [B, block_table_stride] int32: page id holding keys
 *                     i*P .. i*P+P-1 of sequence b; stride >= ceil(L_max / P);
 *                     only the entries covering kv_len[b] keys are read;
 *   page_size (P)     a power of two, 64 .. 2^20;
 *   kv_len            [B] int32, required, in [n_q, L_max]; the block's own
 *                     K/V sit at keys kv_len-n_q .. kv_len-1 as in the
 *                     contiguous call;
 *   L_max             largest kv_len (sizes the launch plan and workspace).
 * Every other argument is as in spec_verify_attention.  A block_table entry
 * outside [0, num_pages) sets SPEC_DEVERR_PAGE; the key range of the split
 * that met it is dropped (the output stays finite, and no memory outside the
 * pool is read).  With pages, num_splits is raised where needed so a split's
 * keys span at most 511 pages.
 */
spec_status_t spec_verify_attention_paged(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
    int32_t block_table_stride, int32_t num_pages, int32_t page_size, void* out, float* lse,
    const int32_t* kv_len, const int32_t* parent, int32_t parent_batch_stride, int32_t B,
    int32_t Hq, int32_t Hkv, int32_t n_q, int32_t D, int32_t L_max, spec_dtype_t dtype,
    float scale, int32_t num_splits, void* workspace, size_t workspace_bytes, int32_t* dev_err,
    hipStream_t stream);

size_t spec_verify_attention_paged_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t n_q,
                                             int32_t D, int32_t L_max, int32_t page_size,
                                             spec_dtype_t dtype, int32_t num_splits);

/*
 * spec_window_attention -- bounded draft attention over sinks + a FIFO ring.
 *
 * Defines: "Guide to MagicDec", section 1 "Fixed-Window KV Cache Decoupling"
 * (the draft keeps only a W-token window managed as a circular FIFO, so its
 * attention cost is O(W) whatever the context length) and section "Best
 * Practices", item 1 (a few dedicated slots keep the first prompt tokens as
 * attention sinks).
 *
 * With T = total_len[b] tokens seen (the current one included), the keys are
 * tokens [0, min(S,T)) (sink slot t) and tokens [max(S, T-W), T) (token t in
 * ring slot (t-S) mod W).  One query per sequence, so no mask is applied.
 *
 *   q        [B, Hq, 1, D]    dtype
 *   k_ring   [B, Hkv, W, D]   dtype   ring slots (written only by the fused append)
 *   v_ring   [B, Hkv, W, D]   dtype
 *   k_sink   [B, Hkv, S, D]   dtype   nullable when S == 0
 *   v_sink   [B, Hkv, S, D]   dtype
 *   k_new    [B, Hkv, 1, D]   dtype, nullable: K/V of token T-1; if given it is
 *   v_new    [B, Hkv, 1, D]            written to its sink/ring slot and used
 *                                      in this same call (fused append)
 *   total_len [B] int32 (>= 1)
 *   out      [B, Hq, 1, D] dtype;  lse [B, Hq, 1] f32 nullable
 *   W >= 1, S >= 0, D in {64, 128}, Hq % Hkv == 0.
 *   num_splits, workspace: as in spec_verify_attention.
 */
spec_status_t spec_window_attention(const void* q, void* k_ring, void* v_ring, void* k_sink,
                                    void* v_sink, const void* k_new, const void* v_new,
                                    const int32_t* total_len, void* out, float* lse, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t D, int32_t W, int32_t S,
                                    spec_dtype_t dtype, float scale, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes, int32_t* dev_err,
                                    hipStream_t stream);

size_t spec_window_attention_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t W,
                                       int32_t S, spec_dtype_t dtype, int32_t num_splits);

/*
 * spec_sample -- acceptance test, residual resample and bonus draw.
 *
 * Defines: "Guide to MagicDec", section 2 (accept x with probability
 * min(1, p_target(x)/p_draft(x)); on rejection resample from the normalised
 * max(0, p_target - p_draft)) and its verifier code (bonus token from the
 * target row after the last draft when all are accepted); "Speculative
 * Decoding & Medusa Architecture", section 2 (one speculative sampling step);
 * "Speculative Decoding in LLM Serving Systems", section "Accepting and
 * rejecting" (walk left to right, stop at the first rejection, 1 .. gamma+1
 * tokens per round).
 *
 * Node view: node 0 is the last accepted token, nodes 1..N-1 are drafted
 * tokens, parent[c] < c.  A chain is N = gamma+1 with parent == NULL.
 *   target_logits [B, N, V] f32   row u: target next-token logits after node u
 *   draft_logits  [B, N, V] f32   row u: draft logits u's children were drawn
 *                                 from (rows of leaves are never read)
 *   tokens        [B, N] int32    drafted token of node c (tokens[b][0] unused)
 *   parent        int32 nullable: NULL = chain; [N] (parent_batch_stride 0)
 *                 or [B, N] (stride N); parent[0] = -1, parent[c] in [0, c).
 *   seed, offset  Philox4x32-10 key = seed; offset < 2^30 selects the round.
 *                 Node c's acceptance uniform is U(ctr = (c, 0, b, 4*offset)),
 *                 U(w) = (2*(w>>9)+1) * 2^-24 from output word 0.  Each node is
 *                 tested; the walk takes, at every node, its first child (in
 *                 index order) that passed.  The draw at the stop row is a
 *                 two-level exponential race over 1024-id chunks (counters
 *                 (chunk, row, b, 4*offset+2) and (id/4, row, b, 4*offset+3),
 *                 word id%4); ties go to the lowest index.
 * Outputs (all [B, ...], device):
 *   out_tokens [B, N] int32   accepted drafted tokens then the drawn token, -1 padded
 *   out_count  [B]    int32   emitted tokens (1 .. depth+1); 0 on a device-data error
 *   out_path   [B, N] int32   nullable: node ids of the accepted path from 0, -1 padded
 *   out_accept [B, N] uint8   nullable: per-node test result (node 0 reported 1)
 * N in 1 .. SPEC_MAX_SAMPLE_NODES, V >= 1.
 */
spec_status_t spec_sample(const float* target_logits, const float* draft_logits,
                          const int32_t* tokens, const int32_t* parent,
                          int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                          uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_count,
                          int32_t* out_path, uint8_t* out_accept, void* workspace,
                          size_t workspace_bytes, int32_t* dev_err, hipStream_t stream);

size_t spec_sample_workspace(int32_t B, int32_t N, int32_t V);

/*
 * spec_sample_bf16 -- spec_sample with bfloat16 logits.
 *
 * Defines: the same computation as spec_sample; the pages fix no logit
 * precision, and bf16 halves the bytes of the sampling tail.  target_logits
 * and draft_logits are [B, N, V] bfloat16 (bit patterns, 16-byte aligned);
 * every logit widens exactly to fp32 and the arithmetic is that of
 * spec_sample.  Workspace: spec_sample_workspace(B, N, V).
 */
spec_status_t spec_sample_bf16(const void* target_logits, const void* draft_logits,
                               const int32_t* tokens, const int32_t* parent,
                               int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                               uint64_t seed, uint64_t offset, int32_t* out_tokens,
                               int32_t* out_count, int32_t* out_path, uint8_t* out_accept,
                               void* workspace, size_t workspace_bytes, int32_t* dev_err,
                               hipStream_t stream);

/*
 * spec_draft_sample -- one draft-step token draw per sequence.
 *
 * Defines: "Guide to MagicDec", step 2 of its reference implementation (the
 * drafter): at each draft step the draft logits of the next position go
 * through a softmax and one token is drawn from the result; the verifier
 * later uses the same distribution (spec_sample recomputes it from the same
 * logits row).  The draw is an exponential race over p = softmax(l): id x
 * scores p_x / E_x with E_x = -ln U_x, U_x = U(ctr = (x/4, node, b,
 * 4*offset+1)) from output word x%4 (U as in spec_sample); the largest score
 * wins, ties go to the lowest id.  The race picks x with probability p_x.
 *
 *   draft_logits  dtype (SPEC_F32 or SPEC_BF16), row b at draft_logits +
 *                 b*row_stride elements, V entries (row_stride 0 = V).  With row_stride = N*V and the pointer
 *                 at row u of spec_sample's [B, N, V] draft logits, the draw
 *                 reads, in place, the row that u's child is drawn from.
 *   node          id of the node being drawn (chain: draft step j draws node
 *                 j+1); distinct nodes of one round get independent uniforms.
 *   seed, offset  as in spec_sample (same round => same offset).
 *   out_token     int32, out_token[b*token_stride] = drawn id (token_stride 0
 *                 = 1; with N it writes column `node` of spec_sample's tokens
 *                 array when out_token points at tokens + node).
 *   out_logprob   [B] fp32 nullable: ln p of the drawn id.
 *   workspace     spec_draft_sample_workspace(B, V) bytes.
 * A row with no finite logit sets SPEC_DEVERR_LOGITS and gets token -1 (and
 * a NaN log-probability).  Logits must be finite or -inf.
 */
spec_status_t spec_draft_sample(const void* draft_logits, spec_dtype_t dtype, int64_t row_stride,
                                int32_t B, int32_t V, uint64_t seed, uint64_t offset, int32_t node,
                                int32_t* out_token, int32_t token_stride, float* out_logprob,
                                void* workspace, size_t workspace_bytes, int32_t* dev_err,
                                hipStream_t stream);

size_t spec_draft_sample_workspace(int32_t B, int32_t V);

/*
 * spec_kv_commit -- keep the accepted path's K/V, drop the rest.
 *
 * Defines: "Speculative Decoding in LLM Serving Systems" (blog notes),
 * section "Core idea" (only the wrong guesses are rolled back), and "Guide to
 * MagicDec", step 3 of its reference implementation (verifier and rollback
 * controller).  Runs after spec_sample on the same round.  For every sequence
 * b with p0 = kv_len[b] - n_q (the block's first cache position, as in
 * spec_verify_attention) and c = count[b]:
 *     K[b,h,p0+j,:] = old K[b,h,p0+path[b][j],:]  and the same for V, j < c;
 *     kv_len[b]     = p0 + c;
 * positions before p0 are not touched, positions p0+c .. are left as they are
 * (stale, outside the new length).  The token drawn by spec_sample has no K/V
 * yet: it is the next round's node 0.
 *
 *   k_cache, v_cache  [B, Hkv, L_cap, D], dtype, updated in place
 *   kv_len            [B] int32, device, updated in place (must not be NULL)
 *   path              [B, n_q] int32 nullable: spec_sample's out_path (N = n_q).
 *                     NULL means a chain: the path is 0, 1, .., c-1 and no row
 *                     moves, only kv_len changes.
 *   count             [B] int32: spec_sample's out_count.  A sequence with
 *                     count 0 (flagged by spec_sample) is left unchanged.
 *   draft_total_len   [B] int32 nullable, device, updated in place: the draft
 *                     ring's total_len (spec_window_attention).  The draft
 *                     appended one entry per chain node 0 .. draft_appended-1
 *                     this round; the entries of nodes >= c are dropped:
 *                     total_len -= max(0, draft_appended - c).  Slots of
 *                     dropped entries are reused by the next appends.
 *   draft_appended    0 .. n_q (ignored when draft_total_len is NULL).
 * Device-data errors (kv_len outside [n_q, L_cap]; c outside [1, n_q]; a path
 * not starting at 0, not strictly increasing or reaching n_q; a rewind below 1)
 * set SPEC_DEVERR_KV_LEN / _PATH / _TOTAL_LEN and leave that sequence's cache
 * rows, kv_len and draft_total_len unchanged.
 * D in {64, 128}; the call needs no workspace.
 */
spec_status_t spec_kv_commit(void* k_cache, void* v_cache, int32_t* kv_len, const int32_t* path,
                             const int32_t* count, int32_t B, int32_t Hkv, int32_t n_q, int32_t D,
                             int32_t L_cap, spec_dtype_t dtype, int32_t* draft_total_len,
                             int32_t draft_appended, int32_t* dev_err, hipStream_t stream);

/*
 * spec_sample_ex -- spec_sample with a logit dtype and a sibling rule.
 *
 * Defines: spec_sample's computation, plus the rule for candidate trees.  The
 * pages name tree verification in the style of SpecInfer and Medusa ("Speculative
 * Decoding in LLM Serving Systems", section "Tree-based variants"; "Speculative
 * Decoding & Medusa Architecture", section 4) without the acceptance rule
 * among siblings.
 *   SPEC_SIBLINGS_FIRST     spec_sample's rule: each node c is tested with its
 *                           own uniform against min(1, p(x_c)/q(x_c)) at its
 *                           parent; the walk takes the first child that passed.
 *   SPEC_SIBLINGS_LOSSLESS  at the node the walk stands on, its children are
 *                           tested in index order against p_i, where p_0 = p
 *                           and p_{i+1} = normalised max(p_i - q, 0) after
 *                           child i is rejected (q the node's draft row); the
 *                           first child with u_c < p_i(x_c)/q(x_c) is taken.
 *                           If all are rejected the draw comes from the last
 *                           p_i (from p if its mass vanishes).  When siblings
 *                           are drawn independently from q, every emitted token
 *                           follows the target distribution.  Each rejected
 *                           sibling costs one pass over the node's two rows, in
 *                           one extra kernel with one work-group per sequence.
 *                           Untested nodes report out_accept 0.
 * For a chain both rules give the same tokens, counts and paths.
 * logits_dtype: SPEC_F32 (as spec_sample) or SPEC_BF16 (as spec_sample_bf16).
 * Other arguments and the workspace are as in spec_sample.
 */
spec_status_t spec_sample_ex(const void* target_logits, const void* draft_logits,
                             spec_dtype_t logits_dtype, spec_sibling_rule_t siblings,
                             const int32_t* tokens, const int32_t* parent,
                             int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                             uint64_t seed, uint64_t offset, int32_t* out_tokens,
                             int32_t* out_count, int32_t* out_path, uint8_t* out_accept,
                             void* workspace, size_t workspace_bytes, int32_t* dev_err,
                             hipStream_t stream);

/*
 * spec_sample_noalloc -- spec_sample_ex without a workspace: allocates nothing.
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same computation, arguments (minus workspace/workspace_bytes),
 * layouts and outputs as spec_sample_ex, with the same kernels.  Instead of a
 * caller workspace the call uses a library-owned device array of
 * SPEC_NOALLOC_SCRATCH_BYTES bytes per GPU (a static device variable: no
 * hipMalloc, hipFree or allocating library routine is called).  Its address
 * is looked up once per device, on the first call made with that device
 * current; the caller's current device must be the device `stream` belongs to.
 *
 * Limit: sizes whose workspace, spec_sample_workspace(B, N, V), exceeds
 * SPEC_NOALLOC_SCRATCH_BYTES return SPEC_ERR_UNSUPPORTED (nothing launched).
 * The array's arrival counters are cleared by a small kernel at the start of
 * every call, so a call never depends on what an earlier call left there.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on the same device (different streams, or several host threads)
 * race on it and must be serialised by the caller.
 */
spec_status_t spec_sample_noalloc(const void* target_logits, const void* draft_logits,
                                  spec_dtype_t logits_dtype, spec_sibling_rule_t siblings,
                                  const int32_t* tokens, const int32_t* parent,
                                  int32_t parent_batch_stride, int32_t B, int32_t N, int32_t V,
                                  uint64_t seed, uint64_t offset, int32_t* out_tokens,
                                  int32_t* out_count, int32_t* out_path, uint8_t* out_accept,
                                  int32_t* dev_err, hipStream_t stream);

/*
 * spec_validate_tree -- host-side check of a parent array (host pointer).
 * Valid: parent[c] in [-1, c) for every c; with require_single_root also
 * parent[0] == -1 and parent[c] >= 0 for c >= 1.  Returns SPEC_OK,
 * SPEC_ERR_BAD_TREE, or SPEC_ERR_INVALID_ARG (NULL pointer, n < 1).
 */
spec_status_t spec_validate_tree(const int32_t* parent_host, int32_t n,
                                 int32_t require_single_root);

/* Static, human-readable name of a status code. */
const char* spec_status_str(spec_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
