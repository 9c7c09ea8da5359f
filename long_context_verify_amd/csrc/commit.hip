// commit.hip -- keep the accepted path's K/V after verification (gfx950).
//
// "Speculative Decoding in LLM Serving Systems", section "Core idea": guess,
// check, and roll back only what turned out wrong; "Guide to MagicDec",
// step 3 of its reference implementation (verifier and rollback controller).
// The verified block's cache rows p0 .. p0+n_q-1 (p0 = kv_len - n_q) hold the
// K/V of every drafted node.  The next round needs the prefix followed by the
// accepted path only:
//     cache[p0 + j] <- cache[p0 + path[j]]   for j < count,
//     kv_len        <- p0 + count.
// The draft model's ring drops the entries of rejected drafts: it appended
// one entry per chain node 0 .. appended-1, of which the first count survive.
//
// Work-group (b, kv head, K|V) stages its source rows in LDS and writes them
// back in path order, so moves that overlap (path[j] > j) never read a row
// that is already overwritten.  A chain's path is the identity and moves
// nothing.  The lengths are updated by a second, tiny kernel, after every
// move of the sequence has read the old kv_len.

#include <hip/hip_runtime.h>

#include "spec_common.hpp"
#include "spec_internal.hpp"

namespace specv {

constexpr int kCommitThreads = 256;

// The path of sequence b, or the identity when no path is given.
__device__ __forceinline__ int path_at(const CommitArgs& a, int b, int j) {
  return a.path ? a.path[(size_t)b * a.n_q + j] : j;
}

// 0 when sequence b can be committed; otherwise the error bits it earns
// (-1: a sequence the sampler already flagged, out_count == 0: left alone).
__device__ __forceinline__ int commit_check(const CommitArgs& a, int b, int& p0, int& count) {
  const int L = a.kv_len[b];
  count = a.count[b];
  p0 = L - a.n_q;
  if (count == 0) return -1;
  if (L < a.n_q || L > a.L_cap) return SPEC_DEVERR_KV_LEN;
  if (count < 1 || count > a.n_q || path_at(a, b, 0) != 0) return SPEC_DEVERR_PATH;
  for (int j = 1; j < count; ++j) {
    const int pj = path_at(a, b, j);
    if (pj <= path_at(a, b, j - 1) || pj >= a.n_q) return SPEC_DEVERR_PATH;
  }
  if (a.draft_total_len && a.draft_total_len[b] - (a.draft_appended - count) < 1 &&
      a.draft_appended > count)
    return SPEC_DEVERR_TOTAL_LEN;
  return 0;
}

__global__ __launch_bounds__(kCommitThreads) void kv_commit_move(CommitArgs a) {
  extern __shared__ u32x4 stage[];  // [count - j0][row_bytes / 16]
  const int unit = blockIdx.x;      // b * Hkv + kv head
  const int b = unit / a.Hkv;
  int p0, count;
  if (commit_check(a, b, p0, count) != 0) return;
  // path[j] == j up to the first moved row j0; after it path[j] > j throughout.
  int j0 = 0;
  while (j0 < count && path_at(a, b, j0) == j0) ++j0;
  if (j0 == count) return;
  const int n16 = a.row_bytes / 16;
  char* base = static_cast<char*>(blockIdx.y ? a.v : a.k) +
               ((size_t)unit * a.L_cap + p0) * (size_t)a.row_bytes;
  const int total = (count - j0) * n16;
  for (int i = threadIdx.x; i < total; i += kCommitThreads) {
    const int j = j0 + i / n16, piece = i % n16;
    const char* src = base + (size_t)path_at(a, b, j) * a.row_bytes;
    stage[i] = reinterpret_cast<const u32x4*>(src)[piece];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < total; i += kCommitThreads) {
    const int j = j0 + i / n16, piece = i % n16;
    reinterpret_cast<u32x4*>(base + (size_t)j * a.row_bytes)[piece] = stage[i];
  }
}

__global__ __launch_bounds__(kCommitThreads) void kv_commit_lengths(CommitArgs a) {
  const int b = blockIdx.x * kCommitThreads + threadIdx.x;
  if (b >= a.B) return;
  int p0, count;
  const int bad = commit_check(a, b, p0, count);
  if (bad) {
    if (bad > 0) report_error(a.dev_err, bad);
    return;
  }
  a.kv_len[b] = p0 + count;
  if (a.draft_total_len && a.draft_appended > count)
    a.draft_total_len[b] -= a.draft_appended - count;
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t stream) {
  dim3 block(kCommitThreads);
  if (a.path) {
    const size_t lds = (size_t)a.n_q * a.row_bytes;
    hipLaunchKernelGGL(kv_commit_move, dim3(a.B * a.Hkv, 2), block, lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kv_commit_lengths, dim3((a.B + kCommitThreads - 1) / kCommitThreads), block,
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace specv
