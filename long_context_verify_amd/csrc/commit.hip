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
// One work-group per sequence stages the source rows of every kv head in LDS
// before writing them back in path order, so moves that overlap
// (path[j] > j) never read a row that is already overwritten, and then sets
// the lengths.  A chain's path is the identity and moves nothing.

#include <hip/hip_runtime.h>

#include "spec_common.hpp"
#include "spec_internal.hpp"

namespace specv {

constexpr int kCommitThreads = 256;
constexpr int kCommitBatch = 2048;   // 16-byte pieces staged per round (32 KB of LDS)

// Validation of one sequence by one wave, all loads issued at once: lane t
// holds path[t] (t < n_q; the identity when no path is given).  status is 0
// when the sequence can be committed, -1 for a sequence the sampler already
// flagged (count 0: left alone, no new error), else the error bits it earns.
struct CommitView {
  int status, p0, count, path;
};

__device__ __forceinline__ CommitView commit_check(const CommitArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  const int L = a.kv_len[b];
  const int count = a.count[b];
  const int T = a.draft_total_len ? a.draft_total_len[b] : 0x40000000;
  int pj = lane;
  if (a.path && lane < a.n_q) pj = a.path[(size_t)b * a.n_q + lane];
  const int prev = __shfl(pj, lane > 0 ? lane - 1 : 0);
  CommitView v{0, L - a.n_q, count, pj};
  if (count == 0) {
    v.status = -1;
  } else if (L < a.n_q || L > a.L_cap) {
    v.status = SPEC_DEVERR_KV_LEN;
  } else if (count < 1 || count > a.n_q) {
    v.status = SPEC_DEVERR_PATH;
  } else {
    // path[0] == 0, strictly increasing, below n_q.
    const bool bad = lane < count && (lane == 0 ? pj != 0 : (pj <= prev || pj >= a.n_q));
    if (__any(bad))
      v.status = SPEC_DEVERR_PATH;
    else if (a.draft_total_len && a.draft_appended > count && T - (a.draft_appended - count) < 1)
      v.status = SPEC_DEVERR_TOTAL_LEN;
  }
  return v;
}

// One work-group per sequence: it alone reads and writes that sequence's
// rows and lengths, so one launch needs no ordering between work-groups.
// The rows to move (every kv head, K and V) are staged through LDS in
// batches of kCommitBatch 16-byte pieces: all loads of a batch, a barrier,
// all stores, a barrier.
__global__ __launch_bounds__(kCommitThreads) void kv_commit(CommitArgs a) {
  __shared__ u32x4 stage[kCommitBatch];
  const int b = blockIdx.x;
  const CommitView cv = commit_check(a, b);
  const int lane = threadIdx.x & 63;
  if (cv.status != 0) {
    if (cv.status > 0 && threadIdx.x == 0) report_error(a.dev_err, cv.status);
    return;
  }
  // path[j] == j up to the first moved row j0; after it path[j] > j throughout.
  const uint64_t moved = __ballot(lane < cv.count && cv.path != lane);
  if (moved) {
    const int j0 = __builtin_ctzll(moved);
    const int n16 = a.row_bytes / 16;
    const int per_pair = (cv.count - j0) * n16;    // pieces per (kv head, K|V)
    const int total = 2 * a.Hkv * per_pair;
    for (int base_i = 0; base_i < total; base_i += kCommitBatch) {
      const int n = min(kCommitBatch, total - base_i);
      char* dst[kCommitBatch / kCommitThreads];
#pragma unroll
      for (int k = 0; k < kCommitBatch / kCommitThreads; ++k) {
        const int t = k * kCommitThreads + threadIdx.x;
        const int i = base_i + (t < n ? t : 0);
        const int pair = i / per_pair, rem = i - pair * per_pair;
        const int j = j0 + rem / n16, piece = rem % n16;
        const int src_row = __shfl(cv.path, j);   // every lane takes part in the shuffle
        char* row0 = static_cast<char*>((pair & 1) ? a.v : a.k) +
                     (((size_t)b * a.Hkv + (pair >> 1)) * a.L_cap + cv.p0) * (size_t)a.row_bytes +
                     (size_t)piece * 16;
        dst[k] = row0 + (size_t)j * a.row_bytes;
        if (t < n) stage[t] = *reinterpret_cast<const u32x4*>(row0 + (size_t)src_row * a.row_bytes);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kCommitBatch / kCommitThreads; ++k) {
        const int t = k * kCommitThreads + threadIdx.x;
        if (t < n) *reinterpret_cast<u32x4*>(dst[k]) = stage[t];
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    a.kv_len[b] = cv.p0 + cv.count;
    if (a.draft_total_len && a.draft_appended > cv.count)
      a.draft_total_len[b] -= a.draft_appended - cv.count;
  }
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_commit, dim3(a.B), dim3(kCommitThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace specv
