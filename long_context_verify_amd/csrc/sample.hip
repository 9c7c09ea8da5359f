// sample.hip -- the speculative-sampling tail on gfx950.
//
// What is computed ("Guide to MagicDec", section 2 and its verifier code;
// "Speculative Decoding & Medusa Architecture", section 2; "Speculative
// Decoding in LLM Serving Systems", section "Accepting and rejecting"):
// per sequence, each drafted token x at node c is tested against
// min(1, p_target(x) / p_draft(x)) taken at c's parent; the walk from the
// root keeps the accepted prefix; at the stop node one token is drawn from
// the normalised max(p_target - p_draft, 0) (after a rejection) or from
// p_target (when the walk ends at a leaf: the bonus token).
//
// Two kernels, back to back on the caller's stream (no work-group waits on
// another; the second phase's last work-group of a sequence finishes it):
//
//   sample_stats   grid (vocab chunks, 2N rows, B).  Streams, once, the rows
//                  the decision needs: the target and draft rows of nodes that
//                  have children (and, for the lossless rule, the target rows
//                  of leaves too), with non-temporal loads, and writes
//                  per-chunk (max, sum of exp(x - max)); fp32 inside a thread,
//                  fp64 across threads.
//   sample_resid   grid (groups, B).  Every work-group of a sequence derives
//                  the same decision (fp64 log-normalisers, one Philox uniform
//                  and acceptance test per node, the walk from the root over
//                  parents held in LDS: a few hundred scalars after one round
//                  of loads), then the residual (or target) mass of its
//                  1024-id race chunks of the stop row (non-temporal loads,
//                  four chunks in flight at once).  When the walk
//                  ends at a leaf whose target row the first kernel skipped,
//                  the groups gather that row's per-chunk (max, sum) instead,
//                  so a leaf row is read once, and only when it is drawn from.
//                  The group that completes the sequence's masses (an arrival
//                  counter per sequence in the workspace) runs the two-level
//                  exponential race in fp64 at the stop row and writes the
//                  outputs.
// With the lossless sibling rule a decide kernel (one work-group per
// sequence) runs between the two and stores the decision record that the
// residual groups read.
//
// Randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11: four 32-bit
// counter words, two key words, ten rounds of two 32x32->64 multiplies with
// the published multipliers and Weyl key bumps), uniform
// U = (2 (w >> 9) + 1) 2^-24.  Counters:
//   accept test of node c:      (c, 0, b, 4*offset + 0), word 0
//   race over chunks at row r:  (chunk, r, b, 4*offset + 2), word 0
//   race over ids in a chunk:   (id / 4, r, b, 4*offset + 3), word id % 4
//   draft-step draw of node c:  (id / 4, c, b, 4*offset + 1), word id % 4

#include <hip/hip_runtime.h>

#include <mutex>

#include "spec_common.hpp"
#include "spec_internal.hpp"

namespace specv {

constexpr int kSampleThreads = 256;
constexpr int kDecideThreads = 512;    // lossless decide: one work-group streams the rows
constexpr int kRaceChunk = 1024;
constexpr int kStatsChunk = 8192;   // ids per stats work-group (32 per thread)
constexpr int kDraftChunkSmall = 2048;   // ids per draft-draw work-group (8 per thread)
constexpr int kDraftChunkLarge = 4096;   // the same at large batch (16 per thread)
constexpr int kArriveFan = 16;      // residual groups per first-level arrival counter
constexpr int kArrivePad = 16;      // counters 64 bytes apart
constexpr int kArriveStride = kArrivePad * (kArriveFan + 1);   // counters per sequence

// Arrival of member `i` of a group of n work-groups at a two-level tree of
// counters (kArriveStride of them at ctr): true in the last to arrive.  A
// hundred work-groups incrementing one counter would serialise on it.
__device__ __forceinline__ bool last_of_group(uint32_t* ctr, int i, int n, int32_t* dev_err) {
  const int sub = i % kArriveFan;
  const int n_sub = (n - 1 - sub) / kArriveFan + 1;
  if (!last_arrival(ctr + kArrivePad * sub, (uint32_t)n_sub, dev_err)) return false;
  return last_arrival(ctr + kArrivePad * kArriveFan, (uint32_t)min(kArriveFan, n), dev_err);
}

__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
}

__device__ __forceinline__ double uniform24(uint32_t w) {
  return ((double)(w >> 9) * 2.0 + 1.0) * 5.9604644775390625e-08;  // 2^-24
}

// Logit loads, fp32 or bf16 in memory, fp32 in registers (bf16 widens exactly).
template <typename T>
__device__ __forceinline__ float ld1(const T* row, size_t e) {
  return (float)row[e];
}
// Ids e .. e+3 (e a multiple of 4, rows aligned to whole vectors): one 16-byte
// (fp32) or 8-byte (bf16) load; NT: non-temporal (data read once).
template <typename T, bool NT = false>
__device__ __forceinline__ f32x4 ld4(const T* row, size_t e) {
  if constexpr (sizeof(T) == 4) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row) + (e >> 2);
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  } else {
    const unsigned long long* p = reinterpret_cast<const unsigned long long*>(row) + (e >> 2);
    unsigned long long v;
    if constexpr (NT) v = __builtin_nontemporal_load(p);
    else v = *p;
    const uint2 w = {(uint32_t)v, (uint32_t)(v >> 32)};
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
  }
}

__device__ __forceinline__ int parent_of(const SampleArgs& a, int b, int c) {
  if (!a.parent) return c - 1;
  return a.parent[(size_t)b * a.parent_stride + c];
}

// Block-wide reductions (256 threads = 4 waves) through a small LDS scratch.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Sum over a work-group of NT threads (NT / 64 waves).
template <int NT>
__device__ __forceinline__ double block_sum_nt(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) t += red[k];
  return t;
}

// Arg-max of (score, index) with ties to the lowest index.
__device__ __forceinline__ void better(double& s, int& i, double s2, int i2) {
  if (s2 > s || (s2 == s && i2 < i)) {
    s = s2;
    i = i2;
  }
}
__device__ __forceinline__ void block_argmax(double& s, int& i, double* reds, int* redi) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double s2 = __shfl_xor(s, off);
    const int i2 = __shfl_xor(i, off);
    better(s, i, s2, i2);
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    reds[w] = s;
    redi[w] = i;
  }
  __syncthreads();
  s = reds[0];
  i = redi[0];
#pragma unroll
  for (int k = 1; k < 4; ++k) better(s, i, reds[k], redi[k]);
}

// ---------------------------------------------------------------------------
// Row statistics.
// ---------------------------------------------------------------------------
template <bool VEC4, typename T>
__global__ __launch_bounds__(kSampleThreads) void sample_stats(SampleArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int chunk = blockIdx.x, rowsel = blockIdx.y, b = blockIdx.z;
  const int kind = rowsel >= a.N;  // 0: target row, 1: draft row
  const int u = rowsel - kind * a.N;
  if (kind || !a.leaf_rows) {
    // Draft rows are needed only at nodes that have children, and so are
    // target rows unless the leaves' are streamed here too (the residual
    // pass reads a leaf's target row if the walk stops there).
    int has;
    if (!a.parent) {
      has = u < a.N - 1;
    } else {
      has = 0;
      for (int c = 1 + threadIdx.x; c < a.N; c += kSampleThreads) has |= parent_of(a, b, c) == u;
      has = __syncthreads_or(has);
    }
    if (!has) return;
  }
  const T* row = static_cast<const T*>(kind ? a.draft : a.target) + ((size_t)b * a.N + u) * a.V;
  const int x0 = chunk * a.vchunk;
  // Node c = 1 + thread (N <= threads): its parent and drafted token, loaded
  // ahead of the row so that their use below waits for nothing else.
  static_assert(SPEC_MAX_SAMPLE_NODES <= kSampleThreads + 1, "one child per thread");
  const int c = 1 + threadIdx.x;
  int pc = -1, xc = -1;
  if (c < a.N) {
    pc = parent_of(a, b, c);
    xc = a.tokens[(size_t)b * a.N + c];
  }
  constexpr int PER = kStatsChunk / kSampleThreads;  // 32
  float x[PER];
  if (VEC4) {
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) {
      const int e = x0 + 4 * (threadIdx.x + kSampleThreads * i);
      f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (e < a.V) v = ld4<T, true>(row, e);   // V % 4 == 0: a vector is wholly in or out
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * i + k] = v[k];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = x0 + threadIdx.x + kSampleThreads * i;
      x[i] = e < a.V ? ld1(row, e) : -INFINITY;
    }
  }
  // The drafted tokens of u's children that fall in this chunk: their logits
  // in this row go to the workspace (stored at the end, so the load is not
  // waited for), and the decision reads them in the same round as the row
  // statistics.
  const bool gather = pc == u && xc >= x0 && xc < x0 + a.vchunk && xc < a.V;
  const float xlogit = gather ? ld1(row, xc) : 0.f;
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < PER; ++i) mx = fmaxf(mx, x[i]);
  mx = block_max(mx, redf);
  float s = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int i = 0; i < PER; ++i) s += fast_exp2((x[i] - mx) * kLog2e);
  }
  const double tot = block_sum((double)s, redd);
  if (threadIdx.x == 0) {
    const size_t o = ((size_t)b * 2 * a.N + rowsel) * a.n_vchunks + chunk;
    a.part_m[o] = mx;
    a.part_s[o] = tot;
  }
  if (gather) a.tok_logit[((size_t)b * 2 + kind) * a.N + c] = xlogit;
}

// ---------------------------------------------------------------------------
// Decision and residual masses.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// The decision of one sequence, computed by a whole work-group: fp64
// log-normalisers from the per-chunk partials, one Philox uniform and
// acceptance test per drafted node, and the walk from the root.  Every global
// load it needs is issued up front, so it costs about two memory round trips.
struct Decision {
  float m[2][SPEC_MAX_SAMPLE_NODES];      // row max (target, draft)
  double lz[2][SPEC_MAX_SAMPLE_NODES];    // row log normaliser
  double s[2][SPEC_MAX_SAMPLE_NODES];     // row sum of exp(x - max)
  uint8_t has_child[SPEC_MAX_SAMPLE_NODES];
  uint8_t acc[SPEC_MAX_SAMPLE_NODES];
  int path[SPEC_MAX_SAMPLE_NODES];
  int tok[SPEC_MAX_SAMPLE_NODES];         // drafted token of each node
  int16_t par[SPEC_MAX_SAMPLE_NODES];     // parent of each node (loaded once)
  int len, bad, stop;
  bool residual;
  double shift;                           // residual weights max(pt - shift * pd, 0)
};

// Per-node inputs of the lossless sibling walk.
struct SiblingTests {
  double ratio0[SPEC_MAX_SAMPLE_NODES];   // p_target(x_c) / p_draft(x_c) at the parent
  double pt[SPEC_MAX_SAMPLE_NODES];       // p_target(x_c) at the parent
  double pd[SPEC_MAX_SAMPLE_NODES];       // p_draft(x_c) at the parent
  float u[SPEC_MAX_SAMPLE_NODES];         // acceptance uniform of node c
  int16_t par[SPEC_MAX_SAMPLE_NODES];
  double red[kDecideThreads / kWave];
};

template <typename T, int NT, bool CACHE>
__device__ void lossless_walk(const SampleArgs& a, int b, Decision& d, SiblingTests& st);

// NT: threads of the calling work-group.
template <typename T, bool LOSSLESS = false, int NT = kSampleThreads, bool CACHE = false>
__device__ __forceinline__ void decide_sequence(const SampleArgs& a, int b, Decision& d,
                                SiblingTests* st = nullptr) {
  const int N = a.N, V = a.V;
  const int tid = threadIdx.x;

  // One round of loads: the drafted tokens, their logits at the parent
  // (gathered by the stats kernel; valid wherever the token and parent are),
  // and this thread's first row partial of the fold below.
  const int nv = a.n_vchunks;
  const int GL = nv >= 64 ? 64 : (nv > 32 ? 64 : nv > 16 ? 32 : nv > 8 ? 16 : nv > 4 ? 8 : 4);
  const int rows_per_pass = NT / GL;
  float pm0 = -INFINITY;
  double ps0 = 0.0;
  if (tid / GL < 2 * N && tid % GL < nv) {
    const size_t o = ((size_t)b * 2 * N + tid / GL) * nv + tid % GL;
    pm0 = a.part_m[o];
    ps0 = a.part_s[o];
  }
  float tl = 0.f, dl = 0.f;
  int x = 0, p = -1;
  const int c_tok = 1 + tid;
  if (c_tok < N) {
    p = parent_of(a, b, c_tok);
    x = a.tokens[(size_t)b * N + c_tok];
    tl = a.tok_logit[(size_t)b * 2 * N + c_tok];
    dl = a.tok_logit[((size_t)b * 2 + 1) * N + c_tok];
  }
  if (tid == 0) d.bad = 0;
  for (int u = tid; u < N; u += NT) d.has_child[u] = 0;
  if (c_tok < N) {
    d.tok[c_tok] = x;
    d.par[c_tok] = (int16_t)p;
  }
  __syncthreads();
  for (int c = 1 + tid; c < N; c += NT) {
    const int pc = c == c_tok ? p : parent_of(a, b, c);
    if (pc < 0 || pc >= c)
      d.bad = 1;
    else
      d.has_child[pc] = 1;
  }
  if (tid == 0 && a.parent && parent_of(a, b, 0) != -1) d.bad = 1;
  __syncthreads();
  const bool bad_tree = d.bad != 0;

  // Fold the per-chunk partials of every needed row: GL lanes per row, all
  // rows side by side (the first partial of each lane was loaded above).
  for (int base = 0; base < 2 * N; base += rows_per_pass) {
    const int rs = base + tid / GL;
    const int k0 = tid % GL;
    const int kind = rs >= N;
    const int u = rs - kind * N;
    const bool need =
        rs < 2 * N && ((!kind && a.leaf_rows) || (!bad_tree && d.has_child[u]));
    const size_t o = ((size_t)b * 2 * N + rs) * nv;
    float mk = -INFINITY;
    double sk = 0.0;
    float m = -INFINITY;
    if (need)
      for (int k = k0; k < nv; k += GL) m = fmaxf(m, (base == 0 && k == k0) ? pm0 : a.part_m[o + k]);
    for (int off = GL >> 1; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    double sum = 0.0;
    if (need && m != -INFINITY)
      for (int k = k0; k < nv; k += GL) {
        const bool first = base == 0 && k == k0;
        mk = first ? pm0 : a.part_m[o + k];
        sk = first ? ps0 : a.part_s[o + k];
        if (mk != -INFINITY) sum += sk * exp((double)mk - (double)m);
      }
    for (int off = GL >> 1; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (need && k0 == 0) {
      d.m[kind][u] = m;
      d.s[kind][u] = sum;
      d.lz[kind][u] = (double)m + log(sum);
    }
  }
  __syncthreads();
  if constexpr (LOSSLESS) {
    // Per-node log-probabilities and uniforms; the walk tests them in order.
    if (tid == 0) d.acc[0] = 1;
    if (c_tok < N) {
      d.acc[c_tok] = 0;
      st->par[c_tok] = (int16_t)p;
      if (!bad_tree) {
        if (x < 0 || x >= V) {
          d.bad = 2;
        } else {
          const double lp = (double)tl - d.lz[0][p], lq = (double)dl - d.lz[1][p];
          // The plain ratio is computed as in the first-accepted rule.
          st->ratio0[c_tok] = (dl == -INFINITY) ? ((tl == -INFINITY) ? 0.0 : INFINITY)
                                                : exp(lp - lq);
          st->pt[c_tok] = exp(lp);
          st->pd[c_tok] = exp(lq);
          uint32_t c0 = (uint32_t)c_tok, c1 = 0u, c2 = (uint32_t)b, c3 = a.ctr3_base + 0u;
          philox4x32_10(c0, c1, c2, c3, a.key0, a.key1);
          st->u[c_tok] = (float)uniform24(c0);
        }
      }
    }
    __syncthreads();
    lossless_walk<T, NT, CACHE>(a, b, d, *st);
    return;
  }
  if (tid == 0) d.acc[0] = 1;
  if (c_tok < N) {
    bool ok = false;
    if (!bad_tree) {
      if (x < 0 || x >= V) {
        d.bad = 2;
      } else {
        double ratio;
        if (dl == -INFINITY)
          ratio = (tl == -INFINITY) ? 0.0 : INFINITY;
        else
          ratio = exp(((double)tl - d.lz[0][p]) - ((double)dl - d.lz[1][p]));
        uint32_t c0 = (uint32_t)c_tok, c1 = 0u, c2 = (uint32_t)b, c3 = a.ctr3_base + 0u;
        philox4x32_10(c0, c1, c2, c3, a.key0, a.key1);
        ok = uniform24(c0) < ratio;
      }
    }
    d.acc[c_tok] = ok;
  }
  __syncthreads();
  const bool bad = d.bad != 0;
  // Walk from the root: at each node take the first child, in index order,
  // that passed its test.  Children have larger indices than their parent.
  if (tid < kWave) {
    int cur = 0, len = 1;
    if (tid == 0) d.path[0] = 0;
    if (!bad) {
      while (true) {
        int nxt = -1;
        for (int base = cur + 1; base < N && nxt < 0; base += kWave) {
          const int c = base + tid;
          const bool hit = c < N && d.acc[c] && d.par[c] == cur;
          const unsigned long long ball = __ballot(hit);
          if (ball) nxt = base + __ffsll((long long)ball) - 1;
        }
        if (nxt < 0) break;
        if (tid == 0) d.path[len] = nxt;
        ++len;
        cur = nxt;
      }
    }
    if (tid == 0) {
      d.len = len;
      d.stop = cur;
      d.residual = d.has_child[cur] != 0;
      d.shift = 1.0;
    }
  }
  __syncthreads();
}

// Sum over the vocabulary of max(pt - shift * pd, 0) at row r (fp32 terms, fp64
// accumulation): the mass left after `shift` draft distributions are taken off.
template <typename T, int NT>
__device__ double residual_mass(const SampleArgs& a, int b, int r, const Decision& d,
                                double shift, double* red) {
  const int N = a.N, V = a.V;
  const T* trow = static_cast<const T*>(a.target) + ((size_t)b * N + r) * V;
  const T* drow = static_cast<const T*>(a.draft) + ((size_t)b * N + r) * V;
  const float tm = d.m[0][r], tinv = (float)(1.0 / d.s[0][r]);
  const float dm = d.m[1][r], dinv = (float)(1.0 / d.s[1][r]);
  const float sh = (float)shift;
  double acc = 0.0;
  if (V % 4 == 0) {
    // Batches of kU vectors per row per thread, all loads issued before any
    // use: one work-group streams the rows, so memory parallelism sets the pace.
    constexpr int kU = 8;
    for (int e0 = 4 * threadIdx.x; e0 < V; e0 += 4 * NT * kU) {
      f32x4 t4[kU], d4[kU];
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int e = e0 + 4 * NT * j;
        t4[j] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        d4[j] = t4[j];
        if (e < V) {
          t4[j] = ld4(trow, e);
          d4[j] = ld4(drow, e);
        }
      }
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < kU; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float pt = fast_exp2((t4[j][k] - tm) * kLog2e) * tinv;
          const float pd = fast_exp2((d4[j][k] - dm) * kLog2e) * dinv;
          part += fmaxf(pt - sh * pd, 0.f);
        }
      acc += (double)part;
    }
  } else {
    for (int e = threadIdx.x; e < V; e += NT) {
      const float pt = fast_exp2((ld1(trow, e) - tm) * kLog2e) * tinv;
      const float pd = fast_exp2((ld1(drow, e) - dm) * kLog2e) * dinv;
      acc += (double)fmaxf(pt - sh * pd, 0.f);
    }
  }
  return block_sum_nt<NT>(acc, red);
}

// Row r's probabilities held in registers: thread t keeps ids 4 t + 4 NT j + k
// (j < kCacheVec, k < 4), the layout of residual_mass's first batch, so the
// sums below add the same terms in the same order.
constexpr int kCacheVec = 16;

template <typename T, int NT>
__device__ __forceinline__ void load_row_probs(const SampleArgs& a, int b, int r,
                                               const Decision& d, float (&cpt)[4 * kCacheVec],
                                               float (&cpd)[4 * kCacheVec]) {
  const int N = a.N, V = a.V;
  const T* trow = static_cast<const T*>(a.target) + ((size_t)b * N + r) * V;
  const T* drow = static_cast<const T*>(a.draft) + ((size_t)b * N + r) * V;
  const float tm = d.m[0][r], tinv = (float)(1.0 / d.s[0][r]);
  const float dm = d.m[1][r], dinv = (float)(1.0 / d.s[1][r]);
  // Two halves, so at most half the raw vectors are live next to the cache.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    constexpr int HV = kCacheVec / 2;
    f32x4 t4[HV], d4[HV];
#pragma unroll
    for (int jj = 0; jj < HV; ++jj) {
      const int e = 4 * threadIdx.x + 4 * NT * (h * HV + jj);
      t4[jj] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      d4[jj] = t4[jj];
      if (e < V) {
        t4[jj] = ld4(trow, e);
        d4[jj] = ld4(drow, e);
      }
    }
#pragma unroll
    for (int jj = 0; jj < HV; ++jj)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cpt[4 * (h * HV + jj) + k] = fast_exp2((t4[jj][k] - tm) * kLog2e) * tinv;
        cpd[4 * (h * HV + jj) + k] = fast_exp2((d4[jj][k] - dm) * kLog2e) * dinv;
      }
  }
}

template <int NT>
__device__ __forceinline__ double cached_mass(const float (&cpt)[4 * kCacheVec],
                                              const float (&cpd)[4 * kCacheVec], double shift,
                                              double* red) {
  const float sh = (float)shift;
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4 * kCacheVec; ++i) part += fmaxf(cpt[i] - sh * cpd[i], 0.f);
  return block_sum_nt<NT>((double)part, red);
}

// Lossless sibling rule: at each node its children are tested in index order
// against p_i = max(p - shift_i q, 0) / mass_i (p_0 = p); after a rejection
// shift_{i+1} = shift_i + mass_i and mass_{i+1} = sum max(p - shift_{i+1} q, 0),
// the closed form of normalising max(p_i - q, 0).  One vocabulary pass per
// rejected sibling.  If every child is rejected the draw uses the residual
// max(p - shift q, 0); a vanished mass falls back to p.
// CACHE: the rows fit in registers (V % 4 == 0, V <= 4 kCacheVec NT).
template <typename T, int NT, bool CACHE>
__device__ void lossless_walk(const SampleArgs& a, int b, Decision& d, SiblingTests& st) {
  const int N = a.N;
  const int tid = threadIdx.x;
  const bool bad = d.bad != 0;
  int cur = 0, len = 1;
  if (tid == 0) d.path[0] = 0;
  bool residual = false;
  double shift = 0.0;
  // With CACHE the node's rows stay in registers while its siblings are
  // tested: one load and one set of exponentials per node.
  float cpt[CACHE ? 4 * kCacheVec : 1], cpd[CACHE ? 4 * kCacheVec : 1];
  if (!bad) {
    while (d.has_child[cur]) {
      double sh = 0.0, mass = 1.0;
      int nxt = -1;
      bool vanished = false, cached = false;
      // Children of cur in index order: one ballot per 64 candidates.
      const int lane = tid & 63;
      for (int base = cur + 1; base < N && nxt < 0 && !vanished; base += kWave) {
        const int cl = base + lane;
        unsigned long long kids = __ballot(cl < N && st.par[cl] == cur);
        while (kids) {
          const int c = base + __builtin_ctzll(kids);
          kids &= kids - 1;
          double ratio;
          if (sh == 0.0) {
            ratio = st.ratio0[c];
          } else if (st.pd[c] == 0.0) {
            ratio = (st.pt[c] - sh * st.pd[c] > 0.0) ? INFINITY : 0.0;
          } else {
            const double pc = st.pt[c] - sh * st.pd[c];
            ratio = pc > 0.0 ? pc / (mass * st.pd[c]) : 0.0;
          }
          if ((double)st.u[c] < ratio) {
            nxt = c;
            break;
          }
          sh += mass;
          if constexpr (CACHE) {
            if (!cached) load_row_probs<T, NT>(a, b, cur, d, cpt, cpd);
            cached = true;
            mass = cached_mass<NT>(cpt, cpd, sh, st.red);
          } else {
            mass = residual_mass<T, NT>(a, b, cur, d, sh, st.red);
          }
          if (!(mass > 0.0)) {
            vanished = true;
            break;
          }
        }
      }
      if (nxt < 0) {
        residual = !vanished;
        shift = vanished ? 0.0 : sh;
        break;
      }
      if (tid == 0) {
        d.acc[nxt] = 1;
        d.path[len] = nxt;
      }
      ++len;
      cur = nxt;
    }
  }
  if (tid == 0) {
    d.len = len;
    d.stop = cur;
    d.residual = residual;
    d.shift = shift;
  }
  __syncthreads();
}

// Store one sequence's decision record (the lossless decide kernel).
__device__ __forceinline__ void store_decision(const SampleArgs& a, int b, const Decision& d) {
  const int N = a.N, tid = threadIdx.x;
  const int r = d.stop;
  int32_t* dec = a.decision + (size_t)b * a.dec_stride;
  for (int c = tid; c < N; c += (int)blockDim.x) {
    dec[4 + c] = c < d.len ? d.path[c] : -1;
    dec[4 + N + c] = d.acc[c];
  }
  if (tid == 0) {
    dec[0] = d.len;
    dec[1] = d.bad;
    dec[2] = d.residual;
    dec[3] = r;
    double* st = a.decision_lz + (size_t)b * kDecisionDoubles;
    st[0] = d.lz[0][r];
    st[1] = d.residual ? d.lz[1][r] : 0.0;
    st[2] = d.residual ? d.shift : 0.0;
    st[3] = d.m[0][r];
    st[4] = 1.0 / d.s[0][r];
    st[5] = d.residual ? d.m[1][r] : 0.0;
    st[6] = d.residual ? 1.0 / d.s[1][r] : 0.0;
  }
}

// grid (B): the lossless walk, one work-group per sequence (its vocabulary
// passes are sequential), stores the decision record.
template <typename T, bool CACHE>
__global__ __launch_bounds__(kDecideThreads) void sample_decide_lossless(SampleArgs a) {
  __shared__ Decision d;
  __shared__ SiblingTests st;
  const int b = blockIdx.x;
  decide_sequence<T, true, kDecideThreads, CACHE>(a, b, d, &st);
  store_decision(a, b, d);
}

// E = -ln U of a race uniform in fp32, within 2e-6 relative: the series of
// -ln(1 - d) near U = 1 (where a logarithm's last-place error would be a
// large relative error), the hardware logarithm elsewhere.  U is exact in
// fp32 (a 24-bit odd numerator over 2^24), and so is d = 1 - U.
__device__ __forceinline__ float race_e32(uint32_t w) {
  const float u = (float)(2u * (w >> 9) + 1u) * 5.9604644775390625e-08f;
  const float d = 1.0f - u;
  if (d < 0.015625f) return d * (1.0f + d * (0.5f + d * (1.0f / 3.0f)));
  return -__builtin_amdgcn_logf(u) * kLn2;
}

// The level-2 race among this thread's ids e0 .. e0+3 (logits lt, ld): id x
// scores w_x / E_x in fp64, with w_x = max(pt - shift pd, 0) when resid, else
// pt, where pt = exp(lt - lzt), pd = exp(ld - lzd); the block's best goes to
// (best, bidx), ties to the lowest id.  The fp64 score is taken only for ids
// whose fp32 upper bound reaches the best fp32 lower bound in the block: the
// bounds carry the fp32 rounding of the exponent (2e-7 of |logit| + |log
// normaliser|, plus 2e-6) on pt and pd, of E (2e-6) and of the quotient, ten
// times over, and 1e-30 for fp32 underflow, so no id left out can win or tie
// in fp64.  Usually one id per block is scored in fp64.
__device__ __forceinline__ void race_ids(const float (&lt)[4], const float (&ld)[4], const uint32_t (&words)[4],
                         int e0, int V, double lzt, double lzd, double shift, bool resid,
                         double& best, int& bidx, double* redd, int* redi) {
  __shared__ float redf[4];
  const float lzt_f = (float)lzt, lzd_f = (float)lzd, sh_f = (float)shift;
  float hi[4], lo_max = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    hi[k] = -1.f;
    if (e0 + k >= V || lt[k] == -INFINITY) continue;
    const float pt = fast_exp2((lt[k] - lzt_f) * kLog2e);
    const float et = 2e-6f * (fabsf(lt[k]) + fabsf(lzt_f)) + 2e-5f;
    float w = pt, eps = et * pt + 1e-30f;
    if (resid) {
      const float pd = ld[k] == -INFINITY ? 0.f : fast_exp2((ld[k] - lzd_f) * kLog2e);
      const float ed = 2e-6f * (fabsf(ld[k]) + fabsf(lzd_f)) + 2e-5f;
      w = pt - sh_f * pd;
      eps += ed * sh_f * pd;
    }
    if (!(w + eps > 0.f)) continue;   // no positive weight in fp64 either
    const float e = race_e32(words[k]);
    hi[k] = (w + eps) / e * (1.f + 1e-4f);
    if (w - eps > 0.f) lo_max = fmaxf(lo_max, (w - eps) / e * (1.f - 1e-4f));
  }
  const float floor_lo = block_max(lo_max, redf);
  uint32_t cand = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (hi[k] > 0.f && hi[k] >= floor_lo) cand |= 1u << k;
  while (__any(cand != 0)) {
    if (cand) {
      const int k = __builtin_ctz(cand);
      cand &= cand - 1;
      float ltk = 0.f, ldk = 0.f;
      uint32_t wk = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == k) {
          ltk = lt[q];
          ldk = ld[q];
          wk = words[q];
        }
      const double pt = exp((double)ltk - lzt);
      double wx = pt;
      if (resid) {
        const double pd = exp((double)ldk - lzd);
        wx = pt - shift * pd > 0.0 ? pt - shift * pd : 0.0;
      }
      if (wx > 0.0) better(best, bidx, wx / -log(uniform24(wk)), e0 + k);
    }
  }
  block_argmax(best, bidx, redd, redi);
}

// ---------------------------------------------------------------------------
// The draw at the stop row and the outputs, run by the last residual
// work-group of a sequence.  The stop node's decision comes from that
// group's own LDS copy, or from the record the lossless decide kernel stored
// (path node ids at dec[4 + c], accept flags at dec[4 + N + c]).  The
// two-level exponential race: chunks race on their masses (level 1), ids
// race inside the winning chunk on their weights (level 2).
// ---------------------------------------------------------------------------
struct StopView {
  int len, bad, r;
  bool residual;
  double lzt, lzd, shift;   // the stop row's fp64 log-normalisers and residual shift
  const int32_t* dec;       // the record, or NULL
  const Decision* d;        // the LDS decision when dec is NULL
};

// Outputs of a sequence whose device data is invalid (bad parent array or token).
__device__ __forceinline__ void emit_bad(const SampleArgs& a, int b, int bad) {
  const int N = a.N, tid = threadIdx.x;
  for (int c = tid; c < N; c += (int)blockDim.x) {
    a.out_tokens[(size_t)b * N + c] = -1;
    if (a.out_path) a.out_path[(size_t)b * N + c] = -1;
    if (a.out_accept) a.out_accept[(size_t)b * N + c] = 0;
  }
  if (tid == 0) {
    a.out_count[b] = 0;
    report_error(a.dev_err, bad == 2 ? SPEC_DEVERR_TOKEN : SPEC_DEVERR_PARENT);
  }
}

// Level 1 of the draw at stop row r: chunks race with score W_c / E1_c.
// After a rejection the weights are the residual masses; if they all vanish,
// the target's (use_resid tells which).  The masses were stored by other
// work-groups of this launch.  Returns the winning chunk.
__device__ __forceinline__ int race_level1(const SampleArgs& a, int b, int r, bool residual,
                                           bool& use_resid, bool held = false,
                                           double w_held = 0.0) {
  __shared__ double redd[4];
  __shared__ int redi[4];
  const int tid = threadIdx.x;
  const double* rw = a.race_w + (size_t)b * a.n_race * 2;
  double w_res = 0.0, w_tgt = 0.0;     // this thread's first chunk, q = tid
  if (held) {
    // Target weights already in registers (one chunk per thread, no residual).
    w_tgt = w_held;
  } else if (tid < a.n_race) {
    w_res = load_coherent(rw + 2 * tid);
    w_tgt = load_coherent(rw + 2 * tid + 1);
  }
  double tot = w_res;
  for (int q = tid + kSampleThreads; q < a.n_race; q += kSampleThreads)
    tot += load_coherent(rw + 2 * q);
  tot = block_sum(tot, redd);
  const bool fallback = residual && !(tot > 0.0);
  use_resid = residual && !fallback;
  double best = -1.0;
  int bidx = 0x7fffffff;
  for (int q = tid; q < a.n_race; q += kSampleThreads) {
    const double W = q == tid ? (use_resid ? w_res : w_tgt)
                              : load_coherent(rw + 2 * q + (use_resid ? 0 : 1));
    if (W > 0.0) {
      uint32_t c0 = (uint32_t)q, c1 = (uint32_t)r, c2 = (uint32_t)b, c3 = a.ctr3_base + 2u;
      philox4x32_10(c0, c1, c2, c3, a.key0, a.key1);
      better(best, bidx, W / -log(uniform24(c0)), q);
    }
  }
  block_argmax(best, bidx, redd, redi);
  return bidx < a.n_race ? bidx : 0;
}

// The level-2 race among this thread's four ids of one race chunk, with the
// logits already in registers (lt, ld; ids past V hold -inf).  Returns the
// winning id of the chunk (block-wide), or a value >= V if no id has positive
// weight.  After a residual race that finds no id with a positive fp64
// residual (the fp32 chunk mass was positive from a cancellation at the 1e-7
// level) the chunk is raced on the target's weights instead.
__device__ __forceinline__ int race_chunk(const SampleArgs& a, int b, int r, int q, const float (&lt)[4],
                          const float (&ld)[4], bool use_resid, double lzt, double lzd,
                          double shift) {
  __shared__ double redd[4];
  __shared__ int redi[4];
  const int e0 = q * kRaceChunk + 4 * (int)threadIdx.x;
  uint32_t w0 = (uint32_t)(e0 >> 2), w1 = (uint32_t)r, w2 = (uint32_t)b, w3 = a.ctr3_base + 3u;
  philox4x32_10(w0, w1, w2, w3, a.key0, a.key1);
  const uint32_t words[4] = {w0, w1, w2, w3};
  double best = -1.0;
  int bidx = 0x7fffffff;
  race_ids(lt, ld, words, e0, a.V, lzt, lzd, use_resid ? shift : 0.0, use_resid, best, bidx,
           redd, redi);
  if (bidx >= a.V && use_resid) {
    best = -1.0;
    bidx = 0x7fffffff;
    race_ids(lt, ld, words, e0, a.V, lzt, lzd, 0.0, false, best, bidx, redd, redi);
  }
  return bidx;
}

// Level 2 of the draw with the winning chunk's logits loaded from memory.
template <typename T>
__device__ __forceinline__ int race_level2(const SampleArgs& a, int b, int r, int cstar, bool use_resid,
                           double lzt, double lzd, double shift) {
  const int N = a.N, V = a.V;
  const T* trow = static_cast<const T*>(a.target) + ((size_t)b * N + r) * V;
  const T* drow = static_cast<const T*>(a.draft) + ((size_t)b * N + r) * V;
  const int e0 = cstar * kRaceChunk + 4 * (int)threadIdx.x;
  float lt[4], ld[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = e0 + k;
    lt[k] = e < V ? ld1(trow, e) : -INFINITY;
    ld[k] = (e < V && use_resid) ? ld1(drow, e) : -INFINITY;
  }
  const int y = race_chunk(a, b, r, cstar, lt, ld, use_resid, lzt, lzd, shift);
  return y < V ? y : 0;
}

// The outputs of a sequence: the accepted path's drafted tokens, then y.
__device__ __forceinline__ void emit_outputs(const SampleArgs& a, int b, const StopView& sv, int y) {
  const int N = a.N, tid = threadIdx.x;
  const int len = sv.len;
  int* out_tok = a.out_tokens + (size_t)b * N;
  auto path_at = [&](int c) -> int {
    if (sv.dec) return sv.dec[4 + c];
    return c < sv.d->len ? sv.d->path[c] : -1;
  };
  for (int c = tid; c < N; c += (int)blockDim.x) {
    int tokv = -1;
    const int pv = path_at(c);
    if (c < len - 1)
      tokv = sv.dec ? a.tokens[(size_t)b * N + path_at(c + 1)] : sv.d->tok[path_at(c + 1)];
    else if (c == len - 1)
      tokv = y;
    out_tok[c] = tokv;
    if (a.out_path) a.out_path[(size_t)b * N + c] = pv;
    if (a.out_accept)
      a.out_accept[(size_t)b * N + c] = (uint8_t)(sv.dec ? sv.dec[4 + N + c] : sv.d->acc[c]);
  }
  if (tid == 0) a.out_count[b] = len;
}

template <typename T>
__device__ void race_emit(const SampleArgs& a, int b, const StopView& sv, bool held = false,
                          double w_held = 0.0) {
  if (sv.bad) {
    emit_bad(a, b, sv.bad);
    return;
  }
  bool use_resid = false;
  const int cstar = race_level1(a, b, sv.r, sv.residual, use_resid, held, w_held);
  const int y = race_level2<T>(a, b, sv.r, cstar, use_resid, sv.lzt, sv.lzd, sv.shift);
  emit_outputs(a, b, sv, y);
}

// Residual (or target) mass of the stop row's 1024-id race chunks q0 .. q1-1
// of this group.  Every work-group of a sequence derives the same decision;
// group 0 stores it.
// With FROM_RECORD the decision comes from the record the lossless decide
// kernel stored.
template <bool VEC4, typename T, bool FROM_RECORD = false>
__global__ __launch_bounds__(kSampleThreads) void sample_resid(SampleArgs a) {
  __shared__ Decision d;
  const int grp = blockIdx.x, b = blockIdx.y;
  const int N = a.N, V = a.V;
  const int tid = threadIdx.x;
  bool bad, residual;
  int r;
  float tm, tinv, dm, dinv, shift;
  double lzt, lzd, shiftd;   // fp64 log-normalisers and shift of the stop row
  if constexpr (FROM_RECORD) {
    const int32_t* dec = a.decision + (size_t)b * a.dec_stride;
    const double* st = a.decision_lz + (size_t)b * kDecisionDoubles;
    bad = dec[1] != 0;
    residual = dec[2] != 0;
    r = dec[3];
    lzt = st[0];
    lzd = st[1];
    shiftd = st[2];
    shift = (float)st[2];
    tm = (float)st[3];
    tinv = (float)st[4];
    dm = (float)st[5];
    dinv = (float)st[6];
  } else {
    decide_sequence<T>(a, b, d);
    bad = d.bad != 0;
    residual = d.residual;
    r = d.stop;
    lzt = d.lz[0][r];
    lzd = residual ? d.lz[1][r] : 0.0;
    shiftd = residual ? d.shift : 0.0;
    shift = 1.f;
    tm = d.m[0][r];
    tinv = (float)(1.0 / d.s[0][r]);
    dm = residual ? d.m[1][r] : 0.f;
    dinv = residual ? (float)(1.0 / d.s[1][r]) : 0.f;
  }
  // A leaf's target row whose statistics the first kernel did not gather
  // (the walk accepted every draft on its path): this pass gathers them too,
  // per race chunk (max, sum of exp), and the draw derives the normaliser.
  const bool row_stats = residual || a.leaf_rows;
  const T* trow = static_cast<const T*>(a.target) + ((size_t)b * N + r) * V;
  const T* drow = static_cast<const T*>(a.draft) + ((size_t)b * N + r) * V;
  const int q0 = (int)((long long)a.n_race * grp / a.n_groups);
  const int q1 = (int)((long long)a.n_race * (grp + 1) / a.n_groups);
  // Per chunk: each wave reduces its lanes with shuffles and parks the two
  // partial sums in LDS; one block pass per batch of chunks adds the waves.
  // The loads of kU chunks are issued together (a group may own several).
  constexpr int kBatch = 64;
  constexpr int kU = 4;
  __shared__ double part[kSampleThreads / kWave][kBatch][2];
  const int wave = tid >> 6, lane = tid & 63;
  for (int qb = q0; qb < q1; qb += kBatch) {
    const int nq = min(kBatch, q1 - qb);
    for (int i0 = 0; i0 < nq; i0 += kU) {
      float tv[kU][4], dv[kU][4];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e0 = (qb + i0 + u) * kRaceChunk + 4 * tid;
        const bool live = i0 + u < nq && !bad;
        if (VEC4) {
          f32x4 t4 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, d4 = t4;
          if (live && e0 < V) {
            t4 = ld4<T, true>(trow, e0);   // non-temporal: the row is read once here
            if (residual) d4 = ld4<T, true>(drow, e0);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            tv[u][k] = t4[k];
            dv[u][k] = d4[k];
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = e0 + k;
            tv[u][k] = (live && e < V) ? ld1(trow, e) : -INFINITY;
            dv[u][k] = (live && e < V && residual) ? ld1(drow, e) : -INFINITY;
          }
        }
      }
      if (row_stats) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (i0 + u >= nq) break;
          float sw = 0.f, spt = 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float pt = fast_exp2((tv[u][k] - tm) * kLog2e) * tinv;
            const float pd = residual ? fast_exp2((dv[u][k] - dm) * kLog2e) * dinv : 0.f;
            spt += pt;
            sw += fmaxf(pt - shift * pd, 0.f);
          }
          const double tw = wave_sum((double)sw);
          const double tp = wave_sum((double)spt);
          if (lane == 0) {
            part[wave][i0 + u][0] = tw;
            part[wave][i0 + u][1] = tp;
          }
        }
      } else {
        // (max, sum of exp(x - max)) of the chunk's target logits, per wave.
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (i0 + u >= nq) break;
          const float mw =
              wave_max(fmaxf(fmaxf(tv[u][0], tv[u][1]), fmaxf(tv[u][2], tv[u][3])));
          float sx = 0.f;
          if (mw != -INFINITY) {
#pragma unroll
            for (int k = 0; k < 4; ++k) sx += fast_exp2((tv[u][k] - mw) * kLog2e);
          }
          const double sw = wave_sum((double)sx);
          if (lane == 0) {
            part[wave][i0 + u][0] = (double)mw;
            part[wave][i0 + u][1] = sw;
          }
        }
      }
    }
    __syncthreads();
    if (tid < nq) {
      double x0 = 0.0, x1 = 0.0;
      if (row_stats) {
#pragma unroll
        for (int w = 0; w < kSampleThreads / kWave; ++w) {
          x0 += part[w][tid][0];
          x1 += part[w][tid][1];
        }
      } else {
        x0 = -INFINITY;
#pragma unroll
        for (int w = 0; w < kSampleThreads / kWave; ++w) x0 = fmax(x0, part[w][tid][0]);
        if (x0 != -INFINITY) {
#pragma unroll
          for (int w = 0; w < kSampleThreads / kWave; ++w)
            if (part[w][tid][0] != -INFINITY)
              x1 += part[w][tid][1] * exp2((part[w][tid][0] - x0) * (double)kLog2e);
        }
      }
      double* o = a.race_w + ((size_t)b * a.n_race + qb + tid) * 2;
      store_coherent(o, x0);
      store_coherent(o + 1, x1);
    }
    __syncthreads();
  }

  // The group that completes the sequence's masses runs the draw.
  if (!last_of_group(a.arrive + (size_t)b * kArriveStride, grp, a.n_groups, a.dev_err)) return;
  // With one race chunk per thread the leaf row's target masses stay in
  // registers and go straight to the level-1 race.
  const bool held = !row_stats && !bad && a.n_race <= kSampleThreads;
  double w_held = 0.0;
  if (!row_stats && !bad) {
    // The stop row's log-normaliser from its race chunks' (max, sum), then
    // each chunk's target mass sum exp(x - lz) in place of the pair.
    __shared__ double redn[4];
    __shared__ float redm[4];
    double* rw = a.race_w + (size_t)b * a.n_race * 2;
    double m0 = -INFINITY, s0 = 0.0;   // this thread's first chunk, q = tid
    if (tid < a.n_race) {
      m0 = load_coherent(rw + 2 * tid);
      s0 = load_coherent(rw + 2 * tid + 1);
    }
    float mx = (float)m0;
    for (int q = tid + kSampleThreads; q < a.n_race; q += kSampleThreads)
      mx = fmaxf(mx, (float)load_coherent(rw + 2 * q));
    mx = block_max(mx, redm);
    double sum = 0.0;
    if (mx != -INFINITY)
      for (int q = tid; q < a.n_race; q += kSampleThreads) {
        const double mq = q == tid ? m0 : load_coherent(rw + 2 * q);
        if (mq != -INFINITY) sum += (q == tid ? s0 : load_coherent(rw + 2 * q + 1)) * exp(mq - (double)mx);
      }
    sum = block_sum(sum, redn);
    lzt = (double)mx + log(sum);
    if (held) {
      w_held = m0 == -INFINITY ? 0.0 : s0 * exp(m0 - lzt);
    } else {
      for (int q = tid; q < a.n_race; q += kSampleThreads) {
        const double mq = load_coherent(rw + 2 * q);
        const double w = mq == -INFINITY ? 0.0 : load_coherent(rw + 2 * q + 1) * exp(mq - lzt);
        store_coherent(rw + 2 * q, 0.0);
        store_coherent(rw + 2 * q + 1, w);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the masses are stored
      __syncthreads();
    }
  }
  StopView sv;
  if constexpr (FROM_RECORD) {
    const int32_t* dec = a.decision + (size_t)b * a.dec_stride;
    sv = StopView{dec[0], dec[1], r, residual, lzt, lzd, shiftd, dec, nullptr};
  } else {
    sv = StopView{d.len, d.bad, r, residual, lzt, lzd, shiftd, nullptr, &d};
  }
  race_emit<T>(a, b, sv, held, w_held);
}


// ---------------------------------------------------------------------------
// Host-side planning and launch.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SamplePlan plan_sample(int32_t B, int32_t N, int32_t V) {
  SamplePlan p{};
  p.vchunk = kStatsChunk;
  p.n_vchunks = (V + kStatsChunk - 1) / kStatsChunk;
  p.n_race = (V + kRaceChunk - 1) / kRaceChunk;
  // Residual work-groups per sequence: one race chunk each while the total
  // stays near 1024 work-groups, more chunks each beyond (every group also
  // re-derives the sequence's decision, so fewer groups is less overhead).
  long long groups = (1024 + (long long)B - 1) / (B > 0 ? B : 1);
  if (groups > p.n_race) groups = p.n_race;
  if (groups < 1) groups = 1;
  p.n_groups = (int)groups;
  p.dec_stride = 4 + 2 * N;
  const size_t rows = (size_t)B * 2 * N * p.n_vchunks;
  p.off_m = align256((size_t)B * kArriveStride * sizeof(uint32_t));
  p.off_s = align256(p.off_m + rows * sizeof(float));
  p.off_g = align256(p.off_s + rows * sizeof(double));
  p.off_w = align256(p.off_g + (size_t)B * 2 * N * sizeof(float));
  p.off_dec = align256(p.off_w + (size_t)B * p.n_race * 2 * sizeof(double));
  p.off_lz = align256(p.off_dec + (size_t)B * p.dec_stride * sizeof(int32_t));
  p.bytes = align256(p.off_lz + (size_t)B * kDecisionDoubles * sizeof(double));
  return p;
}

template <typename T>
static hipError_t launch_sample_t(const SampleArgs& a, hipStream_t stream) {
  const bool vec4 = (a.V % 4) == 0;
  dim3 g1(a.n_vchunks, 2 * a.N, a.B), g2(a.n_groups, a.B), g3(a.B), blk(kSampleThreads);
  if (vec4)
    hipLaunchKernelGGL((sample_stats<true, T>), g1, blk, 0, stream, a);
  else
    hipLaunchKernelGGL((sample_stats<false, T>), g1, blk, 0, stream, a);
  if (a.lossless) {
    // The sibling walk needs sequential vocabulary passes: one work-group per
    // sequence decides, the residual groups read its record.
    if (vec4 && a.V <= 4 * kCacheVec * kDecideThreads)
      hipLaunchKernelGGL((sample_decide_lossless<T, true>), g3, dim3(kDecideThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((sample_decide_lossless<T, false>), g3, dim3(kDecideThreads), 0, stream,
                         a);
    if (vec4)
      hipLaunchKernelGGL((sample_resid<true, T, true>), g2, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((sample_resid<false, T, true>), g2, blk, 0, stream, a);
  } else if (vec4) {
    hipLaunchKernelGGL((sample_resid<true, T>), g2, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL((sample_resid<false, T>), g2, blk, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  return a.logits_bf16 ? launch_sample_t<__bf16>(a, stream) : launch_sample_t<float>(a, stream);
}

// ---------------------------------------------------------------------------
// Library-owned scratch of spec_sample_noalloc (callers that cannot allocate).
// One array per device, in the code object's static device memory.  In host
// code `scratch` names a host-side stand-in, not device memory: kernels and
// fills only ever get the device address that hipGetSymbolAddress returns,
// kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[SPEC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t stream) {
  const uint32_t n = (uint32_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  const uint32_t grid = n / 256u + 1u < 256u ? n / 256u + 1u : 256u;
  hipLaunchKernelGGL(zero_words, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Draft-step draw ("Guide to MagicDec", step 2 of its reference
// implementation: softmax of the draft logits, then one multinomial draw).
// An exponential race over softmax(l): id x scores p_x / E_x with
// E_x = -ln U_x, the largest score wins (ties: lowest id).  In log2 units the
// score ln p_x - ln E_x is l_x - ln(-ln U_x) plus a constant, so the race
// needs neither the row max nor the normaliser; it is evaluated in fp64, the
// precision the reference draw decides in.  Max and normaliser are still
// gathered (per chunk: max and sum of exp2) for the drawn token's
// log-probability.  One launch: the work-group that completes a row's last
// chunk (arrival counters in the workspace) combines the chunk partials.
// ---------------------------------------------------------------------------
// Arg-max of (score, id) with ties to the lowest id, carrying the winner's
// scaled logit along.
struct RaceBest {
  double s;
  int i;
  float x;
};

__device__ __forceinline__ void better_f(RaceBest& r, double s2, int i2, float x2) {
  if (s2 > r.s || (s2 == r.s && i2 < r.i)) r = RaceBest{s2, i2, x2};
}

__device__ __forceinline__ void block_argmax_f(RaceBest& r, RaceBest* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double s2 = __shfl_xor(r.s, off);
    const int i2 = __shfl_xor(r.i, off);
    const float x2 = __shfl_xor(r.x, off);
    better_f(r, s2, i2, x2);
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = r;
  __syncthreads();
  r = red[0];
#pragma unroll
  for (int k = 1; k < 4; ++k) better_f(r, red[k].s, red[k].i, red[k].x);
}

// Combines the chunk partials of row b: the race winner (chunks are in id
// order, so ties still go to the lowest id), the fp64 log2 normaliser, and
// the winner's log-probability.  The partials were stored by other
// work-groups of this launch.
__device__ void draft_finish_row(const DraftArgs& a, int b, float* redf, double* redd,
                                 RaceBest* redr) {
  const size_t o = (size_t)b * a.n_chunks;
  float mx = -INFINITY;
  RaceBest best{-INFINITY, 0x7fffffff, -INFINITY};
  for (int c = threadIdx.x; c < a.n_chunks; c += kSampleThreads) {
    better_f(best, load_coherent(a.part_best + o + c),
             __hip_atomic_load(a.part_idx + o + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
             load_coherent(a.part_x + o + c));
    mx = fmaxf(mx, load_coherent(a.part_m + o + c));
  }
  block_argmax_f(best, redr);
  mx = block_max(mx, redf);
  double sum = 0.0;
  if (mx != -INFINITY)
    for (int c = threadIdx.x; c < a.n_chunks; c += kSampleThreads) {
      const float m = load_coherent(a.part_m + o + c);
      if (m != -INFINITY) sum += load_coherent(a.part_s + o + c) * exp2((double)m - (double)mx);
    }
  sum = block_sum(sum, redd);
  if (threadIdx.x == 0) {
    int tok = best.i;
    float lp = NAN;
    if (best.s == -INFINITY || best.s != best.s || tok < 0 || tok >= a.V) {
      tok = -1;
      report_error(a.dev_err, SPEC_DEVERR_LOGITS);
    } else {
      lp = (float)(((double)best.x - (double)mx - log2(sum)) * 0.6931471805599453);
    }
    a.out_token[(size_t)b * a.token_stride] = tok;
    if (a.out_logprob) a.out_logprob[b] = lp;
  }
}

// grid (chunks of CH ids, B).  Thread t holds the id groups
// g = chunk*CH/4 + t + 256*i (i < CH/1024), four consecutive ids per group,
// so one Philox call serves one 16-byte load.  Small chunks give many
// work-groups: the Philox rounds, not the bytes, set the time of a 0.5 MB
// row.  At large batch there are work-groups enough either way, and chunks
// twice as long spread each work-group's three block reductions over twice
// the ids.
template <bool VEC4, typename T, int CH>
__global__ __launch_bounds__(kSampleThreads) void draft_partial(DraftArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  __shared__ RaceBest redr[4];
  const int chunk = blockIdx.x, b = blockIdx.y;
  const T* row = static_cast<const T*>(a.logits) + (size_t)b * a.row_stride;
  constexpr int GROUPS = CH / 4 / kSampleThreads;  // 2 or 4
  const int g0 = chunk * (CH / 4) + threadIdx.x;
  float x[4 * GROUPS], lraw[4 * GROUPS];   // logit * log2(e), and the logit
#pragma unroll
  for (int i = 0; i < GROUPS; ++i) {
    const int e = 4 * (g0 + kSampleThreads * i);
    if (VEC4) {
      f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (e < a.V) v = ld4(row, e);
#pragma unroll
      for (int k = 0; k < 4; ++k) lraw[4 * i + k] = v[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) lraw[4 * i + k] = e + k < a.V ? ld1(row, e + k) : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) x[4 * i + k] = lraw[4 * i + k] * kLog2e;
  }
  // Race: one Philox block per group of four ids.  The fp32 score of every
  // id picks each thread's candidates cheaply; only ids within delta of the
  // thread's fp32 best get the fp64 score that decides (delta is far above
  // the fp32 error, so no id left out could win in fp64).
  float s32[4 * GROUPS];
  uint32_t word[4 * GROUPS];
  float m32 = -INFINITY;
#pragma unroll
  for (int i = 0; i < GROUPS; ++i) {
    const int g = g0 + kSampleThreads * i;
    uint32_t c0 = (uint32_t)g, c1 = (uint32_t)a.node, c2 = (uint32_t)b, c3 = a.ctr3;
    philox4x32_10(c0, c1, c2, c3, a.key0, a.key1);
    const uint32_t w[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // E = -ln U within 2e-6 relative, also for U near 1 (a series there).
      const float e = race_e32(w[k]);
      word[4 * i + k] = w[k];
      s32[4 * i + k] = lraw[4 * i + k] - __builtin_amdgcn_logf(e) * 0.6931471805599453f;
      m32 = fmaxf(m32, s32[4 * i + k]);   // ids past V carry -inf
    }
  }
  const float delta = 1e-3f + 1e-6f * fabsf(m32);
  // Candidate mask; the fp64 scores are taken one candidate per lane per
  // round (ids in increasing order), so the wave runs as many rounds as its
  // busiest lane has candidates -- almost always one.
  uint32_t cand = 0;
#pragma unroll
  for (int j = 0; j < 4 * GROUPS; ++j)
    if (s32[j] != -INFINITY && s32[j] >= m32 - delta) cand |= 1u << j;
  RaceBest best{-INFINITY, 0x7fffffff, -INFINITY};
  while (__any(cand != 0)) {
    if (cand) {
      const int j = __builtin_ctz(cand);
      cand &= cand - 1;
      float l = 0.f, xs = 0.f;
      uint32_t wj = 0;
#pragma unroll
      for (int q = 0; q < 4 * GROUPS; ++q)
        if (q == j) {
          l = lraw[q];
          xs = x[q];
          wj = word[q];
        }
      const double sc = (double)l - log(-log(uniform24(wj)));
      better_f(best, sc, 4 * (g0 + kSampleThreads * (j >> 2)) + (j & 3), xs);
    }
  }
  block_argmax_f(best, redr);
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 4 * GROUPS; ++i) mx = fmaxf(mx, x[i]);
  mx = block_max(mx, redf);
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 4 * GROUPS; ++i) sum += fast_exp2(x[i] - mx);
  }
  const double tot = block_sum((double)sum, redd);
  if (threadIdx.x == 0) {
    const size_t o = (size_t)b * a.n_chunks + chunk;
    store_coherent(a.part_best + o, best.s);
    __hip_atomic_store(a.part_idx + o, best.i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_coherent(a.part_x + o, best.x);
    store_coherent(a.part_m + o, mx);
    store_coherent(a.part_s + o, tot);
  }
  // The work-group that completes the row's chunks combines them.
  if (last_of_group(a.arrive + (size_t)b * kArriveStride, chunk, a.n_chunks, a.dev_err))
    draft_finish_row(a, b, redf, redd, redr);
}

DraftPlan plan_draft(int32_t B, int32_t V) {
  DraftPlan p{};
  // Long chunks once short ones would give more than eight work-groups per
  // CU (at 64 x 128256: 23-25 against 28 us; at 8 x 128256 short chunks
  // stay faster, 9.4-10.5 against 10.5-11 us).
  const long long small = (long long)B * ((V + kDraftChunkSmall - 1) / kDraftChunkSmall);
  p.chunk = small > 8 * 256 ? kDraftChunkLarge : kDraftChunkSmall;
  p.n_chunks = (V + p.chunk - 1) / p.chunk;
  const size_t n = (size_t)B * p.n_chunks;
  p.off_best = align256((size_t)B * kArriveStride * sizeof(uint32_t));   // arrival counters first
  p.off_idx = align256(p.off_best + n * sizeof(double));
  p.off_x = align256(p.off_idx + n * sizeof(int32_t));
  p.off_m = align256(p.off_x + n * sizeof(float));
  p.off_s = align256(p.off_m + n * sizeof(float));
  p.bytes = align256(p.off_s + n * sizeof(double));
  return p;
}

template <int CH>
static void launch_draft_chunks(const DraftArgs& a, bool vec4, hipStream_t stream) {
  dim3 g1(a.n_chunks, a.B), blk(kSampleThreads);
  if (a.logits_bf16) {
    if (vec4)
      hipLaunchKernelGGL((draft_partial<true, __bf16, CH>), g1, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((draft_partial<false, __bf16, CH>), g1, blk, 0, stream, a);
  } else {
    if (vec4)
      hipLaunchKernelGGL((draft_partial<true, float, CH>), g1, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((draft_partial<false, float, CH>), g1, blk, 0, stream, a);
  }
}

hipError_t launch_draft(const DraftArgs& a, bool vec4, hipStream_t stream) {
  if (a.chunk == kDraftChunkLarge)
    launch_draft_chunks<kDraftChunkLarge>(a, vec4, stream);
  else if (a.chunk == kDraftChunkSmall)
    launch_draft_chunks<kDraftChunkSmall>(a, vec4, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace specv
