// attention.hip -- split-K attention of a query block against a long KV cache (gfx950).
//
// Verification attention ("Guide to MagicDec", section 2: the target verifies
// the drafted tokens with attention over the full context; "Speculative
// Decoding in LLM Serving Systems", sections "The algorithm" and "Tree-based
// variants": the drafted block is causal within itself, or a tree where each
// node sees only its ancestors) and the draft's bounded window attention
// ("Guide to MagicDec", section 1, fixed window as a FIFO ring, and "Best
// Practices" item 1, attention sinks) share one streaming core:
//
//   * a work-group owns one (sequence, kv head) unit, one slice of its query
//     rows (the g query heads of the GQA group times the n_q block nodes, all
//     served by the same K/V tiles) and one contiguous range of 32-key chunks;
//   * each of its four waves walks every fourth chunk on its own, with no
//     barrier in the loop: K and V rows are streamed with non-temporal
//     16-byte loads (the wave's next chunk in flight while it computes the
//     current one) straight into MFMA operand registers (V as eight 16-byte
//     row pieces transposed in-register; the loop-invariant Q operands sit in
//     LDS), S^T = K Q^T and O^T = V^T P^T run on
//     v_mfma_f32_16x16x32_bf16, and an online softmax in the log2 domain keeps
//     every per-query quantity in the lanes of that query;
//   * the mask is evaluated only on chunks that reach the block's own keys or
//     the end of the sequence: a key is visible if it precedes the block or is
//     an ancestor of the query's node (a 64-bit mask built from the parent
//     array);
//   * the four waves merge through LDS once at the end; the split partials
//     (unnormalised O, running max, sum) go to the workspace and the
//     work-group that completes a unit's last split (an arrival counter per
//     unit in the workspace) combines them in a fixed order.
//
// Wide query blocks (candidate trees with g * n_q > 32 rows) go to a second
// bf16 kernel, attn_tree_mfma below, in which all waves of a work-group share
// each K/V chunk through LDS instead of streaming it once per 32-row slice.
//
// The fp32 path is a plain VALU kernel (one wave per query row, lanes over
// the head dimension) with the same partial format, merged by the merge kernel.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "spec_common.hpp"
#include "spec_internal.hpp"

namespace specv {

constexpr int kChunk = 32;          // keys per wave step (two MFMA row blocks of 16)
constexpr int kWaves = 4;           // waves per work-group
constexpr int kThreads = kWaves * kWave;
constexpr int kValuSlice = 4;       // query rows per work-group on the VALU path

// ---------------------------------------------------------------------------
// Key geometry of one (sequence, kv head) unit.
// ---------------------------------------------------------------------------
struct UnitGeom {
  int b, hk, unit;
  int n_keys;   // logical keys 0 .. n_keys-1
  int p0;       // keys >= p0 are the block's own keys (masked by ancestry)
  int key_new;  // window: logical key served from k_new/v_new (-1: none)
  int ns;       // window: number of sink keys (keys < ns are sinks)
};

template <bool WINDOW>
__device__ __forceinline__ UnitGeom unit_geom(const AttnArgs& a, int unit, bool report) {
  UnitGeom u;
  u.unit = unit;
  u.b = unit / a.Hkv;
  u.hk = unit - u.b * a.Hkv;
  u.key_new = -1;
  u.ns = 0;
  if (!WINDOW) {
    int L = a.lens ? a.lens[u.b] : a.L_cap;
    if (L < a.n_q || L > a.L_cap) {
      if (report) report_error(a.dev_err, SPEC_DEVERR_KV_LEN);
      L = 0;
    }
    u.n_keys = L;
    u.p0 = L - a.n_q;
  } else {
    int T = a.lens[u.b];
    if (T < 1) {
      if (report) report_error(a.dev_err, SPEC_DEVERR_TOTAL_LEN);
      u.n_keys = 0;
      u.p0 = 0;
      return u;
    }
    int ns = T < a.S ? T : a.S;
    int nr = T - a.S;
    nr = nr < 0 ? 0 : (nr > a.W ? a.W : nr);
    u.ns = ns;
    u.n_keys = ns + nr;
    u.p0 = u.n_keys;  // one query per sequence: nothing inside the window is masked
    if (a.k_new) u.key_new = (T - 1 < a.S) ? (T - 1) : ns + (T - 1 - a.S) % a.W;
  }
  return u;
}

// Byte address of logical key `key` of a unit, for the K (kv=0) or V (kv=1) side.
template <bool WINDOW>
__device__ __forceinline__ const char* key_row(const AttnArgs& a, const UnitGeom& u, int key,
                                               int kv, size_t row_bytes) {
  if (!WINDOW) {
    const char* base = static_cast<const char*>(kv ? a.v : a.k);
    return base + ((size_t)u.unit * a.L_cap + key) * row_bytes;
  } else {
    if (key == u.key_new)
      return static_cast<const char*>(kv ? a.v_new : a.k_new) + (size_t)u.unit * row_bytes;
    if (key < u.ns)
      return static_cast<const char*>(kv ? a.v_sink : a.k_sink) +
             ((size_t)u.unit * a.S + key) * row_bytes;
    return static_cast<const char*>(kv ? a.v : a.k) +
           ((size_t)u.unit * a.W + (key - u.ns)) * row_bytes;
  }
}

// ---------------------------------------------------------------------------
// Paged caches (verify only).  K and V live in a pool of pages
// [num_pages, Hkv, P, D] with P = 2^page_shift keys, and block_table[b][i]
// names the page holding keys i*P .. i*P+P-1 of sequence b.  P is a multiple
// of every kernel's chunk, so a chunk never straddles pages.  A work-group
// stages the page ids of its key range in LDS once (the launch plan keeps
// the range within kPageCap pages) and each chunk reads its page from there.
// ---------------------------------------------------------------------------
constexpr int kPageCap = 512;

// Stage the page ids of keys [key_begin, key_end) of unit u; doubles as the
// work-group barrier that follows the Q staging.  False (and an error bit) if
// a page id lies outside the pool: the caller then drops its key range.
template <bool PAGED>
__device__ __forceinline__ bool stage_pages(const AttnArgs& a, const UnitGeom& u, int key_begin,
                                            int key_end, int32_t* lds_pages, int& first) {
  int bad = 0;
  first = 0;
  if (PAGED && key_end > key_begin) {
    first = key_begin >> a.page_shift;
    const int n = ((key_end - 1) >> a.page_shift) - first + 1;
    const int32_t* bt = a.block_table + (size_t)u.b * a.bt_stride + first;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int pid = bt[i];
      bad |= pid < 0 || pid >= a.num_pages;
      lds_pages[i] = pid;
    }
  }
  bad = __syncthreads_or(bad);
  if (bad && threadIdx.x == 0) report_error(a.dev_err, SPEC_DEVERR_PAGE);
  return !bad;
}

// Address of key `key` of unit u (K: kv = 0, V: kv = 1) in the verify cache,
// contiguous [B, Hkv, L_cap, D] or paged; with pages, `key` must lie in the
// staged range.  Keys of one chunk are consecutive rows from the chunk's base.
template <bool PAGED>
__device__ __forceinline__ const char* cache_row(const AttnArgs& a, const UnitGeom& u, int key,
                                                 int kv, size_t row_bytes,
                                                 const int32_t* lds_pages, int first) {
  const char* pool = static_cast<const char*>(kv ? a.v : a.k);
  if (!PAGED) return pool + ((size_t)u.unit * a.L_cap + key) * row_bytes;
  const int page = lds_pages[(key >> a.page_shift) - first];
  const size_t in_page = (size_t)(key & ((1 << a.page_shift) - 1));
  return pool + ((((size_t)page * a.Hkv + u.hk) << a.page_shift) + in_page) * row_bytes;
}

// Ancestor bitmask of block node i (bit t set: node t is i or an ancestor of i).
__device__ __forceinline__ uint64_t ancestor_mask(const AttnArgs& a, int b, int i) {
  if (!a.parent) return (i >= 63) ? ~0ull : ((2ull << i) - 1ull);
  const int32_t* par = a.parent + (size_t)b * a.parent_stride;
  uint64_t m = 0;
  int cur = i;
  for (int step = 0; step < 64 && cur >= 0; ++step) {
    m |= 1ull << cur;
    int p = par[cur];
    if (p >= cur || p < -1) {  // not a forest with parent < child: treat as a root
      report_error(a.dev_err, SPEC_DEVERR_PARENT);
      break;
    }
    cur = p;
  }
  return m;
}

// Work-group -> (tile, query slice).  Tiles are (unit, split) pairs.  When a unit
// has several query slices, all slices of a tile are placed on the same XCD
// (work-groups are dealt round-robin over the 8 XCDs) and dispatched back to
// back, so the K/V they share is served from that XCD's L2.
__device__ __forceinline__ bool decode_tile(const AttnArgs& a, int& unit, int& split, int& qs) {
  int id = blockIdx.x;
  int tile;
  if (a.n_qs == 1) {
    tile = id;
    qs = 0;
  } else {
    int xcd = id & 7;
    int local = id >> 3;
    int tix = local / a.n_qs;
    qs = local - tix * a.n_qs;
    tile = tix * 8 + xcd;
  }
  if (tile >= a.n_tiles) return false;
  unit = tile / a.n_splits;
  split = tile - unit * a.n_splits;
  return true;
}

__device__ __forceinline__ void chunk_range(int n_keys, int split, int n_splits, int& c0, int& c1) {
  long long nch = (n_keys + kChunk - 1) / kChunk;
  c0 = (int)(nch * split / n_splits);
  c1 = (int)(nch * (split + 1) / n_splits);
}

// Fused append of the window kernel: the current token's K/V go to its slot.
// Only the (split 0, slice 0) work-group of a unit writes; every reader of that
// key takes it from k_new/v_new instead, so no reader sees the slot mid-write.
template <bool WINDOW>
__device__ __forceinline__ void window_append(const AttnArgs& a, const UnitGeom& u, int split,
                                              int qs, size_t row_bytes) {
  if (!WINDOW) return;
  if (u.key_new < 0 || split != 0 || qs != 0) return;
  const int n16 = (int)(row_bytes / 16);
  for (int t = threadIdx.x; t < 2 * n16; t += blockDim.x) {
    int kv = t / n16, piece = t - kv * n16;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(kv ? a.v_new : a.k_new) + (size_t)u.unit * row_bytes);
    char* dst;
    if (u.key_new < u.ns)
      dst = static_cast<char*>(kv ? a.v_sink_w : a.k_sink_w) +
            ((size_t)u.unit * a.S + u.key_new) * row_bytes;
    else
      dst = static_cast<char*>(kv ? a.v_ring_w : a.k_ring_w) +
            ((size_t)u.unit * a.W + (u.key_new - u.ns)) * row_bytes;
    reinterpret_cast<u32x4*>(dst)[piece] = src[piece];
  }
}

// ---------------------------------------------------------------------------
// Split merge, separate kernel: output row `row` (0 .. M-1) of a
// unit, head-dim entries d0 .. d0+3.  Splits are combined in a fixed order,
// so the result is deterministic.
// ---------------------------------------------------------------------------
template <int D, typename OutT>
__device__ __forceinline__ void merge_item(const MergeArgs& a, int unit, int row, int d0) {
  const int qs = row / a.slice_rows;
  const int rr = row - qs * a.slice_rows;
  const size_t part0 = ((size_t)unit * a.n_qs + qs) * a.n_splits;
  const size_t pstride = (size_t)a.slice_rows;   // rows between consecutive splits

  // Every split's loads are independent, so they are all in flight together.
  const float* ml = a.ws_ml + (part0 * a.slice_rows + rr) * 2;
  const float* src = a.ws_o + (part0 * a.slice_rows + rr) * D + d0;
  float mx = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < a.n_splits; ++s) {
    const float ms = ml[s * pstride * 2];
    const float ls = ml[s * pstride * 2 + 1];
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + s * pstride * D);
    float s_old, s_new;
    merge_scales(mx, ms, s_old, s_new);
    acc = acc * s_old + v * s_new;
    l = l * s_old + ls * s_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int b = unit / a.Hkv, hk = unit - b * a.Hkv;
  const size_t orow = (size_t)(b * a.Hq + hk * a.g) * a.n_q + row;
  OutT* out = static_cast<OutT*>(a.out) + orow * D + d0;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (OutT)(acc[e] * inv);
  if (a.lse && d0 == 0) a.lse[orow] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// bf16 MFMA split kernel.  QB = MFMA query blocks (16 rows each) per slice.
// ---------------------------------------------------------------------------
template <int D, int QB, bool WINDOW, int NW = kWaves, bool PAGED = false>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void attn_split_mfma(AttnArgs a) {
  constexpr int DS = D / 32;             // MFMA k-steps over the head dim for S
  constexpr int SR = 16 * QB;            // query rows per slice
  constexpr int LDS_STRIDE = D + 1;
  __shared__ float lds_o[NW][SR][LDS_STRIDE];
  __shared__ float lds_ml[NW][SR][2];
  __shared__ bf16x8 lds_q[QB][DS][kWave];
  __shared__ int32_t lds_pages[PAGED ? kPageCap : 1];

  int unit, split, qs;
  if (!decode_tile(a, unit, split, qs)) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;   // MFMA column: query within a block; also V row piece
  const int h = lane >> 4;   // MFMA k-group
  const size_t row_bytes = (size_t)D * 2;

  const UnitGeom u = unit_geom<WINDOW>(a, unit, split == 0 && qs == 0 && threadIdx.x == 0);
  window_append<WINDOW>(a, u, split, qs, row_bytes);

  int c0, c1;
  chunk_range(u.n_keys, split, a.n_splits, c0, c1);
  int pfirst = 0;
  const int last = u.n_keys - 1;
  // K operands (A side): lane holds K[kbase + 16 kb + r][32 s + 8 h .. +8].
  auto row_of = [&](int key, int kv, int kbase) -> const char* {
    if constexpr (!PAGED) {
      return key_row<WINDOW>(a, u, key, kv, row_bytes);
    } else {
      // One page lookup per chunk; the chunk's keys are consecutive rows.
      return cache_row<PAGED>(a, u, kbase, kv, row_bytes, lds_pages, pfirst) +
             (size_t)(key - kbase) * row_bytes;
    }
  };
  auto load_k = [&](int kbase, bf16x8 (&kop)[2][DS]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int key = kbase + 16 * kb + r;
      key = key < last ? key : last;
      const char* p = row_of(key, 0, kbase);
#pragma unroll
      for (int s = 0; s < DS; ++s)
        kop[kb][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p + (32 * s + 8 * h) * 2));
    }
  };
  // V row pieces: lane holds V[key(h,t)][8 r .. 8 r + 7] for its eight keys
  // key(h,t) = kbase + 16 (t/4) + 4 h + t%4 -- the keys whose scores the
  // S^T accumulators leave in this lane.
  auto load_v = [&](int kbase, u32x4 (&vraw)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      int key = kbase + 16 * (t >> 2) + 4 * h + (t & 3);
      key = key < last ? key : last;
      if (8 * r < D)
        vraw[t] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(row_of(key, 1, kbase) + r * 16));
      else
        vraw[t] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  bf16x8 kop[2][DS];
  u32x4 vraw[8];
  // The window's waves take one chunk or two: their first K/V loads go out
  // before the Q staging and its barrier, so the two latencies overlap.
  if constexpr (WINDOW) {
    if (c0 + wave < c1) {
      load_k((c0 + wave) * kChunk, kop);
      load_v((c0 + wave) * kChunk, vraw);
    }
  }

  // Query operands (B side of S^T = K Q^T): lane holds Q[row][32 s + 8 h .. +8].
  // They are loop-invariant; wave 0 stages them in LDS in operand order and
  // every wave re-reads them per chunk (conflict-free 16-byte reads), which
  // keeps 32 VGPRs free for the in-flight K/V of the next chunk.
  const char* qbase = static_cast<const char*>(a.q) +
                      ((size_t)(u.b * a.Hq + u.hk * a.g) * a.n_q) * row_bytes;
  uint64_t anc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qs * SR + qb * 16 + r;
    const bool live = row < a.M;
    if (wave == 0) {
#pragma unroll
      for (int s = 0; s < DS; ++s)
        lds_q[qb][s][lane] = live ? *reinterpret_cast<const bf16x8*>(
                                        qbase + (size_t)row * row_bytes + (32 * s + 8 * h) * 2)
                                  : bf16x8{};
    }
    anc[qb] = (!WINDOW && live) ? ancestor_mask(a, u.b, row % a.n_q) : 1ull;
  }

  if constexpr (PAGED) {
    // The page-table staging doubles as the barrier after the Q staging.
    if (!stage_pages<PAGED>(a, u, c0 * kChunk, min(c1 * kChunk, u.n_keys), lds_pages, pfirst))
      c1 = c0;
  } else {
    __syncthreads();
  }

  float m[QB], lsum[QB];
  f32x4 oacc[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    lsum[qb] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Software pipeline: the loads of the wave's next chunk are issued as soon
  // as the current chunk has consumed the registers they land in (K after the
  // S^T products, V after its transpose), so HBM traffic stays in flight
  // while the wave computes.  The prefetch is never behind a branch, which
  // keeps the compiler's wait counts exact.
  auto chunk_step = [&](auto prefetch, int kbase, int nbase) {
    constexpr bool kPrefetch = decltype(prefetch)::value;

    // S^T blocks: sacc[qb][kb][e] = score(key kbase + 16 kb + 4 h + e, query qb*16 + r).
    f32x4 sacc[QB][2];
    int qlane = lane;
    asm volatile("" : "+v"(qlane));  // keep the LDS reads of Q inside the loop
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 qv = lds_q[qb][s][qlane];
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][s], qv, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][s], qv, acc1, 0, 0, 0);
      }
      sacc[qb][0] = acc0;
      sacc[qb][1] = acc1;
    }
    if constexpr (kPrefetch) load_k(nbase, kop);

    const bool need_mask = kbase + kChunk > u.p0;
    bf16x8 pop[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Raw scores; the softmax scale (> 0, in log2 units) is applied to the
      // max and folded into the exponent's FMA.
      float sv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) sv[t] = sacc[qb][t >> 2][t & 3];
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int key = kbase + 16 * (t >> 2) + 4 * h + (t & 3);
          const int rel = key - u.p0;   // block node index when 0 <= rel < n_q
          const bool in_block = rel >= 0;
          const bool anc_ok = ((anc[qb] >> (rel & 63)) & 1ull) != 0;
          const bool ok = key < u.n_keys && (!in_block || anc_ok);
          sv[t] = ok ? sv[t] : -INFINITY;
        }
      }
      float cm = sv[0];
#pragma unroll
      for (int t = 1; t < 8; ++t) cm = fmaxf(cm, sv[t]);
      cm = xgroup_max(cm) * a.scale_log2;
      const float mn = fmaxf(m[qb], cm);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(m[qb] - mu);
      m[qb] = mn;
      float p[8];
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        p[t] = fast_exp2(fmaf(sv[t], a.scale_log2, -mu));
        ps += p[t];
      }
      lsum[qb] = lsum[qb] * alpha + ps;
#pragma unroll
      for (int j = 0; j < 8; ++j) oacc[qb][j] *= alpha;
      u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                  pack_bf16x2(p[6], p[7])};
      pop[qb] = __builtin_bit_cast(bf16x8, pk);
    }

    // In-register 8x8 transpose: vop[j] holds V[key(h,t)][8 r + j] for t = 0..7,
    // the A operand of O^T = V^T P^T whose row r stands for head-dim index 8 r + j.
    bf16x8 vop[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = vraw[2 * e][j >> 1];
        const uint32_t hi = vraw[2 * e + 1][j >> 1];
        // one byte-select per dword: low (even j) or high (odd j) halves of lo, hi
        w[e] = __builtin_amdgcn_perm(hi, lo, (j & 1) ? 0x07060302u : 0x05040100u);
      }
      vop[j] = __builtin_bit_cast(bf16x8, w);
    }
    if constexpr (kPrefetch) load_v(nbase, vraw);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        oacc[qb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[j], pop[qb], oacc[qb][j], 0, 0, 0);
  };

  int c = c0 + wave;
  if (c < c1) {
    if constexpr (!WINDOW) {
      load_k(c * kChunk, kop);
      load_v(c * kChunk, vraw);
    }
    if constexpr (WINDOW) {
      // A few chunks per wave: peel the last one so nothing is read twice.
      for (; c + NW < c1; c += NW)
        chunk_step(std::true_type{}, c * kChunk, (c + NW) * kChunk);
      chunk_step(std::false_type{}, c * kChunk, 0);
    } else {
      // Tens of chunks per wave: a branch-free loop whose last iteration
      // re-reads its own chunk schedules better than the peeled form.
      for (; c < c1; c += NW)
        chunk_step(std::true_type{}, c * kChunk, (c + NW < c1 ? c + NW : c) * kChunk);
    }
  }

  // Wave partial -> LDS.  oacc[qb][j][e] is O(row qb*16 + r, head-dim 8 (4 h + e) + j).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = xgroup_sum(lsum[qb]);
    const int row = qb * 16 + r;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 8 * (4 * h + e) + j;
        if (d < D) lds_o[wave][row][d] = oacc[qb][j][e];
      }
    if (h == 0) {
      lds_ml[wave][row][0] = m[qb];
      lds_ml[wave][row][1] = l;
    }
  }
  __syncthreads();

  // Merge the waves.  With a single split per unit this is the final result
  // (normalised and stored straight to the output); otherwise the work-group
  // partial goes to the workspace, and the work-group that completes the
  // unit's last split merges the splits.
  const size_t part = ((size_t)unit * a.n_qs + qs) * a.n_splits + split;
  float* wo = a.ws_o + part * SR * D;
  float* wml = a.ws_ml + part * SR * 2;
  const bool direct = a.n_splits == 1;
  const size_t orow0 = (size_t)(u.b * a.Hq + u.hk * a.g) * a.n_q + (size_t)qs * SR;
  // Thread t serves row t / TPR and, with j = t % TPR, the head-dim entries
  // dim(k) = 4 j + 4 TPR (k / 4) + k % 4, k < PER: each group of four is one
  // 16-byte piece, and the TPR threads of a row store whole 64-byte runs.
  constexpr int NT = NW * kWave;
  constexpr int TPR = NT / SR;
  constexpr int PER = D / TPR;
  constexpr bool VEC = PER % 4 == 0;
  static_assert(TPR * SR == NT && PER * TPR == D, "epilogue mapping");
  const int row = threadIdx.x / TPR;
  const int jr = threadIdx.x - row * TPR;
  auto dim = [&](int k) { return VEC ? 4 * jr + 4 * TPR * (k >> 2) + (k & 3) : jr * PER + k; };
  const int d0 = dim(0);
  const bool live = qs * SR + row < a.M;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, lds_ml[w][row][0]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float o[PER], l = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float sc = fast_exp2(lds_ml[w][row][0] - mu);
    l += sc * lds_ml[w][row][1];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] += sc * lds_o[w][row][dim(k)];
  }
  __bf16* orow = static_cast<__bf16*>(a.out) + (orow0 + row) * D;
  if (direct) {
    if (live) {
#pragma unroll
      for (int k = 0; k < PER; ++k) orow[dim(k)] = (__bf16)(l > 0.f ? o[k] / l : 0.f);
      if (d0 == 0 && a.lse) a.lse[orow0 + row] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t own_o = coherent_view(wo, SR * D * 4);
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < PER; k += 4)
      store4_coherent(own_o, (row * D + dim(k)) * 4, f32x4{o[k], o[k + 1], o[k + 2], o[k + 3]});
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) store_coherent(wo + row * D + dim(k), o[k]);
  }
  if (d0 == 0) {
    store_coherent(wml + row * 2 + 0, mx);
    store_coherent(wml + row * 2 + 1, l);
  }
  if (!last_arrival(a.arrive + (size_t)unit * a.n_qs + qs, (uint32_t)a.n_splits, a.dev_err))
    return;

  // Split merge in split order: this work-group's partial is in registers,
  // the others' are loaded KS splits at a time (all in flight together).
  constexpr int KS = PER >= 16 ? 2 : (PER >= 8 ? 4 : 8);
  const size_t part0 = part - split;
  float gm = -INFINITY, gl = 0.f, ga[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) ga[k] = 0.f;
  for (int s0 = 0; s0 < a.n_splits; s0 += KS) {
    float vo[KS][PER], vm[KS], vl[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int s = s0 + j;
      const bool other = live && s < a.n_splits && s != split;
      const size_t ps = part0 + (other ? s : split);
      const __amdgpu_buffer_rsrc_t vw_o = coherent_view(a.ws_o + ps * SR * D, SR * D * 4);
      const __amdgpu_buffer_rsrc_t vw_ml = coherent_view(a.ws_ml + ps * SR * 2, SR * 2 * 4);
      vm[j] = mx;
      vl[j] = l;
#pragma unroll
      for (int k = 0; k < PER; ++k) vo[j][k] = o[k];
      if (other) {
        vm[j] = load_coherent(vw_ml, row * 8);
        vl[j] = load_coherent(vw_ml, row * 8 + 4);
        if constexpr (VEC) {
#pragma unroll
          for (int k = 0; k < PER; k += 4) {
            const f32x4 v = load4_coherent(vw_o, (row * D + dim(k)) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) vo[j][k + e] = v[e];
          }
        } else {
#pragma unroll
          for (int k = 0; k < PER; ++k) vo[j][k] = load_coherent(vw_o, (row * D + dim(k)) * 4);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (s0 + j >= a.n_splits) break;
      float s_old, s_new;
      merge_scales(gm, vm[j], s_old, s_new);
      gl = gl * s_old + vl[j] * s_new;
#pragma unroll
      for (int k = 0; k < PER; ++k) ga[k] = ga[k] * s_old + vo[j][k] * s_new;
    }
  }
  if (live) {
    const float inv = gl > 0.f ? 1.f / gl : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) orow[dim(k)] = (__bf16)(ga[k] * inv);
    if (d0 == 0 && a.lse) a.lse[orow0 + row] = gl > 0.f ? (gm + __log2f(gl)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel for wide query blocks (candidate trees): all waves of a
// work-group share every K/V chunk through LDS.
//
// Each wave owns 32 query rows (two MFMA blocks, Q in registers); the
// work-group covers WAVES*32 rows of one (sequence, kv head) unit, so one
// pass over the keys serves them all.  Chunks of 64 keys are copied HBM ->
// LDS with direct-to-LDS loads (global_load_lds_dwordx4: lane l's 16 bytes
// land at base + 16 l), the K rows into one ring of 16 KB tiles and the V
// rows into another:
//   K tile: 64 rows x 256 B, 16-byte pieces XOR-swizzled by row (loaded as
//      1 KB contiguous runs; the A operand of lane (h,r), K[16 kb + r][32 s +
//      8 h .. +8], is one conflict-free 16-byte read);
//   V tile: 64 rows x 256 B, 32-byte granules XOR-swizzled by row -- each
//      wave builds its MFMA operands with gfx950's transposing LDS reads
//      (ds_read_b64_tr_b16), so no register transpose is needed.
//
// Per chunk c a wave runs an MFMA block M_c = {O += V_{c-1}^T P_{c-1}^T,
// S_c = K_c Q^T} and a VALU block X_c = {softmax of S_c -> P_c}; the PV
// product of a chunk is deferred into the next chunk's MFMA block.  The
// work-group has one barrier per chunk, B_c: before it each wave waits for
// its own copies of the tile it reads next (explicit vmcnt waits; the copies
// are inline assembly, see lds_dma16), after it the copy of K chunk c+4 goes
// into the tile K chunk c-1 used and the copy of V chunk c+3 into the tile V
// chunk c-2 used.  Waves 0-3 pass B_c right
// before M_c; waves 4-7 right before X_{c-1}, i.e. half a chunk earlier in
// their own program.  Waves are placed on the four SIMDs in turn, so each
// SIMD holds one wave of each group, and the barrier keeps them in opposite
// phases: while one runs its MFMA block the other runs its softmax.  Either
// way every wave reads only K tile c and V tile c-1 between B_c and B_{c+1},
// so each ring needs one tile being read and the rest can be in flight: with
// five tiles per ring (160 KB) the K of chunks c+1..c+4 and the V of chunks
// c..c+3 are in flight, 128 KB per CU, twice what one ring of whole chunks
// leaves room for.
//
// The softmax of a row runs once per chunk over its 16 scores per lane.  The
// running max is only moved (and O rescaled) when a chunk exceeds it by more
// than 2^8 (log2 domain); otherwise the exponentials are taken against the
// old max and stay below 256, which keeps the rescale off the VALU in the
// common case.  Row sums of P come from one more MFMA per 32 keys with an
// all-ones A operand, so they sum exactly the bf16 weights that multiply V.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// XOR applied to the 16-byte piece index of V row `row` in an LDS tile
// (flips 32-byte granules: granule g of the row is stored at g ^ (row % 8)).
__device__ __forceinline__ int v_swizzle(int row) { return (row & 7) << 1; }
// XOR applied to the 16-byte piece index of K row `row` in an LDS tile.
__device__ __forceinline__ int k_swizzle(int row) { return row & 15; }

constexpr int kTreeChunk = 64;        // keys per chunk
constexpr int kTreeNK = 5;            // K tiles in the ring
constexpr int kTreeNV = 5;            // V tiles in the ring (4 with a page table in LDS)
constexpr float kRescaleTau = 8.0f;   // log2 units

// The copy is issued as inline assembly on purpose: the compiler treats a
// direct-to-LDS load as a pending write to every LDS location, and before the
// next LDS read it would wait for all loads in flight (vmcnt(0)), chunks
// copied ahead included, which serialises the copies with the compute.  The
// kernel orders its tiles itself: an explicit vmcnt wait on this wave's own
// copies, then a work-group barrier, before any wave reads a tile.  M0 holds
// the (wave-uniform) LDS destination; one wait state separates its write from
// the load that reads it.  M0 is a register the compiler reserves, so the
// statement saves it and puts it back instead of declaring it clobbered.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// Wait until at most n of this wave's vector-memory operations are pending
// (expcnt / lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};

template <int WAVES, bool PAGED = false>
__global__ __launch_bounds__(WAVES * kWave, 1) void attn_tree_mfma(AttnArgs a) {
  static_assert(WAVES == 8, "two groups of four waves: one wave of each group per SIMD");
  constexpr int D = 128, DS = 4, QB = 2;
  constexpr int SR = WAVES * 32;              // query rows per work-group
  constexpr int UPW = 32 / WAVES;             // 1 KB load units per wave per chunk
  constexpr int NK = kTreeNK;
  constexpr int NV = PAGED ? kTreeNV - 1 : kTreeNV;
  __shared__ __attribute__((aligned(16))) char ktiles[NK][16384];
  __shared__ __attribute__((aligned(16))) char vtiles[NV][16384];
  __shared__ int32_t lds_pages[PAGED ? kPageCap : 1];

  int unit, split, qs;
  if (!decode_tile(a, unit, split, qs)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Waves 4-7 take each barrier before their softmax block instead of their
  // MFMA block.  They also copy the V rows of every chunk, waves 0-3 the K rows.
  const bool late = wave >= WAVES / 2;
  const int r = lane & 15;
  const int h = lane >> 4;
  const size_t row_bytes = (size_t)D * 2;
  const UnitGeom u = unit_geom<false>(a, unit, split == 0 && qs == 0 && threadIdx.x == 0);
  const int n_keys = __builtin_amdgcn_readfirstlane(u.n_keys);
  const int p0 = __builtin_amdgcn_readfirstlane(u.p0);

  const char* qbase = static_cast<const char*>(a.q) +
                      ((size_t)(u.b * a.Hq + u.hk * a.g) * a.n_q) * row_bytes;
  const int row0 = qs * SR + wave * 32;       // first row of this wave
  const bool wave_live = row0 < a.M;
  bf16x8 qop[QB][DS];
  uint64_t anc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = row0 + qb * 16 + r;
    const bool live = row < a.M;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qop[qb][s] = live ? *reinterpret_cast<const bf16x8*>(qbase + (size_t)row * row_bytes +
                                                           (32 * s + 8 * h) * 2)
                        : bf16x8{};
    anc[qb] = live ? ancestor_mask(a, u.b, row % a.n_q) : 1ull;
  }

  // This split's range of 64-key chunks.
  const long long nch = (n_keys + kTreeChunk - 1) / kTreeChunk;
  const int c0 = (int)(nch * split / a.n_splits);
  int c1 = (int)(nch * (split + 1) / a.n_splits);
  const int last = n_keys - 1;
  int pfirst = 0;
  if constexpr (PAGED) {
    if (!stage_pages<PAGED>(a, u, c0 * kTreeChunk, min(c1 * kTreeChunk, n_keys), lds_pages,
                            pfirst))
      c1 = c0;
  }

  // This wave's share of a chunk: UPW 1 KB units (4 rows each) of the K rows
  // (waves 0-3) or the V rows (waves 4-7).  Slot (lane & 15) of a row takes the
  // 16-byte piece (lane & 15) ^ swizzle(row), so the operand reads below (16
  // rows, same column) hit distinct banks.  The offsets are loop-invariant.
  const bool dma_v = late;
  int drow[UPW];
  uint32_t doff[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int row = 4 * ((wave * UPW + i) & 15) + (lane >> 4);
    const int piece = (lane & 15) ^ (dma_v ? v_swizzle(row) : k_swizzle(row));
    drow[i] = row;
    doff[i] = (uint32_t)(row * 256 + piece * 16);
  }
  const char* dsrc =
      static_cast<const char*>(dma_v ? a.v : a.k) + (size_t)u.unit * a.L_cap * row_bytes;
  auto issue = [&](int c) {
    const int kbase = c * kTreeChunk;
    char* dst = (dma_v ? vtiles[c % NV] : ktiles[c % NK]) + ((wave * UPW) & 15) * 1024;
    // Keys kbase .. kbase+63 are consecutive rows from src: the unit's stream
    // in a contiguous cache, or the chunk's page (one lookup per chunk).
    const char* src = PAGED ? cache_row<PAGED>(a, u, kbase, dma_v ? 1 : 0, row_bytes, lds_pages,
                                               pfirst)
                            : dsrc + (size_t)kbase * row_bytes;
    if (kbase + kTreeChunk <= n_keys) {
#pragma unroll
      for (int i = 0; i < UPW; ++i) lds_dma16(src + doff[i], dst + i * 1024);
    } else {
      // Last, partial chunk: rows past the end repeat the last key (masked below).
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const int key = min(kbase + drow[i], last);
        lds_dma16(src + (size_t)(key - kbase) * row_bytes + (doff[i] & 255u), dst + i * 1024);
      }
    }
  };
  // Barrier B_k.  Before it, this wave's copies of the tile read next have
  // landed: K of chunk k (waves 0-3; up to NK-2 later K tiles may still be in
  // flight) or V of chunk k-1 (waves 4-7; up to NV-2 later V tiles).  After
  // it, the copy of K chunk k+NK-1 goes into the tile K chunk k-1 used, or of
  // V chunk k+NV-2 into the tile V chunk k-2 used.
  auto sync = [&](int k) {
    const int after = dma_v ? min(NV - 2, c1 - k) : min(NK - 2, c1 - 1 - k);
    wait_vmcnt(UPW * max(after, 0));
    __syncthreads();
    const int next = dma_v ? k + NV - 2 : k + NK - 1;
    if (next < c1) issue(next);
  };

  float m[QB];
  f32x4 lacc[QB];
  f32x4 oacc[QB][8];
  f32x4 sacc[QB][4];
  bf16x8 pop[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(
      bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  // S^T for both 32-key halves of a chunk: sacc[qb][kb][e] = score(key 16 kb + 4 h + e,
  // row qb*16 + r).
  auto qk = [&](const char* tile) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 kop[2][DS];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int s = 0; s < DS; ++s)
          kop[kk][s] = *reinterpret_cast<const bf16x8*>(
              tile + (32 * half + 16 * kk + r) * 256 + (((4 * s + h) ^ k_swizzle(r)) << 4));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][s], qop[qb][s], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][s], qop[qb][s], acc1, 0, 0, 0);
        }
        sacc[qb][2 * half] = acc0;
        sacc[qb][2 * half + 1] = acc1;
      }
    }
  };

  // O^T += V^T P^T and l += 1^T P^T.  The A operand of dim block blk is, in
  // lane (h, r), V[key(h, t)][16 blk + r] for t = 0..7 (key(h, t) = 16 (t / 4)
  // + 4 h + t % 4 within the half): two transposing LDS reads, each of four
  // keys.  In a read, lane (h, r) points at 4 dims (16 blk + 4 (r % 4) ..) of
  // key 4 h + r / 4 (+16 for the second), and the hardware hands lane r the
  // dim 16 blk + r of all four keys.
  auto pv = [&](const char* tile) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop[qb][half], lacc[qb], 0, 0, 0);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        v4i16 part[2];
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
          const int vrow = 32 * half + 16 * sec + 4 * h + (r >> 2);
          const int gp = 2 * blk + ((r & 3) >> 1);          // global 16-byte piece
          const char* src = tile + vrow * 256 + ((gp ^ v_swizzle(vrow)) << 4) +
                            ((r & 1) << 3);
          part[sec] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(src));
        }
        const v8i16 w = {part[0][0], part[0][1], part[0][2], part[0][3],
                         part[1][0], part[1][1], part[1][2], part[1][3]};
        const bf16x8 vop = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][blk] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[qb][half], oacc[qb][blk], 0, 0, 0);
      }
    }
  };

  // Scores of chunk c -> bf16 weights P_c (and the running max / rescale).
  // Chunks that reach the block's own keys (or the end) apply the tree mask;
  // the loop below runs the other chunks through a mask-free copy.
  auto softmax = [&](int c, auto masked) {
    const int kbase = c * kTreeChunk;
    constexpr bool need_mask = decltype(masked)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Raw scores; the softmax scale (> 0, in log2 units) is applied to the
      // max and folded into the exponent's FMA.
      float sv[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) sv[t] = sacc[qb][t >> 2][t & 3];
      if constexpr (need_mask) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = kbase + 16 * (t >> 2) + 4 * h + (t & 3);
          const int rel = key - p0;
          const bool anc_ok = ((anc[qb] >> (rel & 63)) & 1ull) != 0;
          const bool ok = key < n_keys && (rel < 0 || anc_ok);
          sv[t] = ok ? sv[t] : -INFINITY;
        }
      }
      // The row max only matters when it passes m + tau, so each lane first
      // tests its own 16 scores; the exact max across the row's four lanes
      // (two cross-lane rounds) is taken only when some lane passes.
      float lm = sv[0];
#pragma unroll
      for (int t = 1; t < 16; ++t) lm = fmaxf(lm, sv[t]);
      if (__any(lm * a.scale_log2 > m[qb] + kRescaleTau)) {
        const float cm = xgroup_max(lm) * a.scale_log2;
        const bool grow = cm > m[qb] + kRescaleTau;
        const float mn = grow ? cm : m[qb];
        const float alpha = grow ? fast_exp2(m[qb] - mn) : 1.f;
        m[qb] = mn;
        lacc[qb] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[qb][j] *= alpha;
      }
      const float mu = (m[qb] == -INFINITY) ? 0.f : m[qb];
      float p[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) p[t] = fast_exp2(fmaf(sv[t], a.scale_log2, -mu));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float* ph = p + 8 * half;
        u32x4 pk = {pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3]),
                    pack_bf16x2(ph[4], ph[5]), pack_bf16x2(ph[6], ph[7])};
        pop[qb][half] = __builtin_bit_cast(bf16x8, pk);
      }
    }
  };

  // Iteration c: [B_c] M_c [B_{c+1} for waves 4-7] X_c.  The last iteration
  // (c = c1) only adds the deferred PV product of chunk c1-1.
  auto step = [&](int c, auto masked) {
    if (!late) sync(c);
    if (wave_live) {
      if (c > c0) pv(vtiles[(c - 1) % NV]);
      if (c < c1) qk(ktiles[c % NK]);
    }
    if (late && c < c1) sync(c + 1);
    if (wave_live && c < c1) softmax(c, masked);
  };
  // Prologue: K chunks c0 .. c0+NK-2, V chunks c0 .. c0+NV-3.  The Q,
  // ancestor and page-table loads are waited for first: the compiler does
  // not see the copies (inline assembly), so otherwise it would wait for
  // every load in flight, copies included, at the first use of Q per chunk.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  const int pre = dma_v ? NV - 2 : NK - 1;
  for (int i = 0; i < pre; ++i)
    if (c0 + i < c1) issue(c0 + i);
  if (late) sync(c0);
  // Chunks below cm hold prefix keys only (every key < p0 <= n_keys).
  const int cm = min(max(p0 / kTreeChunk, c0), c1);
  for (int c = c0; c < cm; ++c) step(c, MaskTag<false>{});
  for (int c = cm; c <= c1; ++c) step(c, MaskTag<true>{});

  if (!wave_live) return;
  // Each wave owns its rows: write them straight to the output (one split) or
  // to the workspace partial of this (unit, slice, split).
  const bool direct = a.n_splits == 1;
  const size_t orow0 = (size_t)(u.b * a.Hq + u.hk * a.g) * a.n_q;
  const size_t part = ((size_t)unit * a.n_qs + qs) * a.n_splits + split;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = lacc[qb][0];                   // every lane of a column holds the row sum
    const int srow = wave * 32 + qb * 16 + r;      // row within the slice
    const int row = qs * SR + srow;
    if (row >= a.M) continue;
    if (direct) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      __bf16* o = static_cast<__bf16*>(a.out) + (orow0 + row) * D;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[16 * blk + 4 * h + e] = (__bf16)(oacc[qb][blk][e] * inv);
      if (h == 0 && a.lse) a.lse[orow0 + row] = l > 0.f ? (m[qb] + __log2f(l)) * kLn2 : -INFINITY;
    } else {
      float* wo = a.ws_o + (part * SR + srow) * D;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) wo[16 * blk + 4 * h + e] = oacc[qb][blk][e];
      if (h == 0) {
        float* wml = a.ws_ml + (part * SR + srow) * 2;
        wml[0] = m[qb];
        wml[1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU split kernel: one wave per query row, lanes over the head dim.
// ---------------------------------------------------------------------------
template <int D, bool WINDOW, bool PAGED = false>
__global__ __launch_bounds__(kThreads) void attn_split_valu(AttnArgs a) {
  constexpr int DPL = D / 64;  // head-dim entries per lane
  __shared__ int32_t lds_pages[PAGED ? kPageCap : 1];
  int unit, split, qs;
  if (!decode_tile(a, unit, split, qs)) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row_bytes = (size_t)D * 4;
  const UnitGeom u = unit_geom<WINDOW>(a, unit, split == 0 && qs == 0 && threadIdx.x == 0);
  window_append<WINDOW>(a, u, split, qs, row_bytes);

  int c0, c1;
  chunk_range(u.n_keys, split, a.n_splits, c0, c1);
  int pfirst = 0;
  if (PAGED &&
      !stage_pages<PAGED>(a, u, c0 * kChunk, min(c1 * kChunk, u.n_keys), lds_pages, pfirst))
    c1 = c0;

  const int row = qs * kValuSlice + wave;
  if (row >= a.M) return;   // no barrier follows
  const float* qrow = reinterpret_cast<const float*>(
      static_cast<const char*>(a.q) +
      ((size_t)(u.b * a.Hq + u.hk * a.g) * a.n_q + row) * row_bytes);
  float qv[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) qv[e] = qrow[lane + 64 * e];
  const uint64_t anc = WINDOW ? 1ull : ancestor_mask(a, u.b, row % a.n_q);

  const int k0 = c0 * kChunk;
  const int k1 = min(c1 * kChunk, u.n_keys);

  float m = -INFINITY, l = 0.f;
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;

  constexpr int KB = 4;  // keys per step
  for (int kk = k0; kk < k1; kk += KB) {
    float s[KB];
    float vv[KB][DPL];
#pragma unroll
    for (int t = 0; t < KB; ++t) {
      int key = kk + t;
      const bool ok_key = key < k1;
      key = ok_key ? key : k1 - 1;
      const float* kr = reinterpret_cast<const float*>(
          WINDOW ? key_row<WINDOW>(a, u, key, 0, row_bytes)
                 : cache_row<PAGED>(a, u, key, 0, row_bytes, lds_pages, pfirst));
      const float* vr = reinterpret_cast<const float*>(
          WINDOW ? key_row<WINDOW>(a, u, key, 1, row_bytes)
                 : cache_row<PAGED>(a, u, key, 1, row_bytes, lds_pages, pfirst));
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        part = fmaf(qv[e], kr[lane + 64 * e], part);
        vv[t][e] = vr[lane + 64 * e];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
      bool ok = ok_key;
      if (ok && key >= u.p0) ok = (anc >> (key - u.p0)) & 1ull;
      s[t] = ok ? part * a.scale_log2 : -INFINITY;
    }
    float cm = s[0];
#pragma unroll
    for (int t = 1; t < KB; ++t) cm = fmaxf(cm, s[t]);
    const float mn = fmaxf(m, cm);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m - mu);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= alpha;
#pragma unroll
    for (int t = 0; t < KB; ++t) {
      const float p = fast_exp2(s[t] - mu);
      l += p;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(p, vv[t][e], o[e]);
    }
  }

  if (a.n_splits == 1) {
    const size_t orow = (size_t)(u.b * a.Hq + u.hk * a.g) * a.n_q + row;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) static_cast<float*>(a.out)[orow * D + lane + 64 * e] = o[e] * inv;
    if (lane == 0 && a.lse) a.lse[orow] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    return;
  }
  const size_t part = ((size_t)unit * a.n_qs + qs) * a.n_splits + split;
  float* wo = a.ws_o + (part * kValuSlice + wave) * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) wo[lane + 64 * e] = o[e];
  if (lane == 0) {
    float* wml = a.ws_ml + (part * kValuSlice + wave) * 2;
    wml[0] = m;
    wml[1] = l;
  }
}

// Separate merge kernel: one thread per (output row, 4 head-dim entries).
template <int D, typename OutT>
__global__ __launch_bounds__(256) void attn_merge(MergeArgs a) {
  constexpr int TPR = D / 4;  // threads per row
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)a.B * a.Hkv * a.M * TPR;
  if (gid >= total) return;
  const long long grow = gid / TPR;
  const int unit = (int)(grow / a.M);
  merge_item<D, OutT>(a, unit, (int)(grow - (long long)unit * a.M), (int)(gid - grow * TPR) * 4);
}

// ---------------------------------------------------------------------------
// Host-side planning and launch.
// ---------------------------------------------------------------------------
static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

AttnPlan plan_attention(int32_t B, int32_t Hkv, int32_t M, int32_t D, int32_t n_keys_max,
                        spec_dtype_t dtype, int32_t num_splits, bool window, int32_t page_size) {
  AttnPlan p{};
  const bool mfma = dtype == SPEC_BF16;
  const long long units = (long long)B * Hkv;
  const int chunks = ceil_div(n_keys_max, kChunk);
  // Query blocks wider than one streaming slice (candidate trees) go to the
  // LDS-shared kernel, so the K/V of a unit is read once for all its rows.
  p.tree_waves = (mfma && !window && D == 128 && M > 32) ? 8 : 0;
  p.slice_rows = p.tree_waves ? 32 * p.tree_waves : (mfma ? (M <= 16 ? 16 : 32) : kValuSlice);
  p.n_qs = ceil_div(M, p.slice_rows);
  if (num_splits > 0) {
    p.n_splits = num_splits;
  } else if (window) {
    // The draft window is a few hundred keys and latency-bound: spread it so
    // that every wave gets one chunk (measured faster than one work-group
    // per unit, which avoids the merge kernel but serialises the chunks).
    p.n_splits = (int)(mfma ? (chunks + kWaves - 1) / kWaves : (chunks + 7) / 8);
    if (p.n_splits < 1) p.n_splits = 1;
  } else {
    // Aim for about one work-group per CU (256 CUs): on the 8B / 32K, 128K
    // and 70B / 16K workloads fewer, longer key ranges streamed faster than
    // more, shorter ones (and need less merge traffic).  Every wave gets at
    // least one chunk.
    const long long target = 256;
    long long s = (target + units * p.n_qs - 1) / (units * p.n_qs);
    long long smax = mfma ? (chunks + kWaves - 1) / kWaves : chunks;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    p.n_splits = (int)s;
  }
  if (page_size > 0) {
    // A split's key range must fit the LDS page table: at most kPageCap - 1
    // pages of keys, so with alignment it touches at most kPageCap pages.
    const int ck = p.tree_waves ? kTreeChunk : kChunk;
    const long long nch = ceil_div(n_keys_max, ck);
    const long long per_split = (long long)(kPageCap - 1) * page_size / ck;   // chunks
    const long long smin = (nch + per_split - 1) / per_split;
    if (p.n_splits < smin) p.n_splits = (int)smin;
  }
  // The streaming kernel (chains, the draft window) merges its splits in the
  // last work-group of each unit: one launch, 4 us less per 8B/32K call than
  // the merge kernel.  The tree kernel keeps the merge kernel: the fused
  // epilogue moved its main-loop schedule (296 -> 354 us at one split).
  p.fuse_merge = mfma && p.n_splits > 1 && p.tree_waves == 0;
  const long long tiles = units * p.n_splits;
  p.grid = (int)(p.n_qs == 1 ? tiles : ((tiles + 7) / 8) * 8 * p.n_qs);
  const size_t parts = (size_t)tiles * p.n_qs;
  p.ws_sync_bytes = (((size_t)units * p.n_qs * sizeof(uint32_t)) + 255) & ~(size_t)255;
  p.ws_o_bytes = ((parts * p.slice_rows * D * sizeof(float)) + 255) & ~(size_t)255;
  p.ws_ml_bytes = ((parts * p.slice_rows * 2 * sizeof(float)) + 255) & ~(size_t)255;
  p.ws_bytes = p.ws_sync_bytes + p.ws_o_bytes + p.ws_ml_bytes;
  return p;
}

template <bool WINDOW, bool PAGED>
static hipError_t launch_split(const AttnArgs& a, spec_dtype_t dtype, hipStream_t stream) {
  dim3 grid(a.grid), block(kThreads);
  if (!WINDOW && a.tree_waves == 8) {
    hipLaunchKernelGGL((attn_tree_mfma<8, PAGED>), grid, dim3(512), 0, stream, a);
  } else if (WINDOW && dtype == SPEC_BF16 && a.n_splits == 1) {
    // One work-group per unit: 8 waves share the window and merge in LDS.
    dim3 wblock(8 * kWave);
    if (a.D == 128) {
      if (a.slice_rows == 16)
        hipLaunchKernelGGL((attn_split_mfma<128, 1, true, 8>), grid, wblock, 0, stream, a);
      else
        hipLaunchKernelGGL((attn_split_mfma<128, 2, true, 8>), grid, wblock, 0, stream, a);
    } else {
      if (a.slice_rows == 16)
        hipLaunchKernelGGL((attn_split_mfma<64, 1, true, 8>), grid, wblock, 0, stream, a);
      else
        hipLaunchKernelGGL((attn_split_mfma<64, 2, true, 8>), grid, wblock, 0, stream, a);
    }
  } else if (dtype == SPEC_BF16) {
    if (a.D == 128) {
      if (a.slice_rows == 16)
        hipLaunchKernelGGL((attn_split_mfma<128, 1, WINDOW, kWaves, PAGED>), grid, block, 0, stream,
                           a);
      else
        hipLaunchKernelGGL((attn_split_mfma<128, 2, WINDOW, kWaves, PAGED>), grid, block, 0, stream,
                           a);
    } else {
      if (a.slice_rows == 16)
        hipLaunchKernelGGL((attn_split_mfma<64, 1, WINDOW, kWaves, PAGED>), grid, block, 0, stream,
                           a);
      else
        hipLaunchKernelGGL((attn_split_mfma<64, 2, WINDOW, kWaves, PAGED>), grid, block, 0, stream,
                           a);
    }
  } else {
    if (a.D == 128)
      hipLaunchKernelGGL((attn_split_valu<128, WINDOW, PAGED>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_split_valu<64, WINDOW, PAGED>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool window, spec_dtype_t dtype, void* out,
                            float* lse, hipStream_t stream) {
  hipError_t e = window           ? launch_split<true, false>(a, dtype, stream)
                 : a.block_table ? launch_split<false, true>(a, dtype, stream)
                                 : launch_split<false, false>(a, dtype, stream);
  if (e != hipSuccess || a.n_splits == 1 || a.arrive) return e;
  MergeArgs m;
  m.ws_o = a.ws_o;
  m.ws_ml = a.ws_ml;
  m.out = out;
  m.lse = lse;
  m.B = a.B;
  m.Hq = a.Hq;
  m.Hkv = a.Hkv;
  m.g = a.g;
  m.n_q = a.n_q;
  m.D = a.D;
  m.M = a.M;
  m.slice_rows = a.slice_rows;
  m.n_qs = a.n_qs;
  m.n_splits = a.n_splits;
  const long long threads = (long long)a.B * a.Hkv * a.M * (a.D / 4);
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (dtype == SPEC_BF16) {
    if (a.D == 128)
      hipLaunchKernelGGL((attn_merge<128, __bf16>), grid, block, 0, stream, m);
    else
      hipLaunchKernelGGL((attn_merge<64, __bf16>), grid, block, 0, stream, m);
  } else {
    if (a.D == 128)
      hipLaunchKernelGGL((attn_merge<128, float>), grid, block, 0, stream, m);
    else
      hipLaunchKernelGGL((attn_merge<64, float>), grid, block, 0, stream, m);
  }
  return hipGetLastError();
}

}  // namespace specv
