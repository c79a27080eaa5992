// EAGLE-2 dynamic draft tree: per-row log-sum-exp and top-k over the vocabulary,
// then the budgeted selection of the tree.
//
// [P3] section 2 (dynamic draft tree: nodes valued by draft confidence, expansion
// deep where confident and wide where not, greedy maximisation of the expected
// acceptance length under a fixed draft-token budget); [P1] innovations list
// items 1 and 3 (top tokens per draft step; pruning to high-probability paths).
// A node's value is its path probability, kept as the cumulative log-probability
// "score"; the budgeted tree is the root plus the best n_nodes-1 candidates.
//
// Kernels:
//   rerank_rows   one workgroup per (row, vocabulary chunk): the chunk's max and
//                 exp-sum, and its top-k in (logit desc, token asc) order, ranked
//                 in parallel over a short candidate list.  Streams the fp32 draft
//                 logits once (the HBM-bound part).
//   rerank_merge  one wave per row: merges the chunk results into the row's lse and
//                 top-k (same order).
//   rerank_tree   one workgroup per sequence: candidate scores depth by depth,
//                 frontier = best k of each depth (ranks counted within the depth),
//                 final = best n_nodes-1 overall (rank within the depth plus binary
//                 searches in the other depths' sorted keys); output breadth first.
#include "common.h"
#include "internal.h"

namespace eagle {

namespace {

constexpr int kRowThreads = 256;
constexpr int kRowPer = 32;                        // elements per thread in rerank_rows
constexpr int kChunk = kRowThreads * kRowPer;      // vocabulary entries per chunk
constexpr int kTreeThreads = 1024;
constexpr int kMaxCand = 2048;                     // candidates per sequence in rerank_tree
constexpr int kMaxRowList = 1024;                  // R * k row-list entries staged in rerank_tree
constexpr int kMaxRows = 512;                      // draft rows per sequence

// (value, index) order: larger value first, then smaller index
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

struct VI {
  float v;
  int i;
};

// (value desc, index asc) as one unsigned 64-bit key: larger key = better.  -0.0 is
// mapped to +0.0 first, so the two zeros rank as equal values (ties then go to the
// lower index), as the (value, index) comparison `better` has them.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ float key_value(uint64_t key) { return ordered_float((uint32_t)(key >> 32)); }
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ uint64_t vi_key(float v, int i) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ VI wave_best(VI a) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    VI b{__shfl_xor(a.v, o), __shfl_xor(a.i, o)};
    if (better(b.v, b.i, a.v, a.i)) a = b;
  }
  return a;
}

// workspace: chunk results [rows][chunks] of (max, sum) + top-k (value, index);
// merged rows [rows][k] (value, index)
struct RrWs {
  float2* chunk_mz;
  float* chunk_v;
  int* chunk_i;
  float* row_v;
  int* row_i;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ __device__ inline RrWs rr_ws(void* ws, const RerankPlan& pl) {
  RrWs w;
  char* p = (char*)ws;
  const size_t rows = (size_t)pl.B * pl.R;
  const size_t nc = rows * pl.chunks;
  w.chunk_mz = (float2*)p;
  p += align256(nc * sizeof(float2));
  w.chunk_v = (float*)p;
  p += align256(nc * pl.k * sizeof(float));
  w.chunk_i = (int*)p;
  p += align256(nc * pl.k * sizeof(int));
  w.row_v = (float*)p;
  p += align256(rows * pl.k * sizeof(float));
  w.row_i = (int*)p;
  return w;
}

// Wave-wide max / sum with every lane holding the result, in registers: DPP steps
// within rows of 16 (lane ^ 1, lane ^ 2, mirror within 8, mirror within 16), then
// the 16- and 32-lane swaps pair each lane with lane ^ 16 and lane ^ 32.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = op(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = op(x, dpp<0x141>(x));   // row_half_mirror
  x = op(x, dpp<0x140>(x));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// k-th largest (1 <= k <= 64) of the wave's 64 values: the largest t (in the
// order-preserving unsigned image) with at least k values >= t, found bit by bit
// with ballots (no cross-lane data movement).
__device__ __forceinline__ float wave_kth_largest(float v, int k) {
  const uint32_t u = ordered_bits(v);
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    if (__popcll(__ballot(u >= c)) >= k) t = c;
  }
  return ordered_float(t);
}

// Rank of key among keys lb .. lb+n-1 of an LDS list: how many come first (larger
// keys first).  Independent LDS reads, unrolled, so the loop is not bound by one
// read's latency per comparison.
__device__ __forceinline__ int rank_in(const uint64_t* keys, int lb, int n, uint64_t key) {
  int rank = 0;
  int o = lb;
  const int end = lb + n;
  for (; o + 8 <= end; o += 8) {
    uint64_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = keys[o + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) rank += v[e] > key ? 1 : 0;
  }
  for (; o < end; ++o) rank += keys[o] > key ? 1 : 0;
  return rank;
}

// One workgroup per (row, vocabulary chunk of kChunk entries).  Max and exp-sum of the chunk,
// and its top-k: every wave keeps the valid elements not below the k-th largest of
// its 64 lane maxima (at least k of its elements are that large, so its top-k is
// among them) and appends them to a short LDS list as (logit desc, token asc) keys;
// each listed key's rank in the list is counted, in parallel over the list, and
// ranks below k are written in rank order (padding past a chunk with fewer than k
// valid entries).  If ties make the list overflow, the whole chunk is searched by k
// rounds instead (same order, same result).
constexpr int kCandCap = 512;

// VEC: 16-byte loads (V % 4 == 0 and 16-byte aligned logits), element e of thread tid
// is x0 + (e/4)*1024 + 4*tid + e%4; otherwise 4-byte loads, element e is
// x0 + e*256 + tid.  Either way every load instruction is coalesced.
template <bool VEC>
__global__ void __launch_bounds__(kRowThreads)
rerank_rows(const float* __restrict__ logits, RerankPlan pl, void* ws) {
  __shared__ float redf[kRowThreads / 64];
  __shared__ uint64_t cand_key[kCandCap];
  __shared__ int ncand_s;
  __shared__ VI red[kRowThreads / 64];
  RrWs w = rr_ws(ws, pl);
  const int chunk = blockIdx.x % pl.chunks;
  const int rr = blockIdx.x / pl.chunks;   // rr-th processed row: sequence rr / nrows
  const size_t row = (size_t)(rr / pl.nrows) * pl.R + pl.row0 + rr % pl.nrows;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int V = pl.V;
  const int x0 = chunk * pl.chunk_len;
  const float* src = logits + row * (size_t)V;

  auto pos_of = [&](int e) {
    return VEC ? x0 + (e >> 2) * (4 * kRowThreads) + 4 * tid + (e & 3) : x0 + e * kRowThreads + tid;
  };
  float val[kRowPer];
  if constexpr (VEC) {
    static_assert(kRowPer % 4 == 0, "whole 16-byte groups per thread");
#pragma unroll
    for (int q = 0; q < kRowPer / 4; ++q) {
      const int x = pos_of(4 * q);   // x % 4 == 0 and V % 4 == 0: x < V covers x + 3
      const f32x4 v = x < V ? *(const f32x4*)(src + x) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int j = 0; j < 4; ++j) val[4 * q + j] = v[j];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kRowPer; ++e) {
      const int x = pos_of(e);
      val[e] = x < V ? src[x] : -INFINITY;
    }
  }
  // index of element e (past the row: the largest index, below every real one)
  auto idx_of = [&](int e) {
    const int x = pos_of(e);
    return x < V ? x : 0x7fffffff;
  };
  float lmax = val[0];
#pragma unroll
  for (int e = 1; e < kRowPer; ++e) lmax = fmaxf(lmax, val[e]);

  // chunk max and exp-sum
  if (tid == 0) ncand_s = 0;
  float mx = wave_reduce<true>(lmax);
  if (lane == 0) redf[wid] = mx;
  __syncthreads();
  mx = redf[0];
#pragma unroll
  for (int i = 1; i < kRowThreads / 64; ++i) mx = fmaxf(mx, redf[i]);
  float z = 0.f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int e = 0; e < kRowPer; ++e) z += __builtin_amdgcn_exp2f((val[e] - mx) * kLog2e);
  }
  z = wave_reduce<false>(z);
  __syncthreads();
  if (lane == 0) redf[wid] = z;

  // candidates of this wave: valid elements >= the k-th largest lane maximum; list
  // slots by LDS adds (the list's order does not matter: ranks are counted)
  const int k = pl.k;
  const float thr = k >= 64 ? -INFINITY : wave_kth_largest(lmax, k);
  int mine = 0;
#pragma unroll
  for (int e = 0; e < kRowPer; ++e) mine += (val[e] >= thr && idx_of(e) < V) ? 1 : 0;
  const int pos0 = mine > 0 ? atomicAdd(&ncand_s, mine) : 0;
  __syncthreads();
  const int ncand = ncand_s;
  if (tid == 0) {
    float zt = 0.f;
    for (int i = 0; i < kRowThreads / 64; ++i) zt += redf[i];
    w.chunk_mz[row * pl.chunks + chunk] = make_float2(mx, zt);
  }
  float* out_v = w.chunk_v + (row * pl.chunks + chunk) * k;
  int* out_i = w.chunk_i + (row * pl.chunks + chunk) * k;
  if (ncand <= kCandCap) {
    int pos = pos0;
#pragma unroll
    for (int e = 0; e < kRowPer; ++e)
      if (val[e] >= thr && idx_of(e) < V) cand_key[pos++] = vi_key(val[e], idx_of(e));
    __syncthreads();
    for (int c = tid; c < ncand; c += kRowThreads) {
      const uint64_t key = cand_key[c];
      const int rank = rank_in(cand_key, 0, ncand, key);
      if (rank < k) {
        out_v[rank] = key_value(key);
        out_i[rank] = key_index(key);
      }
    }
    for (int r = ncand + tid; r < k; r += kRowThreads) {
      out_v[r] = -INFINITY;
      out_i[r] = 0x7fffffff;
    }
    return;
  }
  // many ties: k rounds over the whole chunk, re-read from memory (a rare path; the
  // registers of the main path stay free)
  float pv = INFINITY;
  int pi = -1;
  for (int r = 0; r < k; ++r) {
    VI best{-INFINITY, 0x7fffffff};
#pragma unroll 1
    for (int e = 0; e < kRowPer; ++e) {
      const int x = x0 + e * kRowThreads + tid;
      const float v = x < V ? src[x] : -INFINITY;
      const int ie = x < V ? x : 0x7fffffff;
      const bool after = v < pv || (v == pv && ie > pi);
      if (after && better(v, ie, best.v, best.i)) best = VI{v, ie};
    }
    best = wave_best(best);
    __syncthreads();
    if (lane == 0) red[wid] = best;
    __syncthreads();
    VI bb = red[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / 64; ++i)
      if (better(red[i].v, red[i].i, bb.v, bb.i)) bb = red[i];
    if (tid == 0) {
      out_v[r] = bb.v;
      out_i[r] = bb.i;
    }
    pv = bb.v;
    pi = bb.i;
  }
}

// One wave per row: merges the chunk results into the row's lse and top-k.  The
// row's k best are not below T = the k-th largest chunk maximum (the k chunks with
// the largest maxima hold k elements >= T), so only chunk entries >= T are kept; each
// kept entry's rank among them is counted, and entries of rank < k are written in
// rank order.
constexpr int kMergeCap = 256;   // kept entries per row (more: every entry is kept and ranked)

__global__ void __launch_bounds__(256)
rerank_merge(RerankPlan pl, void* ws, float* __restrict__ draft_lse) {
  __shared__ uint64_t keys[4][1024];
  RrWs w = rr_ws(ws, pl);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int rr = blockIdx.x * 4 + wid;
  if (rr >= pl.B * pl.nrows) return;
  const int row = (rr / pl.nrows) * pl.R + pl.row0 + rr % pl.nrows;
  const int k = pl.k, chunks = pl.chunks;
  const float* cv = w.chunk_v + (size_t)row * chunks * k;
  const int* ci = w.chunk_i + (size_t)row * chunks * k;
  const int n_all = chunks * k;
  // every load the wave needs is requested here, before any of it is used: the chunk
  // (max, exp-sum) pairs, the chunk maxima for the threshold, and the first
  // kMergePre * 64 list entries (one memory round trip for the usual sizes)
  constexpr int kMergePre = 4;
  float2 mz[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    mz[u] = c < chunks ? w.chunk_mz[(size_t)row * chunks + c] : make_float2(-INFINITY, 0.f);
  }
  const bool use_thr = chunks <= 64 && k <= chunks;
  const float cm = (use_thr && lane < chunks) ? cv[(size_t)lane * k] : -INFINITY;
  float pv[kMergePre];
  int pi[kMergePre];
#pragma unroll
  for (int u = 0; u < kMergePre; ++u) {
    const int e = 64 * u + lane;
    pv[u] = e < n_all ? cv[e] : -INFINITY;
    pi[u] = e < n_all ? ci[e] : 0;
  }
  float mx = fmaxf(mz[0].x, mz[1].x);
  for (int c = lane + 128; c < chunks; c += 64) mx = fmaxf(mx, w.chunk_mz[(size_t)row * chunks + c].x);
  mx = wave_reduce<true>(mx);
  float z = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (mz[u].x > -INFINITY) z += mz[u].y * __builtin_amdgcn_exp2f((mz[u].x - mx) * kLog2e);
  for (int c = lane + 128; c < chunks; c += 64) {
    const float2 e = w.chunk_mz[(size_t)row * chunks + c];
    if (e.x > -INFINITY) z += e.y * __builtin_amdgcn_exp2f((e.x - mx) * kLog2e);
  }
  z = wave_reduce<false>(z);
  if (lane == 0) draft_lse[row] = mx + logf(z);

  // threshold: k-th largest chunk maximum (entry 0 of each chunk list); chunks <= 64
  // whenever chunks * k <= 1024 and k >= 16, otherwise keep everything
  const float thr = use_thr ? wave_kth_largest(cm, k) : -INFINITY;
  // keep entries >= thr (lane-major over the chunks * k entries)
  uint64_t* kk = keys[wid];
  int kept = 0;
  for (int base = 0; base < n_all; base += 64) {
    const int e = base + lane;
    const int u = base / 64;
    float v;
    int vi;
    if (u < kMergePre) {
      v = u == 0 ? pv[0] : (u == 1 ? pv[1] : (u == 2 ? pv[2] : pv[3]));
      vi = u == 0 ? pi[0] : (u == 1 ? pi[1] : (u == 2 ? pi[2] : pi[3]));
    } else {
      v = e < n_all ? cv[e] : -INFINITY;
      vi = e < n_all ? ci[e] : 0;
    }
    const bool keep = e < n_all && v >= thr;
    const uint64_t m = __ballot(keep);
    if (keep) kk[kept + __popcll(m & ((1ull << lane) - 1ull))] = vi_key(v, vi);
    kept += __popcll(m);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's own LDS writes are done
  // rank by counting; distinct keys (distinct token ids) give distinct ranks
  for (int e = lane; e < kept; e += 64) {
    const uint64_t key = kk[e];
    int rank = 0;
    for (int o = 0; o < kept; ++o) rank += kk[o] > key ? 1 : 0;
    if (rank < k) {
      w.row_v[(size_t)row * k + rank] = key_value(key);
      w.row_i[(size_t)row * k + rank] = key_index(key);
    }
  }
}

// Adds to rank[c] (c in lb .. lb+n-1) how many of the candidates lb .. lb+n-1 come
// first (LDS adds; rank[] must start at zero).  Each candidate's count is split over
// P = 8, 4, 2 or 1 threads (n <= 128, 256, 512 or more): thread tid takes candidate
// tid % (1024/P) and part tid / (1024/P).  No barrier.
__device__ void rank_level(const uint64_t* keys, int lb, int n, int* rank) {
  static_assert(kTreeThreads == 1024, "the thread split below assumes 1024 threads");
  const int tid = threadIdx.x;
  const int lg = n <= 128 ? 7 : (n <= 256 ? 8 : (n <= 512 ? 9 : 10));   // log2(1024/P)
  const int P = kTreeThreads >> lg;
  const int per = (n + P - 1) >> (10 - lg);   // ceil(n / P)
  const int part = tid >> lg;
  const int lo = part * per;
  const int cnt = min(per, n - lo);
  for (int c = tid & ((1 << lg) - 1); c < n; c += 1 << lg)
    if (cnt > 0) atomicAdd(&rank[lb + c], rank_in(keys, lb + lo, cnt, keys[lb + c]));
}

// Candidate arrays of one sequence in LDS.  Level 1 = the root's proposals; level
// d+1 = the proposals of the frontier of level d (its best k candidates, which take
// rows 1 + (d-1)k .. in rank order).  Ids: level 1 = [0, k), level d+1 =
// [k + (d-1)k^2, k + d k^2).  c_rank = rank within the candidate's level.
struct TreeLds {
  int c_rank[kMaxCand];
  float c_score[kMaxCand];
  uint64_t c_key[kMaxCand];
  uint64_t c_sorted[kMaxCand];   // each level's keys in rank order (final selection)
  int c_tok[kMaxCand];
  short c_par[kMaxCand];
  short c_row[kMaxCand];
  short c_pos[kMaxCand];
  float s_rv[kMaxRowList];
  int s_ri[kMaxRowList];
  float s_lse[kMaxRows];
};

__device__ __forceinline__ int level_base(int d, int k) { return d == 1 ? 0 : k + (d - 2) * k * k; }
__device__ __forceinline__ int level_size(int d, int k) { return d == 1 ? k : k * k; }

// stages the sequence's row lists (rows 0..nrows-1) and normalisers
__device__ void stage_rows(const RerankPlan& pl, const RrWs& w, const float* draft_lse, int b,
                           int nrows, TreeLds& t) {
  const int k = pl.k, R = pl.R;
  for (int e = threadIdx.x; e < nrows * k; e += kTreeThreads) {
    t.s_rv[e] = w.row_v[(size_t)b * R * k + e];
    t.s_ri[e] = w.row_i[(size_t)b * R * k + e];
  }
  for (int r = threadIdx.x; r < nrows; r += kTreeThreads) t.s_lse[r] = draft_lse[(size_t)b * R + r];
  __syncthreads();
}

// candidates (score, token, parent, key) and within-level ranks of levels 1..L, and
// the frontier rows of levels 1..L-1 (c_row, -1 elsewhere); ends with a barrier
__device__ void grow_levels(const RerankPlan& pl, int L, TreeLds& t) {
  const int tid = threadIdx.x;
  const int k = pl.k;
  const int total = k + (L - 1) * k * k;
  const float* rv = t.s_rv;
  const int* ri = t.s_ri;
  const float* lse = t.s_lse;
  for (int c = tid; c < total; c += kTreeThreads) {
    t.c_row[c] = -1;
    t.c_rank[c] = 0;
  }
  for (int r = tid; r < k; r += kTreeThreads) {
    const float sc = rv[r] - lse[0];
    t.c_score[r] = sc;
    t.c_key[r] = vi_key(sc, r);
    t.c_tok[r] = ri[r];
    t.c_par[r] = -1;
  }
  __syncthreads();
  for (int d = 1; d <= L; ++d) {
    const int lb = level_base(d, k), ln = level_size(d, k);
    rank_level(t.c_key, lb, ln, t.c_rank);
    __syncthreads();
    if (d == L) break;
    // frontier: the level's best k take rows 1 + (d-1)k + rank
    for (int c = lb + tid; c < lb + ln; c += kTreeThreads) {
      const int rank = t.c_rank[c];
      if (rank < k) {
        t.c_row[c] = (short)(1 + (d - 1) * k + rank);
        t.c_pos[rank] = (short)c;   // frontier slot -> candidate
      }
    }
    __syncthreads();
    // the k proposals of every frontier slot, one thread each (slot = e / 64,
    // proposal r = e % 64 < k)
    const int base = lb + ln;
    for (int e = tid; e < k * 64; e += kTreeThreads) {
      const int slot = e >> 6, r = e & 63;
      if (r >= k) continue;
      const int c = t.c_pos[slot];
      const int row = 1 + (d - 1) * k + slot;
      const int id = base + slot * k + r;
      const float sc = t.c_score[c] + (rv[(size_t)row * k + r] - lse[row]);
      t.c_score[id] = sc;
      t.c_key[id] = vi_key(sc, id);
      t.c_tok[id] = ri[(size_t)row * k + r];
      t.c_par[id] = (short)c;
    }
    __syncthreads();
  }
}

// Depth (level) of candidate c, from the level bases (no division).
__device__ __forceinline__ int level_of(int c, int k, int L) {
  int d = 1;
  for (int e = 2; e <= L; ++e) d += c >= level_base(e, k) ? 1 : 0;
  return d;
}

// For every level d in d0 .. d0+7 (<= L, != skip): adds how many keys of level d
// (descending in sorted) are larger than key.  Binary searches over the largest power
// of two not above the largest level, the levels in step, with clamped reads issued
// together: one LDS round trip per step.
__device__ __forceinline__ int count_larger8(const uint64_t* sorted, int d0, int L, int skip, int k,
                                             uint64_t key) {
  int lo[8], n[8], base[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = d0 + j;
    const bool on = d <= L && d != skip;
    n[j] = on ? level_size(d, k) : 0;
    base[j] = on ? level_base(d, k) : 0;
    lo[j] = 0;
  }
  const int nmax = k * k;
  int step = 1;
  while (step * 2 <= nmax) step *= 2;
  for (; step > 0; step >>= 1) {
    uint64_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = sorted[base[j] + min(lo[j] + step, max(n[j], 1)) - 1];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (lo[j] + step <= n[j] && v[j] > key) lo[j] += step;
  }
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += lo[j];
  return sum;
}

__global__ void __launch_bounds__(kTreeThreads)
rerank_tree(RerankPlan pl, const int32_t* __restrict__ root_token, const float* __restrict__ draft_lse,
            void* ws, int32_t* __restrict__ tokens, int32_t* __restrict__ parents,
            int32_t* __restrict__ depths, float* __restrict__ scores, int32_t* __restrict__ draft_row) {
  __shared__ TreeLds t;
  RrWs w = rr_ws(ws, pl);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = pl.k;
  const int L = pl.depth;
  const int total = k + (L - 1) * k * k;
  stage_rows(pl, w, draft_lse, b, pl.R, t);
  grow_levels(pl, L, t);
  // Final selection: the best n_nodes-1 candidates overall.  A candidate's overall
  // rank is its rank within its level plus, for every other level, how many of that
  // level's keys are larger (a binary search in the level's keys in rank order).
  const int keep = pl.n_nodes - 1;
  for (int c = tid; c < total; c += kTreeThreads)
    t.c_sorted[level_base(level_of(c, k, L), k) + t.c_rank[c]] = t.c_key[c];
  __syncthreads();
  for (int c = tid; c < total; c += kTreeThreads) {
    const int dc = level_of(c, k, L);
    const uint64_t key = t.c_key[c];
    int rank = t.c_rank[c];
    for (int d0 = 1; d0 <= L; d0 += 8) rank += count_larger8(t.c_sorted, d0, L, dc, k, key);
    t.c_pos[c] = (short)(rank < keep ? 1 : 0);
  }
  __syncthreads();
  // breadth-first positions: 1 + number of selected candidates with a smaller id.
  // Selected counts per 64-candidate group, then each candidate adds the counts of
  // the groups before its own.
  const int lane = tid & 63, wv = tid >> 6;
  const int ngroups = (total + 63) >> 6;   // <= kMaxCand / 64 = 32
  __shared__ int group_cnt[kMaxCand / 64];
  for (int g = wv; g < ngroups; g += kTreeThreads / 64) {
    const int c = (g << 6) + lane;
    const uint64_t m = __ballot(c < total && t.c_pos[c] != 0);
    if (lane == 0) group_cnt[g] = __popcll(m);
  }
  __syncthreads();
  for (int g = wv; g < ngroups; g += kTreeThreads / 64) {
    const int c = (g << 6) + lane;
    const bool sel = c < total && t.c_pos[c] != 0;
    const uint64_t m = __ballot(sel);
    int run = 0;
    for (int j = 0; j < g; ++j) run += group_cnt[j];
    if (sel) t.c_pos[c] = (short)(1 + run + __popcll(m & ((1ull << lane) - 1ull)));
  }
  __syncthreads();
  const size_t ob = (size_t)b * pl.n_nodes;
  if (tid == 0) {
    tokens[ob] = root_token[b];
    parents[ob] = -1;
    depths[ob] = 0;
    scores[ob] = 0.f;
    draft_row[ob] = 0;
  }
  for (int c = tid; c < total; c += kTreeThreads) {
    const int pos = t.c_pos[c];
    if (pos == 0) continue;
    const int dep = level_of(c, k, L);
    const int pc = t.c_par[c];
    tokens[ob + pos] = t.c_tok[c];
    parents[ob + pos] = pc < 0 ? 0 : t.c_pos[pc];
    depths[ob + pos] = dep;
    scores[ob + pos] = t.c_score[c];
    draft_row[ob + pos] = t.c_row[c];
  }
}

// Frontier of depth d (1 <= d < depth) for the per-depth draft expansion: the best k
// candidates of level d, in rank order, become rows 1 + (d-1)k + j; each row gets its
// candidate's token and the row of the node that proposed it.  Needs the row lists
// of rows 0 .. (d-1)k.
__global__ void __launch_bounds__(kTreeThreads)
draft_frontier(RerankPlan pl, int d, const float* __restrict__ draft_lse, void* ws,
               int32_t* __restrict__ row_token, int32_t* __restrict__ parent_row) {
  __shared__ TreeLds t;
  RrWs w = rr_ws(ws, pl);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = pl.k;
  stage_rows(pl, w, draft_lse, b, 1 + (d - 1) * k, t);
  grow_levels(pl, d, t);
  const int lb = level_base(d, k), ln = level_size(d, k);
  for (int c = lb + tid; c < lb + ln; c += kTreeThreads) {
    const int rank = t.c_rank[c];
    if (rank >= k) continue;
    const size_t row = (size_t)b * pl.R + 1 + (d - 1) * k + rank;
    const int pc = t.c_par[c];
    row_token[row] = t.c_tok[c];
    parent_row[row] = pc < 0 ? 0 : t.c_row[pc];
  }
}

}  // namespace

RerankPlan plan_rerank(int B, int V, int top_k, int depth, int n_nodes) {
  RerankPlan pl{};
  pl.B = B;
  pl.V = V;
  pl.k = top_k;
  pl.depth = depth;
  pl.R = 1 + (depth - 1) * top_k;
  pl.n_nodes = n_nodes;
  pl.chunk_len = kChunk;
  pl.chunks = (V + kChunk - 1) / kChunk;
  pl.row0 = 0;
  pl.nrows = pl.R;
  return pl;
}

size_t rerank_workspace_bytes(const RerankPlan& pl) {
  const size_t rows = (size_t)pl.B * pl.R;
  const size_t nc = rows * pl.chunks;
  return align256(nc * sizeof(float2)) + align256(nc * pl.k * sizeof(float)) +
         align256(nc * pl.k * sizeof(int)) + align256(rows * pl.k * sizeof(float)) +
         align256(rows * pl.k * sizeof(int)) + 256;
}

int rerank_max_candidates() { return kMaxCand; }
int rerank_chunk_len() { return kChunk; }
int rerank_max_row_list() { return kMaxRowList; }

hipError_t launch_rerank_rows(const RerankPlan& pl, const float* draft_logits, float* draft_lse,
                              void* workspace, hipStream_t stream) {
  const int rows = pl.B * pl.nrows;
  if (pl.V % 4 == 0 && ((uintptr_t)draft_logits & 15) == 0)
    hipLaunchKernelGGL(rerank_rows<true>, dim3(rows * pl.chunks), dim3(kRowThreads), 0, stream,
                       draft_logits, pl, workspace);
  else
    hipLaunchKernelGGL(rerank_rows<false>, dim3(rows * pl.chunks), dim3(kRowThreads), 0, stream,
                       draft_logits, pl, workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rerank_merge, dim3((rows + 3) / 4), dim3(256), 0, stream, pl, workspace,
                     draft_lse);
  return hipGetLastError();
}

hipError_t launch_rerank_tree(const RerankPlan& pl, const int32_t* root_token, const float* draft_lse,
                              void* workspace, int32_t* tokens, int32_t* parents, int32_t* depths,
                              float* scores, int32_t* draft_row, hipStream_t stream) {
  hipLaunchKernelGGL(rerank_tree, dim3(pl.B), dim3(kTreeThreads), 0, stream, pl, root_token,
                     draft_lse, workspace, tokens, parents, depths, scores, draft_row);
  return hipGetLastError();
}

hipError_t launch_draft_frontier(const RerankPlan& pl, int d, const float* draft_lse, void* workspace,
                                 int32_t* row_token, int32_t* parent_row, hipStream_t stream) {
  hipLaunchKernelGGL(draft_frontier, dim3(pl.B), dim3(kTreeThreads), 0, stream, pl, d, draft_lse,
                     workspace, row_token, parent_row);
  return hipGetLastError();
}

hipError_t launch_rerank(const RerankPlan& pl, const float* draft_logits, const int32_t* root_token,
                         int32_t* tokens, int32_t* parents, int32_t* depths, float* scores,
                         int32_t* draft_row, float* draft_lse, void* workspace, hipStream_t stream) {
  const hipError_t e = launch_rerank_rows(pl, draft_logits, draft_lse, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_rerank_tree(pl, root_token, draft_lse, workspace, tokens, parents, depths, scores,
                            draft_row, stream);
}

}  // namespace eagle
