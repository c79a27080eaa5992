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
//                 exp-sum, and its top-k by k rounds of "best element strictly after
//                 the previous pick" in (logit desc, token asc) order.  Streams the
//                 fp32 draft logits once (the HBM-bound part).
//   rerank_merge  one wave per row: merges the chunk results into the row's lse and
//                 top-k (same extraction order).
//   rerank_tree   one workgroup per sequence: candidate scores depth by depth,
//                 frontier = best k of each depth, final = best n_nodes-1 overall,
//                 all by counting ranks; output breadth first.
#include "common.h"
#include "internal.h"

namespace eagle {

namespace {

constexpr int kRowThreads = 256;
constexpr int kRowPer = 16;                        // elements per thread in rerank_rows
constexpr int kChunk = kRowThreads * kRowPer;      // vocabulary entries per chunk
constexpr int kTreeThreads = 256;
constexpr int kMaxCand = 4096;                     // candidates per sequence in rerank_tree

// (value, index) order: larger value first, then smaller index
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

struct VI {
  float v;
  int i;
};

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

__global__ void __launch_bounds__(kRowThreads)
rerank_rows(const float* __restrict__ logits, RerankPlan pl, void* ws) {
  __shared__ VI red[kRowThreads / 64];
  __shared__ float redf[kRowThreads / 64];
  RrWs w = rr_ws(ws, pl);
  const int chunk = blockIdx.x % pl.chunks;
  const size_t row = blockIdx.x / pl.chunks;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int V = pl.V;
  const int x0 = chunk * pl.chunk_len;
  const float* src = logits + row * (size_t)V;

  float val[kRowPer];
  int idx[kRowPer];
#pragma unroll
  for (int e = 0; e < kRowPer; ++e) {
    const int x = x0 + e * kRowThreads + tid;
    const bool ok = x < V && e * kRowThreads + tid < pl.chunk_len;
    val[e] = ok ? src[x] : -INFINITY;
    idx[e] = ok ? x : 0x7fffffff;
  }
  // max and exp-sum of the chunk
  float mx = val[0];
#pragma unroll
  for (int e = 1; e < kRowPer; ++e) mx = fmaxf(mx, val[e]);
  mx = wave_max(mx);
  if (lane == 0) redf[wid] = mx;
  __syncthreads();
  mx = redf[0];
#pragma unroll
  for (int i = 1; i < kRowThreads / 64; ++i) mx = fmaxf(mx, redf[i]);
  float z = 0.f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int e = 0; e < kRowPer; ++e)
      z += __builtin_amdgcn_exp2f((val[e] - mx) * kLog2e);
  }
  z = wave_sum(z);
  __syncthreads();
  if (lane == 0) redf[wid] = z;
  __syncthreads();
  if (tid == 0) {
    float zt = 0.f;
    for (int i = 0; i < kRowThreads / 64; ++i) zt += redf[i];
    w.chunk_mz[blockIdx.x] = make_float2(mx, zt);
  }
  // top-k by repeated extraction
  float pv = INFINITY;
  int pi = -1;
  for (int r = 0; r < pl.k; ++r) {
    VI best{-INFINITY, 0x7fffffff};
#pragma unroll
    for (int e = 0; e < kRowPer; ++e) {
      const bool after = val[e] < pv || (val[e] == pv && idx[e] > pi);
      if (after && better(val[e], idx[e], best.v, best.i)) best = VI{val[e], idx[e]};
    }
    best = wave_best(best);
    __syncthreads();
    if (lane == 0) red[wid] = best;
    __syncthreads();
    VI b = red[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / 64; ++i)
      if (better(red[i].v, red[i].i, b.v, b.i)) b = red[i];
    if (tid == 0) {
      w.chunk_v[(size_t)blockIdx.x * pl.k + r] = b.v;
      w.chunk_i[(size_t)blockIdx.x * pl.k + r] = b.i;
    }
    pv = b.v;
    pi = b.i;
  }
}

__global__ void __launch_bounds__(256)
rerank_merge(RerankPlan pl, void* ws, float* __restrict__ draft_lse) {
  RrWs w = rr_ws(ws, pl);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= pl.B * pl.R) return;
  // lse
  float mx = -INFINITY;
  for (int c = lane; c < pl.chunks; c += 64) mx = fmaxf(mx, w.chunk_mz[(size_t)row * pl.chunks + c].x);
  mx = wave_max(mx);
  float z = 0.f;
  for (int c = lane; c < pl.chunks; c += 64) {
    const float2 e = w.chunk_mz[(size_t)row * pl.chunks + c];
    if (e.x > -INFINITY) z += e.y * __builtin_amdgcn_exp2f((e.x - mx) * kLog2e);
  }
  z = wave_sum(z);
  if (lane == 0) draft_lse[row] = mx + logf(z);
  // top-k over chunks * k candidates
  const int ncand = pl.chunks * pl.k;
  const float* cv = w.chunk_v + (size_t)row * ncand;
  const int* ci = w.chunk_i + (size_t)row * ncand;
  float pv = INFINITY;
  int pi = -1;
  for (int r = 0; r < pl.k; ++r) {
    VI best{-INFINITY, 0x7fffffff};
    for (int c = lane; c < ncand; c += 64) {
      const float v = cv[c];
      const int i = ci[c];
      const bool after = v < pv || (v == pv && i > pi);
      if (after && better(v, i, best.v, best.i)) best = VI{v, i};
    }
    best = wave_best(best);
    if (lane == 0) {
      w.row_v[(size_t)row * pl.k + r] = best.v;
      w.row_i[(size_t)row * pl.k + r] = best.i;
    }
    pv = best.v;
    pi = best.i;
  }
}

__global__ void __launch_bounds__(kTreeThreads)
rerank_tree(RerankPlan pl, const int32_t* __restrict__ root_token, const float* __restrict__ draft_lse,
            void* ws, int32_t* __restrict__ tokens, int32_t* __restrict__ parents,
            int32_t* __restrict__ depths, float* __restrict__ scores, int32_t* __restrict__ draft_row) {
  __shared__ float c_score[kMaxCand];
  __shared__ int c_tok[kMaxCand];
  __shared__ short c_par[kMaxCand];
  __shared__ short c_row[kMaxCand];
  __shared__ short c_pos[kMaxCand];

  RrWs w = rr_ws(ws, pl);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = pl.k, R = pl.R;
  const float* rv = w.row_v + (size_t)b * R * k;
  const int* ri = w.row_i + (size_t)b * R * k;
  const float* lse = draft_lse + (size_t)b * R;
  const int total = k + (pl.depth - 1) * k * k;

  for (int c = tid; c < total; c += kTreeThreads) c_row[c] = -1;
  // depth 1: the root's proposals
  for (int r = tid; r < k; r += kTreeThreads) {
    c_score[r] = rv[r] - lse[0];
    c_tok[r] = ri[r];
    c_par[r] = -1;
  }
  __syncthreads();
  int lb = 0, ln = k, base = k;
  for (int d = 1; d < pl.depth; ++d) {
    // frontier: rank within the level
    for (int c = lb + tid; c < lb + ln; c += kTreeThreads) {
      int rank = 0;
      for (int o = lb; o < lb + ln; ++o) rank += better(c_score[o], o, c_score[c], c) ? 1 : 0;
      if (rank < k) c_row[c] = (short)(1 + (d - 1) * k + rank);
    }
    __syncthreads();
    for (int c = lb + tid; c < lb + ln; c += kTreeThreads) {
      const int row = c_row[c];
      if (row < 0) continue;
      const int slot = row - (1 + (d - 1) * k);
      for (int r = 0; r < k; ++r) {
        const int id = base + slot * k + r;
        c_score[id] = c_score[c] + (rv[(size_t)row * k + r] - lse[row]);
        c_tok[id] = ri[(size_t)row * k + r];
        c_par[id] = (short)c;
      }
    }
    __syncthreads();
    lb = base;
    ln = k * k;
    base += k * k;
  }
  // final selection by overall rank, then breadth-first positions
  const int keep = pl.n_nodes - 1;
  for (int c = tid; c < total; c += kTreeThreads) {
    int rank = 0;
    const float s = c_score[c];
    for (int o = 0; o < total; ++o) rank += better(c_score[o], o, s, c) ? 1 : 0;
    c_pos[c] = (short)(rank < keep ? 1 : 0);
  }
  __syncthreads();
  // exclusive scan of the selection flags in id order (one pass per thread range)
  const int per = (total + kTreeThreads - 1) / kTreeThreads;
  const int c0 = tid * per, c1 = min(total, c0 + per);
  int cnt = 0;
  for (int c = c0; c < c1; ++c) cnt += c_pos[c];
  __shared__ int tcount[kTreeThreads];
  tcount[tid] = cnt;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < tid; ++i) before += tcount[i];
  __syncthreads();
  int run = before;
  for (int c = c0; c < c1; ++c) {
    const bool s = c_pos[c] != 0;
    c_pos[c] = s ? (short)(1 + run) : (short)0;
    run += s ? 1 : 0;
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
  // depth of a candidate from its id: level 1 = [0, k), level d+1 = [k + (d-1)k^2, k + d k^2)
  for (int c = tid; c < total; c += kTreeThreads) {
    const int pos = c_pos[c];
    if (pos == 0) continue;
    const int dep = c < k ? 1 : 2 + (c - k) / (k * k);
    const int pc = c_par[c];
    tokens[ob + pos] = c_tok[c];
    parents[ob + pos] = pc < 0 ? 0 : c_pos[pc];
    depths[ob + pos] = dep;
    scores[ob + pos] = c_score[c];
    draft_row[ob + pos] = c_row[c];
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

hipError_t launch_rerank(const RerankPlan& pl, const float* draft_logits, const int32_t* root_token,
                         int32_t* tokens, int32_t* parents, int32_t* depths, float* scores,
                         int32_t* draft_row, float* draft_lse, void* workspace, hipStream_t stream) {
  const int rows = pl.B * pl.R;
  hipLaunchKernelGGL(rerank_rows, dim3(rows * pl.chunks), dim3(kRowThreads), 0, stream, draft_logits,
                     pl, workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rerank_merge, dim3((rows + 3) / 4), dim3(256), 0, stream, pl, workspace,
                     draft_lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rerank_tree, dim3(pl.B), dim3(kTreeThreads), 0, stream, pl, root_token,
                     draft_lse, workspace, tokens, parents, depths, scores, draft_row);
  return hipGetLastError();
}

}  // namespace eagle
