// Per-depth EAGLE-2 draft expansion: the glue kernels around the one-layer draft head.
//
// [P2] auto-regression head and workflow paragraphs: the head reads the parent's
// feature and the embedding of the node's token, predicts the node's feature, and
// the frozen LM head turns it into the next-token distribution; [P2] training
// paragraph: the head is a single transformer layer.  The layer, per expansion row:
//     u = [f ; E[t]];  x = W_fc u;  h = x + W_o Attn(rms(x) g1);
//     y = h + W_down(silu(W_gate b) * (W_up b)),  b = rms(h) g2;  logits = W_lm y
// The GEMMs run on the LM-head kernel (weight-streaming MFMA GEMM, fp32 out), the
// attention on the tree-attention kernel over the expanded rows; the kernels here
// gather, normalise, scatter and apply the activation between them.  GEMM inputs
// are bf16, accumulation and the residual stream fp32.
//
// Rows of one depth: row0 .. row0 + nr - 1 of every sequence (row 0 = the root,
// rows 1 + (d-1)k + j = frontier slot j of depth d); processed row m = b * nr + j.
#include "common.h"
#include "internal.h"

namespace eagle {

namespace {

constexpr int kGlueThreads = 256;

__device__ __forceinline__ int seq_row(int m, int nr, int row0, int R, int* b_out) {
  const int b = m / nr;
  *b_out = b;
  return b * R + row0 + (m - b * nr);
}

// X[m] = [feature ; E[token]] (bf16, 2H): the root reads f0 and the root token, other
// rows the feature of their parent row and their own token.  16-byte pieces.
__global__ void __launch_bounds__(kGlueThreads)
draft_gather_input(DraftDims dd, int row0, int nr, const uint16_t* __restrict__ f0,
                   const int32_t* __restrict__ root_token, const uint16_t* __restrict__ embed,
                   const uint16_t* __restrict__ feats, const int32_t* __restrict__ row_token,
                   const int32_t* __restrict__ parent_row, uint16_t* __restrict__ X) {
  const int m = blockIdx.x;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const int r = grow - b * dd.R;
  const int H = dd.H;
  const uint16_t* fsrc;
  int tok;
  if (r == 0) {
    fsrc = f0 + (size_t)b * H;
    tok = root_token[b];
  } else {
    const int pr = min(max(parent_row[grow], 0), dd.R - 1);
    fsrc = feats + ((size_t)b * dd.R + pr) * H;
    tok = row_token[grow];
  }
  tok = min(max(tok, 0), dd.V - 1);
  const uint16_t* esrc = embed + (size_t)tok * H;
  uint16_t* dst = X + (size_t)m * 2 * H;
  for (int e = threadIdx.x * 8; e < H; e += kGlueThreads * 8) {
    *(u32x4*)(dst + e) = *(const u32x4*)(fsrc + e);
    *(u32x4*)(dst + H + e) = *(const u32x4*)(esrc + e);
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kGlueThreads / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}

// s = a (+ res); res_out = s (fp32); norm_out = bf16(s / sqrt(mean(s^2) + eps) * gain)
__global__ void __launch_bounds__(kGlueThreads)
draft_rms(int H, float eps, const float* __restrict__ a, int lda, const float* __restrict__ res,
          const float* __restrict__ gain, float* __restrict__ res_out, uint16_t* __restrict__ norm_out) {
  __shared__ float red[kGlueThreads / 64];
  const int m = blockIdx.x;
  const float* ar = a + (size_t)m * lda;
  const float* rr = res ? res + (size_t)m * H : nullptr;
  float ss = 0.f;
  for (int e = threadIdx.x; e < H; e += kGlueThreads) {
    const float s = ar[e] + (rr ? rr[e] : 0.f);
    res_out[(size_t)m * H + e] = s;
    ss += s * s;
  }
  const float inv = rsqrtf(block_sum(ss, red) / (float)H + eps);
  for (int e = 2 * threadIdx.x; e < H; e += 2 * kGlueThreads) {
    const float s0 = res_out[(size_t)m * H + e], s1 = res_out[(size_t)m * H + e + 1];
    *(uint32_t*)(norm_out + (size_t)m * H + e) = pack_bf16x2(s0 * inv * gain[e], s1 * inv * gain[e + 1]);
  }
}

// qkv fp32 [M][(Hq + 2 Hkv) D] -> q bf16 at [b][r][Hq][D]; k, v bf16 at cache row P + r
__global__ void __launch_bounds__(kGlueThreads)
draft_qkv_scatter(DraftDims dd, int row0, int nr, const float* __restrict__ qkv,
                  uint16_t* __restrict__ qbuf, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  const int m = blockIdx.x;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const int r = grow - b * dd.R;
  const int D = dd.D, qn = dd.Hq * D, kn = dd.Hkv * D;
  const float* src = qkv + (size_t)m * (qn + 2 * kn);
  for (int e = 2 * threadIdx.x; e < qn + 2 * kn; e += 2 * kGlueThreads) {
    const uint32_t pk = pack_bf16x2(src[e], src[e + 1]);
    if (e < qn) {
      *(uint32_t*)(qbuf + (size_t)grow * qn + e) = pk;
    } else {
      const int f = (e - qn) % kn;
      const int g = f / D, c = f % D;
      uint16_t* cache = e < qn + kn ? kc : vc;
      *(uint32_t*)(cache + (((size_t)b * dd.Hkv + g) * dd.kv_cap + dd.P + r) * D + c) = pk;
    }
  }
}

// attention output rows of this depth, [b][r][Hq][D] -> dense [M][Hq D]
__global__ void __launch_bounds__(kGlueThreads)
draft_gather_rows(DraftDims dd, int row0, int nr, int width, const uint16_t* __restrict__ src,
                  uint16_t* __restrict__ dst) {
  const int m = blockIdx.x;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  for (int e = threadIdx.x * 8; e < width; e += kGlueThreads * 8)
    *(u32x4*)(dst + (size_t)m * width + e) = *(const u32x4*)(src + (size_t)grow * width + e);
}

// gu fp32 [M][2I] (gate, then up) -> z = bf16(silu(gate) * up) [M][I]
__global__ void __launch_bounds__(kGlueThreads)
draft_silu_mul(int I, const float* __restrict__ gu, uint16_t* __restrict__ z) {
  const int m = blockIdx.x;
  const float* g = gu + (size_t)m * 2 * I;
  for (int e = 2 * threadIdx.x; e < I; e += 2 * kGlueThreads) {
    const float g0 = g[e], g1 = g[e + 1];
    const float s0 = g0 / (1.f + __expf(-g0)), s1 = g1 / (1.f + __expf(-g1));
    *(uint32_t*)(z + (size_t)m * I + e) = pack_bf16x2(s0 * g[I + e], s1 * g[I + e + 1]);
  }
}

// y = bf16(h + d): dense [M][H] (the LM head input) and the row's feature [b][r][H]
__global__ void __launch_bounds__(kGlueThreads)
draft_output(DraftDims dd, int row0, int nr, const float* __restrict__ d, const float* __restrict__ h,
             uint16_t* __restrict__ y, uint16_t* __restrict__ feats) {
  const int m = blockIdx.x;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const int H = dd.H;
  for (int e = 2 * threadIdx.x; e < H; e += 2 * kGlueThreads) {
    const size_t i = (size_t)m * H + e;
    const uint32_t pk = pack_bf16x2(h[i] + d[i], h[i + 1] + d[i + 1]);
    *(uint32_t*)(y + i) = pk;
    *(uint32_t*)(feats + (size_t)grow * H + e) = pk;
  }
}

// logits [M][V] -> the rows' slots of draft_logits [B][R][V]
__global__ void __launch_bounds__(kGlueThreads)
draft_place_logits(DraftDims dd, int row0, int nr, const float* __restrict__ src,
                   float* __restrict__ draft_logits) {
  const int m = blockIdx.y;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const size_t V = dd.V;
  for (size_t e = (size_t)blockIdx.x * kGlueThreads + threadIdx.x; e < V; e += (size_t)gridDim.x * kGlueThreads)
    draft_logits[(size_t)grow * V + e] = src[(size_t)m * V + e];
}

// every row starts without a parent (the root keeps -1) and with token 0; row 0 of a
// sequence carries its root token
__global__ void draft_init_rows(int B, int R, const int32_t* __restrict__ root_token,
                                int32_t* __restrict__ row_token, int32_t* __restrict__ parent_row) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B * R) {
    row_token[i] = (i % R == 0) ? root_token[i / R] : 0;
    parent_row[i] = -1;
  }
}

}  // namespace

hipError_t launch_draft_gather_input(const DraftDims& dd, int row0, int nr, const void* f0,
                                     const int32_t* root_token, const void* embed, const void* feats,
                                     const int32_t* row_token, const int32_t* parent_row, void* X,
                                     hipStream_t s) {
  hipLaunchKernelGGL(draft_gather_input, dim3(dd.B * nr), dim3(kGlueThreads), 0, s, dd, row0, nr,
                     (const uint16_t*)f0, root_token, (const uint16_t*)embed, (const uint16_t*)feats,
                     row_token, parent_row, (uint16_t*)X);
  return hipGetLastError();
}

hipError_t launch_draft_rms(int M, int H, float eps, const float* a, int lda, const float* res,
                            const float* gain, float* res_out, void* norm_out, hipStream_t s) {
  hipLaunchKernelGGL(draft_rms, dim3(M), dim3(kGlueThreads), 0, s, H, eps, a, lda, res, gain, res_out,
                     (uint16_t*)norm_out);
  return hipGetLastError();
}

hipError_t launch_draft_qkv_scatter(const DraftDims& dd, int row0, int nr, const float* qkv, void* qbuf,
                                    void* k_cache, void* v_cache, hipStream_t s) {
  hipLaunchKernelGGL(draft_qkv_scatter, dim3(dd.B * nr), dim3(kGlueThreads), 0, s, dd, row0, nr, qkv,
                     (uint16_t*)qbuf, (uint16_t*)k_cache, (uint16_t*)v_cache);
  return hipGetLastError();
}

hipError_t launch_draft_gather_rows(const DraftDims& dd, int row0, int nr, int width, const void* src,
                                    void* dst, hipStream_t s) {
  hipLaunchKernelGGL(draft_gather_rows, dim3(dd.B * nr), dim3(kGlueThreads), 0, s, dd, row0, nr, width,
                     (const uint16_t*)src, (uint16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_draft_silu_mul(int M, int I, const float* gu, void* z, hipStream_t s) {
  hipLaunchKernelGGL(draft_silu_mul, dim3(M), dim3(kGlueThreads), 0, s, I, gu, (uint16_t*)z);
  return hipGetLastError();
}

hipError_t launch_draft_output(const DraftDims& dd, int row0, int nr, const float* d, const float* h,
                               void* y, void* feats, hipStream_t s) {
  hipLaunchKernelGGL(draft_output, dim3(dd.B * nr), dim3(kGlueThreads), 0, s, dd, row0, nr, d, h,
                     (uint16_t*)y, (uint16_t*)feats);
  return hipGetLastError();
}

hipError_t launch_draft_place_logits(const DraftDims& dd, int row0, int nr, const float* src,
                                     float* draft_logits, hipStream_t s) {
  const int xblocks = (int)((dd.V + kGlueThreads * 8 - 1) / (kGlueThreads * 8));
  hipLaunchKernelGGL(draft_place_logits, dim3(xblocks, dd.B * nr), dim3(kGlueThreads), 0, s, dd, row0,
                     nr, src, draft_logits);
  return hipGetLastError();
}

hipError_t launch_draft_init_rows(int B, int R, const int32_t* root_token, int32_t* row_token,
                                  int32_t* parent_row, hipStream_t s) {
  hipLaunchKernelGGL(draft_init_rows, dim3((B * R + 255) / 256), dim3(256), 0, s, B, R, root_token,
                     row_token, parent_row);
  return hipGetLastError();
}

}  // namespace eagle
