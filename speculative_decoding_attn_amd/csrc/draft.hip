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

// The elementwise kernels take a 2-D grid: blockIdx.y = processed row m, blockIdx.x
// = a slice of kSlice columns, 8 columns (16-byte pieces) per thread.  Widths are
// multiples of 8 (H, I multiples of 64; D 64 or 128).
constexpr int kSlice = kGlueThreads * 8;

// X[m] = [feature ; E[token]] (bf16, 2H): the root reads f0 and the root token, other
// rows the feature of their parent row and their own token.
__global__ void __launch_bounds__(kGlueThreads)
draft_gather_input(DraftDims dd, int row0, int nr, const uint16_t* __restrict__ f0,
                   const int32_t* __restrict__ root_token, const uint16_t* __restrict__ embed,
                   const uint16_t* __restrict__ feats, const int32_t* __restrict__ row_token,
                   const int32_t* __restrict__ parent_row, uint16_t* __restrict__ X) {
  const int m = blockIdx.y;
  const int H = dd.H;
  const int e = (blockIdx.x * kGlueThreads + threadIdx.x) * 8;   // column of [f ; E[t]]
  if (e >= 2 * H) return;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const int r = grow - b * dd.R;
  const uint16_t* src;
  if (e < H) {
    const int pr = r == 0 ? -1 : min(max(parent_row[grow], 0), dd.R - 1);
    src = (r == 0 ? f0 + (size_t)b * H : feats + ((size_t)b * dd.R + pr) * H) + e;
  } else {
    const int tok = min(max(r == 0 ? root_token[b] : row_token[grow], 0), dd.V - 1);
    src = embed + (size_t)tok * H + (e - H);
  }
  *(u32x4*)(X + (size_t)m * 2 * H + e) = *(const u32x4*)src;
}

// 16 bytes of a GEMM output given as split-K slices, summed in slice order (the
// order of the GEMM's own summing pass)
__device__ __forceinline__ f32x4 load4(const F32Slices& a, size_t i) {
  f32x4 v = *(const f32x4*)(a.p + i);
  for (int s = 1; s < a.S; ++s) v += *(const f32x4*)(a.p + (size_t)s * a.stride + i);
  return v;
}

constexpr int kRmsThreads = 1024;
constexpr int kRmsRegs = 4;   // float4 pieces per thread kept in registers: H <= 16384

// s = a (+ res); res_out = s (fp32); norm_out = bf16(s / sqrt(mean(s^2) + eps) * gain).
// One 1024-thread workgroup per row; for H <= 16384 every thread keeps its pieces of
// s in registers, beyond that s is re-read from res_out.
__global__ void __launch_bounds__(kRmsThreads)
draft_rms(int H, float eps, F32Slices a, const float* __restrict__ res,
          const float* __restrict__ gain, float* __restrict__ res_out, uint16_t* __restrict__ norm_out) {
  __shared__ float red[kRmsThreads / 64];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int nq = H / 4;
  const size_t a0 = (size_t)m * H;   // this row's first entry in each slice of a
  const f32x4* rr = res ? (const f32x4*)(res + (size_t)m * H) : nullptr;
  f32x4* so = (f32x4*)(res_out + (size_t)m * H);
  f32x4 sv[kRmsRegs];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRmsRegs; ++j) {
    const int q = tid + j * kRmsThreads;
    if (q < nq) {
      f32x4 v = load4(a, a0 + 4 * (size_t)q);
      if (rr) v += rr[q];
      sv[j] = v;
      so[q] = v;
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
  }
  for (int q = tid + kRmsRegs * kRmsThreads; q < nq; q += kRmsThreads) {
    f32x4 v = load4(a, a0 + 4 * (size_t)q);
    if (rr) v += rr[q];
    so[q] = v;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kRmsThreads / 64; ++i) tot += red[i];
  const float inv = rsqrtf(tot / (float)H + eps);
  uint16_t* no = norm_out + (size_t)m * H;
  auto put = [&](int q, f32x4 v) {
    const int e = 4 * q;
    *(uint2*)(no + e) = make_uint2(pack_bf16x2(v[0] * inv * gain[e], v[1] * inv * gain[e + 1]),
                                   pack_bf16x2(v[2] * inv * gain[e + 2], v[3] * inv * gain[e + 3]));
  };
#pragma unroll
  for (int j = 0; j < kRmsRegs; ++j) {
    const int q = tid + j * kRmsThreads;
    if (q < nq) put(q, sv[j]);
  }
  for (int q = tid + kRmsRegs * kRmsThreads; q < nq; q += kRmsThreads) put(q, so[q]);
}

// qkv fp32 [M][(Hq + 2 Hkv) D] -> q bf16 at [b][r][Hq][D]; k, v bf16 at cache row P + r.
// A thread's 8 columns stay inside one head (D and the q / k / v widths are multiples of 8).
__global__ void __launch_bounds__(kGlueThreads)
draft_qkv_scatter(DraftDims dd, int row0, int nr, F32Slices qkv,
                  uint16_t* __restrict__ qbuf, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  const int m = blockIdx.y;
  const int D = dd.D, qn = dd.Hq * D, kn = dd.Hkv * D;
  const int e = (blockIdx.x * kGlueThreads + threadIdx.x) * 8;
  if (e >= qn + 2 * kn) return;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const int r = grow - b * dd.R;
  const size_t i = (size_t)m * (qn + 2 * kn) + e;
  const f32x4 v0 = load4(qkv, i), v1 = load4(qkv, i + 4);
  const u32x4 pk = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                    pack_bf16x2(v1[2], v1[3])};
  if (e < qn) {
    *(u32x4*)(qbuf + (size_t)grow * qn + e) = pk;
  } else {
    const int f = (e - qn) % kn;
    const int g = f / D, c = f % D;
    uint16_t* cache = e < qn + kn ? kc : vc;
    *(u32x4*)(cache + (((size_t)b * dd.Hkv + g) * dd.kv_cap + dd.P + r) * D + c) = pk;
  }
}

// attention output rows of this depth, [b][r][Hq][D] -> dense [M][Hq D]
__global__ void __launch_bounds__(kGlueThreads)
draft_gather_rows(DraftDims dd, int row0, int nr, int width, const uint16_t* __restrict__ src,
                  uint16_t* __restrict__ dst) {
  const int m = blockIdx.y;
  const int e = (blockIdx.x * kGlueThreads + threadIdx.x) * 8;
  if (e >= width) return;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  *(u32x4*)(dst + (size_t)m * width + e) = *(const u32x4*)(src + (size_t)grow * width + e);
}

// gu fp32 [M][2I] (gate, then up) -> z = bf16(silu(gate) * up) [M][I]
__global__ void __launch_bounds__(kGlueThreads)
draft_silu_mul(int I, const float* __restrict__ gu, uint16_t* __restrict__ z) {
  const int m = blockIdx.y;
  const int e = (blockIdx.x * kGlueThreads + threadIdx.x) * 8;
  if (e >= I) return;
  const f32x4* g = (const f32x4*)(gu + (size_t)m * 2 * I + e);
  const f32x4* u = (const f32x4*)(gu + (size_t)m * 2 * I + I + e);
  const f32x4 g0 = g[0], g1 = g[1], u0 = u[0], u1 = u[1];
  auto sm = [](float x, float up) { return x / (1.f + __expf(-x)) * up; };
  *(u32x4*)(z + (size_t)m * I + e) =
      u32x4{pack_bf16x2(sm(g0[0], u0[0]), sm(g0[1], u0[1])), pack_bf16x2(sm(g0[2], u0[2]), sm(g0[3], u0[3])),
            pack_bf16x2(sm(g1[0], u1[0]), sm(g1[1], u1[1])), pack_bf16x2(sm(g1[2], u1[2]), sm(g1[3], u1[3]))};
}

// y = bf16(h + d): dense [M][H] (the LM head input) and the row's feature [b][r][H]
__global__ void __launch_bounds__(kGlueThreads)
draft_output(DraftDims dd, int row0, int nr, F32Slices d, const float* __restrict__ h,
             uint16_t* __restrict__ y, uint16_t* __restrict__ feats) {
  const int m = blockIdx.y;
  const int H = dd.H;
  const int e = (blockIdx.x * kGlueThreads + threadIdx.x) * 8;
  if (e >= H) return;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const size_t i = (size_t)m * H + e;
  const f32x4 h0 = *(const f32x4*)(h + i), h1 = *(const f32x4*)(h + i + 4);
  const f32x4 d0 = load4(d, i), d1 = load4(d, i + 4);
  const u32x4 pk = {pack_bf16x2(h0[0] + d0[0], h0[1] + d0[1]), pack_bf16x2(h0[2] + d0[2], h0[3] + d0[3]),
                    pack_bf16x2(h1[0] + d1[0], h1[1] + d1[1]), pack_bf16x2(h1[2] + d1[2], h1[3] + d1[3])};
  *(u32x4*)(y + i) = pk;
  *(u32x4*)(feats + (size_t)grow * H + e) = pk;
}

// logits [M][V] -> the rows' slots of draft_logits [B][R][V] (16-byte pieces when
// V % 4 == 0, which keeps every row 16-byte aligned)
template <bool VEC>
__global__ void __launch_bounds__(kGlueThreads)
draft_place_logits(DraftDims dd, int row0, int nr, const float* __restrict__ src,
                   float* __restrict__ draft_logits) {
  const int m = blockIdx.y;
  int b;
  const int grow = seq_row(m, nr, row0, dd.R, &b);
  const size_t V = dd.V;
  const size_t e = ((size_t)blockIdx.x * kGlueThreads + threadIdx.x) * 8;
  if (VEC) {
    if (e >= V) return;
    const f32x4* s4 = (const f32x4*)(src + (size_t)m * V + e);
    f32x4* d4 = (f32x4*)(draft_logits + (size_t)grow * V + e);
    d4[0] = s4[0];
    if (e + 4 < V) d4[1] = s4[1];
  } else {
    for (size_t x = e; x < e + 8 && x < V; ++x) draft_logits[(size_t)grow * V + x] = src[(size_t)m * V + x];
  }
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
  hipLaunchKernelGGL(draft_gather_input, dim3((2 * dd.H + kSlice - 1) / kSlice, dd.B * nr),
                     dim3(kGlueThreads), 0, s, dd, row0, nr,
                     (const uint16_t*)f0, root_token, (const uint16_t*)embed, (const uint16_t*)feats,
                     row_token, parent_row, (uint16_t*)X);
  return hipGetLastError();
}

hipError_t launch_draft_rms(int M, int H, float eps, F32Slices a, const float* res,
                            const float* gain, float* res_out, void* norm_out, hipStream_t s) {
  hipLaunchKernelGGL(draft_rms, dim3(M), dim3(kRmsThreads), 0, s, H, eps, a, res, gain, res_out,
                     (uint16_t*)norm_out);
  return hipGetLastError();
}

hipError_t launch_draft_qkv_scatter(const DraftDims& dd, int row0, int nr, F32Slices qkv, void* qbuf,
                                    void* k_cache, void* v_cache, hipStream_t s) {
  const int width = (dd.Hq + 2 * dd.Hkv) * dd.D;
  hipLaunchKernelGGL(draft_qkv_scatter, dim3((width + kSlice - 1) / kSlice, dd.B * nr), dim3(kGlueThreads),
                     0, s, dd, row0, nr, qkv,
                     (uint16_t*)qbuf, (uint16_t*)k_cache, (uint16_t*)v_cache);
  return hipGetLastError();
}

hipError_t launch_draft_gather_rows(const DraftDims& dd, int row0, int nr, int width, const void* src,
                                    void* dst, hipStream_t s) {
  hipLaunchKernelGGL(draft_gather_rows, dim3((width + kSlice - 1) / kSlice, dd.B * nr), dim3(kGlueThreads),
                     0, s, dd, row0, nr, width,
                     (const uint16_t*)src, (uint16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_draft_silu_mul(int M, int I, const float* gu, void* z, hipStream_t s) {
  hipLaunchKernelGGL(draft_silu_mul, dim3((I + kSlice - 1) / kSlice, M), dim3(kGlueThreads), 0, s, I, gu,
                     (uint16_t*)z);
  return hipGetLastError();
}

hipError_t launch_draft_output(const DraftDims& dd, int row0, int nr, F32Slices d, const float* h,
                               void* y, void* feats, hipStream_t s) {
  hipLaunchKernelGGL(draft_output, dim3((dd.H + kSlice - 1) / kSlice, dd.B * nr), dim3(kGlueThreads), 0, s,
                     dd, row0, nr, d, h,
                     (uint16_t*)y, (uint16_t*)feats);
  return hipGetLastError();
}

hipError_t launch_draft_place_logits(const DraftDims& dd, int row0, int nr, const float* src,
                                     float* draft_logits, hipStream_t s) {
  const int xblocks = (int)((dd.V + kSlice - 1) / kSlice);
  if (dd.V % 4 == 0)
    hipLaunchKernelGGL(draft_place_logits<true>, dim3(xblocks, dd.B * nr), dim3(kGlueThreads), 0, s, dd,
                       row0, nr, src, draft_logits);
  else
    hipLaunchKernelGGL(draft_place_logits<false>, dim3(xblocks, dd.B * nr), dim3(kGlueThreads), 0, s, dd,
                       row0, nr, src, draft_logits);
  return hipGetLastError();
}

hipError_t launch_draft_init_rows(int B, int R, const int32_t* root_token, int32_t* row_token,
                                  int32_t* parent_row, hipStream_t s) {
  hipLaunchKernelGGL(draft_init_rows, dim3((B * R + 255) / 256), dim3(256), 0, s, B, R, root_token,
                     row_token, parent_row);
  return hipGetLastError();
}

}  // namespace eagle
