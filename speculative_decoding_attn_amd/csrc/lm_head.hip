// Frozen LM head fused with per-row max / argmax / second max / log-sum-exp.
//
// [P2] paragraphs on the auto-regression head and the workflow: the target's
// frozen classification head gives the next-token distribution of every tree
// node; [P1] greedy decoding needs its top-1.
//
// logits^T tile = W (vocab rows, A operand) x hidden^T (tree rows, B operand) on the
// 32x32x16 bf16 MFMA.  A workgroup owns WV*VT*32 vocabulary rows and WM*MT*32 hidden
// rows; W is streamed from HBM exactly once, straight into registers in the MFMA
// operand layout (one 64-column block ahead), while the hidden rows of the current
// 64-column block are staged in LDS (XOR-swizzled 16-byte chunks, conflict-free
// reads) and shared by all waves.  In the output layout every lane holds 16
// vocabulary entries of ONE row, so the epilogue reduces in registers, then across
// lane l ^ 32, then across the waves of the workgroup, and writes one partial
// (max, second, sum of exp(x - max), argmax) per (row, vocabulary tile).  A second
// kernel merges the partials of a row.  No atomics: the result is deterministic.
#include "common.h"
#include "internal.h"

namespace eagle {

namespace {

struct Top2 {
  float mx;
  float sec;
  float z;   // sum of exp(x - mx)
  int idx;
};

// Union of two disjoint index sets (any order): top-2 values, first index of the
// max, rescaled exp-sum.
__device__ __forceinline__ Top2 merge_top2(Top2 a, Top2 b) {
  Top2 r;
  const bool a_wins = a.mx > b.mx || (a.mx == b.mx && a.idx < b.idx);
  r.mx = a_wins ? a.mx : b.mx;
  r.idx = a_wins ? a.idx : b.idx;
  r.sec = fmaxf(fminf(a.mx, b.mx), fmaxf(a.sec, b.sec));
  const float za = (a.mx == -INFINITY) ? 0.f : a.z * expf(a.mx - r.mx);
  const float zb = (b.mx == -INFINITY) ? 0.f : b.z * expf(b.mx - r.mx);
  r.z = za + zb;
  return r;
}

__device__ __forceinline__ Top2 shfl_xor_top2(Top2 a, int m) {
  Top2 r;
  r.mx = __shfl_xor(a.mx, m);
  r.sec = __shfl_xor(a.sec, m);
  r.z = __shfl_xor(a.z, m);
  r.idx = __shfl_xor(a.idx, m);
  return r;
}

template <int MT, int VT, int WV, int WM>
__global__ void __launch_bounds__(WV * WM * 64, 1)
lm_head_gemm(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, LmPlan pl,
             f32x4* __restrict__ part, float* __restrict__ logits) {
  constexpr int THREADS = WV * WM * 64;
  constexpr int MROWS = WM * MT * 32;
  constexpr int VROWS = WV * VT * 32;
  constexpr int HB = 64;                               // hidden columns per block
  constexpr int H_UNITS = MROWS * (HB / 8);            // 16-byte chunks per hidden block
  constexpr int H_PER = (H_UNITS + THREADS - 1) / THREADS;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * MROWS * HB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wv = wid % WV;
  const int wm = wid / WV;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int nwg = gridDim.x;
  const int w = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const int mb = logical % pl.nmb;
  const int vt = logical / pl.nmb;
  const int M = pl.M, H = pl.H, V = pl.V;
  const int m0 = mb * MROWS;
  const int v0 = vt * VROWS + wv * VT * 32;

  // W rows of this lane (A operand rows), clamped loads for rows past V
  const uint16_t* wrow[VT];
  bool wvalid[VT];
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int row = v0 + 32 * j + l32;
    wvalid[j] = row < V;
    wrow[j] = W + (size_t)(wvalid[j] ? row : 0) * H + 8 * half;
  }

  f32x16 acc[VT][MT];
#pragma unroll
  for (int j = 0; j < VT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  u32x4 wcur[VT][4], wnxt[VT][4];
  u32x4 hreg[H_PER];

  auto load_w = [&](u32x4 (&dst)[VT][4], int hb) {
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dst[j][s] = wvalid[j] ? *(const u32x4*)(wrow[j] + hb + 16 * s) : u32x4{0, 0, 0, 0};
  };
  auto load_h = [&](int hb) {
#pragma unroll
    for (int it = 0; it < H_PER; ++it) {
      const int u = tid + it * THREADS;
      hreg[it] = u32x4{0, 0, 0, 0};
      if (u < H_UNITS) {
        const int m = m0 + u / (HB / 8);
        const int ch = u % (HB / 8);
        if (m < M) hreg[it] = *(const u32x4*)(hidden + (size_t)m * H + hb + 8 * ch);
      }
    }
  };
  auto store_h = [&](int st) {
    uint16_t* base = lds + st * MROWS * HB;
#pragma unroll
    for (int it = 0; it < H_PER; ++it) {
      const int u = tid + it * THREADS;
      if (u < H_UNITS) {
        const int m = u / (HB / 8);
        const int ch = u % (HB / 8);
        *(u32x4*)(base + m * HB + ((ch ^ (m & 7)) * 8)) = hreg[it];
      }
    }
  };

  const int nhb = H / HB;
  load_w(wcur, 0);
  load_h(0);
  store_h(0);
  __syncthreads();

  for (int hbi = 0; hbi < nhb; ++hbi) {
    const int st = hbi & 1;
    const bool more = hbi + 1 < nhb;
    if (more) {
      load_w(wnxt, (hbi + 1) * HB);
      load_h((hbi + 1) * HB);
    }
    const uint16_t* hs = lds + st * MROWS * HB;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + half;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = wm * MT * 32 + 32 * i + l32;
        const bf16x8 hf = *(const bf16x8*)(hs + m * HB + ((ch ^ (m & 7)) * 8));
#pragma unroll
        for (int j = 0; j < VT; ++j) acc[j][i] = mfma32(as_bf16x8(wcur[j][s]), hf, acc[j][i]);
      }
    }
    if (more) store_h(st ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) wcur[j][s] = wnxt[j][s];
    }
  }

  // ---- epilogue: per-lane top-2 / exp-sum over its 16*VT vocabulary entries
  f32x4* red = (f32x4*)lds;   // [WV][MROWS] partials of this workgroup (reuses the staging LDS)
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int mloc = wm * MT * 32 + 32 * i + l32;
    const int m = m0 + mloc;
    Top2 t{-INFINITY, -INFINITY, 0.f, 0x7fffffff};
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vocab = v0 + 32 * j + 8 * (r >> 2) + 4 * half + (r & 3);
        const float x = vocab < V ? acc[j][i][r] : -INFINITY;
        if (x > t.mx) {
          t.sec = t.mx;
          t.mx = x;
          t.idx = vocab;
        } else if (x > t.sec) {
          t.sec = x;
        }
      }
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vocab = v0 + 32 * j + 8 * (r >> 2) + 4 * half + (r & 3);
        if (vocab < V) z += __builtin_amdgcn_exp2f((acc[j][i][r] - t.mx) * kLog2e);
      }
    t.z = z;
    if (logits != nullptr && m < M) {
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int vocab = v0 + 32 * j + 8 * q4 + 4 * half;
          float* dst = logits + (size_t)m * V + vocab;
          if (vocab + 3 < V && (V & 3) == 0) {
            *(f32x4*)dst = f32x4{acc[j][i][4 * q4], acc[j][i][4 * q4 + 1], acc[j][i][4 * q4 + 2],
                                 acc[j][i][4 * q4 + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (vocab + e < V) dst[e] = acc[j][i][4 * q4 + e];
          }
        }
    }
    t = merge_top2(t, shfl_xor_top2(t, 32));
    if (half == 0) red[wv * MROWS + mloc] = f32x4{t.mx, t.sec, t.z, __int_as_float(t.idx)};
  }
  __syncthreads();
  for (int mloc = tid; mloc < MROWS; mloc += THREADS) {
    const int m = m0 + mloc;
    if (m >= M) continue;
    f32x4 e0 = red[mloc];
    Top2 t{e0[0], e0[1], e0[2], __float_as_int(e0[3])};
#pragma unroll
    for (int q = 1; q < WV; ++q) {
      const f32x4 e = red[q * MROWS + mloc];
      t = merge_top2(t, Top2{e[0], e[1], e[2], __float_as_int(e[3])});
    }
    part[(size_t)m * pl.nvt + vt] = f32x4{t.mx, t.sec, t.z, __int_as_float(t.idx)};
  }
}

// One wave per row: merge the row's vocabulary-tile partials.
__global__ void __launch_bounds__(256)
lm_head_merge(LmPlan pl, const f32x4* __restrict__ part, float* __restrict__ out_max,
              int32_t* __restrict__ out_argmax, float* __restrict__ out_lse,
              float* __restrict__ out_second) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (m >= pl.M) return;
  Top2 t{-INFINITY, -INFINITY, 0.f, 0x7fffffff};
  for (int p = lane; p < pl.nvt; p += 64) {
    const f32x4 e = part[(size_t)m * pl.nvt + p];
    t = merge_top2(t, Top2{e[0], e[1], e[2], __float_as_int(e[3])});
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t = merge_top2(t, shfl_xor_top2(t, o));
  if (lane == 0) {
    out_max[m] = t.mx;
    out_argmax[m] = t.idx;
    out_lse[m] = t.mx + logf(t.z);
    if (out_second) out_second[m] = t.sec;
  }
}

template <int MT, int VT, int WV, int WM>
hipError_t launch_gemm(const LmPlan& pl, const void* hidden, const void* W, f32x4* part,
                       float* logits, hipStream_t stream) {
  hipLaunchKernelGGL((lm_head_gemm<MT, VT, WV, WM>), dim3(pl.nvt * pl.nmb), dim3(WV * WM * 64), 0,
                     stream, (const uint16_t*)hidden, (const uint16_t*)W, pl, part, logits);
  return hipGetLastError();
}

}  // namespace

LmPlan plan_lm_head(int M, int H, int V) {
  LmPlan pl{};
  pl.M = M;
  pl.H = H;
  pl.V = V;
  // tile shapes: (MT m-tiles, VT v-tiles) per wave, WV x WM waves
  if (M > 64) {
    pl.variant = 2;          // MT=4 VT=2 WV=4 WM=2: 256 rows x 256 vocab per workgroup
    pl.mrows = 256;
    pl.vrows = 256;
  } else if (M > 32) {
    pl.variant = 1;          // MT=2 VT=2 WV=4 WM=1: 64 rows x 256 vocab
    pl.mrows = 64;
    pl.vrows = 256;
  } else {
    pl.variant = 0;          // MT=1 VT=1 WV=4 WM=1: 32 rows x 128 vocab
    pl.mrows = 32;
    pl.vrows = 128;
  }
  pl.nvt = (V + pl.vrows - 1) / pl.vrows;
  pl.nmb = (M + pl.mrows - 1) / pl.mrows;
  return pl;
}

size_t lm_head_workspace_bytes(const LmPlan& pl) {
  return (size_t)pl.M * pl.nvt * sizeof(f32x4) + 256;
}

hipError_t launch_lm_head(const LmPlan& pl, const void* hidden, const void* W, float* out_max,
                          int32_t* out_argmax, float* out_lse, float* out_second, float* out_logits,
                          void* workspace, hipStream_t stream) {
  f32x4* part = (f32x4*)workspace;
  hipError_t e;
  switch (pl.variant) {
    case 2: e = launch_gemm<4, 2, 4, 2>(pl, hidden, W, part, out_logits, stream); break;
    case 1: e = launch_gemm<2, 2, 4, 1>(pl, hidden, W, part, out_logits, stream); break;
    default: e = launch_gemm<1, 1, 4, 1>(pl, hidden, W, part, out_logits, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_head_merge, dim3((pl.M + 3) / 4), dim3(256), 0, stream, pl,
                     (const f32x4*)part, out_max, out_argmax, out_lse, out_second);
  return hipGetLastError();
}

}  // namespace eagle
