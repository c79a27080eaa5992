// Frozen LM head fused with per-row max / argmax / second max / log-sum-exp.
//
// [P2] paragraphs on the auto-regression head and the workflow: the target's
// frozen classification head gives the next-token distribution of every tree
// node; [P1] greedy decoding needs its top-1.
//
// logits^T tile = W (vocab rows, A operand) x hidden^T (tree rows, B operand) on the
// 32x32x16 bf16 MFMA.  A workgroup of WV waves owns WV*VT*32 vocabulary rows and
// MT*32 hidden rows; every wave multiplies its own VT vocabulary tiles with all MT
// row tiles.  W is streamed from HBM exactly once, straight into registers in the
// MFMA operand layout, PF 64-column blocks ahead (enough bytes in flight per CU to
// cover HBM latency), while the hidden rows of the current 64-column block are
// staged in LDS (XOR-swizzled 16-byte chunks, conflict-free reads) and shared by
// all waves.  In the output layout every lane holds 16
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

template <int MT, int VT, int WV, int PF, int OCC>
__global__ void __launch_bounds__(WV * 64, OCC)
lm_head_gemm(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, LmPlan pl,
             f32x4* __restrict__ part, float* __restrict__ logits) {
  constexpr int THREADS = WV * 64;
  constexpr int MROWS = MT * 32;
  constexpr int VROWS = WV * VT * 32;
  constexpr int HB = 64;                               // hidden columns per block
  constexpr int HSTAGE = MROWS * HB;                   // bf16 per LDS stage
  constexpr int H_PER = MROWS * (HB / 8) / THREADS;    // 16-byte loads per thread per block
  static_assert(MROWS * (HB / 8) % THREADS == 0, "hidden staging must cover the block exactly");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * HSTAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
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

  // W rows of this lane (A operand rows); rows past V read row 0 and are masked later
  const uint16_t* wrow[VT];
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int row = v0 + 32 * j + l32;
    wrow[j] = W + (size_t)(row < V ? row : 0) * H + 8 * half;
  }

  f32x16 acc[VT][MT];
#pragma unroll
  for (int j = 0; j < VT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // Software pipeline.  W blocks stay in flight in a ring of PF register slots (W
  // streams from HBM) and hidden blocks in a ring of 2 register slots (a hidden block
  // is loaded two iterations before it is stored to LDS; it comes from L2 / Infinity
  // Cache).  The loop's global loads are issued with inline assembly and waited for
  // with explicit vmcnt counts: the compiler's wait-counter tracking cannot follow a
  // register ring across the loop back-edge and would drain every load at each block.
  // Issue order per iteration i: hidden loads H_i (block i+2), then W loads W_i (block
  // i+PF).  Loads past the last block re-read it (addresses are clamped), so every
  // iteration issues the same count and the counts below are exact; their data is
  // never used (the hidden rows of a padding block are zeroed).
  static_assert(PF % 2 == 0, "the loop is unrolled by PF and the hidden ring has 2 slots");
  constexpr int W_LOADS = VT * 4;
  constexpr int H_LOADS = H_PER;
  // compute(i) needs W_{i-PF}; issued after it: (PF-1) x (H + W) of later iterations + H_i
  constexpr int WAIT_W = (PF - 1) * (H_LOADS + W_LOADS) + H_LOADS;
  // store of hidden block i+1 needs H_{i-1}; issued after it: W_{i-1}, H_i, W_i
  constexpr int WAIT_H = 2 * W_LOADS + H_LOADS;
  static_assert(WAIT_W <= 63 && WAIT_H <= 63, "vmcnt is a 6-bit counter");
  u32x4 wbuf[PF][VT][4];
  u32x4 hreg[2][H_PER];

  const int nhb = H / HB;
  const int nhb_pad = (nhb + PF - 1) / PF * PF;   // blocks past nhb are zero blocks
  auto load_w = [&](u32x4 (&dst)[VT][4], int hbi) {
    const int hb = min(hbi, nhb - 1) * HB;
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[j][s] = gload_async(wrow[j] + hb + 16 * s);
  };
  auto load_h = [&](u32x4 (&dst)[H_PER], int hbi) {
    const int hb = min(hbi, nhb - 1) * HB;
#pragma unroll
    for (int it = 0; it < H_PER; ++it) {
      const int u = tid + it * THREADS;
      const int m = m0 + u / (HB / 8);
      const int ch = u % (HB / 8);
      dst[it] = gload_async(hidden + (size_t)min(m, M - 1) * H + hb + 8 * ch);
    }
  };
  // zero the rows past M and the blocks past nhb, then store to LDS (after the wait)
  auto store_h = [&](const u32x4 (&src)[H_PER], int st, int hbi) {
    uint16_t* base = lds + st * HSTAGE;
#pragma unroll
    for (int it = 0; it < H_PER; ++it) {
      const int u = tid + it * THREADS;
      const int m = u / (HB / 8);
      const int ch = u % (HB / 8);
      const u32x4 v = (m0 + m < M && hbi < nhb) ? src[it] : u32x4{0, 0, 0, 0};
      *(u32x4*)(base + m * HB + ((ch ^ (m & 7)) * 8)) = v;
    }
  };
  // One block: 4 k-steps x MT row tiles = 4*MT operand reads from LDS, each feeding
  // VT MFMAs.  The reads run LA groups ahead of the MFMAs that consume them; a
  // scheduling fence after each group keeps that order (the scheduler would otherwise
  // sink each read to its use and wait for it).
  auto compute = [&](int st, const u32x4 (&wb)[VT][4]) {
    const uint16_t* hs = lds + st * HSTAGE;
    constexpr int NG = 4 * MT;   // groups: g = s * MT + i
    constexpr int LA = 3;        // reads in flight ahead of the MFMAs
    auto rd = [&](int g) {
      const int s = g / MT, i = g % MT;
      const int m = 32 * i + l32;
      const int ch = 2 * s + half;
      return *(const bf16x8*)(hs + m * HB + ((ch ^ (m & 7)) * 8));
    };
    bf16x8 hf[LA + 1];
#pragma unroll
    for (int g = 0; g < LA; ++g) hf[g] = rd(g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + LA < NG) hf[(g + LA) % (LA + 1)] = rd(g + LA);
      const int s = g / MT, i = g % MT;
#pragma unroll
      for (int j = 0; j < VT; ++j) acc[j][i] = mfma32(as_bf16x8(wb[j][s]), hf[g % (LA + 1)], acc[j][i]);
      __builtin_amdgcn_sched_barrier(0);   // keep program order: read g+LA, then the MFMAs of g
    }
  };

  // prologue: W blocks 0..PF-1 and hidden blocks 0, 1; drained before the loop
#pragma unroll
  for (int u = 0; u < PF; ++u) load_w(wbuf[u], u);
  load_h(hreg[0], 0);
  load_h(hreg[1], 1);
  wait_vmcnt<0>();
#pragma unroll
  for (int u = 0; u < PF; ++u)
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) after_wait(wbuf[u][j][s]);
#pragma unroll
  for (int it = 0; it < H_PER; ++it) {
    after_wait(hreg[0][it]);
    after_wait(hreg[1][it]);
  }
  store_h(hreg[0], 0, 0);
  __syncthreads();

  // iteration i: issue H_i into ring slot i%2 (its block i was stored last
  // iteration), compute block i from LDS stage i%2 with W slot i%PF, refill that
  // slot with block i+PF, store hidden block i+1 into LDS stage (i+1)%2
  for (int hb0 = 0; hb0 < nhb_pad; hb0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int hbi = hb0 + u;
      load_h(hreg[u & 1], hbi + 2);
      wait_vmcnt<WAIT_W>();
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) after_wait(wbuf[u][j][s]);
      compute(u & 1, wbuf[u]);
      load_w(wbuf[u], hbi + PF);
      wait_vmcnt<WAIT_H>();
#pragma unroll
      for (int it = 0; it < H_PER; ++it) after_wait(hreg[(u + 1) & 1][it]);
      store_h(hreg[(u + 1) & 1], (u + 1) & 1, hbi + 1);
      __syncthreads();
    }
  }
  // The last loads of the rings are never read, so to the compiler their
  // destination registers are dead and free for reuse while the loads are still in
  // flight.  Waiting here and then touching every ring register keeps them reserved
  // until the data has landed.
  wait_vmcnt<0>();
#pragma unroll
  for (int u = 0; u < PF; ++u)
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) after_wait(wbuf[u][j][s]);
#pragma unroll
  for (int it = 0; it < H_PER; ++it) {
    after_wait(hreg[0][it]);
    after_wait(hreg[1][it]);
  }

  // ---- epilogue: per-lane top-2 / exp-sum over its 16*VT vocabulary entries
  f32x4* red = (f32x4*)lds;   // [WV][MROWS] partials of this workgroup (reuses the staging LDS)
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int mloc = 32 * i + l32;
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

template <int MT, int VT, int WV, int PF, int OCC>
hipError_t launch_gemm(const LmPlan& pl, const void* hidden, const void* W, f32x4* part,
                       float* logits, hipStream_t stream) {
  hipLaunchKernelGGL((lm_head_gemm<MT, VT, WV, PF, OCC>), dim3(pl.nvt * pl.nmb), dim3(WV * 64), 0,
                     stream, (const uint16_t*)hidden, (const uint16_t*)W, pl, part, logits);
  return hipGetLastError();
}

}  // namespace

LmPlan plan_lm_head(int M, int H, int V) {
  LmPlan pl{};
  pl.M = M;
  pl.H = H;
  pl.V = V;
  // tile shapes: every wave covers all MT m-tiles of the workgroup's rows and VT
  // 32-row vocabulary tiles; W blocks 4 deep in flight
  if (M > 128) {
    pl.variant = 3;          // MT=8 VT=2: 256 rows x 256 vocab, 1 wave/SIMD (accumulators in AGPRs)
    pl.mrows = 256;
    pl.vrows = 256;
  } else if (M > 64) {
    pl.variant = 2;          // MT=4 VT=2: 128 rows x 256 vocab
    pl.mrows = 128;
    pl.vrows = 256;
  } else if (M > 32) {
    pl.variant = 1;          // MT=2 VT=2: 64 rows x 256 vocab, 2 waves/SIMD
    pl.mrows = 64;
    pl.vrows = 256;
  } else {
    pl.variant = 0;          // MT=1 VT=1: 32 rows x 128 vocab, 2 waves/SIMD
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
    case 3: e = launch_gemm<8, 2, 4, 4, 1>(pl, hidden, W, part, out_logits, stream); break;
    case 2: e = launch_gemm<4, 2, 4, 4, 1>(pl, hidden, W, part, out_logits, stream); break;
    case 1: e = launch_gemm<2, 2, 4, 4, 2>(pl, hidden, W, part, out_logits, stream); break;
    default: e = launch_gemm<1, 1, 4, 4, 2>(pl, hidden, W, part, out_logits, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_head_merge, dim3((pl.M + 3) / 4), dim3(256), 0, stream, pl,
                     (const f32x4*)part, out_max, out_argmax, out_lse, out_second);
  return hipGetLastError();
}

}  // namespace eagle
