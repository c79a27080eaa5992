// Frozen LM head fused with per-row max / argmax / second max / log-sum-exp.
//
// [P2] paragraphs on the auto-regression head and the workflow: the target's
// frozen classification head gives the next-token distribution of every tree
// node; [P1] greedy decoding needs its top-1.
//
// logits^T tile = W (vocab rows, A operand) x hidden^T (tree rows, B operand) on the
// 32x32x16 bf16 MFMA.  A workgroup's waves form a grid over its vocabulary rows and
// hidden rows; every wave multiplies its VT vocabulary tiles with its MT row tiles
// (for the largest M: 8 waves, two per SIMD, so one wave's MFMAs cover the other's
// waits).  Both operands are staged in LDS, 64 columns (128 bytes per row) at
// a time, by global->LDS DMA loads that read whole 128-byte lines (8 rows per wave
// instruction) into XOR-swizzled rows; W is streamed from HBM exactly once (non-
// temporal loads, so it does not evict the hidden rows from L2) and runs
// two to three blocks ahead, the hidden rows (L2-resident) one to two.  In the output
// layout every lane holds 16 vocabulary entries of ONE row, so the epilogue reduces
// in registers, then across lane l ^ 32, then across the waves of the workgroup, and
// writes one partial (max, second, sum of exp(x - max), argmax) per (row, vocabulary
// tile).  A second kernel merges the partials of a row.  No atomics: the result is
// deterministic.
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

// 16-byte chunk position of logical chunk c (of 8) in row r of a 128-byte-row LDS
// tile: XOR-swizzled so that any 16 consecutive lanes reading rows r..r+15 at one
// logical chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

constexpr int kLmStagesW = 3;   // W blocks: b+2 in flight while b and b+1 are resident

template <int MT, int VT, int WVV, int WVM>
constexpr int lm_lds_bytes() {
  return kLmStagesW * (WVV * VT * 32) * 128 + 2 * (WVM * MT * 32) * 128;
}

// Waves form a WVV x WVM grid: wave (wvv, wvm) multiplies vocabulary tiles
// wvv*VT .. wvv*VT+VT-1 with hidden row tiles wvm*MT .. wvm*MT+MT-1 of the workgroup.
template <int MT, int VT, int WVV, int WVM, int LA>
__global__ void __launch_bounds__(WVV * WVM * 64)
lm_head_gemm(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, LmPlan pl,
             f32x4* __restrict__ part, float* __restrict__ logits) {
  constexpr int WV = WVV * WVM;
  constexpr int THREADS = WV * 64;
  constexpr int NW = kLmStagesW;
  constexpr int MROWS = WVM * MT * 32;
  constexpr int VROWS = WVV * VT * 32;
  constexpr int RB = 128;                    // bytes per row of a 64-column block
  constexpr int WSTAGE = VROWS * RB;
  constexpr int HSTAGE = MROWS * RB;
  constexpr int W_DMA = VROWS / (8 * WV);    // per wave and block: 8 rows per instruction
  constexpr int H_DMA = MROWS / (8 * WV);
  static_assert(W_DMA * 8 * WV == VROWS && H_DMA * 8 * WV == MROWS,
                "the waves load whole 8-row groups of both tiles");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // The 192-row tile keeps its accumulators in AGPRs: an AGPR operand anywhere in the
  // kernel lets the compiler select the AGPR-result form of the MFMAs (396 against
  // 404 us at 185 rows).  The 256-row tile stays in VGPRs: with the register file
  // split in halves its other values no longer fit and it ran slower.
  if constexpr (MT == 3) asm volatile("" ::"a"(0));
  uint8_t* const wst = smem;                 // [NW][VROWS][128 B] W blocks
  uint8_t* const hst = smem + NW * WSTAGE;   // [2][MROWS][128 B] hidden blocks

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (DMA bases)
  const int wvv = wv % WVV, wvm = wv / WVV;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int nwg = gridDim.x;
  const int w = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const int tiles = pl.nmb * pl.nvt;
  const int ks = logical / tiles;            // split-K slice
  const int mb = (logical % tiles) % pl.nmb;
  const int vt = (logical % tiles) / pl.nmb;
  const int M = pl.M, H = pl.H, V = pl.V;
  const int m0 = mb * MROWS;
  const int v0 = vt * VROWS + wvv * VT * 32;   // this wave's first vocabulary row

  // DMA sources for block 0 (a block adds 128 bytes).  Instruction t of wave wv fills
  // the 8 whole rows 8*(wv*N + t) .. +7 of a stage (full 128-byte lines): lane i
  // takes row +i/8 and stores its chunk at position i%8, i.e. it reads the logical
  // chunk that position holds.  Rows past V / M re-read the last row; those outputs
  // are never written.
  const uint32_t base = lds_addr(smem);
  // this split's 64-column blocks kb0 .. kb0 + nhb - 1
  const int kb0 = ks * pl.kb_per;
  const int nhb = min(pl.kb_per, H / 64 - kb0);
  const uint8_t* wsrc[W_DMA];
#pragma unroll
  for (int t = 0; t < W_DMA; ++t) {
    const int r = 8 * (wv * W_DMA + t) + (lane >> 3);          // row within the W tile
    const int row = min(vt * VROWS + r, V - 1);
    wsrc[t] = (const uint8_t*)(W + (size_t)row * H + (size_t)kb0 * 64) + 16 * swz(r, lane & 7);
  }
  const uint8_t* hsrc[H_DMA];
#pragma unroll
  for (int t = 0; t < H_DMA; ++t) {
    const int r = 8 * (wv * H_DMA + t) + (lane >> 3);          // row within the hidden tile
    const int row = min(m0 + r, M - 1);
    hsrc[t] = (const uint8_t*)(hidden + (size_t)row * H + (size_t)kb0 * 64) + 16 * swz(r, lane & 7);
  }
  // one DMA instruction t (8 rows) of W / hidden block blk into stage st; hidden
  // groups wholly past M are skipped (their rows are never written out)
  // Small row tiles (<= 64 hidden rows): pipeline block blk reads column block
  // (blk + rot) mod nhb, so the workgroups start their K walks at different columns
  // and the W rows streamed at one moment spread over the HBM channels instead of
  // sharing one column offset (60 rows: 331 -> 316 us).  Larger tiles walk in order:
  // there the hidden block every workgroup reads at one moment is shared in L2, and
  // scattered walks cost 35% more HBM traffic for no gain.  The sum order per
  // workgroup is fixed, so results are deterministic.
  const int rot = MROWS <= 64 ? (vt * 37) % nhb : 0;
  auto phys = [&](int blk) {
    const int x = blk + rot;
    return x >= nhb ? x - nhb : x;
  };
  auto issue_w = [&](int blk, int st, int t) {
    dma16_nt(wsrc[t] + (size_t)phys(blk) * RB, base + st * WSTAGE + 8 * (wv * W_DMA + t) * RB);
  };
  auto issue_h = [&](int blk, int st, int t) {
    if (m0 + 8 * (wv * H_DMA + t) < M)
      dma16(hsrc[t] + (size_t)phys(blk) * RB,
            base + NW * WSTAGE + st * HSTAGE + 8 * (wv * H_DMA + t) * RB);
  };

  // The last row tile of the second row half holds at most 16 real rows when M sits
  // just past a multiple of 32 below the tile's end (240 rows in the 256-row tile:
  // rows 224-239).  Its waves then multiply that tile on the 16x16x32 MFMA (16 hidden
  // rows x 16 vocabulary rows, half the matrix-core time of a 32-row tile) and the
  // other tiles as usual: HALF below.  The switch is wave-uniform; both paths run the
  // same barriers.
  const bool half_tail = WVM > 1 && wvm == WVM - 1 && M - (m0 + MROWS - 32) <= 16;
  f32x4* red = (f32x4*)smem;   // [WVV][MROWS] partials of this workgroup (reuses the staging LDS)
  auto body = [&](auto HALFC) __attribute__((always_inline)) {
  constexpr bool HALF = decltype(HALFC)::value;
  f32x16 acc[VT][MT];
#pragma unroll
  for (int j = 0; j < VT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
  f32x4 acc16[2 * VT];   // HALF: vocabulary rows 16q .. 16q+15 of the last row tile
#pragma unroll
  for (int q = 0; q < 2 * VT; ++q) acc16[q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS fragment reads.  A block is NG = 4*MT groups g = (k-step s, row tile i); group
  // g multiplies the VT W fragments of step s with hidden fragment (s, i).
  constexpr int NG = 4 * MT;
  auto w_frag = [&](int stage, int s, int j) {
    const int r = wvv * VT * 32 + 32 * j + l32;
    return *(const bf16x8*)(wst + stage * WSTAGE + r * RB + 16 * swz(r, 2 * s + half));
  };
  auto h_frag32 = [&](int stage, int g) {
    const int s = g / MT, i = g % MT;
    const int r = wvm * MT * 32 + 32 * i + l32;
    return *(const bf16x8*)(hst + stage * HSTAGE + r * RB + 16 * swz(r, 2 * s + half));
  };
  // 16x16x32 operands of the last row tile (HALF): lane l holds row l % 16 of its 16
  // rows and columns 32kk + 8(l/16) .. +7 of the block (k-steps 2kk, 2kk+1)
  const int l16 = lane & 15, q16 = lane >> 4;
  auto h_frag16 = [&](int stage, int kk) {
    const int r = wvm * MT * 32 + 32 * (MT - 1) + l16;
    return *(const bf16x8*)(hst + stage * HSTAGE + r * RB + 16 * swz(r, 4 * kk + q16));
  };
  auto w_frag16 = [&](int stage, int kk, int q) {
    const int r = wvv * VT * 32 + 16 * q + l16;
    return *(const bf16x8*)(wst + stage * WSTAGE + r * RB + 16 * swz(r, 4 * kk + q16));
  };
  // hidden operand of group g: with HALF the last tile's groups of odd k-steps carry the
  // 16x16x32 operand of k-steps s-1, s, those of even k-steps none
  auto h_frag = [&](int stage, int g) {
    if (HALF && g % MT == MT - 1)
      return (g / MT) % 2 == 1 ? h_frag16(stage, (g / MT) / 2) : bf16x8{};
    return h_frag32(stage, g);
  };

  // Pipeline.  Block b's W is in stage b%3, its hidden rows in stage b%2.  Hidden
  // fragments are read LA groups ahead of their MFMAs and W fragments one k-step
  // ahead.  Once the last read of block b is issued (group NG-LA) the waves wait for
  // it and meet at a barrier that also publishes block b+1, then read block b+1
  // while the last LA groups of block b are multiplied, so the matrix cores do not
  // wait for the barrier.  The DMA instructions are spread over the block instead of
  // issued in bursts (a burst fills the vector L1's miss queue and stalls the wave's
  // in-order issue, MFMAs included): W block b+2 over groups WSTART..NG-LA-1 (its stage
  // was freed at block b-1's barrier), hidden block b+2 over the last LA groups (its
  // stage is block b's, freed at this barrier).  Hidden loads are issued after the W
  // loads of the same block, so at block b's barrier only W block b+2 may be
  // outstanding beyond what block b+1 needs.
  static_assert(NG % (LA + 1) == 0, "the hidden fragment ring continues across blocks");
  static_assert(LA <= MT, "the barrier falls in step 3, after step 2 last used wf[0]");
  constexpr int NGI = NG - LA;
  // first group that issues W block b+2: with two row halves (the large-M tile) the W
  // loads go out over the second half of the block only, which keeps fewer of them in
  // flight and measured faster there; the smaller tiles spread them over the block
  constexpr int WSTART = WVM > 1 ? NGI / 2 : 0;
  // Hidden-stage rows of the 8-row groups wholly past M are never loaded, but the
  // MFMAs still read them: zero them once (both stages) so that those products run on
  // zeros instead of whatever an earlier kernel left in LDS.  The chip is power-
  // limited and zero operands draw less (240 rows: 527 -> 517 us after an attention
  // call); their outputs are never written either way.
  {
    const int r0 = min(MROWS, (max(0, M - m0) + 7) & ~7);
    const int n16 = (MROWS - r0) * (RB / 16);
    for (int i = tid; i < 2 * n16; i += THREADS) {
      const int st = i / n16, k = i - st * n16;
      *(uint4*)(hst + st * HSTAGE + r0 * RB + k * 16) = uint4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int t = 0; t < W_DMA; ++t) issue_w(0, 0, t);
#pragma unroll
  for (int t = 0; t < H_DMA; ++t) issue_h(0, 0, t);
  if (nhb > 1) {
#pragma unroll
    for (int t = 0; t < W_DMA; ++t) issue_w(1, 1, t);
    wait_vmcnt<W_DMA>();   // W 0 and hidden 0
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  if (nhb > 1) {
#pragma unroll
    for (int t = 0; t < H_DMA; ++t) issue_h(1, 1, t);
  }

  bf16x8 wf[2][VT];
  bf16x8 w16[2 * VT];   // HALF: the last tile's W operands of the current odd k-step
  bf16x8 hf[LA + 1];
#pragma unroll
  for (int j = 0; j < VT; ++j) wf[0][j] = w_frag(0, 0, j);
#pragma unroll
  for (int g = 0; g < LA; ++g) hf[g] = h_frag(0, g);

  for (int b = 0; b < nhb; ++b) {
    const int sw = b % NW, sh = b & 1;
    const int sw1 = (b + 1) % NW, sh1 = sh ^ 1;   // block b+1 (stale past the last block)
    const int sw2 = (b + 2) % NW;                 // == (b-1) % NW
    const bool more = b + 2 < nhb;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int s = g / MT, i = g % MT;
      if (g + LA < NG) hf[(g + LA) % (LA + 1)] = h_frag(sh, g + LA);
      if (i == 0 && s < 3) {
#pragma unroll
        for (int j = 0; j < VT; ++j) wf[(s + 1) & 1][j] = w_frag(sw, s + 1, j);
      }
#pragma unroll
      for (int t = 0; t < W_DMA; ++t)
        if (WSTART + (t * (NGI - WSTART)) / W_DMA == g && more) issue_w(b + 2, sw2, t);
      if (g == NGI) {
        if (more) wait_vmcnt<W_DMA>();
        else wait_vmcnt<0>();
        __syncthreads();   // block b+1 visible; every wave is done reading block b
#pragma unroll
        for (int j = 0; j < VT; ++j) wf[0][j] = w_frag(sw1, 0, j);   // step 3 uses wf[1]
      }
#pragma unroll
      for (int t = 0; t < H_DMA; ++t)
        if (NGI + (t * LA) / H_DMA == g && more) issue_h(b + 2, sh, t);
      if (g >= NGI) hf[(g + LA) % (LA + 1)] = h_frag(sh1, g + LA - NG);
      if constexpr (HALF) {
        if (i == 0 && s % 2 == 1) {
#pragma unroll
          for (int q = 0; q < 2 * VT; ++q) w16[q] = w_frag16(sw, s / 2, q);
        }
      }
      if (HALF && i == MT - 1) {
        if (s % 2 == 1) {
#pragma unroll
          for (int q = 0; q < 2 * VT; ++q)
            acc16[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w16[q], hf[g % (LA + 1)], acc16[q], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < VT; ++j) acc[j][i] = mfma32(wf[s & 1][j], hf[g % (LA + 1)], acc[j][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();   // every wave is done with the stages; the epilogue reuses them

  // ---- epilogue: per-lane top-2 / exp-sum over its 16*VT vocabulary entries
  if constexpr (HALF) {
    // the 16x16x32 tile: lane l holds hidden row l % 16 and, per q, vocabulary rows
    // 16q + 4(l/16) .. +3; the four lanes of a row are l % 16 + 16 {0, 1, 2, 3}
    const int mloc = wvm * MT * 32 + 32 * (MT - 1) + l16;
    const int m = m0 + mloc;
    Top2 t{-INFINITY, -INFINITY, 0.f, 0x7fffffff};
#pragma unroll
    for (int q = 0; q < 2 * VT; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vocab = v0 + 16 * q + 4 * q16 + r;
        const float x = vocab < V ? acc16[q][r] : -INFINITY;
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
    for (int q = 0; q < 2 * VT; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vocab = v0 + 16 * q + 4 * q16 + r;
        if (vocab < V) z += __builtin_amdgcn_exp2f((acc16[q][r] - t.mx) * kLog2e);
      }
    t.z = z;
    if (logits != nullptr && m < M) {
#pragma unroll
      for (int q = 0; q < 2 * VT; ++q) {
        const int vocab = v0 + 16 * q + 4 * q16;
        float* dst = logits + ((size_t)ks * M + m) * V + vocab;   // split-K: slice ks
        if (vocab + 3 < V && (V & 3) == 0) {
          *(f32x4*)dst = acc16[q];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (vocab + e < V) dst[e] = acc16[q][e];
        }
      }
    }
    t = merge_top2(t, shfl_xor_top2(t, 16));
    t = merge_top2(t, shfl_xor_top2(t, 32));
    if (q16 == 0) red[wvv * MROWS + mloc] = f32x4{t.mx, t.sec, t.z, __int_as_float(t.idx)};
  }
#pragma unroll
  for (int i = 0; i < (HALF ? MT - 1 : MT); ++i) {
    const int mloc = wvm * MT * 32 + 32 * i + l32;
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
          float* dst = logits + ((size_t)ks * M + m) * V + vocab;   // split-K: slice ks
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
    if (half == 0) red[wvv * MROWS + mloc] = f32x4{t.mx, t.sec, t.z, __int_as_float(t.idx)};
  }
  };
  if (half_tail)
    body(std::true_type{});
  else
    body(std::false_type{});
  __syncthreads();
  if (pl.ksplit > 1) return;   // partial sums: no row statistics
  for (int mloc = tid; mloc < MROWS; mloc += THREADS) {
    const int m = m0 + mloc;
    if (m >= M) continue;
    f32x4 e0 = red[mloc];
    Top2 t{e0[0], e0[1], e0[2], __float_as_int(e0[3])};
#pragma unroll
    for (int q = 1; q < WVV; ++q) {
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
  // up to PB partials per lane are loaded before any of them is merged (one memory
  // round trip per row for up to 64*PB vocabulary tiles)
  constexpr int PB = 8;
  for (int p0 = 0; p0 < pl.nvt; p0 += 64 * PB) {
    f32x4 e[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int p = p0 + 64 * u + lane;
      e[u] = p < pl.nvt ? part[(size_t)m * pl.nvt + p] : f32x4{-INFINITY, -INFINITY, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < PB; ++u)
      if (p0 + 64 * u + lane < pl.nvt)
        t = merge_top2(t, Top2{e[u][0], e[u][1], e[u][2], __float_as_int(e[u][3])});
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

// out[i] = sum over the split-K slices of part[s][i] (n = M*N entries)
__global__ void __launch_bounds__(256)
gemm_splitk_sum(size_t n, int S, const float* __restrict__ part, float* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 3 < n) {
    f32x4 a = *(const f32x4*)(part + i);
    for (int s = 1; s < S; ++s) a += *(const f32x4*)(part + (size_t)s * n + i);
    *(f32x4*)(out + i) = a;
  } else {
    for (size_t e = i; e < n; ++e) {
      float a = 0.f;
      for (int s = 0; s < S; ++s) a += part[(size_t)s * n + e];
      out[e] = a;
    }
  }
}

template <int MT, int VT, int WVV, int WVM, int LA>
hipError_t launch_gemm(const LmPlan& pl, const void* hidden, const void* W, f32x4* part,
                       float* logits, hipStream_t stream) {
  constexpr int bytes = lm_lds_bytes<MT, VT, WVV, WVM>();
  static_assert(bytes <= 160 * 1024, "MI355X LDS is 160 KiB per workgroup");
  static_assert(WVV * WVM * MT * 32 * 16 <= bytes, "the epilogue's partials reuse the staging LDS");
  // once per process; function-local static initialisation is thread-safe
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)lm_head_gemm<MT, VT, WVV, WVM, LA>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((lm_head_gemm<MT, VT, WVV, WVM, LA>), dim3(pl.nvt * pl.nmb * pl.ksplit),
                     dim3(WVV * WVM * 64), bytes, stream, (const uint16_t*)hidden,
                     (const uint16_t*)W, pl, part, logits);
  return hipGetLastError();
}

}  // namespace

LmPlan plan_lm_head(int M, int H, int V) {
  LmPlan pl{};
  pl.M = M;
  pl.H = H;
  pl.V = V;
  // tile shapes (LDS holds 3 W stages of vrows x 128 B and 2 hidden stages of
  // mrows x 128 B)
  if (M > 192) {
    pl.variant = 3;          // 8 waves (4 vocab x 2 row halves), 2 per SIMD: 256 rows x 256 vocab
    pl.mrows = 256;
    pl.vrows = 256;
  } else if (M > 128) {
    pl.variant = 4;          // the same grid with three row tiles per half: 192 rows x 256 vocab
    pl.mrows = 192;
    pl.vrows = 256;
  } else if (M > 64) {
    pl.variant = 2;          // 4 waves, MT=4 VT=2: 128 rows x 256 vocab
    pl.mrows = 128;
    pl.vrows = 256;
  } else if (M > 32) {
    pl.variant = 1;          // 4 waves, MT=2 VT=2: 64 rows x 256 vocab
    pl.mrows = 64;
    pl.vrows = 256;
  } else {
    pl.variant = 0;          // 4 waves, MT=1 VT=1: 32 rows x 128 vocab
    pl.mrows = 32;
    pl.vrows = 128;
  }
  pl.nvt = (V + pl.vrows - 1) / pl.vrows;
  pl.nmb = (M + pl.mrows - 1) / pl.mrows;
  pl.ksplit = 1;
  pl.kb_per = H / 64;
  return pl;
}

namespace {

// split-K for plain GEMMs: enough slices to give every CU about two workgroups, each
// slice at least 16 blocks of 64 columns long
LmPlan plan_gemm_f32(int M, int K, int N) {
  LmPlan pl = plan_lm_head(M, K, N);
  if (pl.variant == 1) {
    // 33-64 rows (the draft expansion's GEMMs, 40 rows at C5 shapes): 128 vocabulary
    // rows per workgroup (64 KB of LDS, two workgroups per CU) instead of 256 (112 KB,
    // one per CU).  These GEMMs stream weights with little arithmetic and split K
    // over short slices, and a second workgroup per CU keeps more of the weight
    // stream in flight: the C5-shaped expansion 5.51 -> 5.14 ms.  The LM head of the
    // verification step (no split) stays on the wider tile, which was 1.4% faster there.
    pl.variant = 5;
    pl.vrows = 128;
    pl.nvt = (N + pl.vrows - 1) / pl.vrows;
  }
  const int nhb = K / 64;
  const int tiles = pl.nvt * pl.nmb;
  int S = 1;
  while (S * 2 * tiles <= 2 * kNumCUs && nhb / (S * 2) >= 16) S *= 2;
  pl.ksplit = S;
  pl.kb_per = (nhb + S - 1) / S;
  pl.ksplit = (nhb + pl.kb_per - 1) / pl.kb_per;
  return pl;
}

}  // namespace

size_t gemm_f32_workspace_bytes(int M, int K, int N) {
  const LmPlan pl = plan_gemm_f32(M, K, N);
  size_t b = lm_head_workspace_bytes(pl);
  if (pl.ksplit > 1) b += (size_t)pl.ksplit * M * N * sizeof(float) + 256;
  return b;
}

hipError_t launch_gemm_f32_slices(int M, int K, int N, const void* X, const void* W, float* out,
                                  void* workspace, F32Slices* result, hipStream_t stream) {
  const LmPlan pl = plan_gemm_f32(M, K, N);
  f32x4* part = (f32x4*)workspace;
  float* dst = out;
  if (pl.ksplit > 1)
    dst = (float*)((char*)workspace + (lm_head_workspace_bytes(pl) + 255) / 256 * 256);
  hipError_t e;
  switch (pl.variant) {
    case 3: e = launch_gemm<4, 2, 4, 2, 3>(pl, X, W, part, dst, stream); break;
    case 4: e = launch_gemm<3, 2, 4, 2, 3>(pl, X, W, part, dst, stream); break;
    case 2: e = launch_gemm<4, 2, 4, 1, 3>(pl, X, W, part, dst, stream); break;
    case 1: e = launch_gemm<2, 2, 4, 1, 1>(pl, X, W, part, dst, stream); break;
    case 5: e = launch_gemm<2, 1, 4, 1, 1>(pl, X, W, part, dst, stream); break;
    default: e = launch_gemm<1, 1, 4, 1, 1>(pl, X, W, part, dst, stream); break;
  }
  *result = F32Slices{dst, pl.ksplit, (size_t)M * N};
  return e;
}

hipError_t launch_gemm_f32(int M, int K, int N, const void* X, const void* W, float* out,
                           void* workspace, hipStream_t stream) {
  F32Slices r;
  const hipError_t e = launch_gemm_f32_slices(M, K, N, X, W, out, workspace, &r, stream);
  if (e != hipSuccess || r.S == 1) return e;
  hipLaunchKernelGGL(gemm_splitk_sum, dim3((unsigned)((r.stride + 1023) / 1024)), dim3(256), 0, stream,
                     r.stride, r.S, r.p, out);
  return hipGetLastError();
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
    case 3: e = launch_gemm<4, 2, 4, 2, 3>(pl, hidden, W, part, out_logits, stream); break;
    case 4: e = launch_gemm<3, 2, 4, 2, 3>(pl, hidden, W, part, out_logits, stream); break;
    case 2: e = launch_gemm<4, 2, 4, 1, 3>(pl, hidden, W, part, out_logits, stream); break;
    case 1: e = launch_gemm<2, 2, 4, 1, 1>(pl, hidden, W, part, out_logits, stream); break;
    default: e = launch_gemm<1, 1, 4, 1, 1>(pl, hidden, W, part, out_logits, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_head_merge, dim3((pl.M + 3) / 4), dim3(256), 0, stream, pl,
                     (const f32x4*)part, out_max, out_argmax, out_lse, out_second);
  return hipGetLastError();
}

}  // namespace eagle
