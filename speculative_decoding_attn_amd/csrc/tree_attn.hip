// Tree-verify attention for gfx950.
//
// [P1] innovations list item 2 / [P2] workflow paragraph: the target verifies
// every path of the draft tree in one pass by masking attention with the tree.
// Node i at query head h attends to the whole prefix and to its own root path.
//
// Work decomposition.  For one (sequence b, KV head g) pair the R = N*G query rows
// (row r = node r/G, head g*G + r%G) share every K/V row, so a workgroup takes a
// block of WAVES*32 rows of one pair and one contiguous range of keys ("split"):
// K and V tiles of 32 keys are staged once in LDS and read by all of its waves.
// Each wave owns 32 rows (one 32-row MFMA tile).
//
// Orientation.  Scores are formed transposed, S^T = K * Q^T, with the 32x32x16 bf16
// MFMA: lane l then holds 16 keys of ONE query row (l % 32), so the row max, the
// exponentials and the row sum stay inside the lane (plus one exchange with lane
// l ^ 32), and the output O^T = V^T * P^T again gives each lane one row.  P^T is fed
// straight from the score registers; V is stored transposed in LDS with its key
// positions permuted (bits 2 and 3 of the key index swapped) so that the key order
// of the P^T registers and of the V^T operand agree.
//
// Mask.  The ancestor-or-self set of each lane's node is a 64-bit mask in
// registers; only the key chunks that reach past the prefix are masked.
//
// Softmax.  Base 2 with scale*log2(e) folded into one FMA.  The general kernel keeps
// an online max that is only raised when a chunk exceeds it by more than 2^8
// (values then stay below 256), so O is rescaled rarely; the branch is taken per
// wave when any lane needs it.  The D = 128 eight-wave kernel takes every weight of
// a split against one reference max per row (its section below).
//
// Splits.  The prefix is cut into S ranges of whole 32-key chunks; the last range
// also covers the tree keys.  With S > 1 every workgroup writes its normalised
// partial output and log-sum-exp in fp32 and a merge kernel combines them.
#include "common.h"
#include "internal.h"


namespace eagle {

namespace {

constexpr int KC = 32;            // keys per chunk
constexpr float kLazy = 8.0f;     // log2 headroom before the running max is raised

template <int D>
struct AttnLds {
  static constexpr int KSTR = D + 8;    // bf16 per K row (16 B pad: conflict-free b128 reads)
  static constexpr int VSTR = KC + 8;   // bf16 per V^T row
  static constexpr int KELEMS = KC * KSTR;
  static constexpr int VELEMS = D * VSTR;
  static constexpr int STAGE = KELEMS + VELEMS;
};

// key index within a 16-key group -> position in the V^T row (swap bits 2 and 3)
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// The (sequence, KV head, row block, key split) a workgroup computes.  Uniform batches:
// every (sequence, KV head) pair is cut into pl.S splits of pl.split_len keys
// (attn_item).  Ragged batches with a device plan: sequence b is cut into its own
// number of splits of one common length, chosen on the device from the real prefix
// lengths (planned_item, below), and blocks past the plan's items have nothing to
// do.  `slot` indexes the split partials: uniform pair * S + split, planned item *
// Hkv + KV head.
struct AttnItem {
  bool valid;
  int b, g, rb, split, nsplit, len, slot;
};

__device__ __forceinline__ AttnItem attn_item(const AttnPlan& pl, int logical) {
  AttnItem it;
  it.rb = logical % pl.RB;
  it.split = (logical / pl.RB) % pl.S;
  const int pair = logical / (pl.RB * pl.S);
  it.b = pair / pl.Hkv;
  it.g = pair % pl.Hkv;
  it.nsplit = pl.S;
  it.len = pl.split_len;
  it.slot = pair * pl.S + it.split;
  it.valid = true;
  return it;
}

// Partial slot of split s of (sequence b, KV head g) (see attn_item).
__device__ __forceinline__ int attn_slot(const AttnPlan& pl, int b, int g, int s) {
  return pl.dplan ? (pl.dplan[2 + b] + s) * pl.Hkv + g : (b * pl.Hkv + g) * pl.S + s;
}
__device__ __forceinline__ int attn_nsplit(const AttnPlan& pl, int b) {
  return pl.dplan ? pl.dplan[2 + pl.B + b] : pl.S;
}

// Shortest split: narrow workgroups (one or two waves) are cheap to start, so their
// splits go down to 128 keys (head dim 64); the eight-wave kernel's stay at
// kMinSplitKeys.  The uniform and the ragged plans use the same bound.
__host__ __device__ inline int min_split_keys(int waves) { return waves <= 2 ? 128 : kMinSplitKeys; }

// Ragged batches: the split length and this workgroup's (sequence, split) item, from
// the real prefix lengths.  The length is the smallest multiple of 32 keys, at least
// min_split_keys, for which the sequences' items (ceil(prefix / length) splits each,
// at least one for the tree keys) number at most the B * S items of the uniform
// plan; with every prefix at the maximum that is the uniform plan's split length
// (the same splits).  Every workgroup computes it (a pure function of the prefix
// lengths, so all agree) instead of a separate plan kernel; workgroup 0 also writes
// the per-sequence table the merge reads.  All threads of the workgroup call it.
__device__ AttnItem planned_item(const AttnPlan& pl, int logical) {
  __shared__ int s_best;
  __shared__ int s_item[4];   // valid, sequence, split, number of splits
  const int B = pl.B, cap = pl.B * pl.S;
  const int lo = min_split_keys(pl.waves) / KC, hi = max(lo, (pl.P + KC - 1) / KC);   // hi: B items
  if (threadIdx.x == 0) s_best = hi;
  __syncthreads();
  // each thread tries its own candidate lengths in increasing order, all at once
  int mine = hi;
  for (int u = lo + (int)threadIdx.x; u < hi; u += blockDim.x) {
    const int len = u * KC;
    int c = 0;
    for (int b = 0; b < B && c <= cap; ++b) {
      const int P = min(max(pl.prefix_len[b], 0), pl.P);
      c += max(1, (P + len - 1) / len);
    }
    if (c <= cap) {
      mine = u;
      break;
    }
  }
  mine = wave_min_i(mine);
  if ((threadIdx.x & 63) == 0) atomicMin(&s_best, mine);
  __syncthreads();
  const int len = s_best * KC;
  const int t = logical / (pl.RB * pl.Hkv);
  if (threadIdx.x == 0) {
    s_item[0] = 0;
    s_item[1] = 0;
    s_item[2] = 0;
    s_item[3] = 1;
    int first = 0;
    for (int b = 0; b < B; ++b) {
      const int P = min(max(pl.prefix_len[b], 0), pl.P);
      const int nb = min(max(1, (P + len - 1) / len), cap - first - (B - 1 - b));
      if (logical == 0) {
        pl.dplan[2 + b] = first;
        pl.dplan[2 + B + b] = nb;
      }
      if (t >= first && t < first + nb) {
        s_item[0] = 1;
        s_item[1] = b;
        s_item[2] = t - first;
        s_item[3] = nb;
      }
      first += nb;
    }
    if (logical == 0) {
      pl.dplan[0] = len;
      pl.dplan[1] = first;
    }
  }
  __syncthreads();
  AttnItem it;
  it.rb = logical % pl.RB;
  it.g = (logical / pl.RB) % pl.Hkv;
  it.valid = s_item[0] != 0;
  it.b = s_item[1];
  it.split = s_item[2];
  it.nsplit = s_item[3];
  it.len = len;
  it.slot = t * pl.Hkv + it.g;
  return it;
}

template <int D, int WAVES, bool PAGED>
__global__ void __launch_bounds__(WAVES * 64, 1)
tree_attn_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ v, const int32_t* __restrict__ parents,
              AttnPlan pl, uint16_t* __restrict__ out, float* __restrict__ lse_out,
              float* __restrict__ part_o, float* __restrict__ part_lse) {
  using L = AttnLds<D>;
  constexpr int THREADS = WAVES * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  // per chunk: 4D K units (16 bytes of one key row) and 4D V units (8 bytes of a key
  // pair, i.e. two 8-byte loads); every thread takes the same number of each, so the
  // per-wave load count of a chunk is a constant (the vmcnt arithmetic below)
  constexpr int UNITS = 4 * D;
  static_assert(UNITS % THREADS == 0, "chunk staging must divide evenly over the threads");
  constexpr int K_PER = UNITS / THREADS;
  constexpr int V_PER = UNITS / THREADS;
  constexpr int LOADS = K_PER + 2 * V_PER;   // vector-memory loads per thread per chunk
  static_assert(LOADS <= 63, "vmcnt is a 6-bit counter");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::STAGE];
  __shared__ int32_t ptab[PAGED ? kMaxSplitPages : 1];   // paged KV: this split's blocks

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // blocks are dealt to the 8 XCDs round-robin; renumber so that consecutive
  // logical blocks (the row blocks of one pair and split) share an XCD's L2
  const int nwg = gridDim.x;
  const int w = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const AttnItem item = pl.dplan ? planned_item(pl, logical) : attn_item(pl, logical);
  if (!item.valid) return;   // a planned ragged batch with fewer items than blocks
  const int rb = item.rb;
  const int split = item.split;
  const int b = item.b;
  const int g = item.g;
  const int pair = b * pl.Hkv + g;
  const int G = pl.G;
  // this sequence's prefix and tree (ragged batches: clamped to the plan's maxima,
  // so every access stays inside the layouts the plan was sized for)
  const int P = pl.prefix_len ? min(max(pl.prefix_len[b], 0), pl.P) : pl.P;
  const int N = pl.tree_len ? min(max(pl.tree_len[b], 1), pl.N) : pl.N;
  // this sequence's query rows (rows past R are padding): its N nodes, or the subset
  const int R = (pl.nq > 0 ? pl.nq : N) * G;
  // split s covers prefix keys [s*len, (s+1)*len) below P (possibly none); the last
  // split also takes the tree keys P .. P+N-1
  const int key_begin = (split == item.nsplit - 1) ? min(split * item.len, P) : split * item.len;
  const int key_end = (split == item.nsplit - 1) ? P + N : min(P, (split + 1) * item.len);
  const int key_lim = P + N;

  const uint16_t* kbase = PAGED ? k : k + (size_t)pair * pl.kv_cap * D;
  const uint16_t* vbase = PAGED ? v : v + (size_t)pair * pl.kv_cap * D;
  const int32_t* par = parents + (size_t)b * pl.N;
  // element offset of cache row `key` (< key_lim) of this (sequence, KV head)
  const int first_page = PAGED ? (key_begin >> pl.page_shift) : 0;
  auto row_off = [&](int key) -> size_t {
    if constexpr (PAGED) {
      const int blk = ptab[(key >> pl.page_shift) - first_page];
      const int slot = key & ((1 << pl.page_shift) - 1);
      return (((size_t)blk * pl.Hkv + g) << pl.page_shift | (size_t)slot) * D;
    } else {
      return (size_t)key * D;
    }
  };

  // ---- Q^T operand (B side of S^T = K Q^T) and ancestor mask of this wave's rows
  const int r_row = rb * (WAVES * 32) + wid * 32 + l32;
  bf16x8 qf[KSTEPS];
  uint64_t anc;
  if (r_row < R) {
    const int il = r_row / G;
    const int i = pl.node0 + il;
    const int h = g * G + (r_row - il * G);
    const uint16_t* qp = q + ((size_t)(b * pl.N + i) * pl.Hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(*(const u32x4*)(qp + 16 * s));
    anc = ancestor_mask(par, i, N);
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
    anc = 1;
  }

  f32x16 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float mc = -INFINITY;   // running max of scale*log2e*s
  float lsum = 0.f;       // this lane's half of the row sum

  const float c = pl.c;
  const uint64_t node_mask = N >= 64 ? ~0ull : ((1ull << N) - 1ull);

  // ---- chunk staging: a ring of two register slots.  Chunk c is loaded two
  // iterations before it is computed (slot c%2), stored to LDS stage c%2 at the end of
  // iteration c-1, and computed in iteration c, so each wave keeps one chunk of loads
  // in flight across a whole chunk of compute.  The slots are indexed with
  // compile-time constants only (the chunk loop is unrolled by two), which lets the
  // compiler keep them in registers and wait for exactly the older slot's loads.
  // Rows past P+N are clamped on load and zeroed on store.
  u32x4 kreg[2][K_PER];
  u32x2 vreg[2][V_PER][2];
  auto load_chunk = [&](int slot, int kb) {
#pragma unroll
    for (int it = 0; it < K_PER; ++it) {
      const int u = tid + it * THREADS;
      const int key = min(kb + u / (D / 8), key_lim - 1);
      const int col = (u % (D / 8)) * 8;
      kreg[slot][it] = *(const u32x4*)(kbase + row_off(key) + col);
    }
#pragma unroll
    for (int it = 0; it < V_PER; ++it) {
      const int u = tid + it * THREADS;
      const int kp = u % (KC / 2);
      const int d0 = (u / (KC / 2)) * 4;
      const int key = kb + 2 * kp;
      vreg[slot][it][0] = *(const u32x2*)(vbase + row_off(min(key, key_lim - 1)) + d0);
      vreg[slot][it][1] = *(const u32x2*)(vbase + row_off(min(key + 1, key_lim - 1)) + d0);
    }
  };
  // registers -> LDS stage (K as [key][d], V transposed as [d][permuted key])
  auto store_chunk = [&](int slot, int st, int kb) {
    uint16_t* Ks = lds + st * L::STAGE;
    uint16_t* Vs = Ks + L::KELEMS;
#pragma unroll
    for (int it = 0; it < K_PER; ++it) {
      const int u = tid + it * THREADS;
      const int key = u / (D / 8);
      const int col = (u % (D / 8)) * 8;
      *(u32x4*)(Ks + key * L::KSTR + col) =
          kb + key < key_lim ? kreg[slot][it] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < V_PER; ++it) {
      const int u = tid + it * THREADS;
      const int kp = u % (KC / 2);
      const int d0 = (u / (KC / 2)) * 4;
      const int key = 2 * kp;
      const int pos = (key & 16) | vt_pos(key & 15);
      const u32x2 a = kb + key < key_lim ? vreg[slot][it][0] : u32x2{0, 0};
      const u32x2 bb = kb + key + 1 < key_lim ? vreg[slot][it][1] : u32x2{0, 0};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // elements 2e and 2e+1 of each key's 4-wide piece
        const uint32_t lo = (a[e] & 0xFFFFu) | (bb[e] << 16);
        const uint32_t hi = (a[e] >> 16) | (bb[e] & 0xFFFF0000u);
        *(uint32_t*)(Vs + (d0 + 2 * e) * L::VSTR + pos) = lo;
        *(uint32_t*)(Vs + (d0 + 2 * e + 1) * L::VSTR + pos) = hi;
      }
    }
  };

  const int n_chunks = key_end > key_begin ? (key_end - key_begin + KC - 1) / KC : 0;
  if constexpr (PAGED) {
    // rows loaded by this split (prefetches run up to two chunks past its end, all
    // clamped below key_lim); their blocks, clamped to the pool
    const int last = min(key_lim - 1, key_begin + (n_chunks + 2) * KC - 1);
    const int npages = min((last >> pl.page_shift) - first_page + 1, kMaxSplitPages);
    const int32_t* bt = pl.block_table + (size_t)b * pl.max_pages + first_page;
    for (int j = tid; j < npages; j += THREADS) ptab[j] = min(max(bt[j], 0), pl.num_blocks - 1);
    __syncthreads();
  }
  if (n_chunks > 0) {
    load_chunk(0, key_begin);
    load_chunk(1, key_begin + KC);   // clamped (and zeroed) if it does not exist
    store_chunk(0, 0, key_begin);
  }
  __syncthreads();

  // unrolled by two: the ring slot and LDS stage of each chunk are compile-time
  // indices (a runtime index would move the ring to scratch memory)
  for (int ch0 = 0; ch0 < n_chunks; ch0 += 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int ch = ch0 + st;
      if (st == 1 && ch >= n_chunks) break;   // chunk ch0 always exists
      const int kb = key_begin + ch * KC;
      // chunk ch+2 into the slot chunk ch came from (its data is in LDS already)
      load_chunk(st, kb + 2 * KC);
      const uint16_t* Ks = lds + st * L::STAGE;
      const uint16_t* Vs = Ks + L::KELEMS;

      // S^T tile for 32 keys
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 kf = *(const bf16x8*)(Ks + l32 * L::KSTR + 16 * s + 8 * half);
        sacc = mfma32(kf, qf[s], sacc);
      }

      // scores of this lane's 16 keys; chunks that reach into the tree (or past it) get
      // the ancestor mask: bit j of `allowed` says whether key kb + j is visible
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = sacc[r];
      if (kb + KC > P) {
        const int off = kb - P;   // >= -31
        // only the last split owns the tree keys: in a ragged batch an earlier split
        // can end inside a chunk at this sequence's prefix end
        const uint64_t tm = (split == item.nsplit - 1) ? (anc & node_mask) : 0ull;
        const uint32_t tree_bits = off >= 0 ? (off < 64 ? (uint32_t)(tm >> off) : 0u)
                                            : (uint32_t)(tm << (-off));
        const uint32_t prefix_bits = off < 0 ? ((1u << (-off)) - 1u) : 0u;
        const uint32_t allowed = (tree_bits | prefix_bits) >> (4 * half);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bit = 8 * (r >> 2) + (r & 3);
          sv[r] = ((allowed >> bit) & 1u) ? sv[r] : -INFINITY;
        }
      }

      bf16x8 pf[2];
      {
        float mx = sv[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxc = mx * c;
        const bool need = mxc > mc + kLazy;
        if (__ballot(need)) {
          const float mnew = need ? mxc : mc;
          const float alpha = need ? exp2f(mc - mnew) : 1.f;
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          mc = mnew;
        }
        const float mcu = (mc == -INFINITY) ? 0.f : mc;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(fmaf(sv[r], c, -mcu));
          lsum += pr[r];
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(pr[8 * cc + 2 * e], pr[8 * cc + 2 * e + 1]);
          pf[cc] = as_bf16x8(pk);
        }
      }

      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 vf = *(const bf16x8*)(Vs + (32 * db + l32) * L::VSTR + 16 * cc + 8 * half);
          oacc[db] = mfma32(vf, pf[cc], oacc[db]);
        }

      // chunk ch+1 (loaded during iteration ch-1) -> LDS stage st^1, while chunk ch+2's
      // loads stay in flight
      if (ch + 1 < n_chunks) store_chunk(st ^ 1, st ^ 1, kb + KC);
      __syncthreads();
    }
  }
  // ---- epilogue
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (r_row >= R) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse = (mc + log2f(ltot)) * kLn2;
  const int il = r_row / G;
  const int i = pl.node0 + il;
  const int h = g * G + (r_row - il * G);
  if (pl.S == 1 && !pl.dplan) {
    uint16_t* op = out + ((size_t)(b * pl.N + i) * pl.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * half;
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv);
        pk[1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *(u32x2*)(op + d0) = pk;
      }
    if (half == 0 && lse_out) lse_out[(size_t)(b * pl.N + i) * pl.Hq + h] = lse;
  } else {
    const size_t prow = (size_t)item.slot * pl.Rpad + r_row;
    float* op = part_o + prow * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * half;
        f32x4 vv = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                    oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv};
        *(f32x4*)(op + d0) = vv;
      }
    if (half == 0) part_lse[prow] = lse;
  }
}

// One wave per (pair, row): combine the S split partials with their lse weights.
// D = 128: one (pair, row) per half wave, 4 entries (16 bytes) per lane; the same
// arithmetic per entry as tree_attn_merge
__global__ void __launch_bounds__(256)
tree_attn_merge_hw(AttnPlan pl, const float* __restrict__ part_o, const float* __restrict__ part_lse,
                   uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 31;
  const int gr = blockIdx.x * (blockDim.x / 32) + (threadIdx.x >> 5);
  const int pairs = pl.B * pl.Hkv;
  if (gr >= pairs * pl.R) return;
  const int pair = gr / pl.R;
  const int r = gr % pl.R;
  const int b = pair / pl.Hkv;
  const int g = pair % pl.Hkv;
  if (pl.tree_len && r >= min(max(pl.tree_len[b], 1), pl.N) * pl.G) return;   // past this tree
  const int ns = attn_nsplit(pl, b);
  float mx = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  constexpr int MS = 16;
  if (ns <= MS) {
    // every split's lse and partial loaded at once (one memory latency, not 2 ns)
    float l[MS];
    f32x4 o[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      if (s < ns) {
        const size_t prow = (size_t)attn_slot(pl, b, g, s) * pl.Rpad + r;
        l[s] = part_lse[prow];
        o[s] = *(const f32x4*)(part_o + prow * D + lane * 4);
      }
    }
#pragma unroll
    for (int s = 0; s < MS; ++s)
      if (s < ns) mx = fmaxf(mx, l[s]);
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      if (s < ns) {
        const float wgt = expf(l[s] - mx);
        wsum += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += wgt * o[s][e];
      }
    }
  } else {
    // more splits: the same arithmetic in two passes over batches of MS splits, each
    // batch's loads issued at once (the max first, then the weighted sum in split order)
    for (int s0 = 0; s0 < ns; s0 += MS) {
      float l[MS];
#pragma unroll
      for (int s = 0; s < MS; ++s)
        if (s0 + s < ns) l[s] = part_lse[(size_t)attn_slot(pl, b, g, s0 + s) * pl.Rpad + r];
#pragma unroll
      for (int s = 0; s < MS; ++s)
        if (s0 + s < ns) mx = fmaxf(mx, l[s]);
    }
    for (int s0 = 0; s0 < ns; s0 += MS) {
      float l[MS];
      f32x4 o[MS];
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        if (s0 + s < ns) {
          const size_t prow = (size_t)attn_slot(pl, b, g, s0 + s) * pl.Rpad + r;
          l[s] = part_lse[prow];
          o[s] = *(const f32x4*)(part_o + prow * D + lane * 4);
        }
      }
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        if (s0 + s < ns) {
          const float wgt = expf(l[s] - mx);
          wsum += wgt;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += wgt * o[s][e];
        }
      }
    }
  }
  const float inv = 1.f / wsum;
  const int il = r / pl.G;
  const int i = pl.node0 + il;
  const int h = g * pl.G + (r - il * pl.G);
  uint16_t* o = out + ((size_t)(b * pl.N + i) * pl.Hq + h) * D + lane * 4;
  u32x2 pk;
  pk[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(u32x2*)o = pk;
  if (lane == 0 && lse_out) lse_out[(size_t)(b * pl.N + i) * pl.Hq + h] = mx + logf(wsum);
}

template <int D>
__global__ void __launch_bounds__(256)
tree_attn_merge(AttnPlan pl, const float* __restrict__ part_o, const float* __restrict__ part_lse,
                uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int pairs = pl.B * pl.Hkv;
  if (gw >= pairs * pl.R) return;
  const int pair = gw / pl.R;
  const int r = gw % pl.R;
  const int b = pair / pl.Hkv;
  const int g = pair % pl.Hkv;
  if (pl.tree_len && r >= min(max(pl.tree_len[b], 1), pl.N) * pl.G) return;   // past this tree
  const int ns = attn_nsplit(pl, b);
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, part_lse[(size_t)attn_slot(pl, b, g, s) * pl.Rpad + r]);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t prow = (size_t)attn_slot(pl, b, g, s) * pl.Rpad + r;
    const float wgt = expf(part_lse[prow] - mx);
    wsum += wgt;
    const float* op = part_o + prow * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += wgt * op[e];
  }
  const float inv = 1.f / wsum;
  const int il = r / pl.G;
  const int i = pl.node0 + il;
  const int h = g * pl.G + (r - il * pl.G);
  uint16_t* o = out + ((size_t)(b * pl.N + i) * pl.Hq + h) * D + lane * PER;
  if (PER == 2) {
    *(uint32_t*)o = pack_bf16x2(acc[0] * inv, acc[PER - 1] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const uint32_t pk = pack_bf16x2(acc[e] * inv, 0.f);
      o[e] = (uint16_t)(pk & 0xFFFFu);
    }
  }
  if (lane == 0 && lse_out) lse_out[(size_t)(b * pl.N + i) * pl.Hq + h] = mx + logf(wsum);
}

// ---------------------------------------------------------------------------
// D = 128: eight waves of 32 query rows (two per SIMD), one 256-row block per
// workgroup, each wave running its own software pipeline over the split.
//
// Staging.  K and V reach LDS by global-to-LDS DMA (each lane moves 16 bytes to
// m0 + 16*lane, non-temporal: the cache streams them through once), in chunks of 64
// keys, four stages deep, one workgroup barrier per chunk.  Rows are stored whole
// (256 bytes) with their 16-byte pieces permuted: K piece c of row r sits at
// c ^ (r & 15), which makes the b128 fragment reads of 16 consecutive rows hit every
// bank once; V piece c of row r sits at c ^ 4*(r & 3), which does the same for the
// transposing reads (ds_read_b64_tr_b16) that hand each lane 4 keys of one V column,
// the V^T operand of the output MFMA, without a transpose in registers.  Past the end
// of the split the DMA repeats the split's last row into a stage that is not read
// again, so every iteration issues and waits alike.
//
// Reference max.  A row's weights are taken against one value for the whole split:
// the exact max of the row's scores in the split's first chunk (every row sees a key
// there: a prefix key, or the root of its tree).  Weights above 1 are exact in fp32
// and bf16 alike, so nothing is rescaled along the way.  A row whose weights sum past
// 2^64 (a later score far above the first chunk's) has the whole workgroup redo the
// split: one walk for the exact row max (scores only), then the walk again with it,
// where no weight exceeds 1.
//
// Pipeline of a wave, iteration j, in a fixed order with no branch.  A chunk's scores
// are two 32-key tiles, each its own MFMA accumulation chain; the two chains
// alternate, so no score MFMA waits on the one before it.
//   region 1, 16 MFMA slots: scores of chunk j+1 (S^T = K Q^T) and the weights of
//     tile 1 (keys 32-63) of chunk j;
//   region 2, 16 MFMA slots: output of chunk j (O^T += V^T P^T) and the weights of
//     tile 0 (keys 0-31) of chunk j+1.
// A weight pair goes through three steps (scale and shift, exponentials, bf16 pack
// and row sum) in consecutive slots, so each slot holds independent vector
// instructions beside its MFMA; the other wave of the SIMD fills the gaps.  LDS
// fragments are read four ahead of their MFMAs.  The iteration's workgroup barrier
// comes after the wave's last LDS read, before its last four output MFMAs; past it
// the DMA of chunk j+4 goes into the stage of chunk j, issued after the iteration's
// work.  A wave whose rows are all padding keeps only the DMAs and the barriers.
constexpr int XROW = 256;            // bytes per K or V row
constexpr int WC = 64;               // keys per chunk (two 32-key score tiles)
constexpr int WNB = 4;               // LDS stages
constexpr int WHALF = WC * XROW;     // one chunk of K (or of V): 16 KB
constexpr int WSTAGE = 2 * WHALF;
constexpr int WLDS = WNB * WSTAGE;   // 128 KB of dynamic LDS
constexpr float kRowSumLimit = 18446744073709551616.0f;   // 2^64

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i16 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

template <bool PAGED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
tree_attn_d128(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const int32_t* __restrict__ parents,
               AttnPlan pl, uint16_t* __restrict__ out, float* __restrict__ lse_out,
               float* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int D = 128;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ int32_t ptab[PAGED ? kMaxSplitPages : 1];
  __shared__ int32_t spar[64];   // a tree has at most 64 nodes (64-bit masks)
  __shared__ int32_t redo;       // some row's weights outgrew the reference max

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int nwg = gridDim.x;
  const int w = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const AttnItem item = pl.dplan ? planned_item(pl, logical) : attn_item(pl, logical);
  if (!item.valid) return;   // a planned ragged batch with fewer items than blocks
  const int rb = item.rb;
  const int split = item.split;
  const int b = item.b;
  const int g = item.g;
  const int pair = b * pl.Hkv + g;
  const int G = pl.G;
  const int P = pl.prefix_len ? min(max(pl.prefix_len[b], 0), pl.P) : pl.P;
  const int N = pl.tree_len ? min(max(pl.tree_len[b], 1), pl.N) : pl.N;
  const int R = (pl.nq > 0 ? pl.nq : N) * G;
  const bool last = split == item.nsplit - 1;
  const int key_begin = last ? min(split * item.len, P) : split * item.len;
  const int key_end = last ? P + N : min(P, (split + 1) * item.len);
  const int key_lim = P + N;
  // keys at or past mask_from are masked: the tree part of the last split, and the
  // tail of a chunk that runs past the end of an earlier split
  const int mask_from = last ? P : key_end;
  const int n = key_end > key_begin ? (key_end - key_begin + WC - 1) / WC : 0;
  // last key any load of this split reads (the DMA past the end repeats it)
  const int kmax = max(0, min(key_lim - 1, key_begin + n * WC - 1));

  const uint16_t* kbase = PAGED ? k : k + (size_t)pair * pl.kv_cap * D;
  const uint16_t* vbase = PAGED ? v : v + (size_t)pair * pl.kv_cap * D;
  const int first_page = PAGED ? (key_begin >> pl.page_shift) : 0;
  auto row_off = [&](int key) -> size_t {
    if constexpr (PAGED) {
      const int blk = ptab[(key >> pl.page_shift) - first_page];
      const int slot = key & ((1 << pl.page_shift) - 1);
      return (((size_t)blk * pl.Hkv + g) << pl.page_shift | (size_t)slot) * D;
    } else {
      return (size_t)key * D;
    }
  };

  // the tree's parent links and (paged) this split's slice of the block table to LDS;
  // this wave's Q^T operand to registers
  if (tid < pl.N) spar[tid] = parents[(size_t)b * pl.N + tid];
  bf16x8 qf[KSTEPS];
  const int r_row = rb * 256 + wv * 32 + l32;
  if (r_row < R) {
    const int il = r_row / G;
    const int h = g * G + (r_row - il * G);
    const uint16_t* qp = q + ((size_t)(b * pl.N + pl.node0 + il) * pl.Hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(*(const u32x4*)(qp + 16 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
  }
  if constexpr (PAGED) {
    const int npages = min((kmax >> pl.page_shift) - first_page + 1, kMaxSplitPages);
    const int32_t* bt = pl.block_table + (size_t)b * pl.max_pages + first_page;
    for (int j = tid; j < npages; j += 512) ptab[j] = min(max(bt[j], 0), pl.num_blocks - 1);
  }
  if (tid == 0) redo = 0;
  __syncthreads();

  const uint32_t xbase = lds_addr(xs);
  // a wave whose 32 rows all lie past R (the padding of the last row block) only moves
  // its share of K and V and keeps the barriers: it computes nothing
  const bool busy = rb * 256 + wv * 32 < R;
  // the pair's K and V bases, in scalar registers
  const uint16_t* const kbase_s = uniform_ptr(kbase);
  const uint16_t* const vbase_s = uniform_ptr(vbase);
  // byte offsets, within a chunk, of the 16 bytes of K and V this lane moves
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * wv + 4 * t + (lane >> 4);
    koff[t] = (uint32_t)(row * XROW + 16 * ((lane & 15) ^ (row & 15)));
    voff[t] = (uint32_t)(row * XROW + 16 * ((lane & 15) ^ (4 * (row & 3))));
  }
  // chunk cidx -> LDS stage cidx % WNB; wave wv moves rows 8wv .. 8wv+7 of K and V.
  // FAST: the chunk lies wholly at or below kmax, so a scalar base plus the fixed lane
  // offsets address it (contiguous cache only); otherwise each row is clamped to kmax.
  auto issue = [&](int cidx, auto FAST) {
    const int kb = key_begin + cidx * WC;
    const uint32_t st = xbase + (uint32_t)(cidx % WNB) * WSTAGE;
    if constexpr (!PAGED && decltype(FAST)::value) {
      const uint16_t* kc = kbase_s + (size_t)kb * D;
      const uint16_t* vc = vbase_s + (size_t)kb * D;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t dst = st + (uint32_t)(8 * wv + 4 * t) * XROW;
        dma16_nt_s(kc, koff[t], dst);
        dma16_nt_s(vc, voff[t], dst + WHALF);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 8 * wv + 4 * t + (lane >> 4);
      const size_t off = row_off(min(kb + row, kmax));
      const uint32_t dst = st + (uint32_t)(8 * wv + 4 * t) * XROW;
      dma16_nt(kbase + off + 8 * ((lane & 15) ^ (row & 15)), dst);
      dma16_nt(vbase + off + 8 * ((lane & 15) ^ (4 * (row & 3))), dst + WHALF);
    }
  };
  if (n > 0) {
    issue(0, std::false_type{});
    issue(1, std::false_type{});
  }

  // ---- ancestor mask of this wave's 32 rows (while chunks 0, 1 are in flight)
  uint64_t tmask;
  {
    uint64_t anc = 1;
    if (r_row < R) {
      const int il = r_row / G;
      const int i = pl.node0 + il;
      anc = 0;
      int nn = i;
      for (int step = 0; step < 64; ++step) {   // root path, bounded
        if (nn < 0 || nn >= N) break;
        anc |= 1ull << nn;
        const int p = spar[nn];
        if (p >= nn) break;
        nn = p;
      }
    }
    tmask = last ? (anc & (N >= 64 ? ~0ull : ((1ull << N) - 1ull))) : 0ull;
  }
  // the Q loads and chunks 0, 1 have landed (a wait the compiler sees, so it puts no
  // wait of its own for the Q loads inside the pipeline); the barrier publishes them
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (n > 0) {
#pragma unroll
    for (int c = 2; c < WNB; ++c) issue(c, std::false_type{});
  }
  // The workgroup barrier of iteration j sits after the wave's last LDS read of the
  // iteration, before its last output MFMAs: it publishes chunk j+2 for iteration j+1
  // (the wait leaves only chunk j+3 in flight), and once every wave is past it the
  // iteration's stages are free, so the DMA of chunk j+WNB into stage j % WNB follows.
  auto sync = [&]() __attribute__((always_inline)) {
    wait_vmcnt<4 * (WNB - 3)>();
    __syncthreads();
  };

  f32x16 oacc[DBLK];   // O^T of the wave's rows, 32 dims per tile
  float mref;          // reference max (scale*log2e units), same in both lanes of a row
  float part[4];       // partial row sums (this lane's half of the row)
  f32x16 sacc[2];      // S^T of the newest chunk, keys 32t .. 32t+31 in tile t
  float scp[16];       // tile 1 (keys 32-63) of the previous chunk: sacc is reused
  u32x4 pk[4];         // bf16 weights being formed (P^T operands, 16 keys each)
  bf16x8 pf[4];        // weights of the chunk whose output is being updated
  const float c = pl.c;
  const int kx = l32 & 15;   // K piece permutation of this lane's row

  // keys of chunk cidx this lane's row may see: the prefix part below mask_from and
  // the tree part on the row's root path (bit = key within the chunk)
  auto mask_bits = [&](int cidx) -> uint64_t {
    const int kb = key_begin + cidx * WC;
    const int npre = mask_from - kb;
    const int off = kb - P;
    uint64_t a = npre <= 0 ? 0ull : (npre >= 64 ? ~0ull : ((1ull << npre) - 1ull));
    a |= off >= 0 ? (off < 64 ? tmask >> off : 0ull) : (-off < 64 ? tmask << (-off) : 0ull);
    return a;
  };
  // value x of score r of tile t (key 32t + 8*(r/4) + 4*half + r%4), or -inf where
  // alw excludes it
  auto masked = [&](float x, int t, int r, uint64_t alw, auto MK) -> float {
    if constexpr (decltype(MK)::value) {
      const int bit = 32 * t + 8 * (r >> 2) + 4 * half + (r & 3);
      return ((alw >> bit) & 1ull) ? x : -INFINITY;
    }
    return x;
  };
  // score r of tile t of the chunk being weighed: tile 0 from the matrix-core output,
  // tile 1 from the copy
  auto score = [&](int t, int r, uint64_t alw, auto MK) -> float {
    return masked(t ? scp[r] : sacc[0][r], t, r, alw, MK);
  };
  auto copy_hi = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) scp[r] = sacc[1][r];
  };
  // S^T of the chunk in LDS stage `stage` into sacc (no overlap)
  auto scores_of = [&](int stage) {
    const uint8_t* Ks = xs + stage * WSTAGE + l32 * XROW;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
    for (int f = 0; f < KSTEPS; ++f)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        sacc[t] = mfma32(*(const bf16x8*)(Ks + 32 * t * XROW + 16 * ((2 * f + half) ^ kx)), qf[f],
                         sacc[t]);
  };
  // row max (scale*log2e units, both lanes of a row) of chunk cidx's scores in sacc
  auto chunk_max = [&](int cidx) -> float {
    const uint64_t alw = mask_bits(cidx);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, masked(sacc[t][r], t, r, alw, std::true_type{}));
    return fmaxf(mx, __shfl_xor(mx, 32)) * c;
  };

  // One pipeline iteration.  MK: chunk j or j+1 reaches past mask_from; LAST: j =
  // n-1, no chunk j+1.  Fragments 0-15 are K of chunk j+1 (tile f%2, k-step f/2: the
  // two tiles' accumulation chains alternate), 16-31 V^T of chunk j (16-key step
  // (f-16)/4, dim tile (f-16)%4).
  auto iteration = [&](int j, auto MK, auto LASTT) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(LASTT)::value;
    constexpr bool MASK = decltype(MK)::value;
    const uint8_t* Ks = xs + ((j + 1) % WNB) * WSTAGE + l32 * XROW;
    const int m = lane & 15;
    const uint8_t* vp = xs + (j % WNB) * WSTAGE + WHALF + (4 * half + (m >> 2)) * XROW + 8 * (m & 1);
    const int vcol = 2 * ((lane >> 4) & 1) + ((m & 3) >> 1);
    const int vx = 4 * (m >> 2);
    auto frag = [&](int f) -> bf16x8 {
      if (f < 16) {
        const int t = f & 1, sk = f >> 1;
        return *(const bf16x8*)(Ks + 32 * t * XROW + 16 * ((2 * sk + half) ^ kx));
      }
      const int cc = (f - 16) >> 2, db = (f - 16) & 3;
      const uint8_t* p0 = vp + 16 * cc * XROW + 16 * ((4 * db + vcol) ^ vx);
      const v4i16 both[2] = {lds_read_tr(p0), lds_read_tr(p0 + 8 * XROW)};
      return __builtin_bit_cast(bf16x8, both);
    };
    const uint64_t alw_j = MASK ? mask_bits(j) : ~0ull;
    const uint64_t alw_n = (MASK && !LAST) ? mask_bits(j + 1) : ~0ull;
    constexpr int F0 = LAST ? 16 : 0;
    constexpr int LA = 4;
    bf16x8 ring[LA];
    static_for<LA>([&](auto I) { ring[(F0 + I) % LA] = frag(F0 + I); });
    float xa[8][2], ex[8][2];
    // pair p (scores 2p, 2p+1 of tile t): A scale and shift, B exponentials, C bf16
    // pack (into the P^T operand of 16-key step 2t + p/4) and row sum
    auto stepA = [&](int t, int p, uint64_t alw) {
      xa[p][0] = fmaf(score(t, 2 * p, alw, MK), c, -mref);
      xa[p][1] = fmaf(score(t, 2 * p + 1, alw, MK), c, -mref);
    };
    auto stepB = [&](int p) {
      ex[p][0] = __builtin_amdgcn_exp2f(xa[p][0]);
      ex[p][1] = __builtin_amdgcn_exp2f(xa[p][1]);
    };
    auto stepC = [&](int t, int p) {
      pk[2 * t + (p >> 2)][p & 3] = pack_bf16x2(ex[p][0], ex[p][1]);
      part[p & 3] += ex[p][0] + ex[p][1];
    };
    // slot s of a region (16 slots) for the 8 pairs of tile t: A of pair s/2 (even s),
    // B of pair (s-1)/2 (odd s), C of pair s/2-1 (even s >= 2); C of pair 7 follows
    auto steps = [&](auto S, int t, uint64_t alw) {
      constexpr int s = S;
      if constexpr (s % 2 == 0) stepA(t, s / 2, alw);
      if constexpr (s % 2 == 1) stepB((s - 1) / 2);
      if constexpr (s % 2 == 0 && s >= 2) stepC(t, s / 2 - 1);
    };
    // region 1: scores of chunk j+1, tile 1 of chunk j
    static_for<16>([&](auto S) {
      constexpr int s = S;
      if constexpr (!LAST) {
        constexpr int t = s & 1, sk = s >> 1;
        if constexpr (s == 0) {   // tile 0 of chunk j was weighed, tile 1 copied
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[tt][r] = 0.f;
        }
        sacc[t] = mfma32(ring[s % LA], qf[sk], sacc[t]);
        ring[s % LA] = frag(s + LA);
      }
      steps(S, 1, alw_j);
      __builtin_amdgcn_sched_barrier(0);
    });
    stepC(1, 7);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pf[cc] = as_bf16x8(pk[cc]);
    if constexpr (!LAST) copy_hi();
    // region 2: output of chunk j, tile 0 of chunk j+1
    static_for<16>([&](auto S) {
      constexpr int s = S;
      constexpr int f = 16 + s;
      constexpr int cc = s >> 2, db = s & 3;
      oacc[db] = mfma32(ring[f % LA], pf[cc], oacc[db]);
      if constexpr (f + LA < 32) ring[f % LA] = frag(f + LA);
      if constexpr (!LAST) steps(S, 0, alw_n);
      if constexpr (!LAST && f + LA == 32) sync();   // after this wave's last LDS read
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!LAST) stepC(0, 7);
  };

  // One walk over the split with the reference max fixed (EXACT: mref already holds
  // the exact row max; else it is taken from chunk 0); ACTIVE false: the DMAs and
  // barriers only.  On entry chunks 0 .. WNB-1 are issued and chunks 0, 1 visible to
  // all waves; on exit no DMA is in flight.
  auto walk = [&](auto EXACT, auto ACTIVE) __attribute__((always_inline)) {
    constexpr bool ACT = decltype(ACTIVE)::value;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] = 0.f;
    // prologue: scores of chunk 0, the reference max, the weights of its tile 0
    if constexpr (ACT) {
      scores_of(0);
      if constexpr (!decltype(EXACT)::value) mref = chunk_max(0);
      copy_hi();
      const uint64_t alw0 = mask_bits(0);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(score(0, 2 * p, alw0, std::true_type{}), c, -mref));
        const float e1 =
            __builtin_amdgcn_exp2f(fmaf(score(0, 2 * p + 1, alw0, std::true_type{}), c, -mref));
        pk[p >> 2][p & 3] = pack_bf16x2(e0, e1);
        part[p & 3] += e0 + e1;
      }
    }
    // iteration j: chunks up to j+WNB-1 are issued and chunks j, j+1 visible to all
    // waves; the DMA of chunk j+WNB is issued after the iteration's work, so the
    // waves go from one iteration's MFMAs straight into the next's.  Iterations whose
    // chunks j, j+1 need no mask come first: chunk c needs none when key_begin +
    // (c+1)*WC <= mask_from.
    const int jm = min(max((mask_from - key_begin) / WC - 1, 0), n - 1);
    auto step = [&](int j, auto MK, auto FAST) __attribute__((always_inline)) {
      if constexpr (ACT)
        iteration(j, MK, std::false_type{});
      else
        sync();
      issue(j + WNB, FAST);
    };
    // iterations below jf run two per pass, so the tile-1 scores one iteration hands
    // to the next alternate between two register sets instead of being copied.  In
    // the contiguous cache the chunk each of them issues lies wholly at or below kmax
    // (the paged issue clamps every row anyway, so there jf = jm).
    const int nfull = (kmax + 1 - key_begin) / WC;
    const int jf = PAGED ? jm : min(jm, max(0, nfull - WNB));
    int j = 0;
    for (; j + 1 < jf; j += 2) {
      step(j, std::false_type{}, std::true_type{});
      step(j + 1, std::false_type{}, std::true_type{});
    }
    for (; j < jm; ++j) step(j, std::false_type{}, std::false_type{});
    for (; j < n - 1; ++j) step(j, std::true_type{}, std::false_type{});
    if constexpr (ACT) iteration(n - 1, std::true_type{}, std::true_type{});
    wait_vmcnt<0>();   // no DMA may still write this workgroup's LDS past this point
  };

  float lsum = 0.f;
  if (n > 0) {
    if (busy)
      walk(std::false_type{}, std::true_type{});
    else
      walk(std::false_type{}, std::false_type{});
    lsum = (part[0] + part[1]) + (part[2] + part[3]);
    const bool big = !((lsum + __shfl_xor(lsum, 32)) <= kRowSumLimit);
    if (__ballot(big) && lane == 0) atomicOr(&redo, 1);
    __syncthreads();   // every wave is past its last LDS read, and redo is final
    if (redo) {
      // exact row max over the split (scores only, one chunk in flight ahead), then
      // the walk again with it
      mref = -INFINITY;
      issue(0, std::false_type{});
      for (int cidx = 0; cidx < n; ++cidx) {
        issue(cidx + 1, std::false_type{});
        wait_vmcnt<4>();
        __syncthreads();
        if (busy) {
          scores_of(cidx % WNB);
          mref = fmaxf(mref, chunk_max(cidx));
        }
        __syncthreads();
      }
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int cidx = 0; cidx < WNB; ++cidx) issue(cidx, std::false_type{});
      wait_vmcnt<4 * (WNB - 2)>();
      __syncthreads();
      if (busy)
        walk(std::true_type{}, std::true_type{});
      else
        walk(std::true_type{}, std::false_type{});
      lsum = (part[0] + part[1]) + (part[2] + part[3]);
    }
  } else {
    mref = -INFINITY;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (r_row >= R) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse = (mref + log2f(ltot)) * kLn2;
  const int il = r_row / G;
  const int i = pl.node0 + il;
  const int h = g * G + (r_row - il * G);
  if (pl.S == 1 && !pl.dplan) {
    uint16_t* op = out + ((size_t)(b * pl.N + i) * pl.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * db + 8 * jj + 4 * half;
        u32x2 pk2;
        pk2[0] = pack_bf16x2(oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv);
        pk2[1] = pack_bf16x2(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
        *(u32x2*)(op + d0) = pk2;
      }
    if (half == 0 && lse_out) lse_out[(size_t)(b * pl.N + i) * pl.Hq + h] = lse;
  } else {
    const size_t prow = (size_t)item.slot * pl.Rpad + r_row;
    float* op = part_o + prow * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * db + 8 * jj + 4 * half;
        f32x4 vv = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv, oacc[db][4 * jj + 2] * inv,
                    oacc[db][4 * jj + 3] * inv};
        *(f32x4*)(op + d0) = vv;
      }
    if (half == 0) part_lse[prow] = lse;
  }
}

template <bool PAGED>
hipError_t launch_d128(const AttnPlan& pl, const void* q, const void* k, const void* v,
                       const int32_t* parents, void* out, float* lse, float* part_o,
                       float* part_lse, hipStream_t stream) {
  // once per process; function-local static initialisation is thread-safe
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)tree_attn_d128<PAGED>, hipFuncAttributeMaxDynamicSharedMemorySize, WLDS);
  if (attr != hipSuccess) return attr;
  const int nwg = pl.B * pl.Hkv * pl.RB * pl.S;
  hipLaunchKernelGGL(tree_attn_d128<PAGED>, dim3(nwg), dim3(512), WLDS, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, parents, pl,
                     (uint16_t*)out, lse, part_o, part_lse);
  return hipGetLastError();
}

template <int D, int WAVES>
hipError_t launch_fwd(const AttnPlan& pl, const void* q, const void* k, const void* v,
                      const int32_t* parents, void* out, float* lse, float* part_o,
                      float* part_lse, hipStream_t stream) {
  const int nwg = pl.B * pl.Hkv * pl.RB * pl.S;
  if (pl.block_table)
    hipLaunchKernelGGL((tree_attn_fwd<D, WAVES, true>), dim3(nwg), dim3(WAVES * 64), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, parents,
                       pl, (uint16_t*)out, lse, part_o, part_lse);
  else
    hipLaunchKernelGGL((tree_attn_fwd<D, WAVES, false>), dim3(nwg), dim3(WAVES * 64), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, parents,
                       pl, (uint16_t*)out, lse, part_o, part_lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const AttnPlan& pl, const void* q, const void* k, const void* v,
                        const int32_t* parents, void* out, float* lse, float* part_o,
                        float* part_lse, hipStream_t stream) {
  if constexpr (D == 128) {   // every D = 128 plan has eight waves (plan_tree_attn_rows)
    if (pl.waves != 8) return hipErrorInvalidValue;
    if (pl.block_table)
      return launch_d128<true>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream);
    return launch_d128<false>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream);
  } else {   // D = 64: at most four waves (chunk staging must divide evenly)
    if (pl.waves == 4) return launch_fwd<D, 4>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream);
    if (pl.waves == 2) return launch_fwd<D, 2>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream);
    return launch_fwd<D, 1>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream);
  }
}

}  // namespace

AttnPlan plan_tree_attn(int B, int N, int Hq, int Hkv, int D, int P, int kv_cap) {
  return plan_tree_attn_rows(B, N, 0, 0, Hq, Hkv, D, P, kv_cap);
}

// Nodes node0 .. node0+nq-1 of an N-node tree (nq = 0: all N); the rows, row blocks and
// splits follow the queried rows.
AttnPlan plan_tree_attn_rows(int B, int N, int node0, int nq, int Hq, int Hkv, int D, int P,
                             int kv_cap) {
  AttnPlan pl{};
  pl.B = B;
  pl.N = N;
  pl.Hq = Hq;
  pl.Hkv = Hkv;
  pl.G = Hq / Hkv;
  pl.D = D;
  pl.P = P;
  pl.kv_cap = kv_cap;
  pl.node0 = nq > 0 ? node0 : 0;
  pl.nq = nq > 0 ? nq : 0;
  pl.R = (nq > 0 ? nq : N) * pl.G;
  // 32 rows per wave (one MFMA row tile); D = 64 uses at most 4 waves (its chunk
  // staging must divide evenly over the threads)
  const int wave_rows = 32;
  const int max_waves = D == 64 ? 4 : 8;
  pl.waves = 1;
  while (pl.waves < max_waves && pl.waves * wave_rows < pl.R) pl.waves *= 2;
  // D = 128 always takes the eight-wave kernel, also for 128 rows or fewer: its waves
  // past the rows only move K and V, and its four 64-key LDS stages keep more of the
  // stream in flight than the narrow kernels' two-chunk register ring (the draft
  // expansion's 80-row queries 114 -> 108 us, its 8-row ones 102 -> 93 us, C2's 26
  // rows 16.7 -> 14.9 us); the narrow kernels serve D = 64
  if (D == 128) pl.waves = 8;
  pl.RB = (pl.R + pl.waves * wave_rows - 1) / (pl.waves * wave_rows);
  pl.Rpad = pl.RB * pl.waves * wave_rows;
  // About one workgroup per CU for the eight-wave kernel; the narrower ones (head dim
  // 64) get three (one wave) or two (two or four waves) per CU, so that every SIMD
  // streams keys with a second wave beside it (the LDS of three fits in a CU); more
  // splits than that cost more in the merge.
  const long long units = (long long)B * Hkv * pl.RB;
  const int wg_per_cu = pl.waves == 1 ? 3 : (pl.waves == 2 || pl.waves == 4 ? 2 : 1);
  int s_target = (int)(((long long)kNumCUs * wg_per_cu + units - 1) / units);
  int s_max = P / min_split_keys(pl.waves);
  int S = s_target < s_max ? s_target : s_max;
  if (S < 1) S = 1;
  if (P <= 0) {
    S = 1;
    pl.split_len = 0;
  } else {
    int len = (P + S - 1) / S;
    len = (len + KC - 1) / KC * KC;
    S = (P + len - 1) / len;
    pl.split_len = len;
  }
  pl.S = S;
  return pl;
}

// Paged KV: as plan_tree_attn, with more splits where a split's slice of the block
// table would not fit the LDS table (rows of one split plus two chunks of prefetch).
AttnPlan plan_tree_attn_paged(int B, int N, int Hq, int Hkv, int D, int P, int page_shift) {
  AttnPlan pl = plan_tree_attn(B, N, Hq, Hkv, D, P, P + N);
  auto fits = [&](int len, int S) {
    const int last_range = (P - (S - 1) * len) + N;   // the last split also has the tree
    const int range = (len > last_range ? len : last_range) + 2 * KC;
    return (range >> page_shift) + 2 <= kMaxSplitPages;
  };
  while (P > 0 && !fits(pl.split_len, pl.S) && pl.split_len > KC) {
    int len = ((pl.split_len / 2) + KC - 1) / KC * KC;
    pl.S = (P + len - 1) / len;
    pl.split_len = len;
  }
  pl.page_shift = page_shift;
  return pl;
}

// split partials (fp32 O rows and lse) and, after them, the ragged batches' item table
static size_t plan_table_offset(const AttnPlan& pl) {
  const size_t rows = (size_t)pl.B * pl.Hkv * pl.S * pl.Rpad;
  return (rows * (size_t)pl.D * sizeof(float) + rows * sizeof(float) + 255) / 256 * 256;
}

size_t tree_attn_workspace_bytes(const AttnPlan& pl) {
  if (pl.S <= 1) return 0;
  return plan_table_offset(pl) + (size_t)(2 + 2 * pl.B) * sizeof(int) + 256;
}

hipError_t launch_tree_attn(const AttnPlan& pl0, float scale, const void* q, const void* k,
                            const void* v, const int32_t* parents, void* out, float* lse,
                            void* workspace, hipStream_t stream) {
  AttnPlan pl = pl0;
  pl.c = scale * kLog2e;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (pl.S > 1) {
    const size_t rows = (size_t)pl.B * pl.Hkv * pl.S * pl.Rpad;
    part_o = (float*)workspace;
    part_lse = part_o + rows * pl.D;
    // ragged prefixes: split lengths from the real prefix lengths, chosen by the
    // attention workgroups themselves (planned_item); the table goes to the merge
    if (pl.prefix_len && !pl.block_table && pl.nq == 0)
      pl.dplan = (int*)((char*)workspace + plan_table_offset(pl));
  }
  const hipError_t e =
      pl.D == 128 ? launch_fwd_d<128>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream)
                  : launch_fwd_d<64>(pl, q, k, v, parents, out, lse, part_o, part_lse, stream);
  if (e != hipSuccess || pl.S == 1) return e;
  const int rows = pl.B * pl.Hkv * pl.R;
  const int blocks = (rows + 3) / 4;
  if (pl.D == 128)
    hipLaunchKernelGGL(tree_attn_merge_hw, dim3((rows + 7) / 8), dim3(256), 0, stream, pl, part_o,
                       part_lse, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL(tree_attn_merge<64>, dim3(blocks), dim3(256), 0, stream, pl, part_o, part_lse,
                       (uint16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace eagle
