// Acceptance of a verified draft tree: greedy and multi-round speculative sampling.
#include "common.h"
#include "internal.h"

namespace eagle {

namespace {

// ---------------------------------------------------------------------------
// Greedy.  [P1] greedy decoding paragraph (match the target's top-1 from the first
// draft on, cut at the first mismatch) and [P2] speculative sampling paragraph
// (alpha accepted drafts give alpha + 1 tokens).  One wave per sequence, lane i =
// node i: each lane walks its root path (at most 64 links, stopping at any link
// that breaks the tree rules) to get its depth and whether every edge matches.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
accept_greedy_kernel(const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
                     const int32_t* __restrict__ top1, const int32_t* __restrict__ tree_len, int B,
                     int N, int max_depth, int32_t* __restrict__ accept_len,
                     int32_t* __restrict__ accept_path, int32_t* __restrict__ out_tokens) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (b >= B) return;
  const int32_t* tok = tokens + (size_t)b * N;
  const int32_t* par = parents + (size_t)b * N;
  const int32_t* am = top1 + (size_t)b * N;
  // ragged batches: nodes past this sequence's tree do not exist
  const int Nb = tree_len ? min(max(tree_len[b], 1), N) : N;

  int key = -1;
  if (lane < Nb) {
    bool ok = true;
    bool reached = (lane == 0);
    int depth = 0;
    int n = lane;
    for (int step = 0; step < 64 && n > 0; ++step) {
      const int p = par[n];
      if (p < 0 || p >= n) {
        ok = false;
        break;
      }
      if (tok[n] != am[p]) ok = false;
      ++depth;
      n = p;
      if (n == 0) reached = true;
    }
    if (ok && reached && depth <= max_depth) key = depth * 64 + (63 - lane);
  }
  const int best = wave_max_i(key);   // >= 63: the root always qualifies
  const int vstar = 63 - (best & 63);
  const int alpha = best >> 6;

  const int cap = max_depth + 1;
  int32_t* path_out = accept_path + (size_t)b * cap;
  int32_t* tok_out = out_tokens + (size_t)b * cap;
  for (int j = lane; j < cap; j += 64) {
    if (j <= alpha) {
      int n = vstar;
      for (int s = 0; s < alpha - j; ++s) n = par[n];   // the node at depth j on the path
      path_out[j] = n;
      if (j < alpha) {
        int c = vstar;
        for (int s = 0; s < alpha - j - 1; ++s) c = par[c];   // the node at depth j + 1
        tok_out[j] = tok[c];
      } else {
        tok_out[j] = am[vstar];
      }
    } else {
      path_out[j] = -1;
      tok_out[j] = -1;
    }
  }
  if (lane == 0) accept_len[b] = alpha;
}

// ---------------------------------------------------------------------------
// Multi-round speculative sampling.  [P1] stochastic verification paragraph (q
// target, p draft; accept below min(1, q/p), else resample from the corrected
// distribution), [P2] multi-round speculative sampling section (the recursive
// tree form), [P3] section 2 (rejection sampling keeps the output law).
//
// Closed form used on the device.  With q the target and p the draft at the current
// node, after j rejections the corrected target is
//     q_j = max(0, q - c_j p) / S(c_j),  S(c) = sum_x max(0, q(x) - c p(x)),
// with c_0 = 0 and c_{j+1} = c_j + S(c_j): one rejection maps max(0, q - c p)/S to
// the normalised positive part of (that - p), which is max(0, q - (c + S) p) up to
// its normaliser.  So each rejection round is one vocabulary reduction of
// max(0, q - c p) with the next c, and the acceptance ratio of token t is
// max(0, q(t) - c p(t)) / (S p(t)).  All of it runs in fp64 on fp64 q and p.
//
// Deterministic siblings (point-mass mode, EAGLE-2's top-k expansion): the draft
// distribution behind child t is the point mass at t, so the same rule accepts t when
// u < q'(t) = q(t) / (1 - removed mass) and a rejection removes q(t) from q'.  Those
// decisions need no vocabulary pass; the final draw is from q with the removed tokens
// zeroed.
//
// Parallel layout.  Each sequence gets `chunks` workgroups, each owning a contiguous
// slice of the vocabulary.  Every workgroup follows the same control flow; the
// vocabulary reductions are exchanged through the workspace in self-validating
// words (each 64-bit word carries the exchange's generation next to 32 bits of a
// partial), so a reader needs no separate arrival counter or ordering wait: it polls
// the words themselves.  Every spin is bounded: on timeout the sequence's accept_len
// is set to -1 and all its workgroups leave; the last workgroup of a sequence to
// leave writes its outputs (an exit counter in the workspace).
// ---------------------------------------------------------------------------
constexpr int kSpecThreads = 256;
constexpr int kSpecRegs = 16;   // entries per thread kept in registers
constexpr int kSpecChunk = kSpecThreads * kSpecRegs;   // planned vocabulary entries per workgroup
constexpr unsigned kSpinLimit = 1u << 24;

struct SpecWs {
  unsigned* exits;      // [B] workgroups of the sequence that have finished (+ abort bit)
  int* abort_flags;     // [B]
  unsigned long long* slots;   // [B][2][chunks][8] tagged halves of the exchanged partials
  double* qbuf;         // [B][V] fp64 q of the current node
  double* pbuf;         // [B][V] fp64 p of the current node
};

// exits[b]: low 16 bits count the workgroups of sequence b that are done, bit 16 is set
// by any workgroup that gave up on a spin
constexpr unsigned kExitAbortBit = 1u << 16;

__device__ __forceinline__ SpecWs spec_ws(void* ws, int B, int chunks, int V) {
  SpecWs w;
  char* base = (char*)ws;
  w.exits = (unsigned*)base;
  w.abort_flags = (int*)(base + 256 * ((B * 4 + 255) / 256));
  size_t off = 2 * 256 * (size_t)((B * 4 + 255) / 256);
  w.slots = (unsigned long long*)(base + off);
  off += (size_t)B * 2 * chunks * 8 * sizeof(unsigned long long);
  off = (off + 255) / 256 * 256;
  w.qbuf = (double*)(base + off);
  off += (size_t)B * V * sizeof(double);
  w.pbuf = (double*)(base + off);
  return w;
}

// Clears the exit counters, abort flags and exchange tags of every sequence; a grid of
// enough workgroups that each thread clears a few words.
__global__ void __launch_bounds__(256) spec_init_kernel(void* ws, int B, int chunks, int V) {
  SpecWs w = spec_ws(ws, B, chunks, V);
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < B; i += stride) {
    w.exits[i] = 0u;
    w.abort_flags[i] = 0;
  }
  // generation tags start at 0: no word left by an earlier call can look current
  const int nslot = B * 2 * chunks * 8;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nslot; i += stride) w.slots[i] = 0ull;
}

// Workgroup-wide sum of a double (all threads get the result).
__device__ __forceinline__ double wg_sum_d(double x, double* red) {
  x = wave_sum_d(x);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kSpecThreads / 64; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ double wg_max_d(double x, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int i = 1; i < kSpecThreads / 64; ++i) t = fmax(t, red[i]);
  return t;
}

// Waits until the exchange word *p carries `tag` in its high half and returns the word in
// `out`.  Gives up (false) once the sequence's abort flag is set, or after kSpinLimit
// polls, when it sets that flag itself.
__device__ __forceinline__ bool poll_word(const unsigned long long* p, unsigned tag, int* abort_flag,
                                          unsigned long long& out) {
  unsigned spins = 0;
  for (;;) {
    const unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((unsigned)(v >> 32) == tag) {
      out = v;
      return true;
    }
    if ((++spins & 63u) == 0u && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      return false;
    if (spins > kSpinLimit) {
      __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Publish this workgroup's first nv partials (of 4) for generation `gen`, wait for
// every chunk of the sequence, and return the chunk-ordered partials in
// lds_all[chunks][4] (entries k < nv).  Returns false on timeout.
//
// A double is sent as two 64-bit words: generation + 1 in the high 32 bits, one half
// of the double in the low 32 bits.  64-bit stores and loads are single-copy atomic,
// so a word whose tag matches holds that half of this generation's value, whatever
// order the words become visible in: readers poll the words directly (relaxed
// agent-scope atomics, coherent across the XCDs' L2 caches) and write the halves
// straight into lds_all, which is the little-endian layout of the doubles.  The two
// buffers alternate by generation; a workgroup can only write generation g + 2 after
// every workgroup has written g + 1, i.e. after all of them have read g.
__device__ bool exchange(const SpecWs& w, int b, int chunks, int me, unsigned gen, int nv,
                         const double (&mine)[4], double* lds_all, int* lds_flag) {
  unsigned long long* slot = w.slots + (((size_t)b * 2 + (gen & 1)) * chunks) * 8;
  const unsigned tag = gen + 1;
  const int nw = 2 * nv;
  if (threadIdx.x < nw) {
    const int k = threadIdx.x >> 1;
    const double val = k == 0 ? mine[0] : (k == 1 ? mine[1] : (k == 2 ? mine[2] : mine[3]));
    const unsigned long long bits = (unsigned long long)__double_as_longlong(val);
    const unsigned half = (threadIdx.x & 1) ? (unsigned)(bits >> 32) : (unsigned)bits;
    __hip_atomic_store(&slot[me * 8 + threadIdx.x], ((unsigned long long)tag << 32) | half,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) *lds_flag = 1;
  __syncthreads();   // lds_flag set; every thread is done with the previous lds_all
  bool ok = true;
  unsigned* words = (unsigned*)lds_all;
  for (int i = threadIdx.x; i < chunks * nw; i += blockDim.x) {
    const int c = i / nw, k = i - c * nw;
    unsigned long long v;
    if (!poll_word(&slot[c * 8 + k], tag, &w.abort_flags[b], v)) {
      ok = false;
      break;
    }
    words[c * 8 + k] = (unsigned)v;
  }
  if (!ok) *lds_flag = 0;
  __syncthreads();
  return *lds_flag != 0;
}

// Sum of one double over the workgroups of a sequence: the workgroup's part (summed over
// its waves in wave order) is published through exchange words as in exchange(), and
// every workgroup adds the chunks' parts in chunk order, so all of them hold the same
// sum.  Two workgroup barriers in all.  Returns false on timeout.
__device__ bool exchange_sum(const SpecWs& w, int b, int chunks, int me, unsigned gen, double part,
                             double* red, double* lds_all, int* lds_flag, double& out) {
  part = wave_sum_d(part);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = part;
  if (threadIdx.x == 0) *lds_flag = 1;
  __syncthreads();   // red complete; every thread is done with the previous lds_all
  unsigned long long* slot = w.slots + (((size_t)b * 2 + (gen & 1)) * chunks) * 8;
  const unsigned tag = gen + 1;
  if (threadIdx.x < 2) {
    double s = red[0];
#pragma unroll
    for (int i = 1; i < kSpecThreads / 64; ++i) s += red[i];
    const unsigned long long bits = (unsigned long long)__double_as_longlong(s);
    const unsigned half = threadIdx.x ? (unsigned)(bits >> 32) : (unsigned)bits;
    __hip_atomic_store(&slot[me * 8 + threadIdx.x], ((unsigned long long)tag << 32) | half,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  bool ok = true;
  unsigned* words = (unsigned*)lds_all;
  for (int i = threadIdx.x; i < chunks * 2; i += blockDim.x) {
    const int c = i >> 1, k = i & 1;
    unsigned long long v;
    if (!poll_word(&slot[c * 8 + k], tag, &w.abort_flags[b], v)) {
      ok = false;
      break;
    }
    words[c * 8 + k] = (unsigned)v;
  }
  if (!ok) *lds_flag = 0;
  __syncthreads();
  if (*lds_flag == 0) return false;
  double s = 0.0;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) s += lds_all[4 * c];
  out = s;
  return true;
}

// REGS: every chunk of the plan has at most kSpecRegs * kSpecThreads entries.  Each
// thread then owns the contiguous entries [t0, t1) of its workgroup's chunk and keeps q
// and p of the current node in registers from the logits load to the final draw; the
// workspace copies of q and p are not used.  Otherwise q and p go through the workspace
// (strided passes; the draw walks the same contiguous ranges).
template <bool REGS>
__global__ void __launch_bounds__(kSpecThreads) __attribute__((amdgpu_waves_per_eu(2)))
accept_spec_kernel(const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
                   const int32_t* __restrict__ draft_row, const float* __restrict__ target_logits,
                   const float* __restrict__ draft_logits, const float* __restrict__ u_accept,
                   const float* __restrict__ u_sample, SpecPlan pl, int32_t* __restrict__ accept_len,
                   int32_t* __restrict__ accept_path, int32_t* __restrict__ out_tokens, void* ws) {
  __shared__ double lds_all[4 * 64];
  __shared__ double red[kSpecThreads / 64];
  __shared__ int lds_flag;
  __shared__ int kids[64];
  __shared__ int nkids_s;
  __shared__ double cterm[128];   // per-chunk softmax terms: q in [0, 64), p in [64, 128)
  // per child (in sibling order): token, q and p of its token, its uniform
  __shared__ int kid_tok[64];
  __shared__ double kid_q[64], kid_p[64];
  __shared__ float kid_u[64];
  __shared__ unsigned long long kid_same[64];   // bit i: child i < j carries child j's token
  __shared__ int path_s[65];
  __shared__ double wtot_s[kSpecThreads / 64];   // draw: wave totals of the residual mass
  __shared__ int wlast_s[kSpecThreads / 64];
  __shared__ int found_s;
  __shared__ int tok_s[64];   // every node's token (the children's are read from here)

  const int chunks = pl.chunks;
  const int b = blockIdx.x / chunks;
  const int me = blockIdx.x % chunks;
  const int N = pl.N, V = pl.V;
  const int chunk_len = (V + chunks - 1) / chunks;
  const int x0 = me * chunk_len;
  const int x1 = min(V, x0 + chunk_len);
  // the thread's contiguous entries [t0, t1) (at most kSpecRegs of them when REGS)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int per = (max(0, x1 - x0) + kSpecThreads - 1) / kSpecThreads;
  const int t0 = x0 + tid * per;
  const int t1 = min(x1, t0 + per);
  SpecWs w = spec_ws(ws, pl.B, chunks, V);
  double* qb = w.qbuf + (size_t)b * V;
  double* pb = w.pbuf + (size_t)b * V;
  const int32_t* tok = tokens + (size_t)b * N;
  const int32_t* par = parents + (size_t)b * N;
  // ragged batches: nodes past this sequence's tree do not exist
  const int Nb = pl.tree_len ? min(max(pl.tree_len[b], 1), N) : N;
  const bool pm = pl.mode != 0;   // deterministic siblings (point-mass draft per child)

  unsigned gen = 0;
  int v = 0;
  int alpha = 0;
  if (tid == 0) path_s[0] = 0;
  bool aborted = false;

  double sample_c = 0.0;   // corrected target for the final draw: max(0, q - c p) / S
  double fallback_c = 0.0; // the previous c, should the residual at sample_c be empty
  int sample_node = 0;
  double qr[kSpecRegs], pr[kSpecRegs];   // REGS: q, p of entries t0 + i (0 past t1)
  // the tree's tokens, read once (published by the first barrier of the node loop)
  if (tid < 64) tok_s[tid] = tid < Nb ? tok[tid] : -1;

  for (;;) {
    const size_t node = (size_t)b * N + v;
    const int row = draft_row[node];
    const bool row_ok = row >= 0 && row < pl.R;
    const float* tl = target_logits + node * V;
    const float* dl = draft_logits + ((size_t)b * pl.R + (row_ok ? row : 0)) * V;
    // the node's logits are requested before its children are known, so that their
    // latency overlaps the tree walk (the draft row only when the node has one)
    float tr[kSpecRegs], dr[kSpecRegs];
    if constexpr (REGS) {
#pragma unroll
      for (int i = 0; i < kSpecRegs; ++i) {
        const int x = t0 + i;
        tr[i] = x < t1 ? tl[x] : 0.f;
        dr[i] = (x < t1 && row_ok && !pm) ? dl[x] : 0.f;
      }
    }
    const float lse_t = pl.target_lse ? pl.target_lse[node] : 0.f;
    const float lse_d = (pl.draft_lse && row_ok && !pm) ? pl.draft_lse[(size_t)b * pl.R + row] : 0.f;
    // children of v in ascending index (none at max_depth)
    if (tid < 64) {
      const bool is_kid = tid < Nb && tid > 0 && par[tid] == v && alpha < pl.max_depth;
      const unsigned long long mask = __ballot(is_kid);
      if (is_kid) kids[__popcll(mask & ((1ull << tid) - 1ull))] = tid;
      if (tid == 0) nkids_s = __popcll(mask);
    }
    __syncthreads();
    const int nk = nkids_s;
    const bool has_draft = nk > 0 && row_ok;
    const bool need_p = has_draft && !pm;   // children tried against the draft distribution
    // the children's tokens and logits, loaded here so that their latency overlaps the
    // softmax below instead of sitting in every rejection round
    int ktok = -1;
    float ktl = 0.f, kdl = 0.f;
    if (tid < nk) {
      const int kid = kids[tid];
      const int t = tok_s[kid];
      if (t >= 0 && t < V) {
        ktok = t;
        ktl = tl[t];
        kdl = need_p ? dl[t] : 0.f;
      }
      kid_tok[tid] = ktok;
      kid_u[tid] = u_accept[(size_t)b * N + kid];
    }

    // ---- q and p of node v.  With the caller's normalisers (target_lse, and draft_lse
    // when the children are tried against the draft distribution) every value is
    // exp(logit - lse) at once; otherwise the chunk max and exp-sum are exchanged first
    // and the normalisers formed from them.
    const bool given = pl.target_lse != nullptr && (!need_p || pl.draft_lse != nullptr);
    double lse_q = 0.0, lse_p = 0.0;
    if (given) {
      lse_q = (double)lse_t;
      if (need_p) lse_p = (double)lse_d;
      if constexpr (REGS) {
#pragma unroll
        for (int i = 0; i < kSpecRegs; ++i) {
          const bool in = t0 + i < t1;
          qr[i] = in ? exp((double)tr[i] - lse_q) : 0.0;
          pr[i] = (in && need_p) ? exp((double)dr[i] - lse_p) : 0.0;
        }
      } else {
        for (int x = x0 + tid; x < x1; x += kSpecThreads) {
          qb[x] = exp((double)tl[x] - lse_q);
          if (!pm) pb[x] = need_p ? exp((double)dl[x] - lse_p) : 0.0;
        }
      }
    } else {
      double mq = -INFINITY, mp = -INFINITY;
      if constexpr (REGS) {
#pragma unroll
        for (int i = 0; i < kSpecRegs; ++i) {
          if (t0 + i < t1) {
            mq = fmax(mq, (double)tr[i]);
            if (need_p) mp = fmax(mp, (double)dr[i]);
          }
        }
      } else {
        for (int x = x0 + tid; x < x1; x += kSpecThreads) {
          mq = fmax(mq, (double)tl[x]);
          if (need_p) mp = fmax(mp, (double)dl[x]);
        }
      }
      mq = wg_max_d(mq, red);
      if (need_p) mp = wg_max_d(mp, red);
      double zq = 0.0, zp = 0.0;
      if constexpr (REGS) {
        // exp(x - chunk max) stays in qr / pr; scaled to q / p once the totals are known
#pragma unroll
        for (int i = 0; i < kSpecRegs; ++i) {
          const bool in = t0 + i < t1;
          qr[i] = in ? exp((double)tr[i] - mq) : 0.0;
          pr[i] = (in && need_p) ? exp((double)dr[i] - mp) : 0.0;
          zq += qr[i];
          zp += pr[i];
        }
      } else {
        for (int x = x0 + tid; x < x1; x += kSpecThreads) {
          zq += exp((double)tl[x] - mq);
          if (need_p) zp += exp((double)dl[x] - mp);
        }
      }
      zq = wg_sum_d(zq, red);
      if (need_p) zp = wg_sum_d(zp, red);
      {
        const double mine[4] = {mq, zq, mp, zp};
        if (!exchange(w, b, chunks, me, gen++, 4, mine, lds_all, &lds_flag)) { aborted = true; break; }
      }
      double Mq = -INFINITY, Mp = -INFINITY;
      for (int c = 0; c < chunks; ++c) {
        Mq = fmax(Mq, lds_all[4 * c]);
        Mp = fmax(Mp, lds_all[4 * c + 2]);
      }
      // chunk terms: one exponential per lane, then summed in chunk order by every
      // thread (an empty chunk adds +0.0, which leaves the sum unchanged)
      if (tid < chunks) {
        cterm[tid] = lds_all[4 * tid] > -INFINITY ? lds_all[4 * tid + 1] * exp(lds_all[4 * tid] - Mq) : 0.0;
      } else if (tid >= 64 && tid < 64 + chunks && need_p) {
        const int c = tid - 64;
        cterm[tid] = lds_all[4 * c + 2] > -INFINITY ? lds_all[4 * c + 3] * exp(lds_all[4 * c + 2] - Mp) : 0.0;
      }
      __syncthreads();
      double Zq = 0.0, Zp = 0.0;
      for (int c = 0; c < chunks; ++c) Zq += cterm[c];
      if (need_p)
        for (int c = 0; c < chunks; ++c) Zp += cterm[64 + c];
      lse_q = Mq + log(Zq);
      lse_p = need_p ? Mp + log(Zp) : 0.0;
      if constexpr (REGS) {
        const double sq = exp(mq - lse_q);
        const double sp = need_p ? exp(mp - lse_p) : 0.0;
#pragma unroll
        for (int i = 0; i < kSpecRegs; ++i) {
          qr[i] *= sq;
          pr[i] *= sp;
        }
      } else {
        for (int x = x0 + tid; x < x1; x += kSpecThreads) {
          qb[x] = exp((double)tl[x] - lse_q);
          if (!pm) pb[x] = need_p ? exp((double)dl[x] - lse_p) : 0.0;
        }
      }
    }
    if (tid < nk) {
      kid_q[tid] = ktok >= 0 ? exp((double)ktl - lse_q) : 0.0;
      kid_p[tid] = (ktok >= 0 && need_p) ? exp((double)kdl - lse_p) : 0.0;
    }
    __syncthreads();

    if (!has_draft) {
      sample_c = 0.0;
      sample_node = v;
      break;
    }

    // ---- children in order against the corrected target
    double cst = 0.0, S = 1.0;
    double last_c = -1.0;
    int accepted = -1;
    if (pm) {
      // Deterministic siblings: the draft distribution behind child t is the point mass
      // at t, so q'(t) = q(t) / (1 - removed) for a token not rejected yet (0 for one
      // that was), and a rejection removes q(t).  Every workgroup takes the same
      // decisions from the same values: no exchange.
      if (tid < nk) {
        unsigned long long same = 0ull;
        for (int i = 0; i < tid; ++i)
          if (kid_tok[i] == ktok) same |= 1ull << i;
        kid_same[tid] = same;
      }
      __syncthreads();
      double removed = 0.0;
      unsigned long long gone = 0ull;   // children whose token was removed from q'
      for (int j = 0; j < nk; ++j) {
        const int t = kid_tok[j];
        const bool dup = (gone & kid_same[j]) != 0ull;
        const double qt = kid_q[j];
        const double ratio = (t < 0 || dup) ? 0.0 : fmin(1.0, qt / (1.0 - removed));
        if ((double)kid_u[j] < ratio) {
          accepted = kids[j];
          break;
        }
        if (t >= 0 && !dup && 1.0 - removed - qt > 0.0) {
          removed += qt;
          gone |= 1ull << j;
        }
      }
      if (accepted < 0) {
        // the draw from q without the removed tokens: zero them in this chunk of q
        if constexpr (REGS) {
          for (int j = 0; j < nk; ++j) {
            const int t = kid_tok[j];
            if (((gone >> j) & 1ull) && t >= t0 && t < t1) {
#pragma unroll
              for (int i = 0; i < kSpecRegs; ++i)
                if (t0 + i == t) qr[i] = 0.0;
            }
          }
        } else {
          if (tid < nk && ((gone >> tid) & 1ull)) {
            const int t = kid_tok[tid];
            if (t >= x0 && t < x1) qb[t] = 0.0;
          }
          __syncthreads();
        }
      }
    }
    for (int j = 0; j < (pm ? 0 : nk); ++j) {
      const int kid = kids[j];
      const double qt = kid_q[j], pt = kid_p[j];
      const double resid = fmax(0.0, qt - cst * pt);
      const double ratio = pt > 0.0 ? fmin(1.0, resid / (S * pt)) : (resid > 0.0 ? 1.0 : 0.0);
      if ((double)kid_u[j] < ratio) {
        accepted = kid;
        break;
      }
      const double c2 = cst + S;
      if (j == nk - 1) {
        // every child rejected: the residual at c2 is drawn from directly; its mass
        // comes with the draw's chunk totals (zero exactly when S(c2) is zero)
        last_c = c2;
        break;
      }
      double part = 0.0;
      if constexpr (REGS) {
        // entries past t1 hold q = p = 0 and add +0.0
#pragma unroll
        for (int i = 0; i < kSpecRegs; ++i) part += fmax(0.0, qr[i] - c2 * pr[i]);
      } else {
        for (int x = x0 + tid; x < x1; x += kSpecThreads) part += fmax(0.0, qb[x] - c2 * pb[x]);
      }
      double S2;
      if (!exchange_sum(w, b, chunks, me, gen++, part, red, lds_all, &lds_flag, S2)) {
        aborted = true;
        break;
      }
      if (S2 > 0.0) {
        cst = c2;
        S = S2;
      }
    }
    if (aborted) break;
    if (accepted < 0) {
      sample_c = pm ? 0.0 : (last_c >= 0.0 ? last_c : cst);
      fallback_c = pm ? 0.0 : cst;
      sample_node = v;
      break;
    }
    v = accepted;
    ++alpha;
    if (tid == 0) path_s[alpha] = v;
    __syncthreads();
  }

  const int cap = pl.max_depth + 1;
  if (!aborted) {
    // ---- inverse-CDF draw from max(0, q - c p) (c = 0: q itself); if the residual at
    // the last c vanished by rounding, the draw falls back to the previous c (the
    // decision every workgroup takes from the same totals)
    double c = sample_c;
    const float us = u_sample[(size_t)b * N + sample_node];
    for (;;) {
      // the thread's mass over its contiguous entries, then an index-order scan of the
      // threads' masses: within each wave by lanes, then over the waves
      double tsum = 0.0;
      int tlast = -1;
      if constexpr (REGS) {
#pragma unroll
        for (int i = 0; i < kSpecRegs; ++i) {
          const double m = pm ? qr[i] : fmax(0.0, qr[i] - c * pr[i]);
          tsum += m;
          if (m > 0.0) tlast = t0 + i;
        }
      } else {
        for (int x = t0; x < t1; ++x) {
          const double m = pm ? qb[x] : fmax(0.0, qb[x] - c * pb[x]);
          tsum += m;
          if (m > 0.0) tlast = x;
        }
      }
      double incl = tsum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      double excl = __shfl_up(incl, 1);
      if (lane == 0) excl = 0.0;
      const int wlast = wave_max_i(tlast);
      if (lane == 63) {
        wtot_s[wid] = incl;
        wlast_s[wid] = wlast;
      }
      if (tid == 0) found_s = INT_MAX;
      __syncthreads();
      double chunk_total = 0.0;
      double before = 0.0;
      int chunk_last = -1;
#pragma unroll
      for (int i = 0; i < kSpecThreads / 64; ++i) {
        if (i == wid) before = chunk_total + excl;
        chunk_total += wtot_s[i];
        chunk_last = max(chunk_last, wlast_s[i]);
      }
      const double mine[4] = {chunk_total, (double)chunk_last, 0.0, 0.0};
      if (!exchange(w, b, chunks, me, gen++, 2, mine, lds_all, &lds_flag)) {
        aborted = true;
        break;
      }
      double total = 0.0, offset = 0.0;
      int glast = -1, glast_owner = 0;
      for (int cc = 0; cc < chunks; ++cc) {
        if (cc == me) offset = total;
        total += lds_all[4 * cc];
        if ((int)lds_all[4 * cc + 1] >= 0) {
          glast = (int)lds_all[4 * cc + 1];
          glast_owner = cc;
        }
      }
      if (!(total > 0.0) && c != fallback_c) {
        c = fallback_c;
        continue;
      }
      const double T = (double)us * total;
      if (T < total && T >= offset && T < offset + chunk_total) {
        const double Tl = T - offset;
        if (Tl >= before && Tl < before + tsum) {
          // the first entry whose running mass passes Tl; threads whose ranges touch at
          // a rounding boundary both report, and the lower index is kept
          double run = before;
          int f = -1;
          if constexpr (REGS) {
#pragma unroll
            for (int i = 0; i < kSpecRegs; ++i) {
              run += pm ? qr[i] : fmax(0.0, qr[i] - c * pr[i]);
              if (f < 0 && run > Tl) f = t0 + i;
            }
          } else {
            for (int x = t0; x < t1; ++x) {
              run += pm ? qb[x] : fmax(0.0, qb[x] - c * pb[x]);
              if (run > Tl) {
                f = x;
                break;
              }
            }
          }
          if (f >= 0) atomicMin(&found_s, f);
        }
        __syncthreads();
        if (tid == 0 && found_s == INT_MAX) found_s = chunk_last;   // rounding inside the chunk
      } else if (!(T < total) && me == glast_owner) {
        if (tid == 0) found_s = glast;                               // rounding past the total
      }
      __syncthreads();
      if (tid == 0 && found_s != INT_MAX && found_s >= 0) out_tokens[(size_t)b * cap + alpha] = found_s;
      break;
    }
  }

  // ---- exit.  The last workgroup of the sequence to finish writes the path, the
  // accepted drafts' tokens and the padding, or -1 everywhere (accept_len too) if any
  // workgroup of the sequence gave up on a spin.  The drawn token was stored by thread
  // 0 of the workgroup that found it before that workgroup's release below, so the
  // last workgroup's acquire orders its -1 after it.
  __shared__ unsigned exit_old;
  __syncthreads();
  if (tid == 0)
    exit_old = __hip_atomic_fetch_add(&w.exits[b], 1u + (aborted ? kExitAbortBit : 0u),
                                      __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const unsigned prior = exit_old;
  if ((prior & 0xFFFFu) == (unsigned)(chunks - 1) && tid < 64) {
    const bool bad = aborted || (prior & kExitAbortBit) != 0u;
    for (int j = tid; j < cap; j += 64) {
      if (bad) {
        accept_path[(size_t)b * cap + j] = -1;
        out_tokens[(size_t)b * cap + j] = -1;
      } else if (j <= alpha) {
        accept_path[(size_t)b * cap + j] = path_s[j];
        if (j < alpha) out_tokens[(size_t)b * cap + j] = tok[path_s[j + 1]];
      } else {
        accept_path[(size_t)b * cap + j] = -1;
        out_tokens[(size_t)b * cap + j] = -1;
      }
    }
    if (tid == 0) accept_len[b] = bad ? -1 : alpha;
  }
}

}  // namespace

hipError_t launch_accept_greedy(const int32_t* tokens, const int32_t* parents,
                                const int32_t* target_argmax, const int32_t* tree_len, int B,
                                int N, int max_depth, int32_t* accept_len, int32_t* accept_path,
                                int32_t* out_tokens, hipStream_t stream) {
  hipLaunchKernelGGL(accept_greedy_kernel, dim3((B + 3) / 4), dim3(256), 0, stream, tokens, parents,
                     target_argmax, tree_len, B, N, max_depth, accept_len, accept_path, out_tokens);
  return hipGetLastError();
}

SpecPlan plan_accept_spec(int B, int N, int V) {
  SpecPlan pl{};
  pl.B = B;
  pl.N = N;
  pl.V = V;
  // about 4K vocabulary entries per workgroup, at most 64 per sequence, and at most
  // 256 workgroups in all so that every workgroup of a sequence is resident at once
  int c = (V + kSpecChunk - 1) / kSpecChunk;
  if (c > 64) c = 64;
  int cap = 256 / (B > 0 ? B : 1);
  if (cap < 1) cap = 1;
  if (c > cap) c = cap;
  if (c < 1) c = 1;
  pl.chunks = c;
  return pl;
}

size_t accept_spec_workspace_bytes(const SpecPlan& pl) {
  size_t off = 2 * 256 * (size_t)((pl.B * 4 + 255) / 256);
  off += (size_t)pl.B * 2 * pl.chunks * 8 * sizeof(unsigned long long);
  off = (off + 255) / 256 * 256;
  off += 2 * (size_t)pl.B * pl.V * sizeof(double);
  return off + 256;
}

hipError_t launch_accept_spec(const SpecPlan& pl, const int32_t* tokens, const int32_t* parents,
                              const int32_t* draft_row, const float* target_logits,
                              const float* draft_logits, const float* u_accept,
                              const float* u_sample, int32_t* accept_len, int32_t* accept_path,
                              int32_t* out_tokens, void* workspace, hipStream_t stream) {
  const int words = pl.B * 2 * pl.chunks * 8;
  int init_blocks = (words + 4 * 256 - 1) / (4 * 256);   // about four words per thread
  init_blocks = init_blocks < 1 ? 1 : (init_blocks > 1024 ? 1024 : init_blocks);
  hipLaunchKernelGGL(spec_init_kernel, dim3(init_blocks), dim3(256), 0, stream, workspace, pl.B,
                     pl.chunks, pl.V);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int chunk_len = (pl.V + pl.chunks - 1) / pl.chunks;
  if (chunk_len <= kSpecChunk)
    hipLaunchKernelGGL(accept_spec_kernel<true>, dim3(pl.B * pl.chunks), dim3(kSpecThreads), 0,
                       stream, tokens, parents, draft_row, target_logits, draft_logits, u_accept,
                       u_sample, pl, accept_len, accept_path, out_tokens, workspace);
  else
    hipLaunchKernelGGL(accept_spec_kernel<false>, dim3(pl.B * pl.chunks), dim3(kSpecThreads), 0,
                       stream, tokens, parents, draft_row, target_logits, draft_logits, u_accept,
                       u_sample, pl, accept_len, accept_path, out_tokens, workspace);
  return hipGetLastError();
}

}  // namespace eagle
