// KV-cache commit after acceptance.
//
// [P3] section 4 (limitations): the dynamic draft tree leaves its key/value rows
// scattered through the cache.  After a root path root = path[0], ..., path[alpha]
// is accepted, its tree rows become the next prefix rows in path order:
// new[P + i] = old[P + path[i]] for i = 0..alpha, in every layer, sequence and KV
// head; all other rows are left alone.
//
// The move is in place and sources and destinations overlap (path[i] >= i, so row
// P + i may be the source of an earlier entry), so each workgroup first reads every
// accepted row of its (layer, sequence, KV head) into registers and writes them
// after a barrier.  A pure HBM copy of (alpha + 1) * D * 2 bytes per (cache, layer,
// sequence, head).
#include "common.h"
#include "internal.h"

namespace eagle {

namespace {

constexpr int kCommitThreads = 256;

template <int D>
__global__ void __launch_bounds__(kCommitThreads)
kv_commit_kernel(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                 const int32_t* __restrict__ accept_len, const int32_t* __restrict__ accept_path,
                 int B, int Hkv, int P, int kv_cap, int path_len) {
  constexpr int ROW_UNITS = D / 8;   // 16-byte units per row
  constexpr int PER = (kMaxCommitRows * ROW_UNITS + kCommitThreads - 1) / kCommitThreads;
  const int wg = blockIdx.x;         // (layer, sequence, KV head)
  const int g = wg % Hkv;
  const int b = (wg / Hkv) % B;
  const int layer = wg / (Hkv * B);
  int alpha = accept_len[b];
  if (alpha < 0) return;             // acceptance failed: nothing to commit (uniform)
  alpha = min(alpha, path_len - 1);
  const size_t base = (((size_t)layer * B + b) * Hkv + g) * (size_t)kv_cap * D;
  const int32_t* path = accept_path + (size_t)b * path_len;
  const int units = (alpha + 1) * ROW_UNITS;

  u32x4 kr[PER], vr[PER];
  bool live[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int u = threadIdx.x + it * kCommitThreads;
    const int i = min(u / ROW_UNITS, path_len - 1);   // in bounds for every lane
    const int node = u < units ? path[i] : -1;
    // rows outside the cache (any path content) are skipped
    live[it] = u < units && node >= 0 && node < kv_cap - P;
    if (live[it]) {
      const size_t off = base + (size_t)(P + node) * D + (u % ROW_UNITS) * 8;
      kr[it] = *(const u32x4*)(kc + off);
      vr[it] = *(const u32x4*)(vc + off);
    }
  }
  __syncthreads();   // every source row is in registers before any row is overwritten
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    if (!live[it]) continue;
    const int u = threadIdx.x + it * kCommitThreads;
    const size_t off = base + (size_t)(P + u / ROW_UNITS) * D + (u % ROW_UNITS) * 8;
    *(u32x4*)(kc + off) = kr[it];
    *(u32x4*)(vc + off) = vr[it];
  }
}

}  // namespace

hipError_t launch_kv_commit(void* k_cache, void* v_cache, const int32_t* accept_len,
                            const int32_t* accept_path, int L, int B, int Hkv, int D, int P,
                            int kv_cap, int path_len, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)L * B * Hkv));
  if (D == 128)
    hipLaunchKernelGGL(kv_commit_kernel<128>, grid, dim3(kCommitThreads), 0, stream,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, accept_len, accept_path, B, Hkv, P,
                       kv_cap, path_len);
  else
    hipLaunchKernelGGL(kv_commit_kernel<64>, grid, dim3(kCommitThreads), 0, stream,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, accept_len, accept_path, B, Hkv, P,
                       kv_cap, path_len);
  return hipGetLastError();
}

}  // namespace eagle
