// C-ABI entry points: argument checks on the host, then kernel launches on the
// caller's stream.  Nothing here allocates device memory or keeps state beyond the
// thread-local text of the last error.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/eagle_mi355.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

eagle_status_t fail(eagle_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
eagle_status_t fail(eagle_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

eagle_status_t ok() {
  g_last_error[0] = '\0';
  return EAGLE_OK;
}

eagle_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(EAGLE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The element type of the attention and LM-head operands: bf16 is the one
// implemented; fp32 operands are a valid request this library does not serve.
eagle_status_t check_dtype(eagle_dtype_t dtype) {
  if (dtype == EAGLE_BF16) return EAGLE_OK;
  if (dtype == EAGLE_F32)
    return fail(EAGLE_ERR_UNSUPPORTED, "dtype EAGLE_F32: only bf16 operands are implemented (round fp32 inputs to bf16)");
  return fail(EAGLE_ERR_INVALID_ARG, "dtype=%d is not an eagle_dtype_t value", (int)dtype);
}

}  // namespace

extern "C" {

int eagle_abi_version(void) { return EAGLE_ABI_VERSION; }

const char* eagle_status_string(eagle_status_t status) {
  switch (status) {
    case EAGLE_OK: return "ok";
    case EAGLE_ERR_NULL: return "null pointer";
    case EAGLE_ERR_INVALID_ARG: return "invalid argument";
    case EAGLE_ERR_UNSUPPORTED: return "unsupported";
    case EAGLE_ERR_WORKSPACE: return "workspace too small";
    case EAGLE_ERR_TREE: return "invalid tree";
    case EAGLE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* eagle_last_error(void) { return g_last_error; }

eagle_status_t eagle_check_tree(const int32_t* parents_host, int32_t B, int32_t N) {
  if (!parents_host) return fail(EAGLE_ERR_NULL, "parents_host is NULL");
  if (B < 1 || N < 1) return fail(EAGLE_ERR_INVALID_ARG, "B=%d N=%d must be >= 1", B, N);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* p = parents_host + (size_t)b * N;
    if (p[0] != -1) return fail(EAGLE_ERR_TREE, "sequence %d: parents[0]=%d, expected -1", b, p[0]);
    for (int32_t i = 1; i < N; ++i)
      if (p[i] < 0 || p[i] >= i)
        return fail(EAGLE_ERR_TREE, "sequence %d: parents[%d]=%d not in [0,%d)", b, i, p[i], i);
  }
  return ok();
}

// ---------------------------------------------------------------- attention
static eagle_status_t check_attn_dims(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t P) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || P < 0)
    return fail(EAGLE_ERR_INVALID_ARG, "need B,N,Hq,Hkv >= 1 and P >= 0 (B=%d N=%d Hq=%d Hkv=%d P=%d)",
                B, N, Hq, Hkv, P);
  if (Hq % Hkv) return fail(EAGLE_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (N > EAGLE_MAX_TREE) return fail(EAGLE_ERR_UNSUPPORTED, "N=%d > %d", N, EAGLE_MAX_TREE);
  if (D != 64 && D != 128) return fail(EAGLE_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  if ((long long)P + N > 0x7fffffffLL / 2) return fail(EAGLE_ERR_INVALID_ARG, "P too large");
  return EAGLE_OK;
}

size_t eagle_tree_verify_attn_workspace(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t P) {
  if (check_attn_dims(B, N, Hq, Hkv, D, P) != EAGLE_OK) return 0;
  return eagle::tree_attn_workspace_bytes(eagle::plan_tree_attn(B, N, Hq, Hkv, D, P, P + N));
}

static eagle_status_t attn_impl(const void* q, const void* k, const void* v,
                                const int32_t* parents, const int32_t* prefix_len,
                                const int32_t* tree_len, int32_t B, int32_t N, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t P, int32_t kv_cap, float scale,
                                eagle_dtype_t dtype, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, const char* name) {
  if (!q || !k || !v || !parents || !out)
    return fail(EAGLE_ERR_NULL, "q, k, v, parents and out must be non-NULL");
  eagle_status_t st = check_dtype(dtype);
  if (st != EAGLE_OK) return st;
  st = check_attn_dims(B, N, Hq, Hkv, D, P);
  if (st != EAGLE_OK) return st;
  if (kv_cap < P + N) return fail(EAGLE_ERR_INVALID_ARG, "kv_cap=%d < P+N=%d", kv_cap, P + N);
  if (!(scale > 0.f) || scale != scale || scale > 1e30f)
    return fail(EAGLE_ERR_INVALID_ARG, "scale must be a positive finite number");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(EAGLE_ERR_INVALID_ARG, "q, k, v, out must be 16-byte aligned");
  eagle::AttnPlan pl = eagle::plan_tree_attn(B, N, Hq, Hkv, D, P, kv_cap);
  pl.prefix_len = prefix_len;
  pl.tree_len = tree_len;
  const size_t need = eagle::tree_attn_workspace_bytes(pl);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (need > 0 && !aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char what[96];
  snprintf(what, sizeof(what), "%s launch", name);
  return hip_status(eagle::launch_tree_attn(pl, scale, q, k, v, parents, out, lse, workspace, stream),
                    what);
}

eagle_status_t eagle_tree_verify_attn(const void* q, const void* k, const void* v,
                                      const int32_t* parents, int32_t B, int32_t N, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t P, int32_t kv_cap,
                                      float scale, eagle_dtype_t dtype, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  return attn_impl(q, k, v, parents, nullptr, nullptr, B, N, Hq, Hkv, D, P, kv_cap, scale, dtype,
                   out, lse, workspace, workspace_bytes, stream, "eagle_tree_verify_attn");
}

static int page_shift_of(int32_t page_size) {
  for (int s = 0; s <= 12; ++s)
    if (page_size == (1 << s)) return s;
  return -1;
}

size_t eagle_tree_verify_attn_paged_workspace(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t P, int32_t page_size) {
  if (check_attn_dims(B, N, Hq, Hkv, D, P) != EAGLE_OK) return 0;
  const int shift = page_shift_of(page_size);
  if (shift < 0) return 0;
  return eagle::tree_attn_workspace_bytes(eagle::plan_tree_attn_paged(B, N, Hq, Hkv, D, P, shift));
}

eagle_status_t eagle_tree_verify_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                                            const int32_t* block_table, const int32_t* parents,
                                            int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                            int32_t D, int32_t P, int32_t page_size,
                                            int32_t max_pages, int32_t num_blocks, float scale,
                                            eagle_dtype_t dtype, void* out, float* lse,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  if (!q || !k_pool || !v_pool || !block_table || !parents || !out)
    return fail(EAGLE_ERR_NULL, "q, k_pool, v_pool, block_table, parents and out must be non-NULL");
  eagle_status_t st = check_dtype(dtype);
  if (st != EAGLE_OK) return st;
  st = check_attn_dims(B, N, Hq, Hkv, D, P);
  if (st != EAGLE_OK) return st;
  const int shift = page_shift_of(page_size);
  if (shift < 0) return fail(EAGLE_ERR_UNSUPPORTED, "page_size=%d (a power of two up to 4096)", page_size);
  if (num_blocks < 1 || max_pages < 1)
    return fail(EAGLE_ERR_INVALID_ARG, "num_blocks=%d and max_pages=%d must be >= 1", num_blocks, max_pages);
  if ((long long)max_pages * page_size < (long long)P + N)
    return fail(EAGLE_ERR_INVALID_ARG, "max_pages * page_size = %lld < P+N=%d",
                (long long)max_pages * page_size, P + N);
  if ((double)num_blocks * Hkv * page_size * (double)D > 4.0e18)
    return fail(EAGLE_ERR_INVALID_ARG, "pool too large");
  if (!(scale > 0.f) || scale != scale || scale > 1e30f)
    return fail(EAGLE_ERR_INVALID_ARG, "scale must be a positive finite number");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(EAGLE_ERR_INVALID_ARG, "q, k_pool, v_pool, out must be 16-byte aligned");
  eagle::AttnPlan pl = eagle::plan_tree_attn_paged(B, N, Hq, Hkv, D, P, shift);
  const int last_range = (P - (pl.S - 1) * pl.split_len) + N;
  const int range = (pl.split_len > last_range ? pl.split_len : last_range) + 64;
  if ((range >> shift) + 2 > eagle::kMaxSplitPages)
    return fail(EAGLE_ERR_UNSUPPORTED, "page_size=%d too small for P=%d (block-table slice per split)",
                page_size, P);
  pl.block_table = block_table;
  pl.max_pages = max_pages;
  pl.num_blocks = num_blocks;
  const size_t need = eagle::tree_attn_workspace_bytes(pl);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (need > 0 && !aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return hip_status(eagle::launch_tree_attn(pl, scale, q, k_pool, v_pool, parents, out, lse,
                                            workspace, stream),
                    "eagle_tree_verify_attn_paged launch");
}

eagle_status_t eagle_tree_verify_attn_ragged(const void* q, const void* k, const void* v,
                                             const int32_t* parents, const int32_t* prefix_len,
                                             const int32_t* tree_len, int32_t B, int32_t N,
                                             int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                             int32_t kv_cap, float scale, eagle_dtype_t dtype,
                                             void* out, float* lse, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  if (!prefix_len && !tree_len)
    return fail(EAGLE_ERR_NULL, "prefix_len and tree_len are both NULL (use eagle_tree_verify_attn)");
  return attn_impl(q, k, v, parents, prefix_len, tree_len, B, N, Hq, Hkv, D, P, kv_cap, scale,
                   dtype, out, lse, workspace, workspace_bytes, stream,
                   "eagle_tree_verify_attn_ragged");
}

// ---------------------------------------------------------------- LM head
static eagle_status_t check_lm_dims(int32_t M, int32_t H, int32_t V) {
  if (M < 1 || H < 1 || V < 2)
    return fail(EAGLE_ERR_INVALID_ARG, "need M >= 1, H >= 1, V >= 2 (M=%d H=%d V=%d)", M, H, V);
  if (H % 64) return fail(EAGLE_ERR_UNSUPPORTED, "H=%d is not a multiple of 64", H);
  return EAGLE_OK;
}

size_t eagle_lm_head_workspace(int32_t M, int32_t H, int32_t V) {
  if (check_lm_dims(M, H, V) != EAGLE_OK) return 0;
  return eagle::lm_head_workspace_bytes(eagle::plan_lm_head(M, H, V));
}

eagle_status_t eagle_lm_head_argmax(const void* hidden, const void* weight, int32_t M, int32_t H,
                                    int32_t V, eagle_dtype_t dtype, float* out_max,
                                    int32_t* out_argmax, float* out_lse, float* out_second,
                                    float* out_logits, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (!hidden || !weight || !out_max || !out_argmax || !out_lse)
    return fail(EAGLE_ERR_NULL, "hidden, weight, out_max, out_argmax and out_lse must be non-NULL");
  eagle_status_t st = check_dtype(dtype);
  if (st != EAGLE_OK) return st;
  st = check_lm_dims(M, H, V);
  if (st != EAGLE_OK) return st;
  if (!aligned16(hidden) || !aligned16(weight) || (out_logits && !aligned16(out_logits)))
    return fail(EAGLE_ERR_INVALID_ARG, "hidden, weight and out_logits must be 16-byte aligned");
  const eagle::LmPlan pl = eagle::plan_lm_head(M, H, V);
  const size_t need = eagle::lm_head_workspace_bytes(pl);
  if (!workspace || workspace_bytes < need)
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return hip_status(eagle::launch_lm_head(pl, hidden, weight, out_max, out_argmax, out_lse,
                                          out_second, out_logits, workspace, stream),
                    "eagle_lm_head_argmax launch");
}

// ---------------------------------------------------------------- LM head without allocation
// The scratch of eagle_lm_head_argmax_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never uses its name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress, once per device
// (with that device current), and is kept here.
}  // extern "C"

static __device__ __align__(256) unsigned char scratch[EAGLE_LM_HEAD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// this device's address of `scratch` (looked up on the device's first call)
eagle_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(EAGLE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(EAGLE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return EAGLE_OK;
}
}  // namespace

extern "C" {

eagle_status_t eagle_lm_head_argmax_noalloc(const void* hidden, const void* weight, int32_t M,
                                            int32_t H, int32_t V, eagle_dtype_t dtype,
                                            float* out_max, int32_t* out_argmax, float* out_lse,
                                            float* out_second, float* out_logits,
                                            hipStream_t stream) {
  if (!hidden || !weight || !out_max || !out_argmax || !out_lse)
    return fail(EAGLE_ERR_NULL, "hidden, weight, out_max, out_argmax and out_lse must be non-NULL");
  eagle_status_t st = check_dtype(dtype);
  if (st != EAGLE_OK) return st;
  st = check_lm_dims(M, H, V);
  if (st != EAGLE_OK) return st;
  if (!aligned16(hidden) || !aligned16(weight) || (out_logits && !aligned16(out_logits)))
    return fail(EAGLE_ERR_INVALID_ARG, "hidden, weight and out_logits must be 16-byte aligned");
  const eagle::LmPlan pl = eagle::plan_lm_head(M, H, V);
  const size_t need = eagle::lm_head_workspace_bytes(pl);
  if (need > (size_t)EAGLE_LM_HEAD_NOALLOC_SCRATCH_BYTES)
    return fail(EAGLE_ERR_UNSUPPORTED,
                "M=%d, V=%d need %zu bytes of scratch, more than the %d bytes of the static "
                "scratch (use eagle_lm_head_argmax with a workspace)",
                M, V, need, EAGLE_LM_HEAD_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != EAGLE_OK) return st;
  return hip_status(eagle::launch_lm_head(pl, hidden, weight, out_max, out_argmax, out_lse,
                                          out_second, out_logits, ws, stream),
                    "eagle_lm_head_argmax_noalloc launch");
}

// ---------------------------------------------------------------- acceptance
static eagle_status_t greedy_impl(const int32_t* tokens, const int32_t* parents,
                                  const int32_t* target_argmax, const int32_t* tree_len, int32_t B,
                                  int32_t N, int32_t max_depth, int32_t* accept_len,
                                  int32_t* accept_path, int32_t* out_tokens, hipStream_t stream) {
  if (!tokens || !parents || !target_argmax || !accept_len || !accept_path || !out_tokens)
    return fail(EAGLE_ERR_NULL, "all pointers must be non-NULL");
  if (B < 1 || N < 1 || max_depth < 0)
    return fail(EAGLE_ERR_INVALID_ARG, "need B,N >= 1 and max_depth >= 0");
  if (N > EAGLE_MAX_TREE) return fail(EAGLE_ERR_UNSUPPORTED, "N=%d > %d", N, EAGLE_MAX_TREE);
  if (max_depth > EAGLE_MAX_TREE) return fail(EAGLE_ERR_INVALID_ARG, "max_depth=%d > %d", max_depth, EAGLE_MAX_TREE);
  return hip_status(eagle::launch_accept_greedy(tokens, parents, target_argmax, tree_len, B, N,
                                                max_depth, accept_len, accept_path, out_tokens,
                                                stream),
                    "eagle_accept_greedy launch");
}

eagle_status_t eagle_accept_greedy(const int32_t* tokens, const int32_t* parents,
                                   const int32_t* target_argmax, int32_t B, int32_t N,
                                   int32_t max_depth, int32_t* accept_len, int32_t* accept_path,
                                   int32_t* out_tokens, hipStream_t stream) {
  return greedy_impl(tokens, parents, target_argmax, nullptr, B, N, max_depth, accept_len,
                     accept_path, out_tokens, stream);
}

eagle_status_t eagle_accept_greedy_ragged(const int32_t* tokens, const int32_t* parents,
                                          const int32_t* target_argmax, const int32_t* tree_len,
                                          int32_t B, int32_t N, int32_t max_depth,
                                          int32_t* accept_len, int32_t* accept_path,
                                          int32_t* out_tokens, hipStream_t stream) {
  if (!tree_len) return fail(EAGLE_ERR_NULL, "tree_len is NULL (use eagle_accept_greedy)");
  return greedy_impl(tokens, parents, target_argmax, tree_len, B, N, max_depth, accept_len,
                     accept_path, out_tokens, stream);
}

size_t eagle_accept_spec_workspace(int32_t B, int32_t N, int32_t V) {
  if (B < 1 || N < 1 || V < 1) return 0;
  return eagle::accept_spec_workspace_bytes(eagle::plan_accept_spec(B, N, V));
}

static eagle_status_t spec_impl(const int32_t* tokens, const int32_t* parents,
                                const int32_t* tree_len, int32_t B, int32_t N, int32_t V,
                                int32_t max_depth, const float* target_logits,
                                const float* target_lse, const float* draft_logits,
                                const float* draft_lse, const int32_t* draft_row,
                                int32_t draft_rows, const float* u_accept, const float* u_sample,
                                eagle_spec_mode_t mode, int32_t* accept_len, int32_t* accept_path,
                                int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, const char* name) {
  if (!tokens || !parents || !draft_row || !target_logits || !draft_logits || !u_accept ||
      !u_sample || !accept_len || !accept_path || !out_tokens)
    return fail(EAGLE_ERR_NULL, "every pointer except target_lse and draft_lse must be non-NULL");
  if (B < 1 || N < 1 || V < 1 || draft_rows < 1 || max_depth < 0)
    return fail(EAGLE_ERR_INVALID_ARG, "need B,N,V,draft_rows >= 1 and max_depth >= 0");
  if (N > EAGLE_MAX_TREE) return fail(EAGLE_ERR_UNSUPPORTED, "N=%d > %d", N, EAGLE_MAX_TREE);
  if (max_depth > EAGLE_MAX_TREE) return fail(EAGLE_ERR_INVALID_ARG, "max_depth=%d > %d", max_depth, EAGLE_MAX_TREE);
  if (mode != EAGLE_SPEC_SAMPLED && mode != EAGLE_SPEC_POINT_MASS)
    return fail(EAGLE_ERR_INVALID_ARG, "mode=%d (EAGLE_SPEC_SAMPLED or EAGLE_SPEC_POINT_MASS)", (int)mode);
  eagle::SpecPlan pl = eagle::plan_accept_spec(B, N, V);
  pl.mode = mode;
  pl.R = draft_rows;
  pl.max_depth = max_depth;
  pl.tree_len = tree_len;
  pl.target_lse = target_lse;
  pl.draft_lse = draft_lse;
  const size_t need = eagle::accept_spec_workspace_bytes(pl);
  if (!workspace || workspace_bytes < need)
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char what[64];
  snprintf(what, sizeof(what), "%s launch", name);
  return hip_status(eagle::launch_accept_spec(pl, tokens, parents, draft_row, target_logits,
                                              draft_logits, u_accept, u_sample, accept_len,
                                              accept_path, out_tokens, workspace, stream),
                    what);
}

eagle_status_t eagle_accept_spec(const int32_t* tokens, const int32_t* parents, int32_t B,
                                 int32_t N, int32_t V, int32_t max_depth,
                                 const float* target_logits, const float* target_lse,
                                 const float* draft_logits, const float* draft_lse,
                                 const int32_t* draft_row, int32_t draft_rows,
                                 const float* u_accept, const float* u_sample,
                                 eagle_spec_mode_t mode, int32_t* accept_len,
                                 int32_t* accept_path, int32_t* out_tokens, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return spec_impl(tokens, parents, nullptr, B, N, V, max_depth, target_logits, target_lse,
                   draft_logits, draft_lse, draft_row, draft_rows, u_accept, u_sample, mode,
                   accept_len, accept_path, out_tokens, workspace, workspace_bytes, stream,
                   "eagle_accept_spec");
}

eagle_status_t eagle_accept_spec_ragged(const int32_t* tokens, const int32_t* parents,
                                        const int32_t* tree_len, int32_t B, int32_t N, int32_t V,
                                        int32_t max_depth, const float* target_logits,
                                        const float* target_lse, const float* draft_logits,
                                        const float* draft_lse, const int32_t* draft_row,
                                        int32_t draft_rows, const float* u_accept,
                                        const float* u_sample, eagle_spec_mode_t mode,
                                        int32_t* accept_len, int32_t* accept_path,
                                        int32_t* out_tokens, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (!tree_len) return fail(EAGLE_ERR_NULL, "tree_len is NULL (use eagle_accept_spec)");
  return spec_impl(tokens, parents, tree_len, B, N, V, max_depth, target_logits, target_lse,
                   draft_logits, draft_lse, draft_row, draft_rows, u_accept, u_sample, mode,
                   accept_len, accept_path, out_tokens, workspace, workspace_bytes, stream,
                   "eagle_accept_spec_ragged");
}

// ---------------------------------------------------------------- rerank
static eagle_status_t check_rerank_dims(int32_t B, int32_t V, int32_t top_k, int32_t depth,
                                        int32_t n_nodes) {
  if (B < 1 || V < 1 || top_k < 1 || depth < 1 || n_nodes < 1)
    return fail(EAGLE_ERR_INVALID_ARG, "need B, V, top_k, depth, n_nodes >= 1");
  if (top_k > EAGLE_MAX_TOPK) return fail(EAGLE_ERR_UNSUPPORTED, "top_k=%d > %d", top_k, EAGLE_MAX_TOPK);
  if (top_k > V) return fail(EAGLE_ERR_INVALID_ARG, "top_k=%d > V=%d", top_k, V);
  if (n_nodes > EAGLE_MAX_TREE) return fail(EAGLE_ERR_UNSUPPORTED, "n_nodes=%d > %d", n_nodes, EAGLE_MAX_TREE);
  const long long cand = (long long)top_k + (long long)(depth - 1) * top_k * top_k;
  if (cand > eagle::rerank_max_candidates())
    return fail(EAGLE_ERR_UNSUPPORTED, "top_k + (depth-1)*top_k^2 = %lld candidates > %d", cand,
                eagle::rerank_max_candidates());
  const long long rows = 1 + (long long)(depth - 1) * top_k;
  const long long chunks = (V + eagle::rerank_chunk_len() - 1) / eagle::rerank_chunk_len();
  if (rows * top_k > eagle::rerank_max_row_list() || rows > 512 || chunks * top_k > 1024)
    return fail(EAGLE_ERR_UNSUPPORTED, "rerank sizes past the kernel limits (rows*top_k=%lld, rows=%lld, "
                "chunks*top_k=%lld)", rows * top_k, rows, chunks * top_k);
  if (n_nodes - 1 > cand)
    return fail(EAGLE_ERR_INVALID_ARG, "n_nodes-1=%d exceeds the %lld candidates", n_nodes - 1, cand);
  return EAGLE_OK;
}

size_t eagle2_rerank_workspace(int32_t B, int32_t V, int32_t top_k, int32_t depth) {
  if (B < 1 || V < 1 || top_k < 1 || depth < 1 || top_k > EAGLE_MAX_TOPK) return 0;
  return eagle::rerank_workspace_bytes(eagle::plan_rerank(B, V, top_k, depth, 1));
}

eagle_status_t eagle2_rerank(const float* draft_logits, const int32_t* root_token, int32_t B,
                             int32_t V, int32_t top_k, int32_t depth, int32_t n_nodes,
                             int32_t* tokens, int32_t* parents, int32_t* depths, float* scores,
                             int32_t* draft_row, float* draft_lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!draft_logits || !root_token || !tokens || !parents || !depths || !scores || !draft_row ||
      !draft_lse)
    return fail(EAGLE_ERR_NULL, "all pointers must be non-NULL");
  eagle_status_t st = check_rerank_dims(B, V, top_k, depth, n_nodes);
  if (st != EAGLE_OK) return st;
  const eagle::RerankPlan pl = eagle::plan_rerank(B, V, top_k, depth, n_nodes);
  const size_t need = eagle::rerank_workspace_bytes(pl);
  if (!workspace || workspace_bytes < need)
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return hip_status(eagle::launch_rerank(pl, draft_logits, root_token, tokens, parents, depths, scores,
                                         draft_row, draft_lse, workspace, stream),
                    "eagle2_rerank launch");
}

// ---------------------------------------------------------------- draft expansion
namespace {

struct DraftLayout {
  eagle::DraftDims dd;
  eagle::RerankPlan rpl;
  int Mmax, maxN, maxW;
  size_t off_rerank, off_X, off_G, off_x, off_h, off_n, off_y, off_q, off_att, off_attws, off_lm,
      total;
  size_t attn_ws, lm_ws;
};

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

DraftLayout draft_layout(int B, int H, int Hq, int Hkv, int D, int I, int V, int P, int kv_cap,
                         int top_k, int depth, int n_nodes) {
  DraftLayout L{};
  const int R = 1 + (depth - 1) * top_k;
  L.dd = eagle::DraftDims{B, H, Hq, Hkv, D, I, V, P, kv_cap, R};
  L.rpl = eagle::plan_rerank(B, V, top_k, depth, n_nodes);
  L.Mmax = B * (depth > 1 ? top_k : 1);
  const int qkvn = (Hq + 2 * Hkv) * D;
  L.maxN = V;
  for (int n : {H, qkvn, 2 * I}) L.maxN = n > L.maxN ? n : L.maxN;
  L.maxW = H;
  for (int w : {Hq * D, I}) L.maxW = w > L.maxW ? w : L.maxW;
  // the attention of depth d computes that depth's rows (queries) over the R-row tree
  L.attn_ws = 0;
  for (int d = 0; d < depth; ++d) {
    const int row0 = d == 0 ? 0 : 1 + (d - 1) * top_k, nr = d == 0 ? 1 : top_k;
    const size_t w = eagle::tree_attn_workspace_bytes(
        eagle::plan_tree_attn_rows(B, R, row0, nr, Hq, Hkv, D, P, kv_cap));
    L.attn_ws = w > L.attn_ws ? w : L.attn_ws;
  }
  L.lm_ws = 0;
  const int shapes[6][2] = {{2 * H, H}, {H, qkvn}, {Hq * D, H}, {H, 2 * I}, {I, H}, {H, V}};
  for (int m : {B, L.Mmax})
    for (auto& kn : shapes) {
      const size_t w = eagle::gemm_f32_workspace_bytes(m, kn[0], kn[1]);
      L.lm_ws = w > L.lm_ws ? w : L.lm_ws;
    }
  const size_t M = L.Mmax;
  size_t o = 0;
  L.off_rerank = o; o += a256(eagle::rerank_workspace_bytes(L.rpl));
  L.off_X = o;      o += a256(M * 2 * H * 2);
  L.off_G = o;      o += a256(M * (size_t)L.maxN * 4);
  L.off_x = o;      o += a256(M * H * 4);
  L.off_h = o;      o += a256(M * H * 4);
  L.off_n = o;      o += a256(M * (size_t)L.maxW * 2);
  L.off_y = o;      o += a256(M * H * 2);
  L.off_q = o;      o += a256((size_t)B * R * Hq * D * 2);
  L.off_att = o;    o += a256((size_t)B * R * Hq * D * 2);
  L.off_attws = o;  o += a256(L.attn_ws);
  L.off_lm = o;     o += a256(L.lm_ws);
  L.total = o + 256;
  return L;
}

eagle_status_t check_draft_dims(int32_t B, int32_t H, int32_t Hq, int32_t Hkv, int32_t D, int32_t I,
                                int32_t V, int32_t P, int32_t top_k, int32_t depth, int32_t n_nodes) {
  if (B < 1 || H < 1 || Hq < 1 || Hkv < 1 || I < 1 || V < 2 || P < 0)
    return fail(EAGLE_ERR_INVALID_ARG, "need B, H, Hq, Hkv, I >= 1, V >= 2, P >= 0");
  if (H % 64 || I % 64)
    return fail(EAGLE_ERR_UNSUPPORTED, "H=%d and I=%d must be multiples of 64", H, I);
  if (Hq % Hkv) return fail(EAGLE_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 64 && D != 128) return fail(EAGLE_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  eagle_status_t st = check_rerank_dims(B, V, top_k, depth, n_nodes);
  if (st != EAGLE_OK) return st;
  const long long R = 1 + (long long)(depth - 1) * top_k;
  if (R > EAGLE_MAX_TREE)
    return fail(EAGLE_ERR_UNSUPPORTED, "1 + (depth-1)*top_k = %lld expansion rows > %d", R, EAGLE_MAX_TREE);
  return EAGLE_OK;
}

hipError_t draft_gemm(int M, int K, int N, const void* X, const void* W, float* out, char* ws,
                      const DraftLayout& L, hipStream_t stream) {
  return eagle::launch_gemm_f32(M, K, N, X, W, out, ws + L.off_lm, stream);
}

// the same GEMM with its split-K slices handed to the consumer kernel, which sums
// them while reading (no separate summing pass)
hipError_t draft_gemm_slices(int M, int K, int N, const void* X, const void* W, float* out, char* ws,
                             const DraftLayout& L, eagle::F32Slices* r, hipStream_t stream) {
  return eagle::launch_gemm_f32_slices(M, K, N, X, W, out, ws + L.off_lm, r, stream);
}

}  // namespace

size_t eagle_draft_expand_workspace(int32_t B, int32_t H, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t I, int32_t V, int32_t P, int32_t kv_cap, int32_t top_k,
                                    int32_t depth) {
  if (B < 1 || H < 1 || Hq < 1 || Hkv < 1 || I < 1 || V < 2 || P < 0 || top_k < 1 || depth < 1 ||
      top_k > EAGLE_MAX_TOPK || Hq % Hkv || (D != 64 && D != 128) || kv_cap < P)
    return 0;
  return draft_layout(B, H, Hq, Hkv, D, I, V, P, kv_cap, top_k, depth, 1).total;
}

eagle_status_t eagle_draft_expand(const eagle_draft_head* head, const void* f0,
                                  const int32_t* root_token, void* k_cache, void* v_cache, int32_t B,
                                  int32_t H, int32_t Hq, int32_t Hkv, int32_t D, int32_t I, int32_t V,
                                  int32_t P, int32_t kv_cap, int32_t top_k, int32_t depth,
                                  int32_t n_nodes, float scale, float eps, int32_t* tokens,
                                  int32_t* parents, int32_t* depths, float* scores,
                                  int32_t* draft_row, float* draft_logits, float* draft_lse,
                                  void* features, int32_t* row_token, int32_t* parent_row,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!head || !head->embed || !head->w_fc || !head->w_qkv || !head->w_o || !head->w_gate_up ||
      !head->w_down || !head->w_lm || !head->g1 || !head->g2)
    return fail(EAGLE_ERR_NULL, "every draft-head pointer must be non-NULL");
  if (!f0 || !root_token || !k_cache || !v_cache || !tokens || !parents || !depths || !scores ||
      !draft_row || !draft_logits || !draft_lse || !features || !row_token || !parent_row)
    return fail(EAGLE_ERR_NULL, "all pointers must be non-NULL");
  eagle_status_t st = check_draft_dims(B, H, Hq, Hkv, D, I, V, P, top_k, depth, n_nodes);
  if (st != EAGLE_OK) return st;
  const int R = 1 + (depth - 1) * top_k;
  if (kv_cap < P + R)
    return fail(EAGLE_ERR_INVALID_ARG, "kv_cap=%d < P + expansion rows = %d", kv_cap, P + R);
  const void* const must_align[] = {head->embed, head->w_fc,  head->w_qkv, head->w_o,
                                    head->w_gate_up, head->w_down, head->w_lm, f0,
                                    features,    k_cache,     v_cache,     draft_logits};
  for (const void* p : must_align)
    if (!aligned16(p)) return fail(EAGLE_ERR_INVALID_ARG, "weights, f0, caches, features and draft_logits must be 16-byte aligned");
  const DraftLayout L = draft_layout(B, H, Hq, Hkv, D, I, V, P, kv_cap, top_k, depth, n_nodes);
  if (!workspace || workspace_bytes < L.total)
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (!aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  char* ws = (char*)workspace;
  void* X = ws + L.off_X;
  float* G = (float*)(ws + L.off_G);
  float* xres = (float*)(ws + L.off_x);
  float* hres = (float*)(ws + L.off_h);
  void* nb = ws + L.off_n;
  void* yb = ws + L.off_y;
  void* qbuf = ws + L.off_q;
  void* att = ws + L.off_att;
  void* rws = ws + L.off_rerank;
  const eagle::DraftDims& dd = L.dd;
  const int qkvn = (Hq + 2 * Hkv) * D;
#define DRAFT_TRY(expr, what)                                   \
  do {                                                          \
    const hipError_t e_ = (expr);                               \
    if (e_ != hipSuccess) return hip_status(e_, what);          \
  } while (0)
  DRAFT_TRY(eagle::launch_draft_init_rows(B, R, root_token, row_token, parent_row, stream), "draft init");
  for (int d = 0; d < depth; ++d) {
    const int row0 = d == 0 ? 0 : 1 + (d - 1) * top_k;
    const int nr = d == 0 ? 1 : top_k;
    const int M = B * nr;
    if (d > 0)
      DRAFT_TRY(eagle::launch_draft_frontier(L.rpl, d, draft_lse, rws, row_token, parent_row, stream),
                "draft frontier");
    DRAFT_TRY(eagle::launch_draft_gather_input(dd, row0, nr, f0, root_token, head->embed, features,
                                               row_token, parent_row, X, stream), "draft gather");
    eagle::F32Slices gs;
    DRAFT_TRY(draft_gemm_slices(M, 2 * H, H, X, head->w_fc, G, ws, L, &gs, stream), "draft fc");
    DRAFT_TRY(eagle::launch_draft_rms(M, H, eps, gs, nullptr, head->g1, xres, nb, stream), "draft norm 1");
    DRAFT_TRY(draft_gemm_slices(M, H, qkvn, nb, head->w_qkv, G, ws, L, &gs, stream), "draft qkv");
    DRAFT_TRY(eagle::launch_draft_qkv_scatter(dd, row0, nr, gs, qbuf, k_cache, v_cache, stream), "draft scatter");
    const eagle::AttnPlan apl = eagle::plan_tree_attn_rows(B, R, row0, nr, Hq, Hkv, D, P, kv_cap);
    DRAFT_TRY(eagle::launch_tree_attn(apl, scale, qbuf, k_cache, v_cache, parent_row, att, nullptr,
                                      ws + L.off_attws, stream), "draft attention");
    DRAFT_TRY(eagle::launch_draft_gather_rows(dd, row0, nr, Hq * D, att, nb, stream), "draft gather rows");
    DRAFT_TRY(draft_gemm_slices(M, Hq * D, H, nb, head->w_o, G, ws, L, &gs, stream), "draft o");
    DRAFT_TRY(eagle::launch_draft_rms(M, H, eps, gs, xres, head->g2, hres, nb, stream), "draft norm 2");
    DRAFT_TRY(draft_gemm(M, H, 2 * I, nb, head->w_gate_up, G, ws, L, stream), "draft gate/up");
    DRAFT_TRY(eagle::launch_draft_silu_mul(M, I, G, nb, stream), "draft silu");
    DRAFT_TRY(draft_gemm_slices(M, I, H, nb, head->w_down, G, ws, L, &gs, stream), "draft down");
    DRAFT_TRY(eagle::launch_draft_output(dd, row0, nr, gs, hres, yb, features, stream), "draft output");
    DRAFT_TRY(draft_gemm(M, H, V, yb, head->w_lm, G, ws, L, stream), "draft lm head");
    DRAFT_TRY(eagle::launch_draft_place_logits(dd, row0, nr, G, draft_logits, stream), "draft place");
    eagle::RerankPlan rp = L.rpl;
    rp.row0 = row0;
    rp.nrows = nr;
    DRAFT_TRY(eagle::launch_rerank_rows(rp, draft_logits, draft_lse, rws, stream), "draft rows");
  }
  DRAFT_TRY(eagle::launch_rerank_tree(L.rpl, root_token, draft_lse, rws, tokens, parents, depths,
                                      scores, draft_row, stream), "draft tree");
#undef DRAFT_TRY
  return ok();
}

// ---------------------------------------------------------------- KV commit
eagle_status_t eagle_kv_commit(void* k_cache, void* v_cache, const int32_t* accept_len,
                               const int32_t* accept_path, int32_t L, int32_t B, int32_t Hkv,
                               int32_t D, int32_t P, int32_t kv_cap, int32_t path_len,
                               hipStream_t stream) {
  if (!k_cache || !v_cache || !accept_len || !accept_path)
    return fail(EAGLE_ERR_NULL, "all pointers must be non-NULL");
  if (L < 1 || B < 1 || Hkv < 1 || P < 0 || path_len < 1)
    return fail(EAGLE_ERR_INVALID_ARG, "need L,B,Hkv,path_len >= 1 and P >= 0 (L=%d B=%d Hkv=%d P=%d path_len=%d)",
                L, B, Hkv, P, path_len);
  if (D != 64 && D != 128) return fail(EAGLE_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  if (path_len > eagle::kMaxCommitRows)
    return fail(EAGLE_ERR_UNSUPPORTED, "path_len=%d > %d", path_len, eagle::kMaxCommitRows);
  if ((long long)P + path_len > kv_cap)
    return fail(EAGLE_ERR_INVALID_ARG, "P + path_len = %lld exceeds kv_cap=%d", (long long)P + path_len, kv_cap);
  if ((long long)L * B * Hkv > 0x7fffffffLL ||
      (double)L * B * Hkv * (double)kv_cap * D > 9.0e18)
    return fail(EAGLE_ERR_INVALID_ARG, "cache too large");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(EAGLE_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  return hip_status(eagle::launch_kv_commit(k_cache, v_cache, accept_len, accept_path, L, B, Hkv,
                                            D, P, kv_cap, path_len, stream),
                    "eagle_kv_commit launch");
}

// ---------------------------------------------------------------- measurement probes
eagle_status_t eagle_calib_stream_read(const void* src, size_t bytes, void* sink,
                                       hipStream_t stream) {
  if (!src || !sink) return fail(EAGLE_ERR_NULL, "src and sink must be non-NULL");
  if (bytes < 16 || bytes % 16) return fail(EAGLE_ERR_INVALID_ARG, "bytes=%zu: a positive multiple of 16", bytes);
  if (!aligned16(src)) return fail(EAGLE_ERR_INVALID_ARG, "src must be 16-byte aligned");
  return hip_status(eagle::launch_calib_stream_read(src, bytes, sink, stream),
                    "eagle_calib_stream_read launch");
}

double eagle_calib_mfma_bf16_flops(int32_t iters) {
  if (iters < 1) return 0.0;
  // workgroups x 4 waves x 4 chains x iters x 32*32*16*2 flop
  return (double)eagle::kCalibMfmaBlocks * 4.0 * 4.0 * (double)iters * 32768.0;
}

eagle_status_t eagle_calib_mfma_bf16(int32_t iters, float* out, size_t out_floats,
                                     hipStream_t stream) {
  if (!out) return fail(EAGLE_ERR_NULL, "out must be non-NULL");
  if (iters < 1) return fail(EAGLE_ERR_INVALID_ARG, "iters=%d must be >= 1", iters);
  if (out_floats < (size_t)eagle::kCalibMfmaBlocks * 256)
    return fail(EAGLE_ERR_WORKSPACE, "out holds %zu floats, need %d", out_floats,
                eagle::kCalibMfmaBlocks * 256);
  return hip_status(eagle::launch_calib_mfma_bf16(iters, out, stream), "eagle_calib_mfma_bf16 launch");
}

}  // extern "C"
