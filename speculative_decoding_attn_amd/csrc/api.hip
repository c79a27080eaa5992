// C-ABI entry points: argument checks on the host, then kernel launches on the
// caller's stream.  Nothing here allocates device memory or keeps state beyond the
// thread-local text of the last error.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

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

}  // namespace

extern "C" {

int eagle_abi_version(void) { return EAGLE_ABI_VERSION; }

const char* eagle_status_string(int status) {
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
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, const char* name) {
  if (!q || !k || !v || !parents || !out)
    return fail(EAGLE_ERR_NULL, "q, k, v, parents and out must be non-NULL");
  eagle_status_t st = check_attn_dims(B, N, Hq, Hkv, D, P);
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
                                      float scale, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return attn_impl(q, k, v, parents, nullptr, nullptr, B, N, Hq, Hkv, D, P, kv_cap, scale, out, lse,
                   workspace, workspace_bytes, stream, "eagle_tree_verify_attn");
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
                                            void* out, float* lse, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_pool || !v_pool || !block_table || !parents || !out)
    return fail(EAGLE_ERR_NULL, "q, k_pool, v_pool, block_table, parents and out must be non-NULL");
  eagle_status_t st = check_attn_dims(B, N, Hq, Hkv, D, P);
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
                                             int32_t kv_cap, float scale, void* out, float* lse,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
  if (!prefix_len && !tree_len)
    return fail(EAGLE_ERR_NULL, "prefix_len and tree_len are both NULL (use eagle_tree_verify_attn)");
  return attn_impl(q, k, v, parents, prefix_len, tree_len, B, N, Hq, Hkv, D, P, kv_cap, scale, out,
                   lse, workspace, workspace_bytes, stream, "eagle_tree_verify_attn_ragged");
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
                                    int32_t V, float* out_max, int32_t* out_argmax,
                                    float* out_lse, float* out_second, float* out_logits,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!hidden || !weight || !out_max || !out_argmax || !out_lse)
    return fail(EAGLE_ERR_NULL, "hidden, weight, out_max, out_argmax and out_lse must be non-NULL");
  eagle_status_t st = check_lm_dims(M, H, V);
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
                                const int32_t* draft_row, const float* target_logits,
                                const float* draft_logits, int32_t draft_rows,
                                const float* u_accept, const float* u_sample,
                                const int32_t* tree_len, int32_t B, int32_t N, int32_t V,
                                int32_t max_depth, int32_t* accept_len, int32_t* accept_path,
                                int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (!tokens || !parents || !draft_row || !target_logits || !draft_logits || !u_accept ||
      !u_sample || !accept_len || !accept_path || !out_tokens)
    return fail(EAGLE_ERR_NULL, "all pointers must be non-NULL");
  if (B < 1 || N < 1 || V < 1 || draft_rows < 1 || max_depth < 0)
    return fail(EAGLE_ERR_INVALID_ARG, "need B,N,V,draft_rows >= 1 and max_depth >= 0");
  if (N > EAGLE_MAX_TREE) return fail(EAGLE_ERR_UNSUPPORTED, "N=%d > %d", N, EAGLE_MAX_TREE);
  if (max_depth > EAGLE_MAX_TREE) return fail(EAGLE_ERR_INVALID_ARG, "max_depth=%d > %d", max_depth, EAGLE_MAX_TREE);
  eagle::SpecPlan pl = eagle::plan_accept_spec(B, N, V);
  pl.R = draft_rows;
  pl.max_depth = max_depth;
  pl.tree_len = tree_len;
  const size_t need = eagle::accept_spec_workspace_bytes(pl);
  if (!workspace || workspace_bytes < need)
    return fail(EAGLE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(EAGLE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return hip_status(eagle::launch_accept_spec(pl, tokens, parents, draft_row, target_logits,
                                              draft_logits, u_accept, u_sample, accept_len,
                                              accept_path, out_tokens, workspace, stream),
                    "eagle_accept_spec launch");
}

eagle_status_t eagle_accept_spec(const int32_t* tokens, const int32_t* parents,
                                 const int32_t* draft_row, const float* target_logits,
                                 const float* draft_logits, int32_t draft_rows,
                                 const float* u_accept, const float* u_sample, int32_t B,
                                 int32_t N, int32_t V, int32_t max_depth, int32_t* accept_len,
                                 int32_t* accept_path, int32_t* out_tokens, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return spec_impl(tokens, parents, draft_row, target_logits, draft_logits, draft_rows, u_accept,
                   u_sample, nullptr, B, N, V, max_depth, accept_len, accept_path, out_tokens,
                   workspace, workspace_bytes, stream);
}

eagle_status_t eagle_accept_spec_ragged(const int32_t* tokens, const int32_t* parents,
                                        const int32_t* draft_row, const float* target_logits,
                                        const float* draft_logits, int32_t draft_rows,
                                        const float* u_accept, const float* u_sample,
                                        const int32_t* tree_len, int32_t B, int32_t N, int32_t V,
                                        int32_t max_depth, int32_t* accept_len,
                                        int32_t* accept_path, int32_t* out_tokens,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  if (!tree_len) return fail(EAGLE_ERR_NULL, "tree_len is NULL (use eagle_accept_spec)");
  return spec_impl(tokens, parents, draft_row, target_logits, draft_logits, draft_rows, u_accept,
                   u_sample, tree_len, B, N, V, max_depth, accept_len, accept_path, out_tokens,
                   workspace, workspace_bytes, stream);
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
  const long long chunks = (V + 4095) / 4096;
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

}  // extern "C"
