// Host-side launch plans and launchers shared between the kernel files and the
// C-ABI entry points.  Plans are pure functions of the problem sizes (the
// workspace queries use them without touching the GPU).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace eagle {

// MI355X: 256 CUs.  Split-KV aims at about one attention workgroup per CU.
constexpr int kNumCUs = 256;
constexpr int kMinSplitKeys = 256;

struct AttnPlan {
  int B, N, Hq, Hkv, G, D, P, kv_cap;
  int R;          // query rows per (sequence, KV head) = N * G
  int waves;      // waves per workgroup
  int RB;         // row blocks per pair
  int Rpad;       // RB * waves * 32
  int S;          // key splits
  int split_len;  // keys per split (multiple of 32); the last split also takes the tree
  float c;        // scale * log2(e)
  // ragged batches (may be null): per-sequence prefix length (<= P) and tree size
  // (<= N); P and N above are then the maxima the plan and the layouts are sized for
  const int32_t* prefix_len;
  const int32_t* tree_len;
  // paged KV (may be null): k, v are pools [num_blocks][Hkv][page_size][D] and row r
  // of sequence b lives in block block_table[b][r / page_size] at slot r % page_size
  const int32_t* block_table;
  int page_shift;   // log2(page_size)
  int max_pages;    // row stride of block_table
  int num_blocks;
  // query subset (nq > 0): only nodes node0 .. node0+nq-1 of the N-node tree are
  // computed (the draft expansion's newest rows); masks and keys cover the whole tree
  int node0, nq;
  // ragged batches with split keys (device memory in the workspace, written by the
  // attention kernel's workgroup 0 from prefix_len for the merge): [0] split length,
  // [1] number of (sequence, split) items, [2, 2+B) first item of each sequence,
  // [2+B, 2+2B) its number of splits.  Non-null also tells the attention kernels to
  // plan the splits themselves.  Null otherwise.
  int* dplan;
};

// paged KV: a split's slice of the block table is staged in LDS
constexpr int kMaxSplitPages = 1024;
AttnPlan plan_tree_attn_paged(int B, int N, int Hq, int Hkv, int D, int P, int page_shift);

AttnPlan plan_tree_attn(int B, int N, int Hq, int Hkv, int D, int P, int kv_cap);
AttnPlan plan_tree_attn_rows(int B, int N, int node0, int nq, int Hq, int Hkv, int D, int P,
                             int kv_cap);
size_t tree_attn_workspace_bytes(const AttnPlan& pl);
hipError_t launch_tree_attn(const AttnPlan& pl, float scale, const void* q, const void* k,
                            const void* v, const int32_t* parents, void* out, float* lse,
                            void* workspace, hipStream_t stream);

struct LmPlan {
  int M, H, V;
  int variant;    // tile-shape variant
  int mrows;      // hidden rows per workgroup
  int vrows;      // vocabulary rows per workgroup
  int nvt;        // vocabulary tiles
  int nmb;        // hidden-row blocks
  int ksplit;     // split-K factor (1: whole rows, with the fused row statistics)
  int kb_per;     // 64-column blocks per split
};

LmPlan plan_lm_head(int M, int H, int V);
size_t lm_head_workspace_bytes(const LmPlan& pl);
// Plain GEMM out[M][N] = X[M][K] W[N][K]^T in fp32 on the LM-head kernel, with split-K
// (fp32 partials summed by a second kernel) when the N tiles alone leave most CUs idle.
// A GEMM output left as its split-K slices: element i is p[i] + p[stride + i] + ... +
// p[(S-1) stride + i], summed in slice order (S = 1: the plain output p).
struct F32Slices {
  const float* p;
  int S;
  size_t stride;
};

size_t gemm_f32_workspace_bytes(int M, int K, int N);
// launch_gemm_f32 without its slice-summing pass: the result as slices (in the
// workspace when the GEMM splits K, else in `out`), for a consumer that sums them
hipError_t launch_gemm_f32_slices(int M, int K, int N, const void* X, const void* W, float* out,
                                  void* workspace, F32Slices* result, hipStream_t stream);
hipError_t launch_gemm_f32(int M, int K, int N, const void* X, const void* W, float* out,
                           void* workspace, hipStream_t stream);
hipError_t launch_lm_head(const LmPlan& pl, const void* hidden, const void* W, float* out_max,
                          int32_t* out_argmax, float* out_lse, float* out_second, float* out_logits,
                          void* workspace, hipStream_t stream);

hipError_t launch_accept_greedy(const int32_t* tokens, const int32_t* parents,
                                const int32_t* target_argmax, const int32_t* tree_len, int B,
                                int N, int max_depth, int32_t* accept_len, int32_t* accept_path,
                                int32_t* out_tokens, hipStream_t stream);

struct SpecPlan {
  int B, N, V, R, max_depth;
  int mode;       // 0: siblings drawn from the draft distribution; 1: deterministic (point mass)
  int chunks;     // vocabulary chunks (one workgroup each) per sequence
  const int32_t* tree_len;   // ragged batches: per-sequence tree size (<= N), may be null
  // the callers' log-sum-exp of every target row [B][N] and draft row [B][R] (may be
  // null: the kernel then forms the normalisers itself)
  const float* target_lse;
  const float* draft_lse;
};
SpecPlan plan_accept_spec(int B, int N, int V);
size_t accept_spec_workspace_bytes(const SpecPlan& pl);
hipError_t launch_accept_spec(const SpecPlan& pl, const int32_t* tokens, const int32_t* parents,
                              const int32_t* draft_row, const float* target_logits,
                              const float* draft_logits, const float* u_accept,
                              const float* u_sample, int32_t* accept_len, int32_t* accept_path,
                              int32_t* out_tokens, void* workspace, hipStream_t stream);

struct RerankPlan {
  int B, V, k, depth, R, n_nodes;
  int chunks;     // vocabulary chunks per row for the top-k / log-sum-exp pass
  int chunk_len;  // vocabulary entries per chunk
  int row0, nrows;   // rows row0 .. row0+nrows-1 of every sequence take the row pass
};
RerankPlan plan_rerank(int B, int V, int top_k, int depth, int n_nodes);
size_t rerank_workspace_bytes(const RerankPlan& pl);
hipError_t launch_rerank(const RerankPlan& pl, const float* draft_logits, const int32_t* root_token,
                         int32_t* tokens, int32_t* parents, int32_t* depths, float* scores,
                         int32_t* draft_row, float* draft_lse, void* workspace, hipStream_t stream);

// measurement probes (calib.hip): grid sizes and launchers
constexpr int kCalibReadBlocks = 4096;   // 256-thread workgroups of the streaming read
constexpr int kCalibMfmaBlocks = 2048;   // 256-thread workgroups of the MFMA loop
hipError_t launch_calib_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream);
hipError_t launch_calib_mfma_bf16(int iters, float* out, hipStream_t stream);

// KV commit: at most max_depth + 1 <= 65 accepted rows per (layer, sequence, head)
constexpr int kMaxCommitRows = 65;
hipError_t launch_kv_commit(void* k_cache, void* v_cache, const int32_t* accept_len,
                            const int32_t* accept_path, int L, int B, int Hkv, int D, int P,
                            int kv_cap, int path_len, hipStream_t stream);

}  // namespace eagle

namespace eagle {
int rerank_max_candidates();
int rerank_chunk_len();      // vocabulary entries per chunk of the row pass
// per-depth draft expansion: the row pass over rows [row0, row0 + nrows) of every
// sequence (plan with those fields set), and the frontier of depth d (d >= 1): for
// slot j, row r = 1 + (d-1)*k + j gets the token of the j-th best depth-d candidate
// and the row of the node that proposed it (0 for the root)
hipError_t launch_rerank_rows(const RerankPlan& pl, const float* draft_logits, float* draft_lse,
                              void* workspace, hipStream_t stream);
hipError_t launch_rerank_tree(const RerankPlan& pl, const int32_t* root_token, const float* draft_lse,
                              void* workspace, int32_t* tokens, int32_t* parents, int32_t* depths,
                              float* scores, int32_t* draft_row, hipStream_t stream);
hipError_t launch_draft_frontier(const RerankPlan& pl, int d, const float* draft_lse, void* workspace,
                                 int32_t* row_token, int32_t* parent_row, hipStream_t stream);
int rerank_max_row_list();   // R * top_k limit (also caps R at 512 and chunks * top_k at 1024)

// per-depth draft expansion (draft.hip): sizes shared by the glue kernels
struct DraftDims {
  int B, H, Hq, Hkv, D, I, V, P, kv_cap, R;
};
hipError_t launch_draft_gather_input(const DraftDims& dd, int row0, int nr, const void* f0,
                                     const int32_t* root_token, const void* embed, const void* feats,
                                     const int32_t* row_token, const int32_t* parent_row, void* X,
                                     hipStream_t s);
hipError_t launch_draft_rms(int M, int H, float eps, F32Slices a, const float* res,
                            const float* gain, float* res_out, void* norm_out, hipStream_t s);
hipError_t launch_draft_qkv_scatter(const DraftDims& dd, int row0, int nr, F32Slices qkv, void* qbuf,
                                    void* k_cache, void* v_cache, hipStream_t s);
hipError_t launch_draft_gather_rows(const DraftDims& dd, int row0, int nr, int width, const void* src,
                                    void* dst, hipStream_t s);
hipError_t launch_draft_silu_mul(int M, int I, const float* gu, void* z, hipStream_t s);
hipError_t launch_draft_output(const DraftDims& dd, int row0, int nr, F32Slices d, const float* h,
                               void* y, void* feats, hipStream_t s);
hipError_t launch_draft_place_logits(const DraftDims& dd, int row0, int nr, const float* src,
                                     float* draft_logits, hipStream_t s);
hipError_t launch_draft_init_rows(int B, int R, const int32_t* root_token, int32_t* row_token,
                                  int32_t* parent_row, hipStream_t s);

}  // namespace eagle

