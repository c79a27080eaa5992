/*
 * eagle_mi355.h - C ABI of the EAGLE / EAGLE-2 tree-verification library for
 * AMD MI355X (gfx950).
 *
 * One verification step of speculative decoding with a draft-token tree:
 *   eagle2_rerank          build the EAGLE-2 dynamic draft tree from draft logits
 *   eagle_tree_verify_attn tree attention of the target over prefix + tree
 *   eagle_lm_head_argmax   frozen LM head fused with per-row max/argmax/softmax stats
 *   eagle_accept_greedy    greedy acceptance (longest matching root path)
 *   eagle_accept_spec      multi-round speculative sampling acceptance
 * with _ragged forms of the attention and the acceptances for batches whose
 * sequences have different prefix and tree sizes, a _paged form of the attention
 * for KV caches kept in fixed-size pages, and, after acceptance:
 *   eagle_kv_commit        move the accepted path's K/V rows to the end of the prefix
 * and, before the step, the draft side that feeds eagle2_rerank:
 *   eagle_draft_expand     grow the EAGLE-2 draft tree depth by depth with a one-layer
 *                          draft head and the frozen LM head
 *
 * Sources (web pages on the method), cited per call below:
 *   [P1] "大模型推理效率突破：EAGLE推测解码算法在摩尔线程GPU的实践与优化" (adg.csdn.net)
 *   [P2] "大模型推理效率无损提升3倍，滑铁卢大学、北京大学等机构发布EAGLE" (www.0359xy.cn)
 *   [P3] "EAGLE-2：動態草稿樹讓 LLM 推論加速 4 倍而不失精度" (friday-blog-bgf.pages.dev)
 *
 * Conventions shared by every call
 * --------------------------------
 * Tree.  A draft tree of N nodes (N <= 64) per sequence is a parent array
 *   parents[b][i]: parents[b][0] == -1 (node 0 is the root: the last token already
 *   emitted) and 0 <= parents[b][i] < i for i > 0.  depth(root) = 0.
 * Memory.  Every pointer is DEVICE memory owned by the caller, except where a
 *   parameter name ends in _host.  The library allocates nothing, frees nothing
 *   and keeps no state between calls; scratch memory is the caller's `workspace`
 *   of at least the size the matching *_workspace() query returns (a query is a
 *   pure function of the sizes and never touches the GPU).  All arrays are dense
 *   row-major (C order) with the shapes given.
 * Types.  bf16 tensors are IEEE bfloat16 bit patterns (uint16 storage); fp32 is
 *   IEEE binary32; indices and tokens are int32.
 * Streams.  Work is enqueued on `stream` (0 = the null stream) and the call
 *   returns without waiting; outputs are valid when the stream reaches that point.
 *   Calls are reentrant; two calls may share a workspace only if they are ordered
 *   on one stream.
 * Errors.  Arguments are checked on the host before anything is launched; a bad
 *   argument returns a status and launches nothing.  EAGLE_ERR_HIP reports a HIP
 *   launch error; eagle_last_error() gives the text (thread-local).  Kernels never
 *   read or write outside the buffers described here whatever the CONTENT of
 *   parents / tokens / draft_row; for contents that break the tree rules the
 *   results are unspecified (eagle_check_tree() validates a tree on the host).
 */
#ifndef EAGLE_MI355_H
#define EAGLE_MI355_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EAGLE_ABI_VERSION 3
#define EAGLE_MAX_TREE 64   /* nodes per sequence, root included */
#define EAGLE_MAX_TOPK 64

typedef enum {
  EAGLE_OK = 0,
  EAGLE_ERR_NULL = 1,          /* a required pointer is NULL */
  EAGLE_ERR_INVALID_ARG = 2,   /* a size is out of range or inconsistent */
  EAGLE_ERR_UNSUPPORTED = 3,   /* valid but not implemented (e.g. N > 64, D not 64/128) */
  EAGLE_ERR_WORKSPACE = 4,     /* workspace missing or smaller than the query's size */
  EAGLE_ERR_TREE = 5,          /* eagle_check_tree: parent array breaks the tree rules */
  EAGLE_ERR_HIP = 6            /* a HIP runtime call failed; see eagle_last_error() */
} eagle_status_t;

/* Element type of the attention and LM-head operands.  EAGLE_BF16 is the one this
 * library implements; EAGLE_F32 names fp32 operands (an fp32 model such as the
 * tiny CPU-scale configuration) and is answered with EAGLE_ERR_UNSUPPORTED: such
 * tensors are rounded to bf16 by the caller.  Any other value is
 * EAGLE_ERR_INVALID_ARG. */
typedef enum {
  EAGLE_BF16 = 0,
  EAGLE_F32 = 1
} eagle_dtype_t;

/* Sibling model of eagle_accept_spec (see there). */
typedef enum {
  EAGLE_SPEC_SAMPLED = 0,
  EAGLE_SPEC_POINT_MASS = 1
} eagle_spec_mode_t;

/* Version of this ABI (EAGLE_ABI_VERSION of the built library). */
int eagle_abi_version(void);

/* Static text for a status value (never NULL). */
const char* eagle_status_string(eagle_status_t status);

/* Detail text of the calling thread's last error (empty string if none). */
const char* eagle_last_error(void);

/*
 * Host-side validation of B parent arrays of N nodes (parents_host[B][N], HOST
 * memory): EAGLE_OK if every array has parents[0] == -1 and 0 <= parents[i] < i,
 * EAGLE_ERR_TREE otherwise, EAGLE_ERR_INVALID_ARG if B < 1 or N < 1.
 */
eagle_status_t eagle_check_tree(const int32_t* parents_host, int32_t B, int32_t N);

/*
 * Tree-verify attention.  [P1] innovations list item 2 and [P2] workflow
 * paragraph: every path of the draft tree is verified in ONE target pass by
 * turning the tree into an attention mask.  For sequence b, tree node i and query
 * head h (KV head g = h / (Hq / Hkv)), with keys
 *     J(i) = {0 .. P-1}  U  {P + a : a is an ancestor of i or a == i}
 * and scores s_j = scale * <q[b][i][h], k[b][g][j]>:
 *     out[b][i][h] = sum_j softmax(s)_j * v[b][g][j]
 *     lse[b][i][h] = log(sum_j exp(s_j))          (natural log)
 * q, k are taken as already position-encoded.
 *
 *   q    bf16 [B][N][Hq][D]
 *   k, v bf16 [B][Hkv][kv_cap][D]: rows 0..P-1 hold the prefix, rows P..P+N-1 the
 *        tree nodes in node order; rows >= P+N are never read.  kv_cap >= P + N.
 *   parents int32 [B][N]
 *   out  bf16 [B][N][Hq][D] (written)
 *   lse  fp32 [B][N][Hq] (written; may be NULL)
 *   scale > 0 (usually 1/sqrt(D)); D in {64, 128}; Hq % Hkv == 0; N <= 64; P >= 0.
 *   dtype  EAGLE_BF16 (the type of q, k, v and out)
 *   kv_cap the row capacity of k and v per (sequence, KV head), so that a cache
 *          allocated once for the longest context can be passed as it is
 * Workspace: eagle_tree_verify_attn_workspace(B, N, Hq, Hkv, D, P) bytes (it holds
 * split-KV partial results; 0 means none is needed and workspace may be NULL).
 */
size_t eagle_tree_verify_attn_workspace(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t P);
eagle_status_t eagle_tree_verify_attn(const void* q, const void* k, const void* v,
                                      const int32_t* parents, int32_t B, int32_t N, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t P, int32_t kv_cap,
                                      float scale, eagle_dtype_t dtype, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * Frozen LM head with fused row statistics.  [P2] paragraphs on the
 * auto-regression head and the workflow: the target's frozen classification head
 * turns a feature into the next-token distribution; [P1] greedy decoding takes its
 * top-1.  logits = hidden @ weight^T, then per row m:
 *     out_max[m]    = max_x logits[m][x]
 *     out_argmax[m] = smallest x attaining that max
 *     out_second[m] = max over x != out_argmax[m]   (judges near-ties; may be NULL)
 *     out_lse[m]    = log(sum_x exp(logits[m][x]))   (natural log)
 *     out_logits    = the fp32 logits [M][V] (may be NULL; needed by eagle_accept_spec)
 *
 *   hidden bf16 [M][H], weight bf16 [V][H] (nn.Linear layout).  H % 64 == 0, V >= 2.
 *   dtype EAGLE_BF16 (the type of hidden and weight)
 *   out_max, out_lse, out_second fp32 [M]; out_argmax int32 [M]
 * Workspace: eagle_lm_head_workspace(M, H, V) bytes (never 0).
 */
size_t eagle_lm_head_workspace(int32_t M, int32_t H, int32_t V);
eagle_status_t eagle_lm_head_argmax(const void* hidden, const void* weight, int32_t M, int32_t H,
                                    int32_t V, eagle_dtype_t dtype, float* out_max,
                                    int32_t* out_argmax, float* out_lse, float* out_second,
                                    float* out_logits, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * eagle_lm_head_argmax without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it).  Same arguments and results as eagle_lm_head_argmax minus the workspace: the
 * scratch (the per-vocabulary-tile row partials) lives in a static device array of
 * EAGLE_LM_HEAD_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until
 * the process ends; its address on a device is looked up on the first call made with
 * that device current.  Sizes whose eagle_lm_head_workspace(M, H, V) exceeds the array
 * return EAGLE_ERR_UNSUPPORTED (at V = 128256 that is M > 1046).  The call allocates
 * nothing.  Every call on one GPU uses the same array: calls that overlap on a GPU (two
 * streams, or two host threads) race and their results are undefined; calls ordered
 * on one stream are safe (nothing in the array needs clearing between them).
 */
#define EAGLE_LM_HEAD_NOALLOC_SCRATCH_BYTES (8 << 20)
eagle_status_t eagle_lm_head_argmax_noalloc(const void* hidden, const void* weight, int32_t M,
                                            int32_t H, int32_t V, eagle_dtype_t dtype,
                                            float* out_max, int32_t* out_argmax, float* out_lse,
                                            float* out_second, float* out_logits,
                                            hipStream_t stream);

/*
 * Greedy acceptance.  [P1] greedy decoding paragraph and the figure paragraph
 * after it; [P2] speculative sampling paragraph.  Node i (i > 0) survives when it
 * and every node above it matches: tokens[i] == target_argmax[parents[i]] and its
 * parent survives (the root always survives).  The winner v* is the deepest
 * surviving node of depth <= max_depth (lowest index among equally deep ones);
 * alpha = depth(v*) drafts are accepted and alpha + 1 tokens are emitted.
 *
 *   tokens, parents, target_argmax int32 [B][N] (target_argmax[b][i] = the target's
 *     top-1 next token after node i; tokens[b][0] is the root token, not checked)
 *   max_depth >= 0: capacity of the path outputs is max_depth + 1
 *   accept_len  int32 [B]                 alpha
 *   accept_path int32 [B][max_depth + 1]  root .. v* node indices, then -1
 *   out_tokens  int32 [B][max_depth + 1]  tokens of path[1..], then target_argmax[v*], then -1
 */
eagle_status_t eagle_accept_greedy(const int32_t* tokens, const int32_t* parents,
                                   const int32_t* target_argmax, int32_t B, int32_t N,
                                   int32_t max_depth, int32_t* accept_len, int32_t* accept_path,
                                   int32_t* out_tokens, hipStream_t stream);

/*
 * Multi-round speculative sampling.  [P1] stochastic verification paragraph (q is
 * the target, p the draft; accept a draft token t when a uniform is below
 * min(1, q(t)/p(t)), otherwise correct the target and retry), [P2] multi-round
 * speculative sampling section (recursive form over the token tree, keeping the
 * target distribution; the draft records each sampled token's probability as it
 * drafts), [P3] section 2, speculative decoding basics.  At the current node v
 * (starting at the root): q = exp(target_logits[b][v] - target_lse[b][v]),
 * p = exp(draft_logits[b][r] - draft_lse[b][r]) with r = draft_row[b][v]; the
 * children of v are tried in ascending node index with u_accept[b][child]: accept
 * when u < min(1, q'(t)/p(t)) where q' is the corrected target (q' = q for the first
 * child); a rejection replaces q' by the normalised positive part of (q' - p).  An
 * accepted child becomes the current node.  When every child is rejected, one
 * token is drawn from q' with u_sample[b][v]; at a node with no children, with
 * draft_row < 0, or at depth max_depth, one token is drawn from q.  Draws are
 * inverse-CDF: the smallest x whose cumulative mass exceeds u times the total.
 *
 * mode selects what the siblings are:
 *   EAGLE_SPEC_SAMPLED     the children were drawn from the node's draft distribution
 *                          p (the pages' rule as stated above; exact for such draws);
 *   EAGLE_SPEC_POINT_MASS  the children are the draft's deterministic proposals, as
 *                          in EAGLE-2's top-k expansion ([P3] section 2): the draft
 *                          distribution behind child t is the point mass at t, so t is
 *                          accepted when u < q'(t), and a rejection sets q'(t) to zero
 *                          and renormalises (exact for any fixed set of siblings).
 *                          draft_logits and draft_lse are not read in this mode; a node
 *                          still needs a valid draft_row to have its children tried.
 * Any other mode value is EAGLE_ERR_INVALID_ARG.
 *
 *   tokens, parents int32 [B][N]; max_depth >= 0
 *   target_logits fp32 [B][N][V]; target_lse fp32 [B][N] (log-sum-exp of each target
 *     row, as eagle_lm_head_argmax writes it to out_lse) or NULL
 *   draft_logits fp32 [B][draft_rows][V]; draft_lse fp32 [B][draft_rows] (as
 *     eagle2_rerank writes it) or NULL
 *   draft_row int32 [B][N] (in [-1, draft_rows)); draft_rows >= 1
 *   u_accept, u_sample fp32 [B][N] in [0, 1)
 *   outputs as eagle_accept_greedy; on a spin timeout inside the kernel (a GPU that
 *     does not run the sequence's workgroups together) every output of that
 *     sequence is -1, accept_len included.
 * When a normaliser is NULL the kernel forms it from the logits itself (one more
 * cross-workgroup exchange per visited node); given ones are used as they are.
 * Workspace: eagle_accept_spec_workspace(B, N, V) bytes.
 */
size_t eagle_accept_spec_workspace(int32_t B, int32_t N, int32_t V);
eagle_status_t eagle_accept_spec(const int32_t* tokens, const int32_t* parents, int32_t B,
                                 int32_t N, int32_t V, int32_t max_depth,
                                 const float* target_logits, const float* target_lse,
                                 const float* draft_logits, const float* draft_lse,
                                 const int32_t* draft_row, int32_t draft_rows,
                                 const float* u_accept, const float* u_sample,
                                 eagle_spec_mode_t mode, int32_t* accept_len,
                                 int32_t* accept_path, int32_t* out_tokens, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Ragged batches.  [P3] section 4 (batch sizes above one are the method's weak spot)
 * and its closing remarks (continuous batching): the sequences of one batch carry
 * prefixes and trees of different sizes.  These calls take the same arguments as
 * the uniform ones, where N and P are now the largest tree and prefix the layouts
 * are sized for, plus device arrays
 *   prefix_len int32 [B]  this sequence's prefix length (clamped to [0, P])
 *   tree_len   int32 [B]  this sequence's tree size     (clamped to [1, N])
 * (for attention either may be NULL, meaning "all equal to the maximum").  Sequence
 * b's tree rows follow its own prefix: k, v row prefix_len[b] + i holds node i.  Only
 * nodes i < tree_len[b] exist: rows of q, parents, tokens, target_argmax, draft_row,
 * u_accept, u_sample and target_logits past them are padding (never read as nodes),
 * and the attention writes no output or lse for them.  The LM head needs no ragged
 * form: its rows are independent, so the trees' rows are passed as one [M][H] block.
 * Workspace sizes: those of the uniform calls at the maxima.
 */
eagle_status_t eagle_tree_verify_attn_ragged(const void* q, const void* k, const void* v,
                                             const int32_t* parents, const int32_t* prefix_len,
                                             const int32_t* tree_len, int32_t B, int32_t N,
                                             int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                             int32_t kv_cap, float scale, eagle_dtype_t dtype,
                                             void* out, float* lse, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);
eagle_status_t eagle_accept_greedy_ragged(const int32_t* tokens, const int32_t* parents,
                                          const int32_t* target_argmax, const int32_t* tree_len,
                                          int32_t B, int32_t N, int32_t max_depth,
                                          int32_t* accept_len, int32_t* accept_path,
                                          int32_t* out_tokens, hipStream_t stream);
eagle_status_t eagle_accept_spec_ragged(const int32_t* tokens, const int32_t* parents,
                                        const int32_t* tree_len, int32_t B, int32_t N, int32_t V,
                                        int32_t max_depth, const float* target_logits,
                                        const float* target_lse, const float* draft_logits,
                                        const float* draft_lse, const int32_t* draft_row,
                                        int32_t draft_rows, const float* u_accept,
                                        const float* u_sample, eagle_spec_mode_t mode,
                                        int32_t* accept_len, int32_t* accept_path,
                                        int32_t* out_tokens, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * Paged KV cache.  [P3] section 4 (limitations: dynamic draft trees strain paged
 * cache management such as PagedAttention).  Same computation as
 * eagle_tree_verify_attn, but the K and V rows of each (sequence, KV head) sit in
 * fixed-size pages of shared pools:
 *   k_pool, v_pool bf16 [num_blocks][Hkv][page_size][D]   (16-byte aligned)
 *   block_table int32 [B][max_pages]: row r (prefix rows, then tree rows in node
 *     order, r < P + N) of sequence b lives in block block_table[b][r / page_size]
 *     at slot r % page_size.  Entries are clamped to [0, num_blocks - 1] on the
 *     device, so any table content stays inside the pools.
 *   page_size: a power of two, 1 .. 4096; max_pages * page_size >= P + N.
 * Very small pages with a long prefix are rejected (EAGLE_ERR_UNSUPPORTED) when a
 * split's slice of the block table would not fit on chip.
 * Workspace: eagle_tree_verify_attn_paged_workspace(B, N, Hq, Hkv, D, P, page_size).
 */
size_t eagle_tree_verify_attn_paged_workspace(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t P, int32_t page_size);
eagle_status_t eagle_tree_verify_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                                            const int32_t* block_table, const int32_t* parents,
                                            int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                            int32_t D, int32_t P, int32_t page_size,
                                            int32_t max_pages, int32_t num_blocks, float scale,
                                            eagle_dtype_t dtype, void* out, float* lse,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/*
 * EAGLE-2 dynamic draft tree.  [P3] section 2 (dynamic draft tree: confidence
 * scoring, deep-where-confident / wide-where-not expansion, greedy maximisation of
 * the expected acceptance length under a draft-token budget); [P1] innovations
 * list items 1 and 3 (top tokens per draft step, pruning to high-probability
 * paths).  Per sequence, draft_logits holds R = 1 + (depth-1)*top_k rows: row 0
 * is the root's draft distribution, row 1 + (d-1)*top_k + j the one of frontier
 * slot j at depth d.  Each expanded node proposes its row's top_k tokens (ties to
 * the lower token id) with score = parent score + log_softmax(row)[token]; the
 * frontier of depth d is the top_k depth-d candidates (score descending, then
 * candidate id ascending; ids count depth by depth, slot by slot, rank by rank);
 * the tree is the root plus the n_nodes - 1 best candidates overall, output
 * breadth first (ascending candidate id).
 *
 *   draft_logits fp32 [B][R][V]; root_token int32 [B]
 *   1 <= top_k <= 64, top_k <= V; depth >= 1; 1 <= n_nodes <= 64;
 *   n_nodes - 1 <= top_k + (depth-1)*top_k*top_k
 *   tokens, parents, depths int32 [B][n_nodes]; scores fp32 [B][n_nodes] (root 0)
 *   draft_row int32 [B][n_nodes]: the row holding the node's own expansion (root 0,
 *     -1 for nodes that were not expanded); draft_lse fp32 [B][R]: log-sum-exp of
 *     every row.
 * Workspace: eagle2_rerank_workspace(B, V, top_k, depth) bytes.
 */
size_t eagle2_rerank_workspace(int32_t B, int32_t V, int32_t top_k, int32_t depth);
eagle_status_t eagle2_rerank(const float* draft_logits, const int32_t* root_token, int32_t B,
                             int32_t V, int32_t top_k, int32_t depth, int32_t n_nodes,
                             int32_t* tokens, int32_t* parents, int32_t* depths, float* scores,
                             int32_t* draft_row, float* draft_lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Per-depth EAGLE-2 draft expansion.  [P2] auto-regression head and workflow
 * paragraphs (the head reads the parent's feature and the embedding of the node's
 * token, predicts the node's feature, and the target's frozen LM head gives the next
 * token distribution; repeated, this grows the draft tree); [P2] training paragraph
 * (the head is one transformer layer); [P3] section 2 (dynamic tree under a token
 * budget).  The layer, for expansion row r with parent feature f and token t:
 *     u = [f ; E[t]];  x = W_fc u;  a = rms(x) g1;  q, k, v = W_qkv a
 *     h = x + W_o Attn_r(q, k, v);  b = rms(h) g2
 *     y = h + W_down( silu(W_gate b) * (W_up b) );  logits_r = W_lm y
 * rms(z) = z / sqrt(mean(z^2) + eps); GEMM inputs are bf16, accumulation and the
 * residual stream fp32, y is stored in bf16.  Attn_r: grouped-query attention with
 * the given scale over the draft cache's prefix rows 0..P-1 and the rows P + a of the
 * ancestors a of r in the expansion (itself included); no position encoding.
 *
 * Rows: row 0 is the root (feature f0[b], token root_token[b]); depth by depth, the
 * top_k best candidates of depth d (by cumulative log-probability, ties to the lower
 * candidate id, exactly as eagle2_rerank ranks them) take rows 1 + (d-1)*top_k + j,
 * read the feature y of the row that proposed them and run the head.  Row r's
 * logits are written to draft_logits[b][r]; after the last depth the tree is built
 * from them as eagle2_rerank would (same outputs), so the tree, draft_logits and
 * draft_lse can go straight to eagle_tree_verify_attn / eagle_accept_spec.
 *
 *   head: the weights, bf16 row-major ([out][in], 16-byte aligned) except the fp32
 *     gains: embed [V][H]; w_fc [H][2H]; w_qkv [(Hq + 2 Hkv) D][H] (q rows, then k
 *     rows, then v rows, head-major); w_o [H][Hq D]; w_gate_up [2I][H] (gate rows,
 *     then up rows); w_down [H][I]; w_lm [V][H] (the frozen LM head); g1, g2 [H]
 *   f0 bf16 [B][H]: the target's feature at the root; root_token int32 [B]
 *   k_cache, v_cache bf16 [B][Hkv][kv_cap][D]: the draft layer's cache; rows 0..P-1
 *     are read, rows P .. P + R - 1 (R = 1 + (depth-1)*top_k) are overwritten with
 *     the expansion rows' keys and values; kv_cap >= P + R
 *   H, I multiples of 64; D in {64, 128}; Hq % Hkv == 0; R <= 64; the eagle2_rerank
 *     limits on V, top_k, depth, n_nodes
 *   outputs: tokens, parents, depths, scores, draft_row [B][n_nodes] and draft_lse
 *     [B][R] as eagle2_rerank; draft_logits fp32 [B][R][V]; features bf16 [B][R][H]
 *     (y of every row); row_token, parent_row int32 [B][R] (the token of each row and
 *     the row that proposed it; -1 for the root)
 * Workspace: eagle_draft_expand_workspace(B, H, Hq, Hkv, D, I, V, P, kv_cap, top_k,
 * depth) bytes (0 for invalid sizes).  All launches go to `stream`.
 */
typedef struct {
  const void* embed;
  const void* w_fc;
  const void* w_qkv;
  const void* w_o;
  const void* w_gate_up;
  const void* w_down;
  const void* w_lm;
  const float* g1;
  const float* g2;
} eagle_draft_head;

size_t eagle_draft_expand_workspace(int32_t B, int32_t H, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t I, int32_t V, int32_t P, int32_t kv_cap, int32_t top_k,
                                    int32_t depth);
eagle_status_t eagle_draft_expand(const eagle_draft_head* head, const void* f0,
                                  const int32_t* root_token, void* k_cache, void* v_cache, int32_t B,
                                  int32_t H, int32_t Hq, int32_t Hkv, int32_t D, int32_t I, int32_t V,
                                  int32_t P, int32_t kv_cap, int32_t top_k, int32_t depth,
                                  int32_t n_nodes, float scale, float eps, int32_t* tokens,
                                  int32_t* parents, int32_t* depths, float* scores,
                                  int32_t* draft_row, float* draft_logits, float* draft_lse,
                                  void* features, int32_t* row_token, int32_t* parent_row,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * KV-cache commit after acceptance.  [P3] section 4 (limitations: the dynamic
 * draft tree fragments the KV cache).  The tree's K/V rows follow the prefix in node
 * order (row P + i holds node i, as eagle_tree_verify_attn reads them).  After a
 * root path path[0] = 0, path[1], ..., path[alpha] is accepted, its rows become the
 * next prefix rows in path order, in place, in every layer, sequence and KV head:
 *     cache[l][b][g][P + i] = old cache[l][b][g][P + path[b][i]],  i = 0 .. alpha;
 * every other row keeps its contents, so the next step's prefix is P + alpha + 1.
 *
 *   k_cache, v_cache bf16 [L][B][Hkv][kv_cap][D] (device, 16-byte aligned), updated
 *     in place; D in {64, 128}
 *   accept_len int32 [B] (alpha; sequences with alpha < 0 are left unchanged) and
 *   accept_path int32 [B][path_len] as written by eagle_accept_greedy /
 *     eagle_accept_spec (path_len = max_depth + 1 <= 65); alpha is capped at
 *     path_len - 1, and path entries that name no row of the cache are skipped
 *   P + path_len <= kv_cap
 */
eagle_status_t eagle_kv_commit(void* k_cache, void* v_cache, const int32_t* accept_len,
                               const int32_t* accept_path, int32_t L, int32_t B, int32_t Hkv,
                               int32_t D, int32_t P, int32_t kv_cap, int32_t path_len,
                               hipStream_t stream);

/*
 * Measurement probes (not part of the verification step).  They measure, on the GPU
 * they run on, the two ceilings the kernels above are judged against: the HBM read
 * bandwidth a streaming kernel reaches and the rate the bf16 matrix cores sustain.
 *
 * eagle_calib_stream_read: reads `bytes` (a positive multiple of 16) from the device
 *   buffer `src` (16-byte aligned) once, in 16-byte non-temporal loads spread over
 *   4096 workgroups; `sink` is a device buffer of at least 4096 uint32 that is
 *   written only in a case that cannot occur (it keeps the loads from being dropped).
 * eagle_calib_mfma_bf16: 2048 workgroups of four waves, each wave running four
 *   independent chains of `iters` v_mfma_f32_32x32x16_bf16 on register operands;
 *   `out` (device, at least 2048 * 256 floats) receives one value per lane.
 *   eagle_calib_mfma_bf16_flops(iters) is the number of flops one call performs
 *   (0 for iters < 1).
 */
eagle_status_t eagle_calib_stream_read(const void* src, size_t bytes, void* sink,
                                       hipStream_t stream);
double eagle_calib_mfma_bf16_flops(int32_t iters);
eagle_status_t eagle_calib_mfma_bf16(int32_t iters, float* out, size_t out_floats,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE_MI355_H */
