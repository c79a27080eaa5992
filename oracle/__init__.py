"""Plain, slow, fp64 CPU oracle for one EAGLE / EAGLE-2 verification step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  The HIP library never
calls it, and it shares no code with the HIP library: no kernels, headers,
helpers, tables or pre/post-processing.  Its inputs come from the seeded
generators in ``synth`` (or from fixtures written by scripts that call only this
package).

Sources, cited in each function by page and passage:
  [P1] "大模型推理效率突破：EAGLE推测解码算法在摩尔线程GPU的实践与优化" (adg.csdn.net)
  [P2] "大模型推理效率无损提升3倍，滑铁卢大学、北京大学等机构发布EAGLE" (www.0359xy.cn)
  [P3] "EAGLE-2：動態草稿樹讓 LLM 推論加速 4 倍而不失精度" (friday-blog-bgf.pages.dev)

Pins (tests/test_oracle_*.py) tie every function here to something other than
itself: library routines on special cases (causal attention, log-softmax, top-k),
closed forms (exact enumeration of the speculative-sampling output law), the
pages' worked examples (tests/golden/), brute force on tiny inputs and
invariants.  No function here is "parity unpinned".
"""
from .tree import ancestor_sets, children_of, node_depths  # noqa: F401
from .attention import tree_verify_attention, tree_verify_attention_node  # noqa: F401
from .lm_head import lm_head_logits, lm_head_row_stats, lm_head  # noqa: F401
from .accept import (accept_greedy, accept_spec, sample_inverse_cdf, spec_node_round,  # noqa: F401
                     spec_node_round_point_mass)
from .rerank import eagle2_rerank, grow_tree  # noqa: F401
from .draft import bf16_round, draft_expand, draft_layer_row  # noqa: F401
from .kv_commit import kv_commit  # noqa: F401
from .ragged import accept_greedy_ragged, accept_spec_ragged, tree_verify_attention_ragged  # noqa: F401
from .paged import gather_pages, tree_verify_attention_paged  # noqa: F401
