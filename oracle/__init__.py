"""fp64 CPU oracle for windowed KV-cache eviction.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product
path (the HIP library and its binding) never calls it, and it shares no
code, table or constant generator with that path.

Plain, slow, obviously-correct definitions in float64 (numpy), each function
citing the passage of the pages it restates:

  [PI]  "A Probabilistic Interpretation of KV Cache Eviction" (Geh, Chen,
        Israel, Grover, Van den Broeck)
  [DK]  "DropKV: Decoupling Residual-Output Perturbation for Near-Optimal
        KV-Cache Eviction"
  [IT]  "Information-Theoretic Token Eviction and KV-Cache Compression for
        Memory-Bounded Long-Context LLM Inference" (research-topic note)

Parity status per function is stated in each module header.
"""
from .attention import window_attention, row_positions  # noqa: F401
from .score import perturbation_scores, group_scores, max_pool, score_workload  # noqa: F401
from .select import (  # noqa: F401
    topk_select, proposal_log, proposal, expected_distinct, expected_samples_search,
    inclusion_prob, gumbel_keys, sample_select, select_workload, global_search, global_sample_select,
    draw_counts, literal_select,
)
from .philox import philox4x64_10, uniform53  # noqa: F401
from .decode import compact, decode_attention, decode_alg1_literal  # noqa: F401
