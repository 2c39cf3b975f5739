"""CPU oracle for the DSV hot path: plain, slow, float64/int64 numpy.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import this package. The HIP library never calls it, and it shares no code,
header, table or helper with the HIP path; the two meet only in the seeded input generator
(`synth`), which holds none of the method's arithmetic.

What it computes, following the DSV technical summaries
("DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT Training",
gist.science/{zh,pt,fr,ko}/paper/2502.07590):
  * geometry  - query groups of spatio-temporally adjacent tokens (zh §2.2 "Query Grouping",
                ko §2나).
  * topk      - low-rank scores Q_lr K_lr^T for every query/key pair (zh §2.1 "critical KV
                estimation"), reduced over each query group, then the k largest per group by a
                full stable sort (zh §2.2 "Fused Kernel": MatMul + Top-K).
  * attention - exact softmax attention restricted to each group's selected keys (zh §2.1
                "sparse computation": full attention on the critical KV pairs only), forward
                and backward, in a dense masked form and in a gathered form.
  * adaptive  - per-group k from the share of the estimated attention mass its keys carry
                (zh §2.1 "critical KV estimation": more than 90 % of the attention score).
  * planning  - head placement over devices by a longest-processing-time greedy and its
                imbalance ratio (zh §2.3, db-SP summary), and the dense-versus-sparse choice
                per head (zh §2.1 "OP Dispatcher").
Readings the pages leave open (group reduction = SUM, ties -> lower key index, ascending
rows, scale = 1/sqrt(d), natural-log LSE, no gradient through the selection) are stated in
each function. Every function here is pinned by the CPU tests (see tests/test_oracle_*.py);
the SUM reduction itself is pinned only to this definition, not to the paper's kernel.
"""
from . import geometry, topk, attention, planning, adaptive  # noqa: F401
