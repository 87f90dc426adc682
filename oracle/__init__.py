"""CPU fp64 oracle for blockwise Ring / Striped causal attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The GPU library
(``striped_blockwise_amd``) never imports it and shares no code with it; the only module both
sides use is ``workloads`` (seeded input generation, no attention arithmetic).

Sources (web pages; cited by title and section):
  * "ICLR 2024論文解説: Ring Attention — 複数GPU間でのブロックワイズ分散アテンションによる超長
    コンテキスト処理" -- below "the Ring Attention review": steps 1-3 of the algorithm, the
    online-softmax equation, the PyTorch sketch ("実装例"), the causal-masking note.
  * "Striped Attention: Faster Ring Attention for Causal Transformers" (paper review) -- below
    "the Striped Attention review": the causal-attention definition and the work formulas
    (section 三 "核心公式"), the partition comparison ("分区策略对比"), the GetMask procedures
    ("GetMask 函数"), tiles ("分块与分瓦片"), position IDs ("位置编码处理") and the 2x limit
    ("理论最大加速比").
  * "Computing Attention Weights in Sequence Parallelism" (1cademy) -- the softmax denominator
    split into per-node sums.

Modules:
  attention  -- the plain definition: softmax(Q K^T / sqrt(d) + C) V and its log-sum-exp.
  ring       -- layouts, the ring schedule, GetMask, the blockwise online-softmax emulation,
                the log-sum-exp merge, and the integer work / tile counts.
  backward   -- gradients dQ, dK, dV: autograd of the definition, and the per-(query block,
                K/V block) chain rule a ring runs, driven by the forward's log-sum-exp.
  rope       -- rotary position embedding applied with the striped permutation (the
                permuted position IDs of the Striped Attention review, "位置编码处理").

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against closed forms,
a library routine (torch's scaled_dot_product_attention in fp64), brute force on tiny inputs,
and the worked partition example printed in the Striped Attention review.  The gradients are
pinned by ``tests/test_oracle_backward_pins.py`` (finite differences, closed forms, invariants),
the rotary embedding by ``tests/test_oracle_rope_pins.py`` (its relative-position property).
"""
from . import attention, backward, ring, rope  # noqa: F401
