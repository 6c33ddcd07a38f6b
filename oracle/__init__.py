"""CPU oracle for the ForkAttention hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that computes what one round of decision
requests must produce when every question ``s (+) q_i`` is run as its own
isolated prompt.  Only the test-suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the product path (the HIP library and its
Python binding) never does, and this package imports nothing from it.

Sources (web pages describing Flide / ForkAttention), cited by title and section:

* "Flide: Accelerating Decision Inference with Exact State Forking"
  (Chinese summary, paper.rainbus.top/paper/2610.42148) — sections
  前置知识 (background: Eq. (1) readout, the gated delta rule), 核心方法
  (core method) and 方法步骤详情 (method steps: stream order, visibility rule,
  sliding window, two-call GDN, conv tail by index, selective readout).
* "Flide는 공유 상태를 정확히 분기해 결정 추론을 최대 9.5배 빠르게 한다"
  (Korean summary, onedev.kr/papers/1551) — sections 어떻게 동작하나
  (problem statement, Eq. (1)), 무엇과 다른가 (flat stream, (j, c, t),
  positions continuing from P, Proposition 3.1) and 어떻게 쓰나 (flat-graph
  execution, capacity buckets, splitting, checkpoints).

Modules:
  layout     — independent builder of the flat-stream metadata and split rule
  attention  — rotary positions and causal softmax attention of one prompt
  gdn        — causal depthwise conv, L2 norm and the per-token gated delta rule
  readout    — option probabilities, Eq. (1)
  round      — a whole round, isolated-prompt ("isolated") or trunk-once ("memo")
  stack      — a multi-layer hybrid stack (pre-norm residual blocks around the token mixers) over the
               same isolated prompts, with the readout on question-final rows

Parity status: every function here is pinned by the CPU tests named in its
docstring; none is "parity unpinned".
"""
from . import attention, gdn, layout, readout, round, stack  # noqa: F401
