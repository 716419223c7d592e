"""CPU oracle for the row-wise autograd hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct implementation of every forward op, every
hand-derived backward, the counter-based dropout RNG and a small reverse-mode
tape, written in numpy float64 (float32 only where the pages fix that
precision: the dropout decision and scale).  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The library (``autograd_row_wise_amd``) never imports it and shares
no code with it; nothing here reads anything the library produced.

Pages cited (by title and section; the text is in Chinese, Swedish and
Chinese respectively):

* [AE] xtrain design document "Phase: Autograd Engine + Op Backward"
  (docs/03-autograd-engine.md): sections "Tape 设计", "梯度累加（扇出求和）",
  the op-backward table "各算子 backward 数学", the RMSNorm, RoPE, Softmax and
  Cross-entropy derivations, "Attention 用组合", "验证方法".
* [BP] "Träna en språkmodell: Backprop i anpassad CUDA" (unhomeschool):
  the kernel-pair table "Varje Forward-op Får En Backward-tvilling",
  "En baklängeskärnas uppgift", "Sparade tensorer",
  "Ackumulation över mikrobatcher".
* [DO] xtrain design document "Phase T18: Dropout (device RNG + mask)"
  (docs/17-dropout.md): "RNG：counter-based", "每个 dropout 站点的确定性 seed",
  "dropout 节点的 backward", "与既有特性的组合", "验证方法".
* [AD] "从零构建自动微分引擎：对偶数、计算图与反向传播的 Rust 深度实战"
  (ybb.press): section 2 worked example, section 3.3 reverse pass.

Readings taken where the pages are silent are stated at each function.

Parity status: every function here is pinned by tests under ``tests/`` that
check it against something other than itself (finite differences, closed
forms, invariants, brute force, published values).  The functions whose
exact convention the pages do not fix (GELU erf form, RoPE frequency
schedule, causal masking, bf16 rounding points) are pinned to the
mathematics of the chosen reading, not to the pages.
"""

from . import numerics, ops, rng, tape, fd  # noqa: F401
