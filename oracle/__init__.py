"""fp64 CPU oracle for RoPE-scaled causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; it is the plain definition of what
the library computes, written in numpy float64 so that a reader can check it
against the source pages by eye.

Sources (cited by title and section):
  * "Long Context: RoPE / YaRN / NTK / MLA" (mathieu0905.github.io), the most
    formal page: RoPE derivation (§2), PI (§4), NTK-aware (§5), YaRN (§6),
    sliding window (§10).
  * "8.3 长上下文技术" (LLM full-stack book, paper.xwysyy.cn): RoPE recap
    (§8.3.1), PI / NTK-aware and the over-extrapolated range (§8.3.2), the
    piecewise gamma(d) of NTK-by-parts and YaRN (§8.3.3), FlashAttention's
    exactness and backward recomputation (§8.3.4), Ring Attention and its Striped / Zig-Zag partitions
    (§8.3.5).
  * "长上下文外推" notebook (doc.minddiy.top): worked 2-D rotation (§4.2),
    printed frequency table (§5.2), printed angles (§6.3), NTK table (§15.1).
  * "长上下文推理：RoPE 扩展、位置插值与 Ring Attention" (plumephp.com):
    NTK base example, FlashAttention and Ring notes.

Modules:
  * ``oracle.rope``      frequency table, temperature, bands, rotation.
  * ``oracle.attention`` softmax attention (row blocks and brute force),
                         sliding-window / sink mask, log-sum-exp merge,
                         single-query decode.
  * ``oracle.ring``      Ring Attention over P simulated devices with
                         contiguous, Striped and Zig-Zag partitions.
  * ``oracle.backward``  gradients dq, dk, dv (chain rule, rotated back by
                         the opposite angle).

Every function here is pinned by a ``-m "not gpu"`` test against values the
pages print, closed forms, invariants or library routines (see
``tests/test_oracle_*.py``).  None is "parity unpinned".
"""
from . import rope, attention, ring, backward  # noqa: F401
