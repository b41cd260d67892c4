"""Plain, slow, fp64 CPU oracle for dynamic coarse-grained block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product path: the two share no code.

Every function here is written for a reader checking it against the pages by
eye: numpy float64, one step per line, no blocking, fusion or reordering
beyond what the cited definition states.  Citations name the page and the
section / equation on it:

  [P2] "2.1 Coarse-grained selection: from content grouping to dynamic sparse
       blocks" (PaperTrace, sparse-attention knowledge 2-1)
  [P3] "From index to kernel" (PaperTrace, sparse-attention knowledge 5-1)
  [P1] the DeepSeek Sparse Attention note in the charlestar.github.io feed

Modules:
  routing    block summaries, pooled scores, candidate sets, selection -> J
  worklist   J -> sorted, deduplicated, forced CSR rows + length buckets
  attention  masked dense attention (full score rows, then mask, softmax, AV),
             and a streaming Eq (3)-(5) evaluation used to pin order invariance
  counting   physical-work counts (Eq 8 / Eq 9 style)
  problem    whole-problem drivers (row order, per-sequence routing, sampled rows)
  cache      decode-cache maintenance: append K/V rows, Eq (11) summary update
  quality    router quality: Eq (10) coverage of the dense attention, recall
  backward   gradients of the masked attention (autograd of the definition, fp64)

Parity status of each function is stated in its docstring; conventions that
no page value fixes are marked "parity unpinned".
"""
from . import routing, worklist, attention, counting, problem, cache, quality, backward  # noqa: F401
