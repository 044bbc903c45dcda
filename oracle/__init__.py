"""CPU oracle for the FVAttn single-GPU hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import or call this package; only the tests, the smoke
check and the CPU-baseline leg of the benchmark do.  It shares no code, table
or helper with the HIP path, and imports nothing from it.

It is a plain, slow, float64 restatement of what the path computes, one module
per step:

  hilbert    3D Hilbert order of the (t, y, x) token grid (Skilling's
             transpose construction), the permutation and its inverse.
  route      block mean-pooling of Q/K, pooled block scores and their
             row softmax, the Top-p cut with the Top-k floor, the block mask,
             kept-block lists, per-head load and density.
  lpt        the longest-processing-time-first greedy work list over
             (head, q-block) tiles.
  attention  softmax attention restricted to the kept key blocks, and dense
             attention in the original token order.

Pages the method comes from (cited by title and section in each module):
  * "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for Video
    Generation", arXiv abstract as shown on the mlsanity.com paper index.
  * aixai.ru blog post on FVAttn (Russian), sections "Top-p vs Top-k",
    "Sparse-routing frontend", "Runtime Load Balancing (RLB)".
  * longzhangge.com PaperDaily article on FVAttn (Chinese), method section.
  * bayesiansapien.github.io wiki note "FVAttn: Adaptive Sparse Attention with
    Runtime Load Balancing", sections "What it is" and "Key findings".

Parity status of each function is stated in its module header.
"""
