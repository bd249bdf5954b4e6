"""CPU oracle for the CSA2 FP4 global-KV decode hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

It is a plain, slow NumPy restatement of what the method computes, written
from three web pages about DeepSeek-V4.1-Flash's KV compression:

  [P1] "KV-cache compression: how far it goes" (long-form post, yomxxx.com,
       2026-09-19); sections numbered 一..六 on the page.
  [P2] "DeepSeek-V4.1-Flash KV compression" (rebasdaily.com, 2026-09-21);
       unnumbered sections, named here by their headings in English:
       "the agent bottleneck moves forward", "halve the long input",
       "same notes, many layers" (the CSA2 section), "why it matters",
       "limits and unknowns".
  [P3] "890 bytes per token: the hidden cost DeepSeek cut" (ailily.cc);
       sections numbered 一..四 under the page's analysis part.

Where the pages leave a step open, each module says which reading it takes.

Modules:
  formats   E2M1 and E4M3FN value sets, exact round-to-nearest-even encoders
  quantize  row quantiser (codes + scales) and dequantiser
  indexer   block keys, collapsed indexer query, pinned-order block scores
  select    top-k selection with the lowest-id tie-break
  attend    softmax attention over selected positions (fp64)
  step      layer-stack driver (Full / Reindex / Reuse, hierarchical pool)
"""
