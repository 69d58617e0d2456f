"""CPU oracle for the FP4 compressed global KV cache and its sparse decode path.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package. The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and this package imports nothing
from the product path.

Everything is plain numpy, written step by step from the pages' statement of
the method, without blocking, fusion or reordering beyond what the
definitions state.

Pages cited (all are web pages about DeepSeek-V4.1-Flash's KV cache):

* [FP4]  "Le cache KV en FP4 — les 890 octets, vérifiés" (mkdocs.reaper.mx,
         chapter 05 of the V4.1-Flash architecture notes) — the only page
         with formulas: entry-cost equations, per-layer table, context table,
         the V1 and sliding-window equations.
* [CS]   "DeepSeek V4.1 Flash : 890 octets de cache KV par token"
         (contextstudios.ai) — the CSA2 layer modes Full / Reindex / Reuse,
         top-512, the 16384-candidate hierarchical indexer.
* [TF]   "DeepSeek-V4.1 Flash compresse le KV-Cache de 4 fois" (techfi24.com)
         — ratio merge with learned per-channel weights, shared 512-d latent.
* [F24]  "KV cache da 890 byte per token" (flash24.org) — the hierarchical
         indexer restricts deeper layers to the Full layer's pool.

Where the pages are silent the reading taken is stated in the docstring.
"""
