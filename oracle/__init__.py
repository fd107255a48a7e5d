"""CPU oracle for confidence-scheduled speculative decoding (test infrastructure).

This package is a plain, slow, fp64 restatement of what the method computes. It
exists only to check the HIP library: the tests, the smoke check and the
benchmark's CPU-baseline leg are its only callers. The product path never
imports it, and it imports nothing from the product package.

Modules (each function cites the passage of the source pages it follows):

* ``philox``   -- Philox4x64-10 counter-based uniforms (Salmon et al., SC'11),
  the one random source both sides implement from its published definition.
* ``schedule`` -- block survival products and the hardware-aware prefix
  scheduler (DSpark study notes, section 5.1-5.2; SGLang article, "SPS cost
  table").
* ``pack``     -- front-packed ragged verify buffer (SGLang article, "Ragged
  verify").
* ``verify``   -- rejection-sampling verify with bonus token, greedy verify and
  greedy tree walk (DSpark study notes, section 1 and Figure 1; PCTree article).
* ``markov``   -- Markov-head sequential stage, greedy chain (DSpark study notes,
  section 4; PCTree article, "z_d = L_d + Markov(y_{d-1})").
* ``pctree``   -- parent-conditioned drafting tree (PCTree article).

Parity status of each function is stated in its module header.
"""
