"""CPU oracle for the batched sampling pipeline (test infrastructure only).

This package is the slow, plain reference that defines what the GPU library must
compute. It is test infrastructure: only the test suite, the smoke entry point and
the benchmark's CPU-baseline leg may import it. The product path (the HIP library
and its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path.

Modules
-------
philox    Counter-based Philox4x32-10 generator, written from its published
          definition, plus the uniform and Gumbel transforms of its words.
pipeline  Per-request logit processing and sampling: penalties, logit bias,
          grammar mask, temperature, top-k, top-p, min-p, inverse-CDF draw.
spec      Speculative verification by rejection sampling of draft tokens.
lmhead    LM-head projection followed by Gumbel-max sampling over vocabulary
          tiles with a cross-tile argmax.

Sources: SonicSampler abstract (arxivdaily page, English abstract) for the
pipeline's components and order; "Accelerating Sonar through speculation"
(Perplexity blog, sections on speculative decoding and draft-target decoding)
for verification; the FlashSampling news item (meineki.news, body) for the
fused LM-head sampler.
"""
