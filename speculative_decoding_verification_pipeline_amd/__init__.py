"""MI355X-native batched LLM sampling: fused logit processing + two-stage top-k
sampler, speculative verification, and a fused LM-head Gumbel-max sampler.

The compute lives in libss_sampler.so (HIP, gfx950); `sampler` is its ctypes
binding and `workloads` builds seeded synthetic inputs.
"""
