"""fp64 CPU oracle for prefix-reuse block-causal attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import anything from this package. The product path (the HIP
library and its Python binding) never imports it, and this package imports nothing from
the product path: the two share no code, tables, constants or helpers.

Pages cited in this package (text of public web pages about Qwen-Image-2.1 serving):
  [blog]   ThakiCloud tech blog, "Qwen-Image-2.1 vLLM-Omni day 0" (thakicloud.com, English)
  [recipe] vLLM recipes, "Qwen/Qwen-Image-2.1" (recipes.vllm.ai)
  [L20]    "Qwen-Image-2.1: SGLang vs vLLM-Omni Measured on a Single L20" (aik8s.run)
  [sglang] "SGLang-Diffusion stöder Qwen-Image-2.1 på dag noll" (orcarouter.ai)

Modules:
  attention   block structure, explicit mask, masked softmax attention in fp64 and the
              three calls of the hot path (prefix build, denoise step, full recompute)
  fp8         OCP E4M3FN value table, round-to-nearest-even saturating encoder, and the
              per-(request, head, K/V) absmax quantisation of the prefix cache
  layout      prefix-cache byte layout, tile classification map, useful-pair counts

Pinning status: every function here is pinned by a CPU test against something other than
itself (brute force, a library routine, a closed form, or a page fact); see tests/.
"""
