"""Float64 CPU oracle for one Introspective Strided Decoding (ISD) step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code, tables or constants with the HIP kernels; the only thing the
two sides have in common is the seeded input generator in ``workloads/``.

Sources (web pages on I-DLM; cited by title and section):

* [project]  I-DLM project page (Traditional-Chinese translation, news.myit.tw):
  the ISD card, the TPF widget, the compute-bound speedup derivation (steps
  1-6) and the caption on geometric acceptance.
* [hypho]    "I-DLM：扩散模型如何用'自省一致性'追上自回归模型质量"
  (blog.hypho.cn): sections "Introspective Strided Decoding（ISD）",
  "三项关键训练创新" and "推理：复用 AR 推理栈".
* [hotdry]   "自省扩散语言模型的 token 生成机制与工程实践" (blog.hotdry.top):
  sections "从质量差距到自省机制", "Token 生成的核心参数与验收机制" (with the
  E[acc]/TPF table) and "服务部署与 SGLang 集成".

Modules:
  philox     Philox4x64-10 and the per-decision uniforms
  attention  strictly causal stride attention over a paged KV cache
  accept     log-normalisers, the p/q acceptance test, residual resampling
  commit     writing the stride rows of the accepted prefix into KV pages
  lora       the gated low-rank delta of R-ISD, and a whole gated projection
  tpf        expected acceptance, tokens per forward, the compute-bound identity
  propose    drawing the next N tokens at the MASK rows (sampling or argmax)
  loop       the multi-step decoding loop: per-request VERIFY / REPROPOSE bookkeeping

Every function is pinned by a test in ``tests/test_oracle_*.py`` against a
closed form, a printed value, a library routine or a brute-force count.
"""

from . import accept, attention, commit, lora, loop, philox, propose, tpf  # noqa: F401
