"""CPU oracle for quantized paged-KV decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library under ``quantized_paged_kv_02_amd/``.

The oracle is written from three web pages on KV-cache quantization:

* [yunthe]   "KV Cache量化压缩技术与vLLM推理引擎显存优化实战" (yunthe.com)
* [oh-bug]   "KV Cache Quantization 生产实战：用低精度缓存降低长上下文推理显存" (oh-bug.com)
* [intelli]  "大模型KV Cache显存优化与量化技术实践" (intelliparadigm.com)

Every function cites the page and section it follows.  Quantization runs in
IEEE fp32 (division correctly rounded, round-half-to-even); attention runs in
fp64 over the exact dequantized values.
"""

from .kvq_oracle import *  # noqa: F401,F403
