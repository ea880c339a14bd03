"""CPU oracle for QK4V8 attention: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct reference of what the QK4V8 path computes,
written in NumPy float64 / integer arithmetic (plus a pure-Python scalar
brute force in ``scalar.py``).  It shares no code with the HIP path and never
imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here; the
product path (``bit_quantized_attention_online_amd``) must never route through
it.

Sources (cited by page title and section):

* "MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践"
  (mhpn.cn/news/2564245), below "MpFA page": §2.1-§2.3 (4-bit Q/K, 8-bit V,
  FP32 accumulator, online softmax), §3.2 (per-block scale computed at run
  time from the block's extreme values), §3.3 (dequantize right after QK^T,
  FP32 accumulation, 16-bit output).
* "小米MiMo-V2.5-Pro-FP4-DFlash：FP4+推测解码的万亿推理提速指南"
  (wmrh.cn/news/72329), below "MiMo page": section "MXFP4专家量化" (MXFP4 =
  FP4 values sharing one block scale per 32 elements), section "DFlash块扩散
  推测解码" (the backbone verifies an 8-token drafted block in one forward
  pass).
* The OCP Microscaling (MX) v1.0 and OCP 8-bit floating point (OFP8)
  specifications, for the bit layouts of E2M1, E8M0 and E4M3FN that the name
  "MXFP4" and "FP8 E4M3" refer to.

Readings where the pages are silent (each also listed in the design notes):
the 4-bit format is MXFP4 with 32-element blocks along head_dim; the block
scale follows the OCP rule X = floor(log2 amax) - emax_elem; rounding is
round-to-nearest-even with saturation; V is FP8 E4M3FN with one power-of-two
(E8M0) scale per tile of rows; attention is evaluated exactly in float64 on
the dequantized operands, causal masks are bottom-right aligned, and GQA maps
query head h to KV head floor(h / G).
"""

from . import formats, quant, attention  # noqa: F401
