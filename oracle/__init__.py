"""CPU oracle for the MXFP4 MoE expert layer — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does, and
the oracle imports nothing from the product package (they share no code).

Floating point is carried in float64 and rounded once to the storage type the
contract fixes (fp32 for router weights, expert outputs and layer output;
bf16 for the SwiGLU activation h).

Sources.  The pages ("MiMo-V2.5-Pro-FP4-DFlash" model card, §1 Introduction
and §2 "FP4 Quantization"; the nxbn.cn article "MiMo-V2.5-Pro-FP4-DFlash
万亿参数大模型推理效率的终极突破", sub-sections "量化策略的智能选择" and
"架构设计与配置详解") state that only the MoE experts are stored in MXFP4 with
block size 32, that the layer has 384 experts with 8 active per token, and
that the rest of the model (activations included) runs in higher precision.
The element and scale encodings are those of the OCP Microscaling (MX)
Formats Specification v1.0 (E2M1 elements, E8M0 shared scale).  Everything
the pages leave open is a stated reading; each function says which.

Modules
  mx       E2M1 / E8M0 decode, unpack, pack (OCP conversion), bf16 rounding
  route    top-k routing with softmax weights renormalised over the chosen k
  permute  per-expert histogram, offsets, gather lists
  layer    the whole layer by its plain per-expert dense definition

Parity pins: every function here is pinned by tests under tests/ that check
it against something other than itself (closed forms, the spec's bit-field
definition, brute force, textbook special cases).  No function is
"parity unpinned" except the layer's agreement with the real model, whose
weights and outputs the pages do not publish.
"""

from . import mx, route, permute, layer  # noqa: F401

__all__ = ["mx", "route", "permute", "layer"]
