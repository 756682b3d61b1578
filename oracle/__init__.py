"""Plain, slow CPU oracle for the NF4-LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the tests, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP path
(no kernels, headers, tables or constant generators); both sides take their
inputs from the `synth` module, which holds no arithmetic of the method.

What it computes, and where each step is defined:

* NF4 code table, blockwise absmax quantization, double quantization of the
  scales, dequantization: "QLoRA: How to fine-tune large language models with
  less memory", sections "1. NormalFloat: Store the base weights in 4 bits"
  and "2. Double quantization: Compress the scales too", and the table in
  "A worked memory budget for 65 billion weights".  The 64-weight block size
  is also fixed by "AQLoRA: A Zero-Search Recipe for Fast Quantized LoRA
  Fine-Tuning", section 3.1 (Profiling pass).
* The LoRA linear Y = X W + s X L1 L2 and its backward pass with no gradient
  for the frozen W: equation (3) in "The algebra: How two small matrices
  change a layer" (QLoRA blog) and "Lesson 17. What QLoRA Actually Costs"
  (Warm-up), with s = alpha / r from "LoRA: Fine-tuning a model by learning a
  small update", section "The algebra, with the paper's notation".
* Per-layer NF4 reconstruction error and the top-K protected set: AQLoRA
  summary, sections 3.1 (Profiling pass) and 3.2 (Precision allocation).

Precision: quantization decisions are taken in fp32 (the precision the
quantized format is defined in: fp32 scales, fp32 division), dequantized
weights are fp32 products; the layer products are computed in fp64 on the
exact values of the bf16 inputs and fp32 dequantized weights.

Parity unpinned: the NF4 code values against any external table (the pages
print none), the 8-bit format of the double-quantized scales and the exact
error formula (the AQLoRA page lost its equation); each is fixed by a stated
reading and pinned only by the closed forms and invariants in the tests.
"""
from .nf4 import (nf4_table, codebook_table, CODEBOOKS, quantize, quantize_residual, dequantize_residual, dequantize, dequantize_bf16_bits, bf16_bits, pack_codes,
                  unpack_codes, layer_error, storage_bytes, protect_count, topk,
                  NF4Quant)
from .lora import fwd, bwd, adapter_grads, merge

__all__ = ["nf4_table", "codebook_table", "CODEBOOKS", "quantize", "quantize_residual", "dequantize_residual", "dequantize", "dequantize_bf16_bits", "bf16_bits", "pack_codes",
           "unpack_codes", "layer_error", "storage_bytes", "protect_count", "topk",
           "NF4Quant", "fwd", "bwd", "adapter_grads", "merge"]
