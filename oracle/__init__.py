"""CPU oracle for AutoRound-style weight quantization -- TEST INFRASTRUCTURE.

A plain, slow, obviously-correct NumPy implementation of what the tuning path
computes, written from the pages (the AutoRound blog "Low-Bit Quantization in
Practice with vLLM", sections 2-4, and its Chinese twin; the quantization
"coordinates" page, section 1.2).  It exists only to check the HIP library:
only tests, the smoke entry point and the benchmark's CPU-baseline leg may
import it.  The product path never calls it, and it shares no code with the
HIP library.

Precision contract:
* quantize-dequantize (QDQ): fp32, fixed operation order, IEEE division,
  round-half-to-even, no fused multiply-add -- these decide integer codes, so
  they are taken in the precision the kernel uses;
* GEMMs, loss and gradients: fp64;
* parameter update: fp32 (the stored parameter precision).

Parity status: every function here is pinned by a CPU test (worked examples
from the pages, closed forms, finite differences, torch autograd, brute force,
round trips) except the free-running trajectory of ``tune_layer`` on the
synthetic workloads, for which the pages print no losses or codes
("parity unpinned" beyond oracle-vs-GPU agreement).
"""
from .autoround_ref import (  # noqa: F401
    bf16_round,
    group_range,
    group_scale_zero,
    quantize_codes,
    dequantize,
    qdq,
    rtn,
    gather_batch,
    loss_and_grads,
    ste_grads,
    lr_table,
    signsgd_step,
    tune_layer,
    pack_int4,
    unpack_int4,
    packed_bytes,
    w4a16_matmul,
)
from .bruteforce import bruteforce_min_loss, bruteforce_block_min_loss  # noqa: F401
from . import decoder_ref  # noqa: F401
from .block_ref import (  # noqa: F401
    LINEARS,
    silu,
    swiglu_forward,
    block_reference,
    block_loss_and_grads,
    tune_block,
    quantized_block_output,
)
