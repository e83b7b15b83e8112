"""MI355X (gfx950) routed-expert MoE layer over 4-bit block-quantized experts with a bf16 LoRA.

The compute lives in libbqm.so (HIP kernels behind the C ABI of include/bqm.h);
this package is its ctypes binding.  Importing it does not load the library:
the first call does, and raises if the library has not been built.
"""
from ._lib import (BQMError, FMT_NF4, FMT_NVFP4, MoEDesc, QTensor, SCALE_PER_ROW, STAGES, STAGE_COUNT,
                   SCALE_PER_TENSOR, alloc_qtensor, bqm_abi_version, bqm_dequantize,
                   bqm_last_error, bqm_lora_grad, bqm_moe_dgrad, bqm_moe_dgrad_colwise, bqm_moe_fwd,
                   bqm_moe_workspace_size, bqm_permute, bqm_permute_workspace_size,
                   bqm_nf4_nest, bqm_quantize_nf4, bqm_quantize_nvfp4, bqm_quantize_nvfp4_noalloc,
                   bqm_quantize_nvfp4_workspace_size,
                   bqm_route, load, nf4_nest_groups, quantize_stack)

__all__ = [n for n in dir() if n.startswith("bqm_")] + [
    "BQMError", "FMT_NF4", "FMT_NVFP4", "MoEDesc", "QTensor", "SCALE_PER_ROW", "SCALE_PER_TENSOR", "STAGES", "STAGE_COUNT",
    "alloc_qtensor", "load", "nf4_nest_groups", "quantize_stack"]
