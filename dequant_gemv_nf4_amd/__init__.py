"""dequant_gemv_nf4_amd -- NF4 fused dequant GEMV / small-M GEMM for MI355X (gfx950).

Thin Python binding over libnf4.so (C ABI in include/nf4.h).  Every call only
marshals arguments (pointers, sizes, the current stream) and hands them to the
library; all arithmetic runs in the HIP kernels.  PyTorch is used for device
memory and streams only.  There is no fallback: if libnf4.so is missing or the
device is not gfx950, calls raise.

The packed format and the operation follow the deep-fold README ("Method"):
4-bit NF4 codes in groups of 64 along K with one FP16 scale per group, and the
product y = dequant(codes, scales) . x computed without forming the matrix.
"""
from ._lib import (  # noqa: F401
    GROUP,
    MAX_K,
    MAX_M,
    EMBED_BAD_ID,
    NF4Error,
    Ring,
    PACK_NONFINITE,
    PACK_SCALE_OVERFLOW,
    embed,
    empty_packed,
    gemm,
    gemv,
    lib_path,
    noalloc_max_bytes,
    nf4_codebook,
    nf4_embed,
    nf4_gemm_prefill,
    nf4_gemm_prefill_ws,
    nf4_gemm_smallm,
    nf4_gemm_smallm_noalloc,
    nf4_gemm_smallm_ws,
    nf4_gemv,
    nf4_pack,
    nf4_unpack,
    pack,
    prefill_workspace_bytes,
    ring_slot_bytes,
    smallm_workspace_bytes,
    unpack,
    workspace_for,
)
