"""MI355X (gfx950) decoder-block library: thin Python binding of the C ABI in
include/blk.h.

Every step of the block runs in the HIP kernels of libblk.so; this module
only marshals torch tensors (device memory) and the current HIP stream into
the C calls, and raises on a non-zero status.  If the library is not built
the import succeeds but every call raises: there is no fallback path.
"""
from .binding import (  # noqa: F401
    BLK_BF16, BLK_F32, BLK_GEMM_FP8_E4M3, BLK_GEMM_NATIVE, BlkError, BlockConfig, DecodeConfig, HeadConfig,
    block_bwd, block_fp8_quantize, block_mfma_probe, block_fp8_quantize_2d, block_fwd, block_saved_bytes, block_scratch_bytes,
    block_strerror, block_timing_enable, block_timing_read, decode_scratch_bytes,
    decode_step, decode_step_noalloc, head_loss_bwd, head_loss_fwd, head_scratch_bytes, layer_window, library, library_path,
)
