"""gemv_shot_all_amd: one rank's fused GEMV + AllReduce (one-shot or two-shot) on
MI355X, and the mixture-of-experts GEMM fused with the combine all-to-all.

The operation runs in hand-written HIP kernels inside libgsa.so (C ABI in
include/gsa.h).  This package is its thin Python binding; PyTorch supplies
device memory and streams.  There is no CPU or PyTorch fallback: if the
library is not built, calls raise.
"""
from ._lib import (  # noqa: F401
    A2ABuffer, GSA_ESPLIT, GSA_MOE_MAX_F, GSA_MOE_MAX_TOKENS, EXPORTS, gsa_a2a_alloc,
    gsa_a2a_buffers, gsa_a2a_free, gsa_a2a_pad_words, gsa_a2a_reset, gsa_a2a_signal_pads,
    gsa_a2a_status, gsa_moe_gemm_all_to_all, GSA_DTYPE_BF16, GSA_DTYPE_F32, GSA_EHIP, GSA_EINVAL, GSA_ENOMEM, GSA_ESTATE,
    GSA_ETIMEOUT, GSA_FLAG_PUBLISHED, GSA_FLAG_GROUP_TILES, GSA_FLAG_GROUP_WORDS,
    GSA_FLAG_TILE_ROWS, flag_word,
    GSA_MOE_TILE_ROWS, GSA_MAX_B, GSA_MAX_W,
    GSA_MAX_X_LDS_BYTES, GSA_OK, GSA_PAD_HEADER_WORDS, GsaError, SymmBuffer, device_view,
    gsa_bias_rmsnorm, gsa_epilogue, gsa_gemv_allreduce, gsa_gemv_allreduce_dtype,
    gsa_gemv_allreduce_rmsnorm, gsa_gemv_allreduce_rmsnorm_noalloc,
    gsa_gemv_allreduce_two_shot,
    gsa_peer_publish, gsa_set_wait_timeout_us, gsa_signal_pad_reset, gsa_signal_pad_row_stride,
    gsa_signal_pad_status, gsa_strerror, gsa_symm_alloc, gsa_symm_alloc_dtype, gsa_symm_free, gsa_symm_gathered,
    gsa_symm_signal_pad, gsa_symm_slots, lib, make_epilogue)
