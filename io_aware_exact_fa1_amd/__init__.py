"""MI355X-native exact attention (FlashAttention forward pass and its backward).

The computation lives in the HIP library ``libfa_mi355x.so`` (sources in
``csrc/``, C ABI in ``include/fa.h``); this package is its thin ctypes
binding.  PyTorch is used only for device buffers and streams.
"""

from ._binding import (  # noqa: F401
    EXPORTED, FA_DTYPE_BF16, FA_DTYPE_F32, FA_ERR_ALIAS, FA_ERR_ALIGN, FA_ERR_HEAD_DIM, FA_ERR_LAUNCH, FA_ERR_NULL, FA_ERR_SCALE,
    FA_ERR_SCRATCH, FA_ERR_SHAPE, FA_ERR_VARIANT, FA_OK, FA_SPLIT_NOALLOC_BYTES, LIB_PATH, FaError, backward,
    fa_bwd, fa_bwd_check_args, fa_check_args, fa_check_args_ex, fa_check_args_split, fa_fwd, fa_fwd_ex,
    fa_fwd_f32, fa_fwd_split, fa_fwd_split_noalloc, fa_split_chunks, fa_strerror, fa_supported, forward, forward_ex,
    forward_split, load_library,
)
