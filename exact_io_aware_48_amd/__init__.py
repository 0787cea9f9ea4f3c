"""FlashAttention forward and backward for AMD MI355X (gfx950), behind a C ABI.

The kernels live in ``csrc/`` and are built into ``libfa_fwd.so``
(``python -m exact_io_aware_48_amd.build``); ``include/fa_fwd.h`` and
``include/fa_bwd.h`` and ``include/fa_split.h`` declare the C ABI and this package
binds it with the same names.
"""

from ._lib import FA_BF16, FA_F32, FA_FP8_E4M3, LIB_PATH
from .api import (FaError, fa_bwd, fa_bwd_workspace_size, fa_fwd, fa_fwd_alibi, fa_fwd_alibi_fp8,
                  fa_fwd_blocksparse, fa_fwd_blocksparse_fp8, fa_fwd_fp8, fa_fwd_gqa, fa_fwd_gqa_fp8, fa_fwd_split, fa_fwd_split_fp8, fa_fwd_split_noalloc, fa_fwd_split_plan, fa_lse_merge, fa_plan,
                  fa_split_scratch_bytes,
                  fa_status_string, fa_version)

__all__ = ["fa_fwd", "fa_fwd_fp8", "fa_fwd_gqa", "fa_fwd_gqa_fp8", "fa_fwd_alibi", "fa_fwd_alibi_fp8",
           "fa_fwd_blocksparse", "fa_fwd_blocksparse_fp8",
           "fa_bwd", "fa_bwd_workspace_size",
           "fa_fwd_split", "fa_fwd_split_fp8", "fa_fwd_split_noalloc", "fa_fwd_split_plan", "fa_lse_merge", "fa_plan", "fa_split_scratch_bytes",
           "fa_status_string", "fa_version",
           "FaError",
           "FA_F32", "FA_BF16", "FA_FP8_E4M3", "LIB_PATH"]
