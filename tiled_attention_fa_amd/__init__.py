"""MI355X (gfx950) FlashAttention forward: Python binding of libfa.so.

The binding only marshals arguments: it reads sizes, dtype, pointers and the
current HIP stream from torch tensors and calls the C ABI declared in
include/fa.h.  Every step of the computation runs in the library's kernels.
There is no fallback: if libfa.so is missing, loading fails with an error
that says how to build it.
"""

from ._lib import (  # noqa: F401
    FA_BF16,
    FA_F16,
    FA_F32,
    FAError,
    STATUS_NAMES,
    fa_forward,
    fa_forward_ex,
    fa_forward_ex_noalloc,
    fa_forward_ex_noalloc_raw,
    fa_forward_ex_raw,
    fa_forward_ex_workspace_bytes,
    fa_forward_raw,
    fa_forward_strided,
    fa_forward_strided_raw,
    fa_naive_forward,
    fa_naive_forward_raw,
    fa_naive_workspace_bytes,
    fa_device_info,
    fa_key_groups_suggest,
    fa_splitkv_suggest,
    fa_status_string,
    fa_version,
    fa_workgroup_shape,
    forward,
    forward_ex,
    library_path,
    load_library,
    naive_forward,
    naive_workspace,
    splitkv_workspace,
)
