"""MI355X-native FVAttn hot path: HIP kernels behind a C ABI (include/fvattn.h),
with a thin ctypes binding.

Importing the package loads nothing; the library is loaded on first use and
a missing library raises ImportError (there is no fallback path).
"""
from ._lib import (BF16, attn_workers, EINVAL, ELAUNCH, EUNSUPPORTED, EWORKSPACE, F32, OK,  # noqa: F401
                   FvattnError, declared_symbols, hilbert_permute, library_path,
                   load_library, pack_v, permute_rows, route, route_workspace_size,
                   schedule, schedule_workspace_size, sparse_attn, status_string)
from .pipeline import FVAttnPath, default_workers  # noqa: F401
