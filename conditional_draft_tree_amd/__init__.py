"""MI355X-native conditional draft-tree builder (DominoTree) -- Python binding.

A thin ctypes layer over ``libdtree.so`` (the C ABI in ``include/dtree.h``).
It only checks and marshals arguments: every step of the method runs in the
library's HIP kernels.  PyTorch provides device memory and the current stream.
There is no CPU fallback: if the library is missing, importing the binding's
entry points raises.
"""
from ._lib import (  # noqa: F401
    DT_BF16, DT_EXPAND_AUTO, DT_EXPAND_FUSED, DT_EXPAND_PERSISTENT, DT_EXPAND_RESIDENT, DT_EXPAND_STEPPED, DT_F32, Builder, DtreeError,
    dt_accept_greedy, dt_build, dt_build_folded, dt_build_marginal, dt_build_noalloc,
    dt_correct, dt_create, dt_destroy, dt_expand_mode, dt_fold_input,
    dt_gru_step, dt_last_error, dt_status_string, dt_timing_enable, dt_timing_read, dt_topm, dt_topm_tail,
    dt_workspace_bytes, lib_path, load_library,
)
