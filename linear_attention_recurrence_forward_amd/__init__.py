"""Gated DeltaNet recurrent forward step on AMD Instinct MI355X (gfx950).

The compute runs in libgdn.so (hand-written HIP kernels behind the C ABI of
include/gdn.h); this package is its thin Python binding, with torch providing
device memory and streams. `workloads` holds the seeded synthetic inputs.

Binding names are loaded on first use, so `workloads` can be imported without
torch or a GPU.
"""

_BINDING_NAMES = (
    "EXPORTS", "GdnError", "GdnParams", "STATUS", "STATUS_CODE", "f32_bits", "forward",
    "gdn_check_params", "gdn_forward", "gdn_forward_bf16", "gdn_forward_capture",
    "gdn_forward_ex", "gdn_rollback", "OPT_BF16_IO", "OPT_NORMALIZE_K",
    "gdn_status_string",
    "library_path", "make_params", "params_for", "scale_bits",
)

__all__ = list(_BINDING_NAMES) + ["workloads"]


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
