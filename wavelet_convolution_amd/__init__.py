"""MI355X-native WTConv: fused HIP kernels for gfx950 behind a C-ABI.

The compute path is ``libwtconv.so`` (HIP, built from ``csrc/``); the Python
functions here only marshal arguments to it. Importing the package does not
load the library; the first call of a binding function does, and raises if
the library is missing.
"""
from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401

_BINDING_NAMES = (
    "wtconv_fwd", "wtconv_bwd_data", "wtconv_bwd_weight",
    "wtconv_naive_fwd", "wtconv_naive_bwd_data", "wtconv_naive_bwd_weight",
    "wtconv_workspace_size", "wtconv_status_string", "load_library", "WTConvError",
    "wtconv_bwd", "wtconv_peak_fma", "wtconv_peak_copy", "layout_of", "wtconv_route",
)

_MODULE_NAMES = ("WTConv2d", "WTConvFunction", "wtconv")

__all__ = ["CONFIGS", "WorkloadConfig", "get_config", *_BINDING_NAMES, *_MODULE_NAMES]


def __getattr__(name):
    # the binding is imported on first use so that CPU-only code (configs,
    # inputs, the I/O model) never needs the HIP runtime
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    if name in _MODULE_NAMES:
        from . import module
        return getattr(module, name)
    raise AttributeError(name)
