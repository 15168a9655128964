"""MI355X-native WTConv: fused HIP kernels for gfx950 behind a C-ABI.

The compute path is ``libwtconv.so`` (HIP, built from ``csrc/``); the Python
functions here only marshal arguments to it. Importing the package does not
load the library; the first call does, and raises if it is missing.
"""
from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401

__all__ = ["CONFIGS", "WorkloadConfig", "get_config"]


def __getattr__(name):
    # the binding is loaded on first use so that CPU-only code (configs,
    # inputs, the I/O model) never needs the HIP runtime
    from . import binding
    if hasattr(binding, name):
        return getattr(binding, name)
    raise AttributeError(name)
