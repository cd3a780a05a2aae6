"""EntropyCache denoising step for bidirectional diffusion LMs on MI355X (gfx950).

The compute lives in libec.so (HIP kernels behind the C ABI of include/ec.h);
this package is its Python binding. Importing it loads nothing; the first
call loads libec.so and raises if it has not been built.
"""
from ._lib import ECError, load  # noqa: F401

__all__ = [
    "ECError", "load", "ec_entropy_max", "ec_entropy_max_noalloc", "ec_cache_scatter", "ec_partial_attn",
    "ec_partial_attn_plan", "ec_rope_table",
    "ec_forward", "DeviceModel", "KVCache", "Decoder", "StepOut", "ec_timing_enable",
    "ec_timing_read",
]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
