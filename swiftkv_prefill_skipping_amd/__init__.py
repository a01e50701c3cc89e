"""SwiftKV prefill on MI355X (gfx950): Python binding of libswiftkv.

The library (C ABI in include/swiftkv.h, HIP kernels in csrc/) does all of
the work; this package only marshals arguments (``_lib``) and provides
device-memory plumbing (``runner``).  Importing it does not load the
library; the first call does, and raises if it has not been built.
"""
from ._lib import (SKV_BF16, SKV_FP32, SkvError, make_config, skv_flops, skv_kv_cache_create,  # noqa: F401
                   skv_kv_cache_destroy, skv_kv_cache_view, skv_model_create, skv_model_destroy,
                   skv_model_load_globals, skv_model_load_layer, skv_num_kv_slots, skv_prefill, skv_profile_enable,
                   skv_profile_read)

__all__ = ["SKV_BF16", "SKV_FP32", "SkvError", "make_config", "skv_flops", "skv_kv_cache_create",
           "skv_kv_cache_destroy", "skv_kv_cache_view", "skv_model_create", "skv_model_destroy",
           "skv_model_load_globals", "skv_model_load_layer", "skv_num_kv_slots", "skv_prefill", "skv_profile_enable",
           "skv_profile_read"]
