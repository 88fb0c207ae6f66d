"""MI355X-native Outlier Tokens Tracing (OTT) decode attention.

The compute path is libott.so (hand-written HIP kernels for gfx950) behind the
C ABI in include/ott.h. This package is its Python binding: ``_lib`` holds the
ctypes calls under the C names, ``OTTLayer`` wraps one layer's arena.
"""
from . import _lib
from ._lib import (OttError, ott_append, ott_decode, ott_destroy, ott_fp16_decode,
                   ott_fp16_decode_workspace, ott_get_layout,
                   ott_get_seq_state, ott_init, ott_prefill, ott_quantize_group,
                   ott_set_num_splits, ott_step,
                   ott_status_string)

__all__ = ["OTTLayer", "OttError", "ott_init", "ott_append", "ott_quantize_group", "ott_decode",
           "ott_destroy", "ott_get_layout", "ott_get_seq_state", "ott_set_num_splits",
           "ott_status_string", "ott_fp16_decode", "ott_fp16_decode_workspace",
           "ott_prefill", "ott_step"]


def __getattr__(name):
    if name == "OTTLayer":
        from .layer import OTTLayer
        return OTTLayer
    raise AttributeError(name)
