"""ctypes binding of libott.so (the OTT C ABI declared in include/ott.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory (the arena, inputs, outputs) and the
current HIP stream. If the library has not been built, importing this module
raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libott.so")

OTT_OK = 0
STATUS_NAMES = {
    0: "OTT_OK", 1: "OTT_ERR_INVALID_ARG", 2: "OTT_ERR_UNSUPPORTED",
    3: "OTT_ERR_ARENA_TOO_SMALL", 4: "OTT_ERR_CAPACITY", 5: "OTT_ERR_STATE", 6: "OTT_ERR_HIP",
    7: "OTT_ERR_SCRATCH_TOO_SMALL",
}
FP16_DECODE_SCRATCH_BYTES = 8 << 20  # OTT_FP16_DECODE_SCRATCH_BYTES in include/ott.h

# Every symbol include/ott.h declares.
EXPORTS = ("ott_init", "ott_append", "ott_quantize_group", "ott_decode", "ott_destroy",
           "ott_get_layout", "ott_get_seq_state", "ott_set_num_splits", "ott_status_string",
           "ott_fp16_decode", "ott_fp16_decode_workspace", "ott_prefill",
           "ott_fp16_decode_noalloc", "ott_step")


class ott_config_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("residual", ctypes.c_int32),
                ("pool_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("retention", ctypes.c_int32)]


class ott_layout_t(ctypes.Structure):
    _fields_ = [("arena_bytes", ctypes.c_uint64), ("page_bytes", ctypes.c_uint64),
                ("pages_per_head", ctypes.c_int32), ("ring_capacity", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("off_counters", ctypes.c_uint64), ("off_pages", ctypes.c_uint64),
                ("off_page_pos", ctypes.c_uint64), ("off_page_nvalid", ctypes.c_uint64),
                ("off_pool_k", ctypes.c_uint64), ("off_pool_v", ctypes.c_uint64),
                ("off_pool_pos", ctypes.c_uint64), ("off_pool_n2", ctypes.c_uint64),
                ("off_ring_k", ctypes.c_uint64), ("off_ring_v", ctypes.c_uint64),
                ("off_partials", ctypes.c_uint64), ("off_tickets", ctypes.c_uint64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def _one_hip_runtime() -> None:
    """PyTorch ships its own HIP runtime (libamdhip64, libhsa-runtime64) under the
    same sonames as the system ROCm copies that libott.so is linked against.
    Imported first, torch's copies are in the process and libott.so binds to
    them; loaded first, libott.so would map the system copies and torch its own,
    and two HIP runtimes initialising the same GPU crash at the first GPU call."""
    try:
        import torch  # noqa: F401
    except ImportError:  # no torch: libott.so brings the system runtime alone
        pass


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    H, P, I32, VP = ctypes.c_void_p, ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
    lib.ott_init.argtypes = [P(ott_config_t), VP, ctypes.c_size_t, P(ctypes.c_size_t), P(H)]
    lib.ott_init.restype = ctypes.c_int
    lib.ott_append.argtypes = [H, VP, VP, P(I32), I32, VP]
    lib.ott_append.restype = ctypes.c_int
    lib.ott_quantize_group.argtypes = [H, VP, P(I32)]
    lib.ott_quantize_group.restype = ctypes.c_int
    lib.ott_decode.argtypes = [H, VP, VP, VP]
    lib.ott_decode.restype = ctypes.c_int
    lib.ott_step.argtypes = [H, VP, VP, VP, VP, VP, P(I32)]
    lib.ott_step.restype = ctypes.c_int
    lib.ott_destroy.argtypes = [H]
    lib.ott_destroy.restype = None
    lib.ott_get_layout.argtypes = [H, P(ott_layout_t)]
    lib.ott_get_layout.restype = ctypes.c_int
    lib.ott_get_seq_state.argtypes = [H, I32, P(I32)]
    lib.ott_get_seq_state.restype = ctypes.c_int
    lib.ott_set_num_splits.argtypes = [H, I32]
    lib.ott_set_num_splits.restype = ctypes.c_int
    lib.ott_prefill.argtypes = [H, VP, VP, P(I32), I32, VP]
    lib.ott_prefill.restype = ctypes.c_int
    lib.ott_fp16_decode.argtypes = [I32, I32, I32, I32, VP, VP, I32, P(I32), VP, VP, ctypes.c_float,
                                    VP, ctypes.c_size_t, I32, VP]
    lib.ott_fp16_decode.restype = ctypes.c_int
    lib.ott_fp16_decode_noalloc.argtypes = [I32, I32, I32, I32, VP, VP, I32, P(I32), VP, VP,
                                            ctypes.c_float, I32, VP]
    lib.ott_fp16_decode_noalloc.restype = ctypes.c_int
    lib.ott_fp16_decode_workspace.argtypes = [I32, I32, I32]
    lib.ott_fp16_decode_workspace.restype = ctypes.c_size_t
    lib.ott_status_string.argtypes = [ctypes.c_int]
    lib.ott_status_string.restype = ctypes.c_char_p
    return lib


_one_hip_runtime()
lib = _load()


class OttError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.ott_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


def _check(status: int, where: str) -> None:
    if status != OTT_OK:
        raise OttError(status, where)


# Batch size of each live handle: ott_append and ott_prefill read exactly that
# many host counts, so a list of another length is refused before the call.
_batch_of = {}


def _host_counts(h, values, what: str):
    n = len(values)
    want = _batch_of.get(getattr(h, "value", h))
    if want is not None and n != want:
        raise ValueError(f"{what} has {n} entries; the handle's batch is {want}")
    return (ctypes.c_int32 * n)(*[int(x) for x in values])


# --- the C calls under their own names --------------------------------------

def ott_init(cfg: ott_config_t, d_arena: Optional[int], arena_bytes: int,
             sizing_only: bool = False):
    """Returns the required arena size when sizing_only, else (handle, required)."""
    req = ctypes.c_size_t(0)
    if sizing_only:
        _check(lib.ott_init(ctypes.byref(cfg), None, 0, ctypes.byref(req), None), "ott_init")
        return int(req.value)
    h = ctypes.c_void_p(0)
    _check(lib.ott_init(ctypes.byref(cfg), ctypes.c_void_p(d_arena), arena_bytes,
                        ctypes.byref(req), ctypes.byref(h)), "ott_init")
    _batch_of[h.value] = int(cfg.batch)
    return h, int(req.value)


def ott_append(h, d_k: int, d_v: int, n_new, max_new: int, stream: int) -> None:
    arr = _host_counts(h, n_new, "n_new")
    _check(lib.ott_append(h, ctypes.c_void_p(d_k), ctypes.c_void_p(d_v), arr, max_new,
                          ctypes.c_void_p(stream)), "ott_append")


def ott_quantize_group(h, stream: int) -> int:
    n = ctypes.c_int32(0)
    _check(lib.ott_quantize_group(h, ctypes.c_void_p(stream), ctypes.byref(n)),
           "ott_quantize_group")
    return int(n.value)


def ott_prefill(h, d_k: int, d_v: int, lens, max_len: int, stream: int) -> None:
    arr = _host_counts(h, lens, "lens")
    _check(lib.ott_prefill(h, ctypes.c_void_p(d_k), ctypes.c_void_p(d_v), arr, max_len,
                           ctypes.c_void_p(stream)), "ott_prefill")


def ott_decode(h, d_q: int, d_out: int, stream: int) -> None:
    _check(lib.ott_decode(h, ctypes.c_void_p(d_q), ctypes.c_void_p(d_out),
                          ctypes.c_void_p(stream)), "ott_decode")


def ott_step(h, d_k: int, d_v: int, d_q: int, d_out: int, stream: int) -> int:
    """Returns the number of sequences quantized in the step."""
    n = ctypes.c_int32(0)
    _check(lib.ott_step(h, ctypes.c_void_p(d_k), ctypes.c_void_p(d_v), ctypes.c_void_p(d_q),
                        ctypes.c_void_p(d_out), ctypes.c_void_p(stream), ctypes.byref(n)),
           "ott_step")
    return int(n.value)


def ott_destroy(h) -> None:
    _batch_of.pop(getattr(h, "value", h), None)
    lib.ott_destroy(h)


def ott_get_layout(h) -> ott_layout_t:
    lay = ott_layout_t()
    _check(lib.ott_get_layout(h, ctypes.byref(lay)), "ott_get_layout")
    return lay


def ott_get_seq_state(h, b: int):
    out = (ctypes.c_int32 * 4)()
    _check(lib.ott_get_seq_state(h, b, out), "ott_get_seq_state")
    return tuple(int(x) for x in out)


def ott_set_num_splits(h, s: int) -> None:
    _check(lib.ott_set_num_splits(h, s), "ott_set_num_splits")


def ott_status_string(status: int) -> str:
    return lib.ott_status_string(status).decode()


def ott_fp16_decode(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, d_k: int,
                    d_v: int, max_len: int, lens, d_q: int, d_out: int, sm_scale: float,
                    d_work: Optional[int], work_bytes: int, num_splits: int, stream: int) -> None:
    if len(lens) != batch:
        raise ValueError(f"lens has {len(lens)} entries; batch is {batch}")
    arr = (ctypes.c_int32 * len(lens))(*[int(x) for x in lens])
    _check(lib.ott_fp16_decode(batch, num_q_heads, num_kv_heads, head_dim, ctypes.c_void_p(d_k),
                               ctypes.c_void_p(d_v), max_len, arr, ctypes.c_void_p(d_q),
                               ctypes.c_void_p(d_out), sm_scale, ctypes.c_void_p(d_work),
                               work_bytes, num_splits, ctypes.c_void_p(stream)), "ott_fp16_decode")


def ott_fp16_decode_noalloc(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            d_k: int, d_v: int, max_len: int, lens, d_q: int, d_out: int,
                            sm_scale: float, num_splits: int, stream: int) -> None:
    if len(lens) != batch:
        raise ValueError(f"lens has {len(lens)} entries; batch is {batch}")
    arr = (ctypes.c_int32 * len(lens))(*[int(x) for x in lens])
    _check(lib.ott_fp16_decode_noalloc(batch, num_q_heads, num_kv_heads, head_dim,
                                       ctypes.c_void_p(d_k), ctypes.c_void_p(d_v), max_len, arr,
                                       ctypes.c_void_p(d_q), ctypes.c_void_p(d_out), sm_scale,
                                       num_splits, ctypes.c_void_p(stream)),
           "ott_fp16_decode_noalloc")


def ott_fp16_decode_workspace(batch: int, num_q_heads: int, num_splits: int) -> int:
    return int(lib.ott_fp16_decode_workspace(batch, num_q_heads, num_splits))
