"""ctypes loader for ``libpagedkv.so`` (the C ABI in ``include/pagedkv.h``).

Loading fails loudly when the library has not been built: there is no fallback.
torch is imported first so that the library binds to the HIP runtime torch has
already loaded (both use the ``libamdhip64.so.7`` soname), which lets device
pointers and stream handles from torch pass straight through.
"""

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime before the library does)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_F32 = 0
PKV_BF16 = 1
PKV_OK = 0
PKV_EINVAL = -1
PKV_EUNSUPPORTED = -2
PKV_ENOMEM = -3
PKV_ELAUNCH = -4
PKV_ENOSEQ = -5
PKV_EWORKSPACE = -6
PKV_ESWAPPED = -7
BLOCK_SIZE = 16
PARTITION_TOKENS = 512
STATIC_WORKSPACE_BYTES = 64 << 20

_i32, _i64, _u64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_p, _sz = ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_write": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "pkv_attention_decode": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p]),
    "pkv_attention_decode_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _i32, _i32,
                                                    _i32, _i32, _i32, ctypes.c_int, _p]),
    "pkv_attention_decode_plan": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p]),
    "pkv_attention_decode_plan_upload": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _i32,
                                                        _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p, _p,
                                                        _p, _sz, _p, _p, _p, _p]),
    "pkv_attention_decode_partitions": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _i32,
                                                       _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p]),
    "pkv_attention_decode_merge": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p]),
    "pkv_attention_decode_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _f32, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p]),
    "pkv_attention_decode_partitions_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _f32, _i32, _i32,
                                                              _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                                              _p, _sz, _p]),
    "pkv_varlen_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_attention_varlen": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _f32, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz, _p]),
    "pkv_attention_varlen_plan_upload": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _f32, _i32, _i32,
                                                        _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz,
                                                        _p, _p, _p, _sz, _p, _p]),
    "pkv_attention_varlen_partitions": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _f32, _i32, _i32,
                                                       _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz,
                                                       _p]),
    "pkv_lse_merge": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, ctypes.c_int, _p]),
    "pkv_copy_blocks": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p]),
    "pkv_swap_blocks": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                       _p]),
    "pkv_decode_graph_create": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _f32, _i32, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _sz]),
    "pkv_decode_graph_launch": (ctypes.c_int, [_p, _p]),
    "pkv_decode_graph_destroy": (None, [_p]),
    "pkv_check_tables": (ctypes.c_int, [_p, _p, _i32, _i32, _i32]),
    "pkv_check_slots": (ctypes.c_int, [_p, _i32, _i32, _i32]),
    "pkv_check_pool": (ctypes.c_int, [_p, _sz]),
    "pkv_alloc_create": (_p, [_i32, _i32, _u64]),
    "pkv_alloc_destroy": (None, [_p]),
    "pkv_alloc_add_seq": (ctypes.c_int, [_p, _i64]),
    "pkv_alloc_fork": (ctypes.c_int, [_p, _i64, _i64]),
    "pkv_alloc_append": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _p]),
    "pkv_alloc_append_batch": (ctypes.c_int, [_p, _p, _p, _i32, _p, _i64, _p, _i32, _p]),
    "pkv_alloc_free_seq": (ctypes.c_int, [_p, _i64]),
    "pkv_alloc_block_table": (ctypes.c_int, [_p, _i64, _p, _i32, _p]),
    "pkv_alloc_block_tables": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _i32, _p]),
    "pkv_alloc_seq_len": (_i64, [_p, _i64]),
    "pkv_alloc_num_free": (_i32, [_p]),
    "pkv_alloc_num_blocks": (_i32, [_p]),
    "pkv_alloc_refcount": (_i32, [_p, _i32]),
    "pkv_alloc_add_seq_tokens": (ctypes.c_int, [_p, _i64, _p, _i32, _u64, _p, _p]),
    "pkv_alloc_append_tokens": (ctypes.c_int, [_p, _i64, _p, _i32, _p, _p, _p]),
    "pkv_alloc_num_cached": (_i32, [_p]),
    "pkv_alloc_set_host_pool": (ctypes.c_int, [_p, _i32]),
    "pkv_alloc_swap_out": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _p]),
    "pkv_alloc_swap_in": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _p]),
    "pkv_alloc_is_swapped": (ctypes.c_int, [_p, _i64]),
    "pkv_alloc_host_table": (ctypes.c_int, [_p, _i64, _p, _i32, _p]),
    "pkv_alloc_num_free_host": (_i32, [_p]),
    "pkv_alloc_host_refcount": (_i32, [_p, _i32]),
}
# The varlen launches one by one take the same arguments as their last three together.
for _name in ("pkv_attention_varlen_plan", "pkv_attention_varlen_decode_partitions",
              "pkv_attention_varlen_prefill_tiles", "pkv_attention_varlen_merge"):
    SIGNATURES[_name] = SIGNATURES["pkv_attention_varlen_partitions"]

_lib = None


def lib():
    """The loaded library (loaded on first use).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python paged_kv_cache_360_amd/build.py` "
                "(the paged-attention path has no fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class PagedKVError(RuntimeError):
    """A C-ABI call returned a negative status."""

    def __init__(self, func, code):
        self.code = code
        msg = lib().pkv_last_error().decode(errors="replace")
        super().__init__(f"{func}: {lib().pkv_strerror(code).decode()} ({code}): {msg}")


def check(func, code):
    if code != PKV_OK:
        raise PagedKVError(func, code)
    return code
