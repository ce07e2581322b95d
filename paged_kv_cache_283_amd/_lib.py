"""ctypes loader for libpagedkv.so (the gfx950 HIP library built in-tree).

The library must have been built (``python -m paged_kv_cache_283_amd.build`` or
``__graft_entry__.build()``); there is no fallback of any kind.
"""
import ctypes
import os

LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

# pkv_status
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EDEVICE = range(5)
STATUS_NAMES = {OK: "PKV_OK", EINVAL: "PKV_EINVAL", EUNSUPPORTED: "PKV_EUNSUPPORTED",
                EWORKSPACE: "PKV_EWORKSPACE", EDEVICE: "PKV_EDEVICE"}

# pkv_dtype
F32, BF16, F16, FP8_E4M3, INT8, FP8_E4M3_CHANNEL, INT8_CHANNEL = range(7)
CAND_REST, CAND_ALL = range(2)

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_F = ctypes.c_float

# name -> (restype, argtypes), mirroring include/pagedkv.h
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "paged_decode_slots": (_I, [_P, _I, _P, _I, _I, _I, _P, _P]),
    "paged_token_slots": (_I, [_P, _I, _I, _P, _P, _I, _I, _I, _P, _P]),
    "paged_kv_write": (_I, [_P, _P, _I, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "paged_decode_attn_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "paged_decode_attn": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                               _F, _I, _I, _P, _I, _P, _Z, _P]),
    "paged_decode_attn_noalloc": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                       _F, _I, _I, _P, _I, _P]),
    "paged_decode_append_attn": (_I, [_P, _I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I,
                                      _I, _I, _I, _F, _I, _I, _P, _I, _P, _Z, _P]),
    "paged_decode_attn_compact_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "paged_decode_attn_compact": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _I, _P, _P,
                                       _I, _I, _I, _I, _I, _I, _I, _F, _P, _I, _P, _I, _P, _Z, _P]),
    "kv_block_copy": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "h2o_select": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P]),
    "paged_kv_append": (_I, [_P, _P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "paged_prefill_attn": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                _I, _I, _F, _P]),
    "kv_swap": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "kv_keep_select": (_I, [_P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P]),
    "kv_compact": (_I, [_P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "pkv_timing_begin": (_I, [_I]),
    "pkv_timing_end": (_I, [ctypes.POINTER(ctypes.c_float), _I]),
    "pkv_probe_read": (_I, [_P, _Z, _P, _P]),
    "pkv_probe_copy": (_I, [_P, _P, _Z, _P]),
}


class PagedKVError(RuntimeError):
    """A non-OK pkv_status, with the library's message."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libpagedkv.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_283_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(fn: str, status: int) -> None:
    if status != OK:
        msg = load().pkv_last_error().decode(errors="replace")
        raise PagedKVError(fn, status, msg)


def call(fn: str, *args) -> None:
    """Call a status-returning entry point and raise PagedKVError on failure."""
    check(fn, getattr(load(), fn)(*args))
