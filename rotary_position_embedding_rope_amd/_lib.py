"""ctypes view of ``librope_mi355x.so`` (the C ABI of include/rope_mi355x.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIBRARY = Path(__file__).resolve().parent / "librope_mi355x.so"

NEOX, GPTJ = 0, 1
BF16, F32, F16 = 0, 1, 2
OK, ERR_NULL, ERR_SHAPE, ERR_BASE, ERR_UNSUPPORTED, ERR_EMPTY_ROW, ERR_TABLE_RANGE, ERR_HIP, ERR_ALIGN, \
    ERR_SCRATCH = range(10)
DECODE_SCRATCH_BYTES = 8 << 20   # ROPE_DECODE_SCRATCH_BYTES

# every symbol include/rope_mi355x.h declares
EXPORTS = ("rope_status_str", "rope_tables_build", "rope_tables_build_scaled", "rope_apply",
           "rope_flash_attn_fwd", "rope_flash_attn_bwd", "rope_flash_attn_bwd_workspace_size",
           "rope_flash_attn_workspace_size", "rope_decode_attn_fwd", "rope_decode_workspace_size",
           "rope_decode_attn_fwd_noalloc")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not LIBRARY.exists():
        raise RuntimeError(
            f"{LIBRARY} is missing: build it first (python -m "
            "rotary_position_embedding_rope_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(str(LIBRARY))
    vp, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.rope_status_str.argtypes = [i32]
    lib.rope_status_str.restype = ctypes.c_char_p
    lib.rope_tables_build.argtypes = [f64, i32, i64, vp, vp, vp]
    lib.rope_tables_build.restype = i32
    lib.rope_tables_build_scaled.argtypes = [f64, i32, i64, f64, vp, vp, vp]
    lib.rope_tables_build_scaled.restype = i32
    lib.rope_apply.argtypes = [vp, i64, i64, i32, vp, i64, i64, i32, vp, i64, vp, vp, i64,
                               i32, i32, i32, i32, vp]
    lib.rope_apply.restype = i32
    lib.rope_flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i64, i64,
                                        vp, vp, i64, i32, i32, i32, f32, i32, vp, i64, vp]
    lib.rope_flash_attn_fwd.restype = i32
    lib.rope_flash_attn_workspace_size.argtypes = [i32, i32, i64, i64, i32, i64, i64, i32, i32]
    lib.rope_flash_attn_workspace_size.restype = i64
    lib.rope_flash_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32,
                                        i64, i64, vp, vp, i64, i32, i32, i32, f32, i32, vp, i64, vp]
    lib.rope_flash_attn_bwd.restype = i32
    lib.rope_flash_attn_bwd_workspace_size.argtypes = [i32, i32, i32, i64, i64, i32, i32, i32]
    lib.rope_flash_attn_bwd_workspace_size.restype = i64
    lib.rope_decode_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32,
                                         vp, vp, i64, i32, i32, f32, i32, vp, i64, vp]
    lib.rope_decode_attn_fwd.restype = i32
    lib.rope_decode_workspace_size.argtypes = [i32, i32, i32, i64, i32]
    lib.rope_decode_workspace_size.restype = i64
    lib.rope_decode_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32,
                                                 vp, vp, i64, i32, i32, f32, i32, vp]
    lib.rope_decode_attn_fwd_noalloc.restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().rope_status_str(int(status)).decode()
