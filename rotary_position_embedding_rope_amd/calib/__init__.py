"""ctypes view of ``librope_calib.so`` (include/rope_calib.h): measurement
kernels timed by bench.py beside the library's own (an in-place 16-byte
stream, and a flash-attention inner step on LDS-resident tiles).  Not part
of the RoPE path; loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIBRARY = Path(__file__).resolve().parent.parent / "librope_calib.so"
OK, ERR_NULL, ERR_SHAPE, ERR_HIP = 0, 1, 2, 7
EXPORTS = ("rope_calib_stream_inplace", "rope_calib_stream_read", "rope_calib_attn_loop")
# (head dim, waves per SIMD, pipelined) variants the loop kernel is built for
LOOP_VARIANTS = tuple((64, w, p) for w in (1, 2, 3, 4) for p in (0, 1)) + \
    tuple((128, w, p) for w in (1, 2) for p in (0, 1))
TILE_KEYS = 64

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not LIBRARY.exists():
        raise RuntimeError(f"{LIBRARY} is missing: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(str(LIBRARY))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rope_calib_stream_inplace.argtypes = [vp, i64, i32, i32, vp]
    lib.rope_calib_stream_inplace.restype = i32
    lib.rope_calib_stream_read.argtypes = [vp, i64, ctypes.c_uint32, vp, vp]
    lib.rope_calib_stream_read.restype = i32
    lib.rope_calib_attn_loop.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.rope_calib_attn_loop.restype = i32
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise RuntimeError(f"{what} failed with status {rc}")


def stream_inplace(buf, n_vec: int, row_vecs: int, span_vecs: int, stream=None) -> None:
    """Add 1 to every 32-bit word of n_vec 16-byte vectors of the device
    tensor `buf` in place: vector v at (v // span_vecs) * row_vecs +
    v % span_vecs."""
    need = -(-n_vec // span_vecs) * row_vecs * 16
    if buf.numel() * buf.element_size() < need:
        raise ValueError(f"buffer holds {buf.numel() * buf.element_size()} bytes, the pattern needs {need}")
    _check(load().rope_calib_stream_inplace(buf.data_ptr(), n_vec, row_vecs, span_vecs,
                                            None if stream is None else stream.cuda_stream),
           "rope_calib_stream_inplace")


def stream_read(buf, n_vec: int, key: int, hit, stream=None) -> None:
    """Read n_vec 16-byte vectors of the device tensor `buf`; a vector of
    four words equal to `key` writes its index into the int64 tensor `hit`."""
    if buf.numel() * buf.element_size() < 16 * n_vec:
        raise ValueError(f"buffer holds {buf.numel() * buf.element_size()} bytes, the read needs {16 * n_vec}")
    if hit.numel() < 1 or hit.element_size() != 8:
        raise ValueError("hit must hold one int64")
    _check(load().rope_calib_stream_read(buf.data_ptr(), n_vec, key & 0xffffffff, hit.data_ptr(),
                                         None if stream is None else stream.cuda_stream),
           "rope_calib_stream_read")


def loop_shapes(head_dim: int, waves_per_simd: int, workgroups: int):
    """Element counts of (k_tile, v_tile, q_rows, out, cycles) for one call."""
    threads = 256 * waves_per_simd
    return (TILE_KEYS * (head_dim + 8), TILE_KEYS * head_dim, 128 * waves_per_simd * head_dim,
            workgroups * threads * (head_dim // 2 + 4), workgroups * 4 * waves_per_simd)


def attn_loop(head_dim: int, waves_per_simd: int, pipelined: int, iters: int, workgroups: int,
              k_tile, v_tile, q_rows, out, cycles=None, stream=None) -> None:
    """One launch of the attention inner-step kernel; tensor sizes are
    checked against loop_shapes()."""
    if (head_dim, waves_per_simd, pipelined) not in LOOP_VARIANTS:
        raise ValueError(f"no loop kernel for {(head_dim, waves_per_simd, pipelined)}")
    want = loop_shapes(head_dim, waves_per_simd, workgroups)
    tensors = (k_tile, v_tile, q_rows, out) + ((cycles,) if cycles is not None else ())
    for t, n in zip(tensors, want):
        if t.numel() < n or not t.is_contiguous():
            raise ValueError(f"tensor of {t.numel()} elements where the kernel reads/writes {n}")
    _check(load().rope_calib_attn_loop(head_dim, waves_per_simd, pipelined, iters, workgroups,
                                       k_tile.data_ptr(), v_tile.data_ptr(), q_rows.data_ptr(),
                                       out.data_ptr(), None if cycles is None else cycles.data_ptr(),
                                       None if stream is None else stream.cuda_stream),
           "rope_calib_attn_loop")
