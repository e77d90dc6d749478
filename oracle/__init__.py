"""fp64 CPU oracle for RoPE and for softmax attention over rotated Q/K.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never loads it, and it imports nothing from the GPU package.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP); this module
compiles it with gcc on first use and wraps it for numpy arrays.  Every
function mirrors one C entry point; see the C file for the passages of
"RoPE and FlashAttention: relative positions and online softmax" and
"Write Triton Rope Kernel" that each follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "oracle.c"
LIBRARY = HERE / "liboracle.so"

NEOX, GPTJ = 0, 1
OK, ERR_ARG, ERR_EMPTY_ROW, ERR_NOMEM = 0, 1, 2, 3

_LAYOUTS = {"neox": NEOX, "gptj": GPTJ, NEOX: NEOX, GPTJ: GPTJ}


class OracleError(ValueError):
    """A non-zero status from the C oracle."""

    def __init__(self, status: int):
        names = {ERR_ARG: "invalid argument", ERR_EMPTY_ROW: "a query row sees no key",
                 ERR_NOMEM: "out of memory"}
        super().__init__(names.get(status, f"status {status}"))
        self.status = status


def compile_library(source: Path | str = SOURCE, output: Path | str = LIBRARY) -> Path:
    """Compile ``source`` into a shared library at ``output`` with gcc."""
    output = Path(output)
    tmp = output.with_name(output.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           str(source), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


class Oracle:
    """numpy front end over one compiled copy of ``oracle.c``."""

    def __init__(self, path: Path | str):
        self.path = str(path)
        lib = ctypes.CDLL(self.path)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_rope.argtypes = [_dp, _dp, i64, i32, i32, _dp, dbl, i32]
        lib.oracle_trig.argtypes = [dbl, i32, i64, dbl, _dp, _dp]
        lib.oracle_attention.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i64, i64, i64, i32, i32,
                                         i64, i64, i32, dbl, dbl, i32, i32, dbl]
        lib.oracle_attention_rows.argtypes = [_dp, _dp, _dp, i64, i64, i64, i64, i64, i32, i32,
                                              i64, i64, i32, dbl, dbl, i32, i32, dbl,
                                              _i64p, i64, _dp]
        lib.oracle_attention_lse.argtypes = [_dp, _dp, _dp, i64, i64, i64, i64, i64, i32,
                                             i64, i64, i32, dbl, dbl, i32, i32, dbl]
        lib.oracle_attention_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, i64, i64, i64, i64,
                                             i64, i32, i32, i64, i64, i32, dbl, dbl, i32, i32, dbl]
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        for fn in (lib.oracle_rope, lib.oracle_trig, lib.oracle_attention,
                   lib.oracle_attention_rows, lib.oracle_attention_lse, lib.oracle_attention_bwd,
                   lib.oracle_threads):
            fn.restype = ctypes.c_int
        self._lib = lib

    def threads(self) -> int:
        """OpenMP threads the oracle's parallel regions use."""
        return int(self._lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        """Use ``n`` OpenMP threads from now on (for single-thread timings)."""
        self._lib.oracle_set_threads(int(n))

    @staticmethod
    def _check(status: int) -> None:
        if status != OK:
            raise OracleError(status)

    def rope(self, x, positions, base: float = 10000.0, rot_dim: int | None = None,
             layout="gptj") -> np.ndarray:
        """Rotate the rows of ``x`` (``[..., rows, head_dim]``) at ``positions``.

        ``positions`` broadcasts against the row axes of ``x``: either one
        value per row of the last two axes' row dimension, or one per row of
        the whole leading shape.
        """
        x = _f64(x)
        head_dim = x.shape[-1]
        rot = head_dim if rot_dim is None else int(rot_dim)
        pos = np.broadcast_to(np.asarray(positions, dtype=np.float64), x.shape[:-1])
        pos = _f64(pos).reshape(-1)
        flat = x.reshape(-1, head_dim)
        out = np.empty_like(flat)
        self._check(self._lib.oracle_rope(_ptr(flat), _ptr(out), flat.shape[0], head_dim, rot,
                                          _ptr(pos), float(base), _LAYOUTS[layout]))
        return out.reshape(x.shape)

    def trig(self, base: float, rot_dim: int, n_pos: int, pos_div: float = 1.0):
        """fp64 (cos, sin) of (p / pos_div) * theta_i, each ``[n_pos, rot_dim/2]``
        (``pos_div`` > 1: position interpolation)."""
        half = rot_dim // 2
        c = np.empty((n_pos, half))
        s = np.empty((n_pos, half))
        self._check(self._lib.oracle_trig(float(base), int(rot_dim), int(n_pos), float(pos_div),
                                          _ptr(c), _ptr(s)))
        return c, s

    def attention(self, q, k, v, q_off: int = 0, k_off: int = 0, rot_dim: int | None = None,
                  base: float = 10000.0, layout="gptj", causal: bool = True,
                  scale: float = 0.0, pos_div: float = 1.0) -> np.ndarray:
        """Forward of softmax attention over rotated Q/K.

        ``q`` ``[B,H,Sq,D]``, ``k`` ``[B,Hkv,Sk,D]``, ``v`` ``[B,Hkv,Sk,Dv]``
        (``Hkv`` divides ``H``; query head h reads key/value head
        h // (H // Hkv)); 2-D or 3-D inputs are promoted.  ``rot_dim=0``
        disables the rotation; ``pos_div`` divides the positions the rotation
        angles use (position interpolation), not the mask's.
        """
        q, k, v = (_f64(a) for a in (q, k, v))
        nd = q.ndim
        while q.ndim < 4:
            q, k, v = q[None], k[None], v[None]
        B, H, Sq, D = q.shape
        Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
        rot = D if rot_dim is None else int(rot_dim)
        o = np.empty((B, H, Sq, Dv))
        self._check(self._lib.oracle_attention(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Hkv, Sq, Sk, D, Dv, int(q_off), int(k_off),
            rot, float(base), float(pos_div), _LAYOUTS[layout], int(bool(causal)), float(scale)))
        return o.reshape(o.shape[4 - nd:])

    def attention_rows(self, q, k, v, rows, q_off: int = 0, k_off: int = 0,
                       rot_dim: int | None = None, base: float = 10000.0, layout="gptj",
                       causal: bool = True, scale: float = 0.0, pos_div: float = 1.0) -> np.ndarray:
        """Output rows ``(b, h, i)`` of the same forward; returns ``[len(rows), Dv]``."""
        q, k, v = (_f64(a) for a in (q, k, v))
        B, H, Sq, D = q.shape
        Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
        rot = D if rot_dim is None else int(rot_dim)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.empty((r.shape[0], Dv))
        self._check(self._lib.oracle_attention_rows(
            _ptr(q), _ptr(k), _ptr(v), B, H, Hkv, Sq, Sk, D, Dv, int(q_off), int(k_off), rot,
            float(base), float(pos_div), _LAYOUTS[layout], int(bool(causal)), float(scale),
            r.ctypes.data_as(_i64p), r.shape[0], _ptr(out)))
        return out


    def attention_lse(self, q, k, q_off: int = 0, k_off: int = 0, rot_dim: int | None = None,
                      base: float = 10000.0, layout="gptj", causal: bool = True,
                      scale: float = 0.0, pos_div: float = 1.0) -> np.ndarray:
        """Natural-log log-sum-exp of each query row's scores, ``[B, H, Sq]``."""
        q, k = _f64(q), _f64(k)
        B, H, Sq, D = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        rot = D if rot_dim is None else int(rot_dim)
        out = np.empty((B, H, Sq))
        self._check(self._lib.oracle_attention_lse(
            _ptr(q), _ptr(k), _ptr(out), B, H, Hkv, Sq, Sk, D, int(q_off), int(k_off), rot,
            float(base), float(pos_div), _LAYOUTS[layout], int(bool(causal)), float(scale)))
        return out

    def attention_bwd(self, q, k, v, dout, q_off: int = 0, k_off: int = 0,
                      rot_dim: int | None = None, base: float = 10000.0, layout="gptj",
                      causal: bool = True, scale: float = 0.0, pos_div: float = 1.0):
        """Gradients (dq, dk, dv) of ``attention`` for the upstream gradient
        ``dout`` (same shape as the output); 4-D inputs."""
        q, k, v, dout = (_f64(a) for a in (q, k, v, dout))
        B, H, Sq, D = q.shape
        Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
        rot = D if rot_dim is None else int(rot_dim)
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        self._check(self._lib.oracle_attention_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, Sq, Sk,
            D, Dv, int(q_off), int(k_off), rot, float(base), float(pos_div), _LAYOUTS[layout],
            int(bool(causal)), float(scale)))
        return dq, dk, dv


_DEFAULT: Oracle | None = None


def build() -> Path:
    """Compile the oracle library in place (always recompiles)."""
    return compile_library()


def load() -> Oracle:
    """The oracle built from ``oracle.c``; compiled on first use if absent or stale."""
    global _DEFAULT
    if _DEFAULT is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            compile_library()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def load_variant(source_text: str, tag: str) -> Oracle:
    """Compile a modified copy of the oracle source (used by tests that plant a
    mistake in the oracle to show that the pins catch it)."""
    d = Path(tempfile.mkdtemp(prefix=f"oracle_{tag}_"))
    src = d / "oracle.c"
    src.write_text(source_text)
    return Oracle(compile_library(src, d / "liboracle.so"))
