"""Python binding of the C ABI over torch tensors.

Argument marshalling only: each function checks tensor devices/dtypes/shapes
that ctypes cannot see, passes data pointers and the current HIP stream to
the library, and raises ``RopeError`` on a non-zero status.  All computation
happens in the HIP kernels; there is no CPU or eager fallback.  torch provides
device memory and streams.
"""
from __future__ import annotations

import torch

from . import _lib


class RopeError(ValueError):
    """Non-zero status from the C library."""

    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.status_str(status)} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != _lib.OK:
        raise RopeError(status, where)


_LAYOUT = {"neox": _lib.NEOX, "gptj": _lib.GPTJ}


def _layout(layout) -> int:
    if isinstance(layout, str):
        return _LAYOUT[layout.lower()]
    return int(layout)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    if t.dtype == torch.float16:
        return _lib.F16
    raise TypeError(f"unsupported dtype {t.dtype}; bfloat16, float16 or float32 expected")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def tables_build(base: float, rot_dim: int, max_pos: int, device="cuda", pos_divisor: float = 1.0):
    """fp32 (cos, sin) tables ``[max_pos, rot_dim/2]`` built on the device;
    ``pos_divisor`` > 1 builds them for position interpolation."""
    lib = _lib.load()
    cos = torch.empty((max_pos, rot_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    if pos_divisor == 1.0:
        _check(lib.rope_tables_build(float(base), int(rot_dim), int(max_pos), cos.data_ptr(),
                                     sin.data_ptr(), _stream(cos)), "rope_tables_build")
    else:
        _check(lib.rope_tables_build_scaled(float(base), int(rot_dim), int(max_pos),
                                            float(pos_divisor), cos.data_ptr(), sin.data_ptr(),
                                            _stream(cos)), "rope_tables_build_scaled")
    return cos, sin


def rope_apply(q: torch.Tensor | None, k: torch.Tensor | None, positions: torch.Tensor,
               cos: torch.Tensor, sin: torch.Tensor, rot_dim: int | None = None,
               layout="neox") -> None:
    """Rotate ``q`` ``[T, H_q, D]`` and ``k`` ``[T, H_kv, D]`` in place at
    ``positions`` (int32 ``[T]``); either may be None.  One kernel launch."""
    lib = _lib.load()
    ref = q if q is not None else k
    if ref is None:
        raise ValueError("need q or k")
    _require_cuda(q, k, positions, cos, sin)
    if positions.dtype != torch.int32 or positions.dim() != 1 or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int32 vector")
    if cos.dtype != torch.float32 or sin.dtype != torch.float32:
        raise ValueError("cos/sin tables must be float32")
    if not (cos.is_contiguous() and sin.is_contiguous() and cos.shape == sin.shape):
        raise ValueError("cos/sin must be contiguous tables of equal shape")
    T, D = ref.shape[0], ref.shape[-1]
    rot = D if rot_dim is None else int(rot_dim)
    if cos.dim() != 2 or cos.shape[1] != rot // 2:
        raise ValueError("table rows must hold rot_dim/2 values")
    args = []
    for t in (q, k):
        if t is None:
            args += [None, 0, 0, 0]
            continue
        if t.dim() != 3 or t.shape[0] != T or t.shape[2] != D or t.stride(2) != 1:
            raise ValueError("q/k must be [tokens, heads, head_dim] with contiguous head_dim")
        if t.dtype != ref.dtype:
            raise ValueError("q and k must share a dtype")
        args += [t.data_ptr(), t.stride(0), t.stride(1), t.shape[1]]
    if positions.numel() != T:
        raise ValueError("one position per token")
    _check(lib.rope_apply(*args, positions.data_ptr(), T, cos.data_ptr(), sin.data_ptr(),
                          cos.shape[0], D, rot, _layout(layout), _dtype(ref), _stream(ref)),
           "rope_apply")


_WORKSPACES: dict = {}


def workspace_for(q: torch.Tensor, Sk: int, q_pos_offset: int, k_pos_offset: int,
                  causal: bool) -> torch.Tensor | None:
    """Workspace for the split-key schedule of this forward, cached per device
    and grown on demand (None when the library would use none).  Calls
    sharing it must be serialised, which holds on one stream."""
    lib = _lib.load()
    B, H, Sq, D = q.shape
    need = lib.rope_flash_attn_workspace_size(B, H, Sq, Sk, D, int(q_pos_offset), int(k_pos_offset),
                                              int(bool(causal)), _dtype(q))
    if need < 0:
        raise RopeError(-need, "rope_flash_attn_workspace_size")
    if need == 0:
        return None
    key = q.device
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        _WORKSPACES[key] = ws
    return ws


def flash_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   cos: torch.Tensor | None = None, sin: torch.Tensor | None = None,
                   q_pos_offset: int = 0, k_pos_offset: int = 0, rot_dim: int | None = None,
                   layout="neox", causal: bool = True, softmax_scale: float = 0.0,
                   out: torch.Tensor | None = None, workspace="auto",
                   lse: torch.Tensor | None = None) -> torch.Tensor:
    """Fused RoPE + attention forward: ``q`` ``[B, H, Sq, D]``, ``k`` and
    ``v`` ``[B, H_kv, Sk, D]`` with H_kv dividing H (query head h reads
    key/value head h // (H // H_kv)).  ``lse``: optional float32
    ``[B, H, Sq]`` tensor that receives each query row's log-sum-exp (the
    row statistics flash_attn_bwd needs).

    ``rot_dim=0`` (or no tables) runs plain attention.  Returns ``out``
    (allocated like ``q`` when not given).  ``workspace``: "auto" (the
    default: a per-device cached buffer of the size the library asks for,
    none when it asks for none; head dim 128 with fewer query-tile pairs than
    CUs then splits the key range across workgroups), None (never split) or
    a uint8 tensor of at least the library's requested size."""
    lib = _lib.load()
    _require_cuda(q, k, v, cos, sin)
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous [B, H, S, D] tensors of one dtype")
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Sk, D) or v.shape != k.shape or Hkv < 1 or H % Hkv != 0:
        raise ValueError("k and v must be [B, H_kv, Sk, D] with H_kv dividing q's H")
    if rot_dim is None:
        rot_dim = D if cos is not None else 0
    if rot_dim > 0:
        if cos is None or sin is None:
            raise ValueError("rotation needs cos/sin tables")
        if cos.dtype != torch.float32 or not cos.is_contiguous() or cos.shape != sin.shape \
                or not sin.is_contiguous() or cos.dim() != 2 or cos.shape[1] != rot_dim // 2:
            raise ValueError("cos/sin must be contiguous float32 [rows, rot_dim/2]")
        cp, sp, rows = cos.data_ptr(), sin.data_ptr(), cos.shape[0]
    else:
        cp, sp, rows = None, None, 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is not None and (lse.shape != (B, H, Sq) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor on q's device")
    if isinstance(workspace, str):
        workspace = workspace_for(q, Sk, q_pos_offset, k_pos_offset, causal)
    wp, wb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) \
        if workspace is not None else (None, 0)
    _check(lib.rope_flash_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None,
                                   B, H, Hkv, Sq, Sk, D, int(q_pos_offset), int(k_pos_offset),
                                   cp, sp, rows, int(rot_dim), _layout(layout), int(bool(causal)),
                                   float(softmax_scale), _dtype(q), wp, wb, _stream(q)),
           "rope_flash_attn_fwd")
    return out


def prepare_flash_attn_fwd(q, k, v, out, cos=None, sin=None, q_pos_offset: int = 0,
                           k_pos_offset: int = 0, rot_dim: int | None = None, layout="neox",
                           causal: bool = True, softmax_scale: float = 0.0, workspace="auto",
                           lse=None):
    """Validate once and return a zero-argument callable that enqueues the
    fused forward on fixed buffers (for repeated launches in timing loops;
    the buffers must stay alive and unchanged in shape)."""
    if isinstance(workspace, str):
        workspace = workspace_for(q, k.shape[2], q_pos_offset, k_pos_offset, causal)
    flash_attn_fwd(q, k, v, cos, sin, q_pos_offset, k_pos_offset, rot_dim, layout, causal,
                   softmax_scale, out, workspace, lse)   # validates and runs once
    lib = _lib.load()
    B, H, Sq, D = q.shape
    rot = (D if cos is not None else 0) if rot_dim is None else int(rot_dim)
    wp, wb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) \
        if workspace is not None else (None, 0)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, B, H, k.shape[1], Sq, k.shape[2], D,
            int(q_pos_offset), int(k_pos_offset), cos.data_ptr() if rot else None,
            sin.data_ptr() if rot else None, cos.shape[0] if rot else 0, rot, _layout(layout),
            int(bool(causal)), float(softmax_scale), _dtype(q), wp, wb, _stream(q))
    fn = lib.rope_flash_attn_fwd

    def launch():
        status = fn(*args)
        if status != _lib.OK:
            raise RopeError(status, "rope_flash_attn_fwd")
    # the callable holds the workspace it launches on: a later call that grows
    # the per-device cache cannot free it under a prepared launch
    launch.workspace = workspace
    return launch


def prepare_rope_apply(q, k, positions, cos, sin, rot_dim: int | None = None, layout="neox"):
    """Validate once and return a zero-argument callable that enqueues
    rope_apply on fixed buffers (in place)."""
    rope_apply(q, k, positions, cos, sin, rot_dim, layout)
    lib = _lib.load()
    ref = q if q is not None else k
    T, D = ref.shape[0], ref.shape[-1]
    rot = D if rot_dim is None else int(rot_dim)
    args = []
    for t in (q, k):
        args += [None, 0, 0, 0] if t is None else [t.data_ptr(), t.stride(0), t.stride(1), t.shape[1]]
    args += [positions.data_ptr(), T, cos.data_ptr(), sin.data_ptr(), cos.shape[0], D, rot,
             _layout(layout), _dtype(ref), _stream(ref)]
    fn = lib.rope_apply

    def launch():
        status = fn(*args)
        if status != _lib.OK:
            raise RopeError(status, "rope_apply")
    return launch


def decode_workspace(q: torch.Tensor, k_cache: torch.Tensor) -> torch.Tensor:
    """Workspace for decode_attn_fwd on these shapes, cached per device and
    grown on demand.  Calls sharing it must be serialised (one stream)."""
    lib = _lib.load()
    B, H, D = q.shape
    need = lib.rope_decode_workspace_size(B, H, k_cache.shape[1], k_cache.shape[2], D)
    if need < 0:
        raise RopeError(-need, "rope_decode_workspace_size")
    key = ("decode", q.device)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        _WORKSPACES[key] = ws
    return ws


_NO_WORKSPACE = object()   # _decode_args marker: the static-scratch entry point takes none


def _decode_args(q, k_new, v_new, k_cache, v_cache, cache_lens, cos, sin, rot_dim, layout,
                 softmax_scale, out, workspace):
    _require_cuda(q, k_new, v_new, k_cache, v_cache, cache_lens, cos, sin, out)
    for t in (q, k_new, v_new, k_cache, v_cache, out):
        if t.dtype not in (torch.bfloat16, torch.float16) or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k_new, v_new, caches and out must be contiguous, all bfloat16 or all "
                             "float16")
    if q.dim() != 3:
        raise ValueError("q must be [B, H, D] (one new query per request)")
    B, H, D = q.shape
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("k_cache must be [B, H_kv, S_max, D]")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D):
        raise ValueError("v_cache like k_cache, k_new/v_new [B, H_kv, D]")
    if out.shape != q.shape:
        raise ValueError("out must be like q")
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (B,) or not cache_lens.is_contiguous():
        raise ValueError("cache_lens must be a contiguous int32 [B] vector")
    rot = (D if cos is not None else 0) if rot_dim is None else int(rot_dim)
    if rot > 0:
        if cos is None or sin is None or cos.dtype != torch.float32 or cos.shape != sin.shape \
                or not cos.is_contiguous() or not sin.is_contiguous() or cos.dim() != 2 \
                or cos.shape[1] != rot // 2:
            raise ValueError("cos/sin must be contiguous float32 [rows, rot_dim/2]")
        cp, sp, rows = cos.data_ptr(), sin.data_ptr(), cos.shape[0]
    else:
        cp, sp, rows = None, None, 0
    if workspace is _NO_WORKSPACE:
        return None, (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                      cache_lens.data_ptr(), out.data_ptr(), B, H, Hkv, S_max, D, cp, sp, rows, rot,
                      _layout(layout), float(softmax_scale), _dtype(q), _stream(q))
    if workspace is None:
        workspace = decode_workspace(q, k_cache)
    return workspace, (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            cache_lens.data_ptr(), out.data_ptr(), B, H, Hkv, S_max, D, cp, sp, rows, rot,
            _layout(layout), float(softmax_scale), _dtype(q), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(q))


def decode_attn_fwd(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, cache_lens: torch.Tensor,
                    cos: torch.Tensor | None = None, sin: torch.Tensor | None = None,
                    rot_dim: int | None = None, layout="neox", softmax_scale: float = 0.0,
                    out: torch.Tensor | None = None, workspace=None) -> torch.Tensor:
    """One decode step: ``q`` ``[B, H, D]``, ``k_new``/``v_new`` ``[B, H_kv, D]``
    at positions ``cache_lens`` (int32 ``[B]``); appends rope(k_new) and v_new
    to ``k_cache``/``v_cache`` ``[B, H_kv, S_max, D]`` and returns the
    attention output ``[B, H, D]`` over the L + 1 cached keys."""
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    _, args = _decode_args(q, k_new, v_new, k_cache, v_cache, cache_lens, cos, sin, rot_dim, layout,
                           softmax_scale, out, workspace)
    _check(lib.rope_decode_attn_fwd(*args), "rope_decode_attn_fwd")
    return out


def decode_attn_fwd_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            k_cache: torch.Tensor, v_cache: torch.Tensor, cache_lens: torch.Tensor,
                            out: torch.Tensor, cos: torch.Tensor | None = None,
                            sin: torch.Tensor | None = None, rot_dim: int | None = None, layout="neox",
                            softmax_scale: float = 0.0) -> torch.Tensor:
    """decode_attn_fwd through rope_decode_attn_fwd_noalloc: the same step on
    the library's static per-GPU scratch, allocating nothing (``out`` is
    required).  Calls that may overlap on one GPU must be serialised."""
    lib = _lib.load()
    _, args = _decode_args(q, k_new, v_new, k_cache, v_cache, cache_lens, cos, sin, rot_dim, layout,
                           softmax_scale, out, _NO_WORKSPACE)
    _check(lib.rope_decode_attn_fwd_noalloc(*args), "rope_decode_attn_fwd_noalloc")
    return out


def prepare_decode_attn_fwd(q, k_new, v_new, k_cache, v_cache, cache_lens, out, cos=None,
                            sin=None, rot_dim: int | None = None, layout="neox",
                            softmax_scale: float = 0.0, workspace=None):
    """Validate once and return a zero-argument callable that enqueues the
    decode step on fixed buffers (each call appends at the same positions)."""
    ws, args = _decode_args(q, k_new, v_new, k_cache, v_cache, cache_lens, cos, sin, rot_dim, layout,
                            softmax_scale, out, workspace)
    fn = _lib.load().rope_decode_attn_fwd

    def launch():
        status = fn(*args)
        if status != _lib.OK:
            raise RopeError(status, "rope_decode_attn_fwd")
    launch.workspace = ws   # kept alive as long as the callable (see prepare_flash_attn_fwd)
    return launch


def bwd_workspace(q: torch.Tensor, k: torch.Tensor, rot_dim: int) -> torch.Tensor:
    """Workspace for flash_attn_bwd on q's and k's shapes, cached per device
    and grown on demand.  Calls sharing it must be serialised (one stream)."""
    lib = _lib.load()
    B, H, Sq, D = q.shape
    need = lib.rope_flash_attn_bwd_workspace_size(B, H, k.shape[1], Sq, k.shape[2], D, int(rot_dim),
                                                  _dtype(q))
    if need < 0:
        raise RopeError(-need, "rope_flash_attn_bwd_workspace_size")
    key = ("bwd", q.device)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        _WORKSPACES[key] = ws
    return ws


def _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, cos, sin, q_pos_offset, k_pos_offset, rot_dim,
              layout, causal, softmax_scale, workspace):
    _require_cuda(q, k, v, o, lse, dout, dq, dk, dv, cos, sin)
    for t in (q, k, v, o, dout, dq, dk, dv):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o, dout and the gradients must be contiguous 4-D tensors of "
                             "one dtype on one device")
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Sk, D) or v.shape != k.shape or Hkv < 1 or H % Hkv != 0:
        raise ValueError("k and v must be [B, H_kv, Sk, D] with H_kv dividing q's H")
    if o.shape != q.shape or dout.shape != q.shape or dq.shape != q.shape or dk.shape != k.shape \
            or dv.shape != k.shape:
        raise ValueError("o, dout, dq must be shaped like q; dk, dv like k")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    if rot_dim is None:
        rot_dim = D if cos is not None else 0
    if rot_dim > 0:
        if cos is None or sin is None or cos.dtype != torch.float32 or not cos.is_contiguous() \
                or cos.shape != sin.shape or not sin.is_contiguous() or cos.dim() != 2 \
                or cos.shape[1] != rot_dim // 2:
            raise ValueError("rotation needs contiguous float32 cos/sin [rows, rot_dim/2]")
        cp, sp, rows = cos.data_ptr(), sin.data_ptr(), cos.shape[0]
    else:
        cp, sp, rows = None, None, 0
    ws = bwd_workspace(q, k, rot_dim) if workspace is None else workspace
    return ws, (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, Sq, Sk, D, int(q_pos_offset),
            int(k_pos_offset), cp, sp, rows, int(rot_dim), _layout(layout), int(bool(causal)),
            float(softmax_scale), _dtype(q), ws.data_ptr(), ws.numel() * ws.element_size(),
            _stream(q))


def flash_attn_bwd(q, k, v, o, lse, dout, cos=None, sin=None, q_pos_offset: int = 0,
                   k_pos_offset: int = 0, rot_dim: int | None = None, layout="neox",
                   causal: bool = True, softmax_scale: float = 0.0, dq=None, dk=None, dv=None,
                   workspace=None):
    """Gradients (dq, dk, dv) of flash_attn_fwd for the upstream gradient
    ``dout``, from the forward's output ``o`` and row statistics ``lse``
    (pass the same rotation and mask arguments as to the forward)."""
    lib = _lib.load()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _, args = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, cos, sin, q_pos_offset, k_pos_offset,
                        rot_dim, layout, causal, softmax_scale, workspace)
    _check(lib.rope_flash_attn_bwd(*args), "rope_flash_attn_bwd")
    return dq, dk, dv


def prepare_flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, cos=None, sin=None,
                           q_pos_offset: int = 0, k_pos_offset: int = 0, rot_dim: int | None = None,
                           layout="neox", causal: bool = True, softmax_scale: float = 0.0,
                           workspace=None):
    """Validate once and return a zero-argument callable that enqueues the
    backward on fixed buffers."""
    ws, args = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, cos, sin, q_pos_offset, k_pos_offset,
                         rot_dim, layout, causal, softmax_scale, workspace)
    fn = _lib.load().rope_flash_attn_bwd

    def launch():
        status = fn(*args)
        if status != _lib.OK:
            raise RopeError(status, "rope_flash_attn_bwd")
    launch.workspace = ws   # kept alive as long as the callable (see prepare_flash_attn_fwd)
    return launch
