"""MI355X (gfx950) RoPE: a fused RoPE + causal FlashAttention-style forward
and a standalone ragged RoPE op, behind the C ABI of ``include/rope_mi355x.h``.

The HIP library is loaded on first use of an entry point; importing the
package (for example for ``workloads``) does not touch the GPU.
"""
__all__ = ["tables_build", "rope_apply", "flash_attn_fwd", "workloads"]


def __getattr__(name):
    if name in ("tables_build", "rope_apply", "flash_attn_fwd", "RopeError"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
