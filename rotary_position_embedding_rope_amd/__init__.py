"""MI355X (gfx950) RoPE: a fused RoPE + causal FlashAttention-style forward
and its backward, a standalone ragged RoPE op and a decode step over a
key/value cache, behind the C ABI of ``include/rope_mi355x.h``.

The HIP library is loaded on first use of an entry point; importing the
package (for example for ``workloads``) does not touch the GPU.
"""
_API = ("tables_build", "rope_apply", "flash_attn_fwd", "flash_attn_bwd", "decode_attn_fwd",
        "decode_attn_fwd_noalloc",
        "prepare_flash_attn_fwd", "prepare_flash_attn_bwd", "prepare_decode_attn_fwd",
        "prepare_rope_apply", "RopeError")
__all__ = list(_API) + ["workloads"]


def __getattr__(name):
    if name in _API:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
