"""Seeded synthetic inputs for the fused attention and the standalone RoPE op.

This module holds none of the method's arithmetic: it only draws random
numbers, rounds them to the storage type and describes the workload shapes.
Both the GPU path (through the tests and the benchmark) and the fp64 oracle
consume what it produces.

Recipe (the pages fix shapes but neither a generator nor seeds):
  * ``numpy.random.default_rng(seed)`` (PCG64), drawing ``standard_normal`` in
    fp64 in the order q, k, v at full shape, as the worked tests of "RoPE and
    FlashAttention: relative positions and online softmax" (section 5) do with
    ``default_rng``.
  * Values are rounded fp64 -> fp32 (round to nearest even), then fp32 -> bf16
    (round to nearest even) for bf16 workloads.
  * The ragged continuous-batching workload ("Write Triton Rope Kernel",
    "Inputs the agent should gather first", item 6) draws, in this order:
    request lengths from distinct cut points, per-token positions iid uniform
    over the table, then Q, then K.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# storage-type rounding (round to nearest even), no method arithmetic


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of ``x`` rounded fp32 -> bf16 to nearest even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact fp32 values of uint16 bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to(x, dtype: str) -> np.ndarray:
    """fp32 array holding ``x`` rounded to ``dtype`` ('f32', 'bf16' or 'f16'),
    nearest even."""
    f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(f)
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(f))
    if dtype == "f16":
        return np.ascontiguousarray(f.astype(np.float16).astype(np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# workload descriptions


@dataclass(frozen=True)
class AttentionWorkload:
    """One fused RoPE + attention forward: q [B,H,Sq,D], k/v [B,H_kv,Sk,D]
    (H_kv None: H; otherwise it divides H)."""

    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    dtype: str            # 'f32' or 'bf16'
    seed: int
    layout: str           # 'neox' or 'gptj'
    base: float = 10000.0
    rot_dim: int | None = None
    q_off: int = 0
    k_off: int = 0
    causal: bool = True
    H_kv: int | None = None

    @property
    def Hkv(self) -> int:
        return self.H if self.H_kv is None else self.H_kv

    @property
    def rot(self) -> int:
        return self.D if self.rot_dim is None else self.rot_dim

    @property
    def table_rows(self) -> int:
        return max(self.q_off + self.Sq, self.k_off + self.Sk)

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask allows, over all heads."""
        if not self.causal:
            return self.B * self.H * self.Sq * self.Sk
        i = np.arange(self.Sq, dtype=np.int64)
        n = np.clip(self.q_off + i - self.k_off + 1, 0, self.Sk)
        return int(self.B * self.H * n.sum())

    def flops(self) -> int:
        """Algorithmic flops: 4*D per visible pair (QK^T and PV, 2 each)."""
        return 4 * self.D * self.visible_pairs()

    def bwd_flops(self) -> int:
        """Algorithmic flops of the backward: 10*D per visible pair (the
        scores rebuilt, dP = dO V^T, dV, dK and dQ, 2*D each)."""
        return 10 * self.D * self.visible_pairs()

    def label(self) -> str:
        kv = "" if self.Hkv == self.H else f"({self.Hkv}kv)"
        return f"{self.B}x{self.H}{kv}x{self.Sq}x{self.Sk}x{self.D}"


@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step over a key/value cache: B requests, one new token
    each at position lens[b] (keys already cached); q [B,H,D], new k/v
    [B,H_kv,D], caches [B,H_kv,S_max,D] bf16."""

    name: str
    B: int
    H: int
    H_kv: int
    D: int
    S_max: int
    seed: int
    layout: str = "neox"
    base: float = 10000.0
    rot_dim: int | None = None
    min_len: int = 0              # cached lengths drawn uniformly from [min_len, S_max - 1]

    @property
    def rot(self) -> int:
        return self.D if self.rot_dim is None else self.rot_dim

    def lens(self) -> np.ndarray:
        rng = np.random.default_rng(self.seed)
        return rng.integers(self.min_len, self.S_max, size=self.B).astype(np.int32)

    def algorithmic_bytes(self) -> int:
        """Bytes one step must move: the cached K and V rows read once, the new
        q, k, v read, the new K and V rows written, the output written (bf16)."""
        cached = int(self.lens().astype(np.int64).sum())
        return 2 * (2 * cached * self.H_kv * self.D + self.B * (self.H + 2 * self.H_kv) * self.D
                    + 2 * self.B * self.H_kv * self.D + self.B * self.H * self.D)


@dataclass(frozen=True)
class RopeApplyWorkload:
    """Standalone in-place RoPE over a ragged continuous batch."""

    name: str
    n_tokens: int
    n_requests: int
    table_rows: int
    H_q: int
    H_kv: int
    D: int
    rot_dim: int
    layout: str
    dtype: str
    seed: int
    base: float = 10000.0
    positions: str = "uniform"   # 'uniform' (iid over the table) or 'contiguous'
    start_positions: tuple = field(default=())

    def algorithmic_bytes(self) -> int:
        """Bytes the op must move: rotated span read+written for every head,
        one cos and one sin row per token, one int32 position per token."""
        elt = 4 if self.dtype == "f32" else 2
        per_tok = 2 * (self.H_q + self.H_kv) * self.rot_dim * elt + 2 * (self.rot_dim // 2) * 4 + 4
        return self.n_tokens * per_tok


# The parity / benchmark workloads.
TINY_F32 = AttentionWorkload("causal_gptj_f32_1x2x128x64", 1, 2, 128, 128, 64, "f32", 0, "gptj")
SMALL_BF16 = AttentionWorkload("causal_gptj_bf16_1x8x512x64", 1, 8, 512, 512, 64, "bf16", 1, "gptj")
SWEEP_BF16 = tuple(
    AttentionWorkload(f"causal_neox_bf16_{b}x8x{s}x64", b, 8, s, s, 64, "bf16", seed, "neox")
    for (b, s), seed in zip(((1, 1024), (1, 2048), (1, 4096), (2, 1024), (4, 1024)), range(2, 7))
)
HEADLINE = SWEEP_BF16[2]   # 1x8x4096x64 bf16 NeoX causal
# the same shape with fp16 storage
HEADLINE_F16 = AttentionWorkload("causal_neox_f16_1x8x4096x64", 1, 8, 4096, 4096, 64, "f16", 4, "neox")
PREFILL_OFFSET = AttentionWorkload("chunked_prefill_neox_bf16_1x32x2048q_16384k_128", 1, 32, 2048,
                                   16384, 128, "bf16", 7, "neox", base=500000.0,
                                   q_off=14336, k_off=0)
RAGGED_ROPE = RopeApplyWorkload("ragged_rope_neox_bf16_8192tok_32q8kv_rot64of128", 8192, 16,
                                32768, 32, 8, 128, 64, "neox", "bf16", 8)
# the same batch with fp16 storage
RAGGED_ROPE_F16 = RopeApplyWorkload("ragged_rope_neox_f16_8192tok_32q8kv_rot64of128", 8192, 16,
                                    32768, 32, 8, 128, 64, "neox", "f16", 11)

# the chunked prefill with 8 key/value heads for the 32 query heads (the
# head counts of the ragged RoPE workload): grouped-query attention
PREFILL_GQA = AttentionWorkload("chunked_prefill_gqa_neox_bf16_1x32q8kv_2048q_16384k_128", 1, 32,
                                2048, 16384, 128, "bf16", 9, "neox", base=500000.0,
                                q_off=14336, k_off=0, H_kv=8)

ATTENTION_WORKLOADS = (TINY_F32, SMALL_BF16) + SWEEP_BF16 + (PREFILL_OFFSET, PREFILL_GQA)

# a decode step of a continuous batch: 16 requests with cached lengths
# uniform in [1024, 32767], the head counts and dims of the ragged RoPE
# workload
DECODE = DecodeWorkload("decode_gqa_neox_bf16_16req_32q8kv_128_ctx1k-32k", 16, 32, 8, 128, 32768, 10,
                        base=500000.0, min_len=1024)


# ---------------------------------------------------------------------------
# generators


def attention_inputs(w: AttentionWorkload):
    """(q, k, v) as fp32 arrays holding values exact in ``w.dtype``."""
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.H, w.Sq, w.D))
    k = rng.standard_normal((w.B, w.Hkv, w.Sk, w.D))
    v = rng.standard_normal((w.B, w.Hkv, w.Sk, w.D))
    return tuple(round_to(a.astype(np.float32), w.dtype) for a in (q, k, v))


def ragged_lengths(rng: np.random.Generator, total: int, n_requests: int) -> np.ndarray:
    """``n_requests`` positive lengths summing to ``total`` from distinct cut points."""
    if n_requests < 1 or n_requests > total:
        raise ValueError("need 1 <= n_requests <= total")
    cuts = np.sort(rng.choice(np.arange(1, total), size=n_requests - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total]])
    return np.diff(edges).astype(np.int64)


def rope_apply_inputs(w: RopeApplyWorkload):
    """dict with 'lengths', 'positions' (int32), 'q' [T,H_q,D], 'k' [T,H_kv,D]
    (fp32 arrays exact in ``w.dtype``)."""
    rng = np.random.default_rng(w.seed)
    lengths = ragged_lengths(rng, w.n_tokens, w.n_requests)
    if w.positions == "uniform":
        positions = rng.integers(0, w.table_rows, size=w.n_tokens)
    elif w.positions == "contiguous":
        starts = list(w.start_positions) or [0] * w.n_requests
        positions = np.concatenate([s + np.arange(n) for s, n in zip(starts, lengths)])
    else:
        raise ValueError(w.positions)
    q = rng.standard_normal((w.n_tokens, w.H_q, w.D)).astype(np.float32)
    k = rng.standard_normal((w.n_tokens, w.H_kv, w.D)).astype(np.float32)
    return {
        "lengths": lengths,
        "positions": positions.astype(np.int32),
        "q": round_to(q, w.dtype),
        "k": round_to(k, w.dtype),
    }


def decode_inputs(w: DecodeWorkload, with_cache: bool = True):
    """dict with 'lens' (int32 [B]), 'q' [B,H,D], 'k_new', 'v_new' [B,H_kv,D]
    and (with_cache) 'k_raw', 'v_cache' [B,H_kv,S_max,D]: the unrotated keys
    and the values of the cached positions (fp32 arrays exact in bf16)."""
    rng = np.random.default_rng(w.seed + 1)
    d = {"lens": w.lens()}
    for name, shape in (("q", (w.B, w.H, w.D)), ("k_new", (w.B, w.H_kv, w.D)),
                        ("v_new", (w.B, w.H_kv, w.D))):
        d[name] = round_to(rng.standard_normal(shape).astype(np.float32), "bf16")
    if with_cache:
        shape = (w.B, w.H_kv, w.S_max, w.D)
        d["k_raw"] = round_to(rng.standard_normal(shape).astype(np.float32), "bf16")
        d["v_cache"] = round_to(rng.standard_normal(shape).astype(np.float32), "bf16")
    return d
