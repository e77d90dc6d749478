"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and turns every invalid argument into its status code before any
HIP call (so these run without a GPU; no compute call is made)."""
import re
from pathlib import Path

import pytest

from rotary_position_embedding_rope_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "rope_mi355x.h"



def slot(i, off=0):
    """A fake device address, never dereferenced: slots are 4 TiB apart, so
    the tensors of one call never overlap unless a test places them so."""
    return (i << 42) + off


FAKE, FAKE2 = slot(1), slot(2)
MISALIGNED = slot(1, 2)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = HEADER.read_text()
    body = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rope_[a-z_0-9]+)\s*\(", body)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_codes_match_header():
    text = HEADER.read_text()
    codes = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"#define (ROPE_\w+) (\d+)", text))
    assert codes["ROPE_OK"] == _lib.OK and codes["ROPE_ERR_NULL"] == _lib.ERR_NULL
    assert codes["ROPE_ERR_SHAPE"] == _lib.ERR_SHAPE and codes["ROPE_ERR_BASE"] == _lib.ERR_BASE
    assert codes["ROPE_ERR_UNSUPPORTED"] == _lib.ERR_UNSUPPORTED
    assert codes["ROPE_ERR_EMPTY_ROW"] == _lib.ERR_EMPTY_ROW
    assert codes["ROPE_ERR_TABLE_RANGE"] == _lib.ERR_TABLE_RANGE
    assert codes["ROPE_ERR_HIP"] == _lib.ERR_HIP and codes["ROPE_ERR_ALIGN"] == _lib.ERR_ALIGN
    assert codes["ROPE_ERR_SCRATCH"] == _lib.ERR_SCRATCH
    assert codes["ROPE_NEOX"] == _lib.NEOX and codes["ROPE_GPTJ"] == _lib.GPTJ
    assert codes["ROPE_BF16"] == _lib.BF16 and codes["ROPE_F32"] == _lib.F32
    assert codes["ROPE_F16"] == _lib.F16


def test_status_strings(lib):
    for s in range(10):
        assert _lib.status_str(s)
    assert _lib.status_str(99) == "unknown status"


# --------------------------------------------------------------------------
# rope_tables_build


@pytest.mark.parametrize("base,rot,maxpos,c,s,want", [
    (0.0, 64, 10, FAKE, FAKE2, _lib.ERR_BASE),
    (-1.0, 64, 10, FAKE, FAKE2, _lib.ERR_BASE),
    (float("inf"), 64, 10, FAKE, FAKE2, _lib.ERR_BASE),
    (float("nan"), 64, 10, FAKE, FAKE2, _lib.ERR_BASE),
    (1e4, 63, 10, FAKE, FAKE2, _lib.ERR_SHAPE),
    (1e4, 0, 10, FAKE, FAKE2, _lib.ERR_SHAPE),
    (1e4, 2048, 10, FAKE, FAKE2, _lib.ERR_SHAPE),
    (1e4, 64, 0, FAKE, FAKE2, _lib.ERR_SHAPE),
    (1e4, 64, 1 << 40, FAKE, FAKE2, _lib.ERR_SHAPE),
    (1e4, 64, 10, None, FAKE2, _lib.ERR_NULL),
    (1e4, 64, 10, FAKE, None, _lib.ERR_NULL),
    (1e4, 64, 10, MISALIGNED, FAKE2, _lib.ERR_ALIGN),
])
def test_tables_build_rejects(lib, base, rot, maxpos, c, s, want):
    assert lib.rope_tables_build(base, rot, maxpos, c, s, None) == want
    # the scaled build validates the same way (divisor 1 is the plain table)
    assert lib.rope_tables_build_scaled(base, rot, maxpos, 1.0, c, s, None) == want


@pytest.mark.parametrize("div", [0.0, -2.0, float("inf"), float("nan")])
def test_tables_build_scaled_rejects_divisor(lib, div):
    assert lib.rope_tables_build_scaled(1e4, 64, 10, div, FAKE, FAKE2, None) == _lib.ERR_BASE


# --------------------------------------------------------------------------
# rope_apply


def apply_args(**over):
    a = dict(q=slot(1), qst=40 * 128, qsh=128, hq=32, k=slot(2), kst=8 * 128, ksh=128, hkv=8,
             pos=slot(3), n=8192, cos=slot(4), sin=slot(5), rows=32768, D=128, rot=64,
             layout=_lib.NEOX, dtype=_lib.BF16)
    a.update(over)
    return [a["q"], a["qst"], a["qsh"], a["hq"], a["k"], a["kst"], a["ksh"], a["hkv"], a["pos"],
            a["n"], a["cos"], a["sin"], a["rows"], a["D"], a["rot"], a["layout"], a["dtype"], None]


@pytest.mark.parametrize("over,want", [
    (dict(D=127), _lib.ERR_SHAPE),
    (dict(D=0), _lib.ERR_SHAPE),
    (dict(D=2048, rot=64), _lib.ERR_SHAPE),
    (dict(rot=130), _lib.ERR_SHAPE),
    (dict(rot=63), _lib.ERR_SHAPE),
    (dict(rot=0), _lib.ERR_SHAPE),
    (dict(n=-1), _lib.ERR_SHAPE),
    (dict(hq=-1), _lib.ERR_SHAPE),
    (dict(qsh=64), _lib.ERR_SHAPE),            # head rows overlap
    (dict(qst=31 * 128), _lib.ERR_SHAPE),      # token rows overlap
    (dict(layout=2), _lib.ERR_UNSUPPORTED),
    (dict(dtype=5), _lib.ERR_UNSUPPORTED),
    (dict(dtype=_lib.F16, q=None), _lib.ERR_NULL),   # fp16 is accepted: validation goes on
    (dict(dtype=_lib.F16, q=slot(1, 1)), _lib.ERR_ALIGN),
    (dict(q=None), _lib.ERR_NULL),
    (dict(k=None), _lib.ERR_NULL),
    (dict(pos=None), _lib.ERR_NULL),
    (dict(cos=None), _lib.ERR_NULL),
    (dict(rows=0), _lib.ERR_TABLE_RANGE),
    (dict(q=slot(1, 1)), _lib.ERR_ALIGN),
    (dict(pos=slot(3, 2)), _lib.ERR_ALIGN),
    (dict(cos=slot(4, 2)), _lib.ERR_ALIGN),
    # 2^31 - 1 tokens x 40 heads: the grid would pass 2^32 - 1 work-items
    (dict(n=2147483647), _lib.ERR_SHAPE),
])
def test_rope_apply_rejects(lib, over, want):
    assert lib.rope_apply(*apply_args(**over)) == want


@pytest.mark.parametrize("over", [dict(n=0), dict(hq=0, hkv=0, q=None, k=None)])
def test_rope_apply_noop_needs_no_device(lib, over):
    # an empty batch is a no-op: OK without any HIP call
    assert lib.rope_apply(*apply_args(**over)) == _lib.OK


# --------------------------------------------------------------------------
# rope_flash_attn_fwd


def fwd_args(**over):
    a = dict(q=slot(1), k=slot(2), v=slot(3), o=slot(4), lse=None, B=1, H=8, Hkv=None, Sq=4096, Sk=4096,
             D=64, qo=0, ko=0, cos=slot(5), sin=slot(6), rows=4096, rot=64, layout=_lib.NEOX,
             causal=1, scale=0.0, dtype=_lib.BF16, ws=None, wsb=0)
    a.update(over)
    hkv = a["H"] if a["Hkv"] is None else a["Hkv"]
    return [a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], hkv, a["Sq"], a["Sk"], a["D"], a["qo"],
            a["ko"], a["cos"], a["sin"], a["rows"], a["rot"], a["layout"], a["causal"], a["scale"],
            a["dtype"], a["ws"], a["wsb"], None]


@pytest.mark.parametrize("over,want", [
    (dict(B=0), _lib.ERR_SHAPE),
    (dict(H=-1), _lib.ERR_SHAPE),
    (dict(Sq=0), _lib.ERR_SHAPE),
    (dict(Sk=0), _lib.ERR_SHAPE),
    (dict(Hkv=0), _lib.ERR_SHAPE),
    (dict(Hkv=3), _lib.ERR_SHAPE),               # 3 does not divide 8
    (dict(Hkv=16), _lib.ERR_SHAPE),
    (dict(D=63), _lib.ERR_SHAPE),
    (dict(rot=66), _lib.ERR_SHAPE),
    (dict(rot=-2), _lib.ERR_SHAPE),
    (dict(qo=-1), _lib.ERR_SHAPE),
    (dict(scale=float("nan")), _lib.ERR_SHAPE),
    (dict(scale=float("inf")), _lib.ERR_SHAPE),
    (dict(o=slot(1)), _lib.ERR_SHAPE),             # o aliases q
    (dict(o=slot(1, 0x1000)), _lib.ERR_SHAPE),     # o overlaps q at an offset
    (dict(o=slot(3, -16)), _lib.ERR_SHAPE),        # o's last bytes overlap v
    (dict(lse=slot(4)), _lib.ERR_SHAPE),           # lse aliases o
    (dict(lse=slot(4, 0x3ffffc)), _lib.ERR_SHAPE), # lse starts inside o (4 MiB)
    (dict(lse=slot(7, 2)), _lib.ERR_ALIGN),
    (dict(D=192, rot=192), _lib.ERR_UNSUPPORTED),   # D/2 = 96 is not a power of two
    (dict(D=96, rot=96), _lib.ERR_UNSUPPORTED),
    (dict(rot=48), _lib.ERR_UNSUPPORTED),
    (dict(dtype=3), _lib.ERR_UNSUPPORTED),
    (dict(dtype=_lib.F16, q=None), _lib.ERR_NULL),  # fp16 accepted: validation goes on
    (dict(layout=7), _lib.ERR_UNSUPPORTED),
    (dict(q=None), _lib.ERR_NULL),
    (dict(v=None), _lib.ERR_NULL),
    (dict(cos=None), _lib.ERR_NULL),
    (dict(qo=0, ko=1, rows=8192), _lib.ERR_EMPTY_ROW),
    (dict(rows=4095), _lib.ERR_TABLE_RANGE),
    (dict(qo=14336, Sq=2048, Sk=16384, rows=16383), _lib.ERR_TABLE_RANGE),
    (dict(cos=slot(5, 4)), _lib.ERR_ALIGN),
    (dict(k=slot(2, 8)), _lib.ERR_ALIGN),
    (dict(ws=None, wsb=1024), _lib.ERR_SHAPE),        # bytes without a buffer
    (dict(ws=slot(8), wsb=-1), _lib.ERR_SHAPE),
    (dict(ws=slot(8, 4), wsb=4096), _lib.ERR_ALIGN),
    (dict(ws=slot(4, 0x100), wsb=4096), _lib.ERR_SHAPE),   # workspace inside o
    (dict(ws=slot(2, 0x100), wsb=4096), _lib.ERR_SHAPE),   # workspace inside k
    # 16 M workgroups of 512 threads: past the 2^32 - 1 work-items of one launch
    (dict(B=2048, H=1024, Sq=1024, Sk=1024), _lib.ERR_SHAPE),
])
def test_flash_rejects(lib, over, want):
    assert lib.rope_flash_attn_fwd(*fwd_args(**over)) == want


def test_flash_without_rotation_needs_no_table(lib):
    # rot_dim = 0: tables may be NULL; a bad shape is still reported first
    assert lib.rope_flash_attn_fwd(*fwd_args(rot=0, cos=None, sin=None, rows=0, B=0)) == _lib.ERR_SHAPE
    # non-causal with q_off < k_off is legal (every key is visible); shape error first
    assert lib.rope_flash_attn_fwd(*fwd_args(causal=0, qo=0, ko=5, rows=8192, H=0)) == _lib.ERR_SHAPE


@pytest.mark.parametrize("args,want", [
    ((0, 8, 4096, 4096, 64, 0, 0, 1, _lib.BF16), _lib.ERR_SHAPE),
    ((1, 8, 4096, 4096, 63, 0, 0, 1, _lib.BF16), _lib.ERR_SHAPE),
    ((1, 8, 4096, 4096, 96, 0, 0, 1, _lib.BF16), _lib.ERR_UNSUPPORTED),
    ((1, 8, 4096, 4096, 64, 0, 0, 1, 7), _lib.ERR_UNSUPPORTED),
    ((1, 8, 4096, 4096, 64, 0, 3, 1, _lib.BF16), _lib.ERR_EMPTY_ROW),
    ((1, 8, 4096, 4096, 64, -1, 0, 1, _lib.BF16), _lib.ERR_SHAPE),
])
def test_workspace_size_rejects(lib, args, want):
    """Invalid shapes come back as minus the status code, before any HIP call."""
    assert lib.rope_flash_attn_workspace_size(*args) == -want


def test_workspace_size_fp32_needs_none(lib):
    # the fp32 kernel has no balanced schedule: no device query, zero bytes
    assert lib.rope_flash_attn_workspace_size(1, 2, 128, 128, 64, 0, 0, 1, _lib.F32) == 0


def decode_args(**over):
    a = dict(q=slot(1), kn=slot(2), vn=slot(3), kc=slot(4), vc=slot(5), lens=slot(6),
             o=slot(7), B=16, H=32, Hkv=8, S=32768, D=128, cos=slot(8), sin=slot(9), rows=32768,
             rot=128, layout=_lib.NEOX, scale=0.0, dtype=_lib.BF16, ws=slot(10), wsb=1 << 30)
    a.update(over)
    return [a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["lens"], a["o"], a["B"], a["H"],
            a["Hkv"], a["S"], a["D"], a["cos"], a["sin"], a["rows"], a["rot"], a["layout"],
            a["scale"], a["dtype"], a["ws"], a["wsb"], None]


@pytest.mark.parametrize("over,want", [
    (dict(B=0), _lib.ERR_SHAPE),
    (dict(Hkv=0), _lib.ERR_SHAPE),
    (dict(Hkv=5), _lib.ERR_SHAPE),                 # 5 does not divide 32
    (dict(S=0), _lib.ERR_SHAPE),
    (dict(D=63), _lib.ERR_SHAPE),
    (dict(rot=130), _lib.ERR_SHAPE),
    (dict(rot=-2), _lib.ERR_SHAPE),
    (dict(scale=float("nan")), _lib.ERR_SHAPE),
    (dict(wsb=1024), _lib.ERR_SHAPE),              # workspace too small
    (dict(wsb=2397183), _lib.ERR_SHAPE),           # one byte short
    (dict(B=1 << 20, S=1 << 24, wsb=1 << 62), _lib.ERR_SHAPE),   # pass counts past 32 bits
    (dict(o=slot(1)), _lib.ERR_SHAPE),             # o aliases q
    (dict(o=slot(4, 1 << 20)), _lib.ERR_SHAPE),    # o inside the key cache
    (dict(vc=slot(4, 1 << 29)), _lib.ERR_SHAPE),   # the caches overlap
    (dict(ws=slot(5, 64)), _lib.ERR_SHAPE),        # workspace inside the value cache
    (dict(D=96, rot=96), _lib.ERR_UNSUPPORTED),
    (dict(Hkv=2), _lib.ERR_UNSUPPORTED),           # 16 query heads per key/value head
    (dict(dtype=_lib.F32), _lib.ERR_UNSUPPORTED),
    (dict(dtype=_lib.F16, q=None), _lib.ERR_NULL),    # fp16 accepted
    (dict(layout=7), _lib.ERR_UNSUPPORTED),
    (dict(q=None), _lib.ERR_NULL),
    (dict(lens=None), _lib.ERR_NULL),
    (dict(ws=None), _lib.ERR_NULL),
    (dict(cos=None), _lib.ERR_NULL),
    (dict(rows=0), _lib.ERR_TABLE_RANGE),
    (dict(kc=slot(4, 8)), _lib.ERR_ALIGN),
    (dict(lens=slot(6, 2)), _lib.ERR_ALIGN),
    (dict(ws=slot(10, 4)), _lib.ERR_ALIGN),
])
def test_decode_rejects(lib, over, want):
    assert lib.rope_decode_attn_fwd(*decode_args(**over)) == want


def test_decode_workspace_size(lib):
    # partial states (m, l, D floats) for each of G query heads in B * Hkv + 1024
    # slots, rounded up to 256 bytes, then one (workgroup, count) pair per slice
    def want(B, H, Hkv, D):
        n = (B * Hkv + 1024) * (H // Hkv) * (D + 2) * 4
        return (n + 255) // 256 * 256 + B * Hkv * 8
    assert lib.rope_decode_workspace_size(16, 32, 8, 32768, 128) == want(16, 32, 8, 128) == 2397184
    assert lib.rope_decode_workspace_size(1, 1, 1, 1, 64) == want(1, 1, 1, 64)
    # the size does not depend on the cache length
    assert lib.rope_decode_workspace_size(16, 32, 8, 1, 128) == want(16, 32, 8, 128)
    assert lib.rope_decode_workspace_size(1, 6, 4, 100, 128) == -_lib.ERR_SHAPE
    assert lib.rope_decode_workspace_size(1, 32, 2, 100, 128) == -_lib.ERR_UNSUPPORTED
    # no rotation: tables may be NULL (a bad shape is still reported)
    assert lib.rope_decode_attn_fwd(*decode_args(rot=0, cos=None, sin=None, rows=0, B=0)) == _lib.ERR_SHAPE


def test_decode_scratch_size_matches_header():
    text = HEADER.read_text()
    m = re.search(r"#define ROPE_DECODE_SCRATCH_BYTES \((\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DECODE_SCRATCH_BYTES


def noalloc_args(**over):
    a = decode_args(**over)
    return a[:19] + [a[21]]   # no workspace pointer or size


@pytest.mark.parametrize("over,want", [
    (dict(B=0), _lib.ERR_SHAPE),
    (dict(Hkv=2), _lib.ERR_UNSUPPORTED),
    (dict(D=96, rot=96), _lib.ERR_UNSUPPORTED),
    # scratch need past ROPE_DECODE_SCRATCH_BYTES: rejected before any HIP call
    (dict(B=2998, Hkv=1, H=4), _lib.ERR_SCRATCH),    # one (request, kv head) too many
    (dict(B=991, Hkv=1, H=8), _lib.ERR_SCRATCH),
    (dict(B=512, Hkv=8, H=32), _lib.ERR_SCRATCH),    # 4096 (request, kv head) pairs
    # fits: the host-side argument checks still run before the scratch lookup
    (dict(B=2997, Hkv=1, H=4, q=None), _lib.ERR_NULL),
    (dict(B=990, Hkv=1, H=8, q=None), _lib.ERR_NULL),
    (dict(rot=130), _lib.ERR_SHAPE),
    (dict(cos=None), _lib.ERR_NULL),
    (dict(rows=0), _lib.ERR_TABLE_RANGE),
    (dict(kc=slot(4, 8)), _lib.ERR_ALIGN),
])
def test_decode_noalloc_rejects_before_any_device_call(lib, over, want):
    # shape, scratch size, pointer, table and alignment rejections come before
    # the scratch lookup (the overlap check, which needs the scratch address,
    # comes after it)
    assert lib.rope_decode_attn_fwd_noalloc(*noalloc_args(**over)) == want


def test_decode_noalloc_limit_matches_workspace_size(lib):
    # the entry point accepts exactly the shapes whose workspace fits
    for G, D, n_fit in [(4, 128, 2997), (8, 128, 990), (4, 64, 6867)]:
        assert lib.rope_decode_workspace_size(n_fit, G, 1, 100, D) <= _lib.DECODE_SCRATCH_BYTES
        assert lib.rope_decode_workspace_size(n_fit + 1, G, 1, 100, D) > _lib.DECODE_SCRATCH_BYTES
        args = noalloc_args(B=n_fit + 1, H=G, Hkv=1, D=D, rot=D)
        assert lib.rope_decode_attn_fwd_noalloc(*args) == _lib.ERR_SCRATCH


# --------------------------------------------------------------------------
# rope_flash_attn_bwd


def bwd_args(**over):
    a = dict(q=slot(1), k=slot(2), v=slot(3), o=slot(4), do=slot(5), lse=slot(6), dq=slot(7),
             dk=slot(8), dv=slot(9), B=1, H=8, Hkv=8, Sq=4096, Sk=4096, D=64, qo=0, ko=0,
             cos=slot(10), sin=slot(11), rows=4096,
             rot=64, layout=_lib.NEOX, causal=1, scale=0.0, dtype=_lib.BF16,
             ws=slot(12), wsb=1 << 24)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "B", "H", "Hkv", "Sq",
                           "Sk", "D", "qo", "ko", "cos", "sin", "rows", "rot", "layout", "causal",
                           "scale", "dtype", "ws", "wsb")] + [None]


@pytest.mark.parametrize("over,want", [
    (dict(B=0), _lib.ERR_SHAPE),
    (dict(Hkv=3), _lib.ERR_SHAPE),
    (dict(Sk=0), _lib.ERR_SHAPE),
    (dict(D=63), _lib.ERR_SHAPE),
    (dict(rot=66), _lib.ERR_SHAPE),
    (dict(qo=-1), _lib.ERR_SHAPE),
    (dict(scale=float("nan")), _lib.ERR_SHAPE),
    (dict(dq=slot(1)), _lib.ERR_SHAPE),           # dq aliases q
    (dict(dq=slot(1, 0x100000)), _lib.ERR_SHAPE), # dq overlaps q at an offset
    (dict(dk=slot(6)), _lib.ERR_SHAPE),           # dk aliases lse
    (dict(dv=slot(7)), _lib.ERR_SHAPE),           # dv aliases dq
    (dict(dv=slot(8, 0x200)), _lib.ERR_SHAPE),    # dv overlaps dk
    (dict(ws=slot(9, 0x3fff00)), _lib.ERR_SHAPE), # workspace overlaps dv's end
    (dict(wsb=1024), _lib.ERR_SHAPE),             # workspace too small (4096 rows x 8 heads x 4 B)
    (dict(dtype=_lib.F32), _lib.ERR_UNSUPPORTED),
    (dict(dtype=_lib.F16, lse=None), _lib.ERR_NULL),  # fp16 accepted
    (dict(D=96, rot=96), _lib.ERR_UNSUPPORTED),
    (dict(rot=48), _lib.ERR_UNSUPPORTED),
    (dict(layout=3), _lib.ERR_UNSUPPORTED),
    (dict(lse=None), _lib.ERR_NULL),
    (dict(do=None), _lib.ERR_NULL),
    (dict(dv=None), _lib.ERR_NULL),
    (dict(ws=None), _lib.ERR_NULL),
    (dict(cos=None), _lib.ERR_NULL),
    (dict(qo=0, ko=1, rows=8192), _lib.ERR_EMPTY_ROW),
    (dict(rows=4095), _lib.ERR_TABLE_RANGE),
    (dict(lse=slot(6, 2)), _lib.ERR_ALIGN),
    (dict(dk=slot(8, 8)), _lib.ERR_ALIGN),
    (dict(ws=slot(12, 4)), _lib.ERR_ALIGN),
])
def test_bwd_rejects(lib, over, want):
    assert lib.rope_flash_attn_bwd(*bwd_args(**over)) == want


def test_bwd_workspace_size(lib):
    f = lib.rope_flash_attn_bwd_workspace_size
    # row sums only without rotation
    assert f(1, 8, 8, 4096, 4096, 64, 0, _lib.BF16) == 8 * 4096 * 4
    assert f(2, 3, 3, 5, 5, 128, 0, _lib.BF16) == 256
    # with rotation: the rotated q and k copies too, each from a 256-byte boundary
    assert f(1, 8, 8, 4096, 4096, 64, 64, _lib.BF16) == 8 * 4096 * 4 + 2 * 8 * 4096 * 64 * 2
    assert f(2, 4, 2, 5, 7, 128, 32, _lib.F16) == 256 + 2 * 4 * 5 * 128 * 2 + 2 * 2 * 7 * 128 * 2
    assert f(1, 2, 1, 3, 3, 64, 64, _lib.BF16) == 256 + 768 + 512
    assert f(1, 8, 8, 0, 16, 64, 0, _lib.BF16) == -_lib.ERR_SHAPE
    assert f(1, 8, 3, 16, 16, 64, 0, _lib.BF16) == -_lib.ERR_SHAPE     # H_kv must divide H
    assert f(1, 8, 8, 16, 16, 64, 66, _lib.BF16) == -_lib.ERR_SHAPE    # rot_dim past head_dim
    assert f(1, 8, 8, 16, 16, 64, 0, _lib.F32) == -_lib.ERR_UNSUPPORTED
    # one byte less than the size the library asks for is rejected, with and
    # without the rotated copies (a call with the full size would reach the
    # device, so it is not made here)
    for rot in (64, 0):
        need = f(1, 8, 8, 4096, 4096, 64, rot, _lib.BF16)
        assert need == 8 * 4096 * 4 + (2 * 8 * 4096 * 64 * 2 if rot else 0)
        assert lib.rope_flash_attn_bwd(*bwd_args(rot=rot, wsb=need - 1)) == _lib.ERR_SHAPE
