"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas retyped.

Each pin takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees.  ``tests/test_oracle_pins.py`` runs every pin on the real
oracle, and runs the whole set on copies of the oracle with a planted mistake
to show that each such mistake fails at least one pin.

Pages cited:
  [RF] "RoPE and FlashAttention: relative positions and online softmax"
  [TR] "Write Triton Rope Kernel"
"""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---------------------------------------------------------------------------
# independent constructions used as references


def rotation_matrix(head_dim: int, rot_dim: int, pos: float, base: float, layout: str) -> np.ndarray:
    """Explicit block rotation matrix R(pos): each pair's plane gets the
    textbook 2x2 rotation [[c, -s], [s, c]] by pos * base**(-2i/rot_dim).
    Built as a dense matrix and applied with a matmul, so it shares no
    per-pair indexing code with the oracle's loop."""
    R = np.eye(head_dim)
    half = rot_dim // 2
    for i in range(half):
        a, b = (2 * i, 2 * i + 1) if layout == "gptj" else (i, i + half)
        ang = pos * np.power(base, -2.0 * i / rot_dim)
        c, s = np.cos(ang), np.sin(ang)
        R[a, a], R[a, b], R[b, a], R[b, b] = c, -s, s, c
    return R


def rope_complex(x: np.ndarray, positions, base: float, rot_dim: int, layout: str) -> np.ndarray:
    """RoPE as complex multiplication: pair i is the complex number
    x_a + j x_b, multiplied by exp(j * pos * theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    half = rot_dim // 2
    if layout == "gptj":
        z = x[..., 0:rot_dim:2] + 1j * x[..., 1:rot_dim:2]
    else:
        z = x[..., :half] + 1j * x[..., half:rot_dim]
    theta = np.power(base, -2.0 * np.arange(half) / rot_dim)
    pos = np.asarray(positions, dtype=np.float64)[..., None]
    w = z * np.exp(1j * pos * theta)
    y = x.copy()
    if layout == "gptj":
        y[..., 0:rot_dim:2], y[..., 1:rot_dim:2] = w.real, w.imag
    else:
        y[..., :half], y[..., half:rot_dim] = w.real, w.imag
    return y


def dense_reference(qr, kr, v, allowed, scale):
    """softmax(scale * qr kr^T + mask) v with scipy's softmax."""
    from scipy.special import softmax
    s = np.where(allowed, scale * (qr @ kr.T), -np.inf)
    return softmax(s, axis=-1) @ v


def offset_mask(Sq: int, Sk: int, q_off: int, k_off: int) -> np.ndarray:
    return (k_off + np.arange(Sk))[None, :] <= (q_off + np.arange(Sq))[:, None]


# ---------------------------------------------------------------------------
# RoPE pins


def pin_worked_example(orc):
    """[RF] section 2, practice solution (tests/golden/worked_example.txt)."""
    rows = []
    for line in (GOLDEN / "worked_example.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            m, n, val, sym = line.split()
            rows.append((int(m), int(n), float(val), sym))
    x = np.array([[1.0, 0.0]])
    for layout in ("gptj", "neox"):
        for m, n, val, sym in rows:
            arg = float(sym[len("cos("):-1])
            assert abs(val - math.cos(arg)) < 1e-16, "fixture value disagrees with its own formula"
            q = orc.rope(x, [m], base=10000.0, layout=layout)
            k = orc.rope(x, [n], base=10000.0, layout=layout)
            score = float(q[0] @ k[0])
            assert abs(score - val) <= 1e-15, (layout, m, n, score, val)


def pin_relative_shift_p2(orc):
    """All-pairs relative-shift invariance with the shapes of [RF] section 2's
    test: q [2,3,7,8] at 4..10, k [2,3,9,8] at 2..10, shift 23, 1e-11."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((2, 3, 7, 8))
    k = rng.standard_normal((2, 3, 9, 8))
    qp, kp = np.arange(4, 11), np.arange(2, 11)
    for layout in ("gptj", "neox"):
        a = orc.rope(q, qp, layout=layout) @ np.swapaxes(orc.rope(k, kp, layout=layout), -1, -2)
        b = orc.rope(q, qp + 23, layout=layout) @ np.swapaxes(orc.rope(k, kp + 23, layout=layout), -1, -2)
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
        wrong = orc.rope(q, qp, layout=layout) @ np.swapaxes(orc.rope(k, kp + 1, layout=layout), -1, -2)
        assert not np.allclose(a, wrong), "shifting only k must change the scores"


def pin_relative_shift_long(orc):
    """Relative-shift invariance at the long-context settings: D=128, base
    500000, positions near 14336..16383, shift 10000.  Tolerance scales with
    the largest angle times fp64 epsilon times D."""
    rng = np.random.default_rng(5)
    D = 128
    q = rng.standard_normal((6, D))
    k = rng.standard_normal((9, D))
    qp, kp = 14336 + np.arange(6) * 300, np.arange(9) * 1800
    shift = 10000
    tol = (16384 + shift) * 2.0 ** -52 * D * 64
    for layout in ("gptj", "neox"):
        a = orc.rope(q, qp, base=5e5, layout=layout) @ orc.rope(k, kp, base=5e5, layout=layout).T
        b = orc.rope(q, qp + shift, base=5e5, layout=layout) @ orc.rope(k, kp + shift, base=5e5, layout=layout).T
        np.testing.assert_allclose(a, b, rtol=0, atol=tol)


def pin_norm_preserved(orc):
    """Rotations preserve norms ([RF] section 1)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 64))
    pos = rng.integers(0, 32768, size=5)
    for layout in ("gptj", "neox"):
        for rot in (64, 32):
            y = orc.rope(x, pos, rot_dim=rot, layout=layout)
            np.testing.assert_allclose((y ** 2).sum(-1), (x ** 2).sum(-1), rtol=1e-13)


def pin_chunked_equals_full(orc):
    """Rotating K in two chunks with their true positions equals rotating it
    whole, bit for bit; restarting the positions of the second chunk at 0
    must differ ([RF] section 2)."""
    rng = np.random.default_rng(43)
    k = rng.standard_normal((2, 3, 9, 8))
    kp = np.arange(2, 11)
    for layout in ("gptj", "neox"):
        full = orc.rope(k, kp, layout=layout)
        chunked = np.concatenate([orc.rope(k[..., :4, :], kp[:4], layout=layout),
                                  orc.rope(k[..., 4:, :], kp[4:], layout=layout)], axis=-2)
        assert np.array_equal(full, chunked)
        restarted = orc.rope(k[..., 4:, :], np.arange(5), layout=layout)
        assert not np.allclose(full[..., 4:, :], restarted)


def pin_position_zero_identity(orc):
    """cos 0 = 1 and sin 0 = 0 exactly: position 0 leaves a row unchanged."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128))
    for layout in ("gptj", "neox"):
        for rot in (128, 64):
            assert np.array_equal(orc.rope(x, 0, rot_dim=rot, layout=layout), x)


def pin_complex_multiplication(orc):
    """RoPE equals multiplying each pair, read as a complex number, by
    exp(i * pos * theta_i); checked for both pairings, partial and full
    rotation, and several bases."""
    rng = np.random.default_rng(17)
    for D, rot, base in ((8, 8, 10000.0), (64, 64, 10000.0), (128, 64, 10000.0),
                         (128, 128, 500000.0), (12, 4, 100.0)):
        x = rng.standard_normal((7, D))
        pos = rng.integers(0, 40000, size=7)
        for layout in ("gptj", "neox"):
            got = orc.rope(x, pos, base=base, rot_dim=rot, layout=layout)
            want = rope_complex(x, pos, base, rot, layout)
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


def pin_brute_force_matrices(orc):
    """On tiny rows (D <= 8) the oracle equals the explicit block rotation
    matrix R(pos) applied by matmul."""
    rng = np.random.default_rng(19)
    for D, rot in ((2, 2), (4, 4), (6, 4), (8, 8), (8, 2)):
        x = rng.standard_normal((5, D))
        pos = [0, 1, 7, 300, 12345]
        for layout in ("gptj", "neox"):
            got = orc.rope(x, pos, base=100.0, rot_dim=rot, layout=layout)
            want = np.stack([rotation_matrix(D, rot, p, 100.0, layout) @ x[r] for r, p in enumerate(pos)])
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_layout_permutation(orc):
    """GPT-J and NeoX are the same functions after permuting the rotated dims
    (slot 2i -> i, 2i+1 -> i + rot/2), bit for bit ([RF] section 2;
    [TR] "Common failure modes")."""
    rng = np.random.default_rng(23)
    for D, rot in ((64, 64), (128, 64)):
        x = rng.standard_normal((6, D))
        pos = rng.integers(0, 32768, size=6)
        half = rot // 2
        perm = np.arange(D)
        perm[:half] = np.arange(0, rot, 2)
        perm[half:rot] = np.arange(1, rot, 2)
        gptj = orc.rope(x, pos, rot_dim=rot, layout="gptj")
        neox = orc.rope(x[:, perm], pos, rot_dim=rot, layout="neox")
        assert np.array_equal(neox, gptj[:, perm])


def pin_partial_tail(orc):
    """Partial RoPE leaves dims >= rot_dim bit-identical, and its first rot_dim
    dims equal a full rotation of those dims alone: the frequency schedule
    depends on rot_dim only ([TR] "Correctness requirements")."""
    rng = np.random.default_rng(29)
    x = rng.standard_normal((8, 128))
    pos = rng.integers(0, 32768, size=8)
    for layout in ("gptj", "neox"):
        y = orc.rope(x, pos, rot_dim=64, layout=layout)
        assert np.array_equal(y[:, 64:], x[:, 64:])
        head = orc.rope(np.ascontiguousarray(x[:, :64]), pos, rot_dim=64, layout=layout)
        assert np.array_equal(y[:, :64], head)


def pin_trig_table(orc):
    """The exact table: row 0 is (1, 0); column 0 is (cos p, sin p) because the
    first frequency is 1 ([RF] section 3); everything matches numpy's trig of
    p * base**(-2i/rot_dim)."""
    for base, rot, n in ((10000.0, 64, 4096), (500000.0, 128, 512)):
        c, s = orc.trig(base, rot, n)
        assert np.array_equal(c[0], np.ones(rot // 2)) and np.array_equal(s[0], np.zeros(rot // 2))
        p = np.arange(n, dtype=np.float64)
        np.testing.assert_allclose(c[:, 0], np.cos(p), rtol=0, atol=1e-15)
        np.testing.assert_allclose(s[:, 0], np.sin(p), rtol=0, atol=1e-15)
        ang = p[:, None] * np.power(base, -2.0 * np.arange(rot // 2) / rot)[None, :]
        np.testing.assert_allclose(c, np.cos(ang), rtol=0, atol=1e-12)
        np.testing.assert_allclose(s, np.sin(ang), rtol=0, atol=1e-12)


def pin_token_permutation(orc):
    """Per-token positions: permuting the tokens (with their positions)
    commutes with the rotation ([TR] "Required reasoning process" step 3)."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((20, 3, 16))
    pos = rng.integers(0, 32768, size=20)
    perm = rng.permutation(20)
    for layout in ("gptj", "neox"):
        y = orc.rope(x, pos[:, None], rot_dim=8, layout=layout)
        yp = orc.rope(x[perm], pos[perm][:, None], rot_dim=8, layout=layout)
        assert np.array_equal(yp, y[perm])


# ---------------------------------------------------------------------------
# attention pins


def pin_attention_p2_example(orc):
    """[RF] section 5's example: Q [7,4], K [9,4], V [9,5] from default_rng(43),
    keys j <= 2 + i visible (query offset 2), scale 1/2, no rotation; equals
    scipy's dense softmax at 1e-12."""
    rng = np.random.default_rng(43)
    Q, K, V = rng.normal(size=(7, 4)), rng.normal(size=(9, 4)), rng.normal(size=(9, 5))
    mask = np.arange(9)[None, :] <= (2 + np.arange(7))[:, None]
    want = dense_reference(Q, K, V, mask, 0.5)
    got = orc.attention(Q, K, V, q_off=2, k_off=0, rot_dim=0, causal=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_attention_vs_scipy_rotated(orc):
    """RoPE attention with offsets equals rotating with the explicit matrices,
    then scipy's dense masked softmax (1e-12)."""
    rng = np.random.default_rng(37)
    for (Sq, Sk, q_off, k_off, D, rot, layout, causal) in (
            (7, 9, 2, 0, 8, 8, "gptj", True), (9, 9, 0, 0, 8, 8, "neox", True),
            (5, 12, 20, 13, 8, 4, "neox", True), (6, 4, 0, 0, 6, 6, "gptj", False)):
        q, k, v = rng.standard_normal((Sq, D)), rng.standard_normal((Sk, D)), rng.standard_normal((Sk, D))
        qr = np.stack([rotation_matrix(D, rot, q_off + i, 10000.0, layout) @ q[i] for i in range(Sq)])
        kr = np.stack([rotation_matrix(D, rot, k_off + j, 10000.0, layout) @ k[j] for j in range(Sk)])
        allowed = offset_mask(Sq, Sk, q_off, k_off) if causal else np.ones((Sq, Sk), bool)
        want = dense_reference(qr, kr, v, allowed, 1.0 / math.sqrt(D))
        got = orc.attention(q, k, v, q_off=q_off, k_off=k_off, rot_dim=rot, layout=layout, causal=causal)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_attention_vs_torch_sdpa(orc):
    """torch's scaled_dot_product_attention in fp64 on the CPU with an
    explicit boolean mask ([RF] sections 5 and 6) agrees at 1e-12."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(41)
    B, H, Sq, Sk, D = 2, 3, 6, 10, 8
    q, k, v = (rng.standard_normal(s) for s in ((B, H, Sq, D), (B, H, Sk, D), (B, H, Sk, D)))
    q_off, k_off = 4, 0
    qr = orc.rope(q, q_off + np.arange(Sq), layout="neox")
    kr = orc.rope(k, k_off + np.arange(Sk), layout="neox")
    mask = torch.tensor(offset_mask(Sq, Sk, q_off, k_off))
    want = F.scaled_dot_product_attention(torch.tensor(qr), torch.tensor(kr), torch.tensor(v),
                                          attn_mask=mask, dropout_p=0.0).numpy()
    got = orc.attention(q, k, v, q_off=q_off, k_off=k_off, layout="neox")
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_attention_closed_forms(orc):
    """Closed forms: zero queries give uniform weights, so causal output row i
    is the mean of V[0..i]; row 0 of a square causal forward is V[0]; a single
    key returns V; all-ones V gives all-ones output (softmax rows sum to 1)."""
    rng = np.random.default_rng(47)
    S, D = 12, 8
    k, v = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    got = orc.attention(np.zeros((S, D)), k, v, layout="gptj")
    want = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    q = rng.standard_normal((S, D))
    got = orc.attention(q, k, v, layout="neox")
    np.testing.assert_allclose(got[0], v[0], rtol=0, atol=1e-15)
    got = orc.attention(q[:1], k[:1], v[:1], layout="neox", causal=False)
    np.testing.assert_allclose(got, v[:1], rtol=0, atol=1e-15)
    got = orc.attention(q, k, np.ones((S, D)), q_off=3, k_off=1, layout="gptj")
    np.testing.assert_allclose(got, np.ones((S, D)), rtol=0, atol=1e-14)


def pin_attention_translation(orc):
    """Moving queries and keys together by the same offset leaves the output
    unchanged up to rounding (the relative-position identity, [RF] section 1)."""
    rng = np.random.default_rng(53)
    q, k, v = (rng.standard_normal((1, 2, 16, 16)) for _ in range(3))
    a = orc.attention(q, k, v, q_off=0, k_off=0, layout="neox")
    b = orc.attention(q, k, v, q_off=777, k_off=777, layout="neox")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)
    c = orc.attention(q, k, v, q_off=1, k_off=0, layout="neox")
    assert not np.allclose(a, c), "changing only the query offset must change the output"


def pin_empty_row_rejected(orc):
    """A query that sees no key is rejected ([RF] section 5)."""
    import oracle as oracle_pkg
    rng = np.random.default_rng(59)
    q, k, v = (rng.standard_normal((4, 8)) for _ in range(3))
    try:
        orc.attention(q, k, v, q_off=0, k_off=1, layout="gptj")
    except oracle_pkg.OracleError as e:
        assert e.status == oracle_pkg.ERR_EMPTY_ROW
    else:
        raise AssertionError("empty row accepted")


def pin_rows_match_full(orc):
    """The sampled-row entry point reproduces the full forward bit for bit."""
    rng = np.random.default_rng(61)
    q, k, v = rng.standard_normal((2, 2, 9, 8)), rng.standard_normal((2, 2, 11, 8)), rng.standard_normal((2, 2, 11, 8))
    full = orc.attention(q, k, v, q_off=5, k_off=3, layout="gptj")
    rows = [(0, 0, 0), (1, 1, 8), (0, 1, 4), (1, 0, 2)]
    got = orc.attention_rows(q, k, v, rows, q_off=5, k_off=3, layout="gptj")
    assert np.array_equal(got, np.stack([full[b, h, i] for b, h, i in rows]))


def pin_gqa_vs_torch_sdpa(orc):
    """Fewer key/value heads than query heads: query head h reads key/value
    head h // (H // Hkv) ([TR] "Inputs the agent should gather first", item 3,
    and "Required reasoning process", step 10, for the two head counts).
    torch's scaled_dot_product_attention with enable_gqa=True, in fp64 on the
    CPU with the explicit offset mask, agrees at 1e-12; so does the
    sampled-row entry point, bit for bit with the full forward."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(43)
    B, H, Hkv, Sq, Sk, D = 2, 6, 2, 5, 9, 8
    q = rng.standard_normal((B, H, Sq, D))
    k, v = rng.standard_normal((B, Hkv, Sk, D)), rng.standard_normal((B, Hkv, Sk, D))
    q_off, k_off = 6, 2
    qr = orc.rope(q, q_off + np.arange(Sq), layout="neox")
    kr = orc.rope(k, k_off + np.arange(Sk), layout="neox")
    mask = torch.tensor(offset_mask(Sq, Sk, q_off, k_off))
    want = F.scaled_dot_product_attention(torch.tensor(qr), torch.tensor(kr), torch.tensor(v),
                                          attn_mask=mask, dropout_p=0.0, enable_gqa=True).numpy()
    got = orc.attention(q, k, v, q_off=q_off, k_off=k_off, layout="neox")
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    rows = [(0, 1, 3), (1, 4, 2), (0, 0, 0), (1, 5, 4)]
    sel = orc.attention_rows(q, k, v, rows, q_off=q_off, k_off=k_off, layout="neox")
    assert np.array_equal(sel, np.stack([got[b, h, i] for b, h, i in rows]))


def pin_gqa_head_count_must_divide(orc):
    """A key/value head count that does not divide the query head count is
    rejected."""
    rng = np.random.default_rng(47)
    q = rng.standard_normal((1, 4, 3, 8))
    k, v = rng.standard_normal((1, 3, 3, 8)), rng.standard_normal((1, 3, 3, 8))
    try:
        orc.attention(q, k, v, layout="neox")
    except Exception:
        return
    raise AssertionError("head counts 4 / 3 accepted")


def pin_decode_step_forms(orc):
    """One decoded token at cache length L: its query sits at position L and
    sees the L cached keys and its own ([RF] sections 2 and 6: rotate the new
    token at its cache position, keep rotated keys in the cache).  Both forms
    the decode tests use must equal a reference built from complex-number
    rotation and scipy's softmax, with query head h reading key/value head
    h // (H // Hkv):
      (a) the oracle's attention of the one query at q_off = L over the raw
          keys 0..L, each rotated at its own position;
      (b) the oracle's attention without rotation of the query rotated at L
          over keys that were rotated once when they were cached."""
    rng = np.random.default_rng(53)
    H, Hkv, D = 4, 2, 8
    for layout in ("gptj", "neox"):
        for L in (0, 1, 6, 13):
            q = rng.standard_normal((1, H, 1, D))
            k = rng.standard_normal((1, Hkv, L + 1, D))
            v = rng.standard_normal((1, Hkv, L + 1, D))
            pos = np.arange(L + 1)
            kr = rope_complex(k, pos, 100.0, D, layout)
            qr = rope_complex(q, [L], 100.0, D, layout)
            want = np.stack([dense_reference(qr[0, h], kr[0, h // 2], v[0, h // 2],
                                             np.ones((1, L + 1), bool), 1 / math.sqrt(D))
                             for h in range(H)])[None]
            a = orc.attention(q, k, v, q_off=L, k_off=0, base=100.0, layout=layout)
            np.testing.assert_allclose(a, want, rtol=0, atol=1e-12)
            b = orc.attention(orc.rope(q, [L], base=100.0, layout=layout),
                              orc.rope(k, pos, base=100.0, layout=layout), v, q_off=L, k_off=0,
                              rot_dim=0)
            np.testing.assert_allclose(b, want, rtol=0, atol=1e-12)


def pin_position_interpolation(orc):
    """Position interpolation divides every position by the extension factor
    before the angle is formed ([RF] section 3).  The table at factor s holds
    at row s*m exactly the plain table's row m; at a fractional factor it
    equals numpy's cos/sin of (p/s) theta_i; and attention with the factor
    equals complex-number rotation at the divided positions plus SciPy's
    softmax, the mask still comparing the undivided positions."""
    for base, rot in ((10000.0, 64), (500000.0, 128)):
        c1, s1 = orc.trig(base, rot, 50)
        c4, s4 = orc.trig(base, rot, 200, pos_div=4.0)
        assert np.array_equal(c4[::4], c1) and np.array_equal(s4[::4], s1)
        cf, sf = orc.trig(base, rot, 300, pos_div=2.5)
        ang = (np.arange(300)[:, None] / 2.5) * np.power(base, -2.0 * np.arange(rot // 2) / rot)[None]
        np.testing.assert_allclose(cf, np.cos(ang), rtol=0, atol=1e-12)
        np.testing.assert_allclose(sf, np.sin(ang), rtol=0, atol=1e-12)
        assert not np.allclose(cf[1:], orc.trig(base, rot, 300)[0][1:])
    rng = np.random.default_rng(59)
    Sq, Sk, D, q_off, k_off, s = 5, 11, 8, 9, 3, 3.0
    for layout in ("gptj", "neox"):
        q = rng.standard_normal((1, 2, Sq, D))
        k, v = rng.standard_normal((1, 2, Sk, D)), rng.standard_normal((1, 2, Sk, D))
        qr = rope_complex(q, (q_off + np.arange(Sq)) / s, 100.0, D, layout)
        kr = rope_complex(k, (k_off + np.arange(Sk)) / s, 100.0, D, layout)
        allowed = offset_mask(Sq, Sk, q_off, k_off)
        want = np.stack([dense_reference(qr[0, h], kr[0, h], v[0, h], allowed, 1 / math.sqrt(D))
                         for h in range(2)])[None]
        got = orc.attention(q, k, v, q_off=q_off, k_off=k_off, base=100.0, layout=layout, pos_div=s)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        rows = orc.attention_rows(q, k, v, [(0, 1, 0), (0, 0, 4)], q_off=q_off, k_off=k_off,
                                  base=100.0, layout=layout, pos_div=s)
        np.testing.assert_allclose(rows, np.stack([want[0, 1, 0], want[0, 0, 4]]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# backward pins


def _loss_grad_fd(orc, q, k, v, dout, h=1e-5, **kw):
    """Central differences of L = sum(dout * attention(q, k, v)) with respect
    to every element of q, k and v."""
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.empty_like(args[which])
        it = np.nditer(args[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            lp = np.sum(dout * orc.attention(*plus, **kw))
            lm = np.sum(dout * orc.attention(*minus, **kw))
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def pin_bwd_finite_differences(orc):
    """The gradients equal central finite differences of the forward (the
    pinned oracle forward) for the loss sum(dout * o): GQA, offsets with the
    causal mask, partial rotation, both pairings, interpolated positions and
    no mask ([RF] section 5: the backward is the derivative of the same
    forward)."""
    rng = np.random.default_rng(61)
    cases = [
        dict(shape=(1, 2, 1, 4, 6, 8), kw=dict(q_off=2, k_off=0, rot_dim=8, layout="neox")),
        dict(shape=(1, 4, 2, 3, 5, 8), kw=dict(q_off=4, k_off=1, rot_dim=4, layout="gptj", base=100.0)),
        dict(shape=(2, 2, 2, 3, 3, 6), kw=dict(rot_dim=6, layout="neox", causal=False, pos_div=2.5)),
    ]
    for c in cases:
        B, H, Hkv, Sq, Sk, D = c["shape"]
        q = rng.standard_normal((B, H, Sq, D))
        k = rng.standard_normal((B, Hkv, Sk, D))
        v = rng.standard_normal((B, Hkv, Sk, D))
        dout = rng.standard_normal((B, H, Sq, D))
        got = orc.attention_bwd(q, k, v, dout, **c["kw"])
        want = _loss_grad_fd(orc, q, k, v, dout, **c["kw"])
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, rtol=0, atol=2e-8)


def _torch_rope(x, pos, base, rot, layout):
    """RoPE in torch fp64 from complex multiplication (built without the
    oracle's pair indexing)."""
    import torch
    half = rot // 2
    theta = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / rot)
    ang = pos[:, None].to(torch.float64) * theta[None, :]
    w = torch.polar(torch.ones_like(ang), ang)
    if layout == "gptj":
        z = torch.complex(x[..., 0:rot:2], x[..., 1:rot:2]) * w
        rotated = torch.stack([z.real, z.imag], dim=-1).flatten(-2)
    else:
        z = torch.complex(x[..., :half], x[..., half:rot]) * w
        rotated = torch.cat([z.real, z.imag], dim=-1)
    return torch.cat([rotated, x[..., rot:]], dim=-1)


def pin_bwd_vs_torch_autograd(orc):
    """fp64 torch autograd through a forward written independently (complex
    rotation, explicit matmul, offset mask, torch.softmax, key/value heads
    repeated for GQA) agrees with the oracle's gradients at 1e-11, and its
    log-sum-exp rows with the oracle's at 1e-12."""
    import torch
    rng = np.random.default_rng(67)
    for layout, rot, causal in (("neox", 8, True), ("gptj", 16, True), ("neox", 16, False)):
        B, H, Hkv, Sq, Sk, D, q_off, k_off, base = 2, 4, 2, 6, 9, 16, 5, 2, 500.0
        arrays = [rng.standard_normal(s) for s in ((B, H, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D),
                                                   (B, H, Sq, D))]
        q, k, v, dout = (torch.tensor(a, requires_grad=i < 3) for i, a in enumerate(arrays))
        qr = _torch_rope(q, torch.arange(Sq) + q_off, base, rot, layout)
        kr = _torch_rope(k, torch.arange(Sk) + k_off, base, rot, layout)
        krr = kr.repeat_interleave(H // Hkv, dim=1)
        vr = v.repeat_interleave(H // Hkv, dim=1)
        s = qr @ krr.transpose(-1, -2) / math.sqrt(D)
        if causal:
            allowed = torch.from_numpy(offset_mask(Sq, Sk, q_off, k_off))
            s = s.masked_fill(~allowed, float("-inf"))
        o = torch.softmax(s, dim=-1) @ vr
        (o * dout).sum().backward()
        kw = dict(q_off=q_off, k_off=k_off, rot_dim=rot, base=base, layout=layout, causal=causal)
        got = orc.attention_bwd(*arrays, **kw)
        for g, t in zip(got, (q.grad, k.grad, v.grad)):
            np.testing.assert_allclose(g, t.numpy(), rtol=0, atol=1e-11)
        lse = torch.logsumexp(s, dim=-1).detach().numpy()
        np.testing.assert_allclose(orc.attention_lse(arrays[0], arrays[1], **kw), lse, rtol=0,
                                   atol=1e-12)


ALL_PINS = [v for name, v in sorted(globals().items()) if name.startswith("pin_")]
