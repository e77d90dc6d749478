"""The blocked online-softmax recurrence that the fused GPU kernel runs,
checked in fp64 against the dense oracle.

Recurrence ("RoPE and FlashAttention: relative positions and online softmax",
section 5): per query row keep a running maximum m, denominator l and
unnormalised numerator u; for each key block with scores s (masked scores are
-inf) take m' = max(m, max s), rescale l and u by exp(m - m'), add exp(s - m')
and its weighted values, and return u / l after the last block.  A block in
which a row sees no key leaves that row's state untouched.  This is also the
exact recurrence of the kernel (which works in base 2 with the scale folded
into the exponent; identical in real arithmetic).
"""
import math

import numpy as np
import pytest

import oracle
from pins import dense_reference, offset_mask


def blocked_attention(q, k, v, allowed, q_block, k_block, rescale=True):
    """Online-softmax attention over key blocks of ``k_block`` keys, query
    blocks of ``q_block`` rows.  ``rescale=False`` drops the correction of
    earlier blocks when the maximum rises (a planted mistake)."""
    Sq, Sk = allowed.shape
    if not allowed.any(axis=1).all():
        raise ValueError("a query row sees no key")
    scale = 1.0 / math.sqrt(q.shape[1])
    out = np.empty((Sq, v.shape[1]))
    for i0 in range(0, Sq, q_block):
        rows = slice(i0, min(i0 + q_block, Sq))
        n = rows.stop - rows.start
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        u = np.zeros((n, v.shape[1]))
        for j0 in range(0, Sk, k_block):
            cols = slice(j0, min(j0 + k_block, Sk))
            s = np.where(allowed[rows, cols], scale * (q[rows] @ k[cols].T), -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            live = m_new > -np.inf              # rows with at least one visible key so far
            ref = np.where(live, m_new, 0.0)    # avoids (-inf) - (-inf)
            alpha = np.where(live, np.exp(m - ref), 1.0) if rescale else np.ones(n)
            p = np.exp(s - ref[:, None])
            l = alpha * l + p.sum(axis=1)
            u = alpha[:, None] * u + p @ v[cols]
            m = m_new
        out[rows] = u / l[:, None]
    return out


@pytest.mark.parametrize("block", [1, 2, 3, 20])
def test_blocked_equals_dense_p2(block):
    """Section 5's example (Q [7,4], K [9,4], V [9,5], keys j <= 2 + i),
    blocks of 1, 2, 3 and longer than the sequence; 1e-12."""
    rng = np.random.default_rng(43)
    Q, K, V = rng.normal(size=(7, 4)), rng.normal(size=(9, 4)), rng.normal(size=(9, 5))
    mask = np.arange(9)[None, :] <= (2 + np.arange(7))[:, None]
    want = oracle.load().attention(Q, K, V, q_off=2, k_off=0, rot_dim=0)
    np.testing.assert_allclose(blocked_attention(Q, K, V, mask, block, block), want,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(want, dense_reference(Q, K, V, mask, 0.5), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("q_block,k_block", [(4, 3), (5, 8), (16, 16), (3, 64)])
def test_blocked_offset_mask_with_all_masked_blocks(q_block, k_block):
    """Rectangular offset mask (queries at 30.., keys at 11..) where some key
    blocks are entirely invisible to some query rows."""
    rng = np.random.default_rng(7)
    Sq, Sk, D = 13, 40, 8
    q, k, v = rng.standard_normal((Sq, D)), rng.standard_normal((Sk, D)), rng.standard_normal((Sk, D))
    mask = offset_mask(Sq, Sk, 30, 11)
    assert not mask.all(axis=1).all() and mask.any(axis=1).all()
    want = oracle.load().attention(q, k, v, q_off=30, k_off=11, rot_dim=0)
    np.testing.assert_allclose(blocked_attention(q, k, v, mask, q_block, k_block), want,
                               rtol=1e-12, atol=1e-12)


def test_rising_maximum_needs_rescale():
    """A rising maximum across blocks: dropping the rescale gives a wrong
    answer, keeping it gives the dense one (section 5's control; the values
    [0, 1, 20] and [3, 4, 9] are that section's)."""
    from scipy.special import softmax
    x = np.array([0.0, 1.0, 20.0])
    values = np.array([3.0, 4.0, 9.0])
    naive_tile_average = (softmax(x[:2]) @ values[:2] + values[2]) / 2
    assert abs(naive_tile_average - softmax(x) @ values) > 1

    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 4))
    k = rng.standard_normal((12, 4)) * np.linspace(0.1, 6.0, 12)[:, None]  # later keys score higher
    v = rng.standard_normal((12, 3))
    mask = np.ones((6, 12), bool)
    want = oracle.load().attention(q, k, v, rot_dim=0, causal=False)
    np.testing.assert_allclose(blocked_attention(q, k, v, mask, 6, 3), want, rtol=1e-12, atol=1e-12)
    assert not np.allclose(blocked_attention(q, k, v, mask, 6, 3, rescale=False), want, atol=1e-3)


def test_empty_row_rejected():
    """Section 5: a row that sees no key at all is rejected."""
    q = np.ones((3, 4))
    with pytest.raises(ValueError):
        blocked_attention(q, q, q, np.zeros((3, 3), bool), 2, 2)
