"""The seeded input generators: shapes, storage-type rounding, raggedness."""
import numpy as np

from rotary_position_embedding_rope_amd import workloads as wl


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 lies exactly between two bf16 values (1 and 1 + 2^-7): ties go to even (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    got = wl.round_to(x, "bf16")
    assert got[0] == 1.0 and got[1] == 1.0 + 2.0 ** -6 and got[2] == -2.5
    assert np.array_equal(wl.bf16_to_f32(wl.bf16_bits(got)), got)


def test_attention_inputs_deterministic_and_exact():
    w = wl.SMALL_BF16
    a = wl.attention_inputs(w)
    b = wl.attention_inputs(w)
    for x, y in zip(a, b):
        assert x.shape == (1, 8, 512, 64) and x.dtype == np.float32
        assert np.array_equal(x, y)
        assert np.array_equal(wl.round_to(x, "bf16"), x)
    assert abs(float(a[0].std()) - 1.0) < 0.02


def test_gqa_inputs():
    w = wl.PREFILL_GQA
    assert (w.H, w.Hkv) == (32, 8)
    small = wl.AttentionWorkload("g", 1, 6, 5, 7, 8, "bf16", 3, "neox", H_kv=2)
    q, k, v = wl.attention_inputs(small)
    assert q.shape == (1, 6, 5, 8) and k.shape == v.shape == (1, 2, 7, 8)
    assert wl.SMALL_BF16.Hkv == wl.SMALL_BF16.H


def test_ragged_workload():
    w = wl.RAGGED_ROPE
    d = wl.rope_apply_inputs(w)
    assert d["lengths"].sum() == 8192 and len(d["lengths"]) == 16 and (d["lengths"] > 0).all()
    assert d["positions"].dtype == np.int32 and d["positions"].min() >= 0
    assert d["positions"].max() < 32768
    assert d["q"].shape == (8192, 32, 128) and d["k"].shape == (8192, 8, 128)
    assert w.algorithmic_bytes() == 86_016_000


def test_flop_counts():
    assert wl.HEADLINE.flops() == 4 * 64 * 8 * 4096 * 4097 // 2
    assert wl.PREFILL_OFFSET.visible_pairs() == 32 * sum(14337 + i for i in range(2048))
    assert wl.TINY_F32.table_rows == 128 and wl.PREFILL_OFFSET.table_rows == 16384
