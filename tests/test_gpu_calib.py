"""The measurement kernels of librope_calib.so do the work they are timed
for: the in-place stream touches exactly the vectors of its pattern, and
the attention inner-step kernel's accumulators and row sums equal the
step's definition (S = K Q^T, P = exp2(S) rounded to bf16, O = P V, l = row
sums of P; "RoPE and FlashAttention", section 5) times the iteration count,
computed here in fp64 from the same bf16 inputs."""
import numpy as np
import pytest
import torch

from rotary_position_embedding_rope_amd import calib
from rotary_position_embedding_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("row,span,n_vec", [(16, 8, 8 * 300), (16, 8, 8 * 300 + 5), (4, 4, 1000), (8, 1, 77)])
def test_stream_touches_exactly_its_pattern(row, span, n_vec):
    rng = np.random.default_rng(row * 100 + span)
    n_rows = -(-n_vec // span)
    words = rng.integers(0, 2 ** 31, size=(n_rows * row + 3) * 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(words.copy()).to(DEV)
    calib.stream_inplace(buf, n_vec, row, span)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    v = np.arange(n_vec)
    touched = (v // span) * row + v % span
    want = words.copy().reshape(-1, 4)
    want[touched] += 1
    assert np.array_equal(got, want.reshape(-1))


@pytest.mark.parametrize("n_vec,at", [(1, 0), (1000, 999), (12345, 4321)])
def test_stream_read_finds_a_planted_vector(n_vec, at):
    key = 0x7A5C3E1D
    words = np.random.default_rng(n_vec).integers(0, 2 ** 31, size=4 * n_vec).astype(np.int32)
    words[4 * at:4 * at + 4] = key
    buf = torch.from_numpy(words).to(DEV)
    hit = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    miss = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    calib.stream_read(buf, n_vec, key, hit)
    calib.stream_read(buf, n_vec, key ^ 1, miss)   # no vector matches: nothing written
    torch.cuda.synchronize()
    assert int(hit.item()) == at and int(miss.item()) == -1


def bf16_round(x):
    return wl.round_to(np.asarray(x, dtype=np.float64), "bf16")


@pytest.mark.parametrize("variant", calib.LOOP_VARIANTS, ids=lambda v: "d%d_w%d_p%d" % v)
def test_attention_loop_computes_the_step(variant):
    D, wps, pipe = variant
    iters, wgs = 4, 2
    rng = np.random.default_rng(D * 10 + wps * 2 + pipe)
    k = bf16_round(rng.normal(0, 0.25, size=(64, D)))
    v = bf16_round(rng.normal(0, 1.0, size=(64, D)))
    q = bf16_round(rng.normal(0, 0.25, size=(128 * wps, D)))
    # device layouts: K rows at pitch D + 8; V chunk c of row r at chunk c ^ 4((r >> 1) & 1)
    k_dev = np.zeros((64, D + 8))
    k_dev[:, :D] = k
    v_dev = np.zeros((64, D))
    for r in range(64):
        for c in range(D // 8):
            p = c ^ (4 * ((r >> 1) & 1))
            v_dev[r, 8 * p:8 * p + 8] = v[r, 8 * c:8 * c + 8]
    kt, vt, qt = (torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(DEV).contiguous()
                  for a in (k_dev, v_dev, q))
    n_k, n_v, n_q, n_out, n_cyc = calib.loop_shapes(D, wps, wgs)
    out = torch.full((n_out,), float("nan"), dtype=torch.float32, device=DEV)
    cyc = torch.zeros(n_cyc, dtype=torch.int64, device=DEV)
    calib.attn_loop(D, wps, pipe, iters, wgs, kt, vt, qt, out, cyc)
    torch.cuda.synchronize()

    s = q @ k.T                                  # [rows, 64 keys]
    assert s.max() < 7.0                         # no row sum reaches the fast-path bound
    p = bf16_round(np.exp2(s))
    o_want = iters * (p @ v)                     # [rows, D]
    l_want = iters * p.sum(axis=1)

    got = out.cpu().numpy().reshape(wgs, 256 * wps, D // 2 + 4)
    lane = np.arange(64)
    for g in range(wgs):
        o = np.full((128 * wps, D), np.nan)
        l = np.zeros(128 * wps)
        for w in range(4 * wps):
            th = got[g, 64 * w:64 * w + 64]      # [lane, values]
            rows = 32 * w + lane % 32
            for b in range(D // 32):
                for r in range(16):
                    dim = 32 * b + 8 * (r // 4) + 4 * (lane // 32) + r % 4
                    o[rows, dim] = th[:, 16 * b + r]
            np.add.at(l, rows, th[:, D // 2:].sum(axis=1))
        tol_o = 4e-3 * np.abs(o_want).max()
        assert np.abs(o - o_want).max() <= tol_o
        assert np.abs(l - l_want).max() <= 4e-3 * l_want.max()
    assert (cyc.cpu().numpy() > 0).all()
