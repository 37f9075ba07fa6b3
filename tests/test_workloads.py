"""Seeded input generator: determinism, shapes, ragged lengths, sweep grid."""
import torch

from parallax_covariance_corrected_amd.workloads import (WORKLOADS, make_inputs, padded_cache,
                                                         sweep_points, algorithmic_bytes)


def test_deterministic_and_seed_dependent():
    wl = WORKLOADS[2].scaled(B=2, ctx=64, d_model=32)
    a, b, c = make_inputs(wl, 0), make_inputs(wl, 0), make_inputs(wl, 1)
    assert torch.equal(a.q, b.q) and torch.equal(a.K[1], b.K[1]) and torch.equal(a.W_R, b.W_R)
    assert not torch.equal(a.q, c.q)
    assert a.q.dtype == torch.bfloat16 and a.q.shape == (2, 16, 128)
    assert a.W_R.shape == (16 * 128, 32) and a.x.shape == (2, 32)
    assert a.K[0].shape == (8, 64, 128) and a.seq_lens.tolist() == [64, 64]


def test_wr_zero_keeps_rest_of_stream():
    wl = WORKLOADS[1]
    a, z = make_inputs(wl, 0), make_inputs(wl, 0, wr_zero=True)
    assert torch.count_nonzero(z.W_R) == 0
    assert torch.equal(a.q, z.q) and torch.equal(a.K[0], z.K[0]) and torch.equal(a.x, z.x)
    assert a.q.dtype == torch.float32 and a.W_R.shape == (128, 128)


def test_ragged_lengths_in_range():
    wl = WORKLOADS[5].scaled(B=64, d_model=16, ctx=32768)
    g = torch.Generator("cpu").manual_seed(0)
    from parallax_covariance_corrected_amd.workloads import draw_lengths
    n = draw_lengths(g, 4096, 128, 32768)
    assert int(n.min()) >= 128 and int(n.max()) <= 32768
    # log-uniform: the median sits near the geometric mean sqrt(128*32768) = 2048
    med = float(n.float().median())
    assert 1500 < med < 2800


def test_padded_cache_nan_padding():
    wl = WORKLOADS[2].scaled(B=2, ctx=10, d_model=8, Hq=2, Hkv=1, d=4)
    s = make_inputs(wl, 0, lengths=[3, 10])
    c = padded_cache(s.K, 12)
    assert c.shape == (2, 1, 12, 4)
    assert torch.equal(c[0, :, :3], s.K[0]) and torch.isnan(c[0, :, 3:].float()).all()
    assert torch.isnan(c[1, :, 10:].float()).all()


def test_sweep_grid_and_bytes():
    pts = sweep_points()
    assert len(pts) == 105 and (512, 32768) in pts and (1024, 32768) not in pts
    b = algorithmic_bytes(WORKLOADS[2], 16 * 4096)
    assert b["kv"] == 268_435_456
