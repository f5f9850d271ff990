"""The seeded generators: deterministic, sliceable, and drawing what they claim."""

import numpy as np

from collective_reduction_amd import inputs as I


def test_affine_worked_example():
    s = I.spec("worked_example_4x20_int64")
    xs = I.all_buffers(s)
    assert xs.shape == (4, 20) and xs.dtype == np.int64
    assert xs[3].tolist() == [300 + i for i in range(20)]


def test_slices_and_positions_regenerate_the_same_values():
    s = I.spec("uniform_8x1048576_fp32", count=3 * I.CHUNK + 17)
    full = I.rank_buffer(s, 5)
    assert full.size == 3 * I.CHUNK + 17
    lo, hi = I.CHUNK - 3, 2 * I.CHUNK + 9
    assert np.array_equal(I.rank_buffer(s, 5, lo, hi), full[lo:hi])
    pos = np.array([0, 7, I.CHUNK - 1, I.CHUNK, 3 * I.CHUNK + 16])
    g = I.gather_positions(s, pos)
    assert g.shape == (8, pos.size)
    assert np.array_equal(g[5], full[pos])
    again = I.rank_buffer(s, 5)
    assert np.array_equal(again, full)


def test_distributions():
    u = I.rank_buffer(I.spec("uniform_8x1048576_fp32"), 0)
    assert u.dtype == np.float32 and u.min() >= -1.0 and u.max() < 1.0
    assert abs(float(u.mean())) < 0.01
    n = I.rank_buffer(I.spec("normal_256x4194304_fp32"), 3, 0, 1 << 18)
    assert abs(float(n.std()) - 1e-3) < 2e-5
    iu = I.rank_buffer(I.spec("intuniform_8x1000003_int32"), 2)
    assert iu.dtype == np.int32 and iu.min() >= -(1 << 20) and iu.max() <= (1 << 20)
    b = I.rank_buffer(I.spec("normal_256x6553600_bf16"), 1, 0, 4096)
    assert b.dtype == np.uint16
    f = (b.astype(np.uint32) << 16).view(np.float32)
    assert 0.5e-3 < float(np.abs(f).mean()) < 1.2e-3


def test_ranks_and_workloads_differ():
    s = I.spec("uniform_8x1048576_fp32", count=1000)
    assert not np.array_equal(I.rank_buffer(s, 0), I.rank_buffer(s, 1))
    a = I.rank_buffer(I.spec("normal_8x1000003_fp32"), 0, 0, 1000)
    b = I.rank_buffer(I.spec("intuniform_8x1000003_int32"), 0, 0, 1000)
    assert not np.array_equal(a.view(np.int32), b)
