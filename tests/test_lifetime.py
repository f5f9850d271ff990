"""Buffer lifetimes: the model against the pages' printed table (CPU), and
the four lifetimes measured on the GPU around the library's collectives."""

import pytest

from collective_reduction_amd import lifetime as LT

MIB = 1 << 20


def test_model_matches_the_printed_table(golden):
    g = golden("lifetime_256mib_world4.json")
    mdl = LT.model(g["payload_mib"] * MIB, g["world"])
    for mode, row in g["rows"].items():
        assert mdl[mode]["steady"] == row["steady_mib"] * MIB, mode
        assert mdl[mode]["peak"] == row["peak_mib"] * MIB, mode
    assert 1 - mdl["reduce_scatter_only"]["steady"] / mdl["allreduce_full"]["steady"] == g["steady_reduction_rs_only"]


@pytest.mark.gpu
@pytest.mark.parametrize("mode", LT.MODES)
def test_measured_lifetimes_direct(golden, mode):
    """With the direct schedule the library allocates nothing and needs no
    workspace, so the measured per-rank steady and peak bytes are exactly the
    model's: 256 MiB per rank over 4 virtual ranks."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    g = golden("lifetime_256mib_world4.json")
    n = g["world"]
    count = g["payload_mib"] * MIB // 4
    got = LT.measure(mode, n, count, "float32", "direct")
    want = LT.model(g["payload_mib"] * MIB, n)[mode]
    assert got["workspace"] == 0
    assert got["steady"] == want["steady"]
    assert got["peak"] == want["peak"]


@pytest.mark.gpu
@pytest.mark.parametrize("mode", LT.MODES)
def test_measured_lifetimes_ring(mode):
    """The ring schedules add only their workspace to the peak."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    n, count = 4, 16 * MIB
    got = LT.measure(mode, n, count, "float32", "ring_stepwise")
    want = LT.model(count * 4, n)[mode]
    assert got["steady"] == want["steady"]
    assert want["peak"] <= got["peak"] <= want["peak"] + got["workspace"]


@pytest.mark.gpu
@pytest.mark.parametrize("mode", LT.MODES)
def test_measured_lifetimes_bench_scale(mode):
    """The same four lifetimes at the bench's scale, 1 GiB per rank over 8
    virtual ranks: measured steady and peak bytes per rank equal the model
    (pinned above by the page's table), e.g. 1024 / 2176 MiB for the naive
    RS + AG and 1024 / 1152 MiB for the optimized one."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    n, count = 8, 1 << 28
    got = LT.measure(mode, n, count, "float32", "direct")
    want = LT.model(count * 4, n)[mode]
    assert got["workspace"] == 0
    assert got["steady"] == want["steady"]
    assert got["peak"] == want["peak"]
