"""The α-β cost model in the C library against every model output the pages
print (tests/golden/alpha_beta_model_printed.json, each with its citation).
Host arithmetic only, no GPU."""

import pytest


@pytest.fixture(scope="module")
def cs():
    from collective_reduction_amd import ccl_sim
    return ccl_sim


def test_printed_cost_model_runs(cs, golden):
    g = golden("alpha_beta_model_printed.json")
    for r in g["runs"]:
        kw = {k: r[k] for k in ("ranks_per_node", "alpha_intra_us", "beta_intra_gbps") if k in r}
        e = cs.ccl_sim_model_estimate(r["coll"], r["algo"], r["n"], r["size_bytes"], r["alpha_us"], r["beta_gbps"], **kw)
        p = r["printed"]
        assert round(e["time_s"] * 1e6, 1) == p["T_us"], r
        assert round(100 * e["latency_fraction"], 1) == p["lat_pct"], r
        assert round(e["algbw_gbps"], 2) == p["algbw"], r
        assert round(e["busbw_gbps"], 2) == p["busbw"], r


def _near(value, printed, unit):
    """The prose tables are rounded by hand: busbw 24.9501 is printed as 24.9,
    so they are held to one unit of their last printed digit (the script's
    printed runs above are held to exact rounding)."""
    return abs(value - printed) <= unit * 1.0001


def test_algbw_busbw_table(cs, golden):
    t = golden("alpha_beta_model_printed.json")["ring_table_1GB"]
    for row in t["rows"]:
        e = cs.ccl_sim_model_estimate("all_reduce", "ring", row["n"], t["size_bytes"], t["alpha_us"], t["beta_gbps"])
        assert _near(e["time_s"] * 1e3, row["T_ms"], 0.1)
        assert _near(e["algbw_gbps"], row["algbw"], 0.1)
        assert _near(e["busbw_gbps"], row["busbw"], 0.1)


def test_core_question_numbers(cs, golden):
    c = golden("alpha_beta_model_printed.json")["core_question"]
    big, small = c["cases"]
    e = cs.ccl_sim_model_estimate("all_reduce", "ring", c["n"], big["size_bytes"], c["alpha_us"], c["beta_gbps"])
    assert round(e["time_s"] * 1e3, 2) == big["T_ms"]
    assert _near(e["algbw_gbps"], big["algbw"], 0.1) and _near(e["busbw_gbps"], big["busbw"], 0.1)
    e = cs.ccl_sim_model_estimate("all_reduce", "ring", c["n"], small["size_bytes"], c["alpha_us"], c["beta_gbps"])
    assert round(e["time_s"] * 1e6) == small["T_us"]
    assert _near(e["algbw_gbps"], small["algbw"], 0.01) and _near(e["busbw_gbps"], small["busbw"], 0.01)


def test_busbw_factors(cs, golden):
    f = golden("alpha_beta_model_printed.json")["busbw_factors_n8"]
    for coll in ("all_reduce", "all_gather", "reduce_scatter", "all_to_all", "broadcast", "reduce"):
        assert cs.ccl_sim_busbw_factor(coll, 8) == f[coll]


def test_ring_page_latency_table(cs, golden):
    r = golden("alpha_beta_model_printed.json")["ring_page"]
    for c in r["cases"]:
        e = cs.ccl_sim_model_estimate("all_reduce", "ring", c["n"], c["size_bytes"], r["alpha_us"], r["beta_gbps"])
        digits = len(str(c["T_ms"]).split(".")[1])
        assert round(e["time_s"] * 1e3, digits) == c["T_ms"], c


def test_ring_knee_is_n_alpha_beta(cs):
    """At S* = nαβ the two ring terms are equal ([PRIMS] §五.6): 2 MB for 8 ranks on IB."""
    n, alpha_us, beta_gbps = 8, 10.0, 25.0
    s_star = n * alpha_us * 1e-6 * beta_gbps * 1e9
    assert s_star == 2_000_000
    e = cs.ccl_sim_model_estimate("all_reduce", "ring", n, s_star, alpha_us, beta_gbps)
    assert abs(e["latency_s"] - e["bandwidth_s"]) < 1e-12


def test_model_rejects_bad_arguments(cs):
    with pytest.raises(cs.CclSimError):
        cs.ccl_sim_model_estimate("all_gather", "tree", 8, 1024)
    with pytest.raises(cs.CclSimError):
        cs.ccl_sim_model_estimate("all_reduce", "2level", 12, 1024, ranks_per_node=8)
    with pytest.raises(cs.CclSimError):
        cs.ccl_sim_model_estimate("all_reduce", "ring", 0, 1024)
    with pytest.raises(cs.CclSimError):
        cs.ccl_sim_model_estimate("all_reduce", "ring", 8, 1024, beta_gbps=0.0)
    e = cs.ccl_sim_model_estimate("all_reduce", "ring", 1, 1024)
    assert e["time_s"] == 0 and e["algbw_gbps"] == 0
