"""The route calibration on the GPU: one problem point measured end to end
(eager and graph-replayed calls of both weight-gradient programs, the
co-run with the CU-holding kernel in both launch orders, the backward and
checkpointed steps), the rule applied to what was measured, and the route
table left as the package installs it."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def drgg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_ragged_grouped_amd as d
    return d


def test_measure_point_small(drgg):
    from dense_ragged_grouped_amd import calibrate, route
    before = drgg.route_count()
    try:
        program, details = calibrate.measure_point(torch, drgg, route, 4, 512, 512, 256, "fp32", None,
                                                   runs=2, reps=1, log=lambda s: None)
        assert program in ("det", "split")
        for mode in ("eager", "graph"):
            d = details[f"op_{mode}"]
            assert d["runs"] == 2 and 0 <= d["wins"] <= 2 and d["median_ratio"] > 0
            # two runs can never reach p < 0.05 (the smallest p is 1/4), so the
            # rule keeps the deterministic program
            assert d["p"] >= 0.25
        assert program == "det"
        assert len(details["corun"]) == 2 * len(route.HOLDER_CUS)
        assert set(details["steps"]) == {str((s, m)) for s in ("bwd", "ckpt") for m in ("eager", "graph")}
        assert all(v > 0 for v in details["median_ms"].values())
    finally:   # measure_point clears the table; reinstall the package's one
        drgg.route_clear()
        if before:
            drgg.load_default_routes()
    assert drgg.route_count() == before
    torch.cuda.synchronize()
