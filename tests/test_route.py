"""The route rule for non-deterministic weight-gradient calls (pure
functions on measured times) and the library's route table (host only)."""
import pytest

from dense_ragged_grouped_amd import route


def test_sign_test_closed_forms():
    # P(X >= k) for X ~ Binomial(n, 1/2)
    assert route.sign_test_p(5, 5) == 1 / 32
    assert route.sign_test_p(4, 4) == 1 / 16
    assert route.sign_test_p(4, 5) == 6 / 32
    assert route.sign_test_p(0, 7) == 1.0
    assert route.sign_test_p(9, 10) == 11 / 1024
    assert abs(sum(route.sign_test_p(k, 12) - route.sign_test_p(k + 1, 12) for k in range(12))
               + route.sign_test_p(12, 12) - 1.0) < 1e-15
    with pytest.raises(ValueError):
        route.sign_test_p(6, 5)


def test_op_level_condition():
    det = [100.0, 101.0, 99.0, 100.5, 100.2]
    fast = [98.0, 98.5, 97.9, 98.1, 98.6]          # every run faster, ratio ~0.98
    kept, d = route.op_level_keeps_split(det, fast)
    assert kept and d["wins"] == 5 and d["p"] == 1 / 32 and d["median_ratio"] < 0.99
    # faster in every run but by less than 1 %
    kept, _ = route.op_level_keeps_split(det, [x * 0.995 for x in det])
    assert not kept
    # one lost run: no longer "every run"
    kept, _ = route.op_level_keeps_split(det, fast[:4] + [101.0])
    assert not kept
    # every run faster but too few runs for p < 0.05
    kept, d = route.op_level_keeps_split(det[:4], fast[:4])
    assert not kept and d["p"] == 1 / 16


def test_corun_and_step_conditions():
    ok = {(8, "split first"): ([100.0] * 3, [102.0] * 3), (32, "det first"): ([100.0] * 3, [103.0] * 3)}
    assert route.corun_keeps_split(ok)[0]
    bad = dict(ok)
    bad[(16, "split first")] = ([100.0] * 3, [103.5] * 3)
    assert not route.corun_keeps_split(bad)[0]
    steps = {("bwd", "eager"): ([200.0] * 3, [202.0] * 3), ("ckpt", "graph"): ([400.0] * 3, [405.2] * 3)}
    assert route.steps_keep_split(steps)[0]        # 1.0100 and 1.0130
    steps[("ckpt", "eager")] = ([400.0] * 3, [405.6] * 3)
    assert not route.steps_keep_split(steps)[0]    # 1.014


def test_choose_program_needs_every_condition():
    det = [100.0, 101.0, 99.0, 100.5, 100.2]
    fast = [98.0, 98.5, 97.9, 98.1, 98.6]
    op = {"eager": (det, fast), "graph": (det, fast)}
    corun = {(c, o): ([100.0] * 3, [101.0] * 3) for c in route.HOLDER_CUS for o in ("det first", "split first")}
    steps = {(s, m): ([100.0] * 3, [99.0] * 3) for s in ("bwd", "ckpt") for m in ("eager", "graph")}
    assert route.choose_program(op, corun, steps)[0] == "split"
    assert route.choose_program({"eager": (det, fast), "graph": (det, det)}, corun, steps)[0] == "det"
    assert route.choose_program(op, {}, steps)[0] == "det"     # a condition not measured
    slow = {k: ([100.0] * 3, [105.0] * 3) for k in corun}
    assert route.choose_program(op, slow, steps)[0] == "det"


def test_route_table_sends_a_point_to_the_split_program():
    import dense_ragged_grouped_amd as drgg
    drgg.route_clear()
    pt = (8, 131072, 1536, 2048, drgg.BF16)
    other = (8, 131072, 1536, 2048, drgg.FP32)
    try:
        assert drgg.wgrad_runs_deterministic(*pt, deterministic=False)
        det_ws = drgg.workspace_size(drgg.OP_WGRAD, *pt[:4], pt[4], False)
        drgg.route_split(*pt)
        drgg.route_split(*pt)                       # no duplicate
        assert drgg.route_count() == 1
        assert not drgg.wgrad_runs_deterministic(*pt, deterministic=False)
        assert drgg.wgrad_runs_deterministic(*pt, deterministic=True)
        assert drgg.wgrad_runs_deterministic(*other, deterministic=False)   # exact match only
        p = drgg.plan(drgg.OP_WGRAD, *pt[:4], pt[4], False, 256)
        assert p["unit"] > 0 and p["chunk_max"] == 0
        assert drgg.workspace_size(drgg.OP_WGRAD, *pt[:4], pt[4], False) != det_ws
        with pytest.raises(drgg.DrggError):
            drgg.route_split(0, 1, 8, 8, drgg.BF16)
    finally:
        drgg.route_clear()
    assert drgg.route_count() == 0
    assert drgg.wgrad_runs_deterministic(*pt, deterministic=False)
    drgg.load_default_routes()


def test_load_routes(tmp_path):
    import json
    import dense_ragged_grouped_amd as drgg
    path = tmp_path / "routes.json"
    path.write_text(json.dumps({"points": [
        {"E": 1, "M": 16384, "N": 512, "K": 4096, "out_dtype": drgg.FP32, "program": "split"},
        {"E": 1, "M": 16384, "N": 48, "K": 4096, "out_dtype": drgg.FP32, "program": "det"}]}))
    drgg.route_clear()
    try:
        assert drgg.load_routes(str(path)) == 1
        assert not drgg.wgrad_runs_deterministic(1, 16384, 512, 4096, drgg.FP32, False)
        assert drgg.wgrad_runs_deterministic(1, 16384, 48, 4096, drgg.FP32, False)
    finally:
        drgg.route_clear()
        drgg.load_default_routes()


def test_shipped_table_follows_its_measurements():
    """The table shipped with the package: every point's program is the one
    the rule gives for its stored ratios' signs, and import installed its
    split points."""
    import json
    import dense_ragged_grouped_amd as drgg
    table = json.load(open(drgg.DEFAULT_ROUTES))
    assert table["compute_units"] == 256 and len(table["points"]) >= 7
    for pt in table["points"]:
        d = pt["details"]
        ok = (all(d[f"op_{m}"]["wins"] == d[f"op_{m}"]["runs"] and d[f"op_{m}"]["p"] < 0.05
                  and d[f"op_{m}"]["median_ratio"] < 0.99 for m in ("eager", "graph"))
              and max(d["corun"].values()) <= 1.03 and max(d["steps"].values()) <= 1.013)
        assert pt["program"] == ("split" if ok else "det"), pt["name"]
        assert drgg.wgrad_runs_deterministic(pt["E"], pt["M"], pt["N"], pt["K"], pt["out_dtype"], False) == \
            (pt["program"] == "det")
