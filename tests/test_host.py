"""Host-side tests of the C ABI (no GPU needed).

* libdrgg.so loads and exports every function include/drgg.h declares;
* argument checks reject bad calls before anything reaches the GPU;
* the planner: the deterministic chunk rule's properties, its independence
  from the CU count, and the bounds the kernels rely on (launched grid and
  partial slots cover every ragged distribution).
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "drgg.h")
LIB = os.path.join(ROOT, "dense_ragged_grouped_amd", "libdrgg.so")


@pytest.fixture(scope="module")
def drgg():
    if not os.path.exists(LIB):   # build only when nothing is built
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_drgg_build", os.path.join(ROOT, "dense_ragged_grouped_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import dense_ragged_grouped_amd as d
    return d


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(drgg):
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(LIB)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"declared in drgg.h but not exported: {missing}"
    assert sorted(drgg.EXPORTS) == names
    assert drgg.abi_version() == 1


def test_status_strings(drgg):
    for code in range(8):
        assert drgg.status_string(code) and drgg.status_string(code) != "unknown status"
    assert drgg.status_string(99) == "unknown status"


# ---- argument checks (all rejected on the host, before any HIP call) ----------

A16 = 0x10000          # a fake, 16-byte aligned "device" address (never dereferenced)


def fwd(drgg, *, X=A16, W=A16, offs=A16, E=2, M=64, N=64, K=64, dt=1, Y=A16):
    return drgg.lib.grouped_gemm_fwd(X, W, offs, E, M, N, K, dt, 1, Y, None, 0, None)


def test_fwd_argument_checks(drgg):
    assert fwd(drgg, E=0) == 1
    assert fwd(drgg, E=1025) == 1
    assert fwd(drgg, dt=7) == 1
    assert fwd(drgg, W=0) == 1
    assert fwd(drgg, X=0) == 1
    assert fwd(drgg, M=-1) == 2
    assert fwd(drgg, N=4) == 2
    assert fwd(drgg, N=12) == 3
    assert fwd(drgg, K=20) == 3
    assert fwd(drgg, X=A16 + 2) == 3
    assert fwd(drgg, offs=A16 + 2) == 3
    assert fwd(drgg, K=2 ** 22 + 8) == 2          # per-lane tile offsets must stay below 2^31
    assert fwd(drgg, M=2 ** 31) == 2


def batched(drgg, op, **kw):
    """A batched call with fake device pointers whose arguments are invalid
    (valid ones would reach the GPU)."""
    f = dict(B=4, T=64, N=64, K=64, a_row=64, a_batch=64 * 64, b_row=64, b_batch=64 * 64,
             o_row=64, o_batch=64 * 64)
    ptr = {k: kw.pop(k) for k in ("X", "W", "Y") if k in kw}
    f.update(kw)
    b = drgg.Batched(**f)
    X, W, Y = ptr.get("X", A16), ptr.get("W", A16), ptr.get("Y", A16)
    lib = drgg.lib
    if op == "fwd":
        return lib.batched_gemm_fwd(X, W, ctypes.byref(b), 1, Y, None)
    if op == "dgrad":
        return lib.batched_gemm_dgrad(X, W, ctypes.byref(b), 1, Y, None, 0, None)
    return lib.batched_gemm_wgrad(X, W, ctypes.byref(b), 1, 1, Y, None, 0, None)


def test_batched_argument_checks(drgg):
    for op in ("fwd", "dgrad", "wgrad"):
        assert batched(drgg, op, B=0) == 1
        assert batched(drgg, op, B=1025) == 1
        assert batched(drgg, op, T=-1) == 2
        assert batched(drgg, op, N=4) == 2
        assert batched(drgg, op, a_row=60) == 2          # a row longer than its stride
        assert batched(drgg, op, a_row=68) == 3          # stride not a multiple of 8
        assert batched(drgg, op, a_batch=12) == 3
        assert batched(drgg, op, a_row=2 ** 22 + 8) == 2
        assert batched(drgg, op, a_batch=2 ** 61) == 4   # last element beyond 2^62
        assert batched(drgg, op, B=2 ** 10, T=2 ** 22) == 2   # B*T beyond int32
        assert batched(drgg, op, X=0) == 1
    assert drgg.lib.batched_gemm_fwd(A16, A16, None, 1, A16, None) == 1
    assert batched(drgg, "wgrad", b_row=32) == 2
    assert batched(drgg, "wgrad", b_batch=4) == 3
    # outputs whose rows would overlap: neither stacked nor interleaved batches
    assert batched(drgg, "fwd", o_row=64, o_batch=64 * 32) == 2
    assert batched(drgg, "fwd", o_row=128, o_batch=64) == 2
    assert batched(drgg, "dgrad", o_row=64, o_batch=0) == 2
    # a strided output layout that is valid passes the checks (and fails on the null X)
    assert batched(drgg, "fwd", o_row=256, o_batch=64, X=0) == 1


def test_wgrad_workspace_checks(drgg):
    lib = drgg.lib
    # deterministic: needs partial slots when experts may be cut into chunks
    need = drgg.workspace_size(drgg.OP_WGRAD, 2, 100000, 256, 256, drgg.FP32, True)
    assert need > 0
    assert lib.grouped_gemm_wgrad(A16, A16, A16, 2, 100000, 256, 256, 1, 1, A16, None, 0, None) == 5
    assert lib.grouped_gemm_wgrad(A16, A16, A16, 2, 100000, 256, 256, 1, 1, A16, A16, need - 1, None) == 5
    assert lib.grouped_gemm_wgrad(A16, A16, A16, 2, 100000, 256, 256, 1, 1, A16, A16 + 8, need, None) == 3
    assert lib.grouped_gemm_wgrad(A16, A16, 0, 2, 100000, 256, 256, 1, 1, A16, A16, need, None) == 1


def test_router_argument_checks(drgg):
    r = drgg.lib.router_gemm_fp32_bf16x3
    assert r(0, A16, 16, 16, 16, A16, None) == 1
    assert r(A16, A16, -1, 16, 16, A16, None) == 2
    assert r(A16, A16, 16, 16, 12, A16, None) == 3
    assert r(A16, A16, 16, 16, 16, A16 + 4, None) == 3
    assert r(A16, A16, 16, 10, 16, A16, None) == 3          # N must be a multiple of 4
    assert r(A16, A16, 16, 16, 2 ** 22 + 8, A16, None) == 2
    assert r(A16, A16, 16, 2 ** 22 + 4, 16, A16, None) == 2   # output offsets stay below 2^31
    assert r(A16, A16, 2 ** 31, 16, 16, A16, None) == 2
    assert r(A16, A16, 2 ** 31 - 1, 16, 2 ** 31 - 8, A16, None) == 2


def test_router_sliced_argument_checks_and_split_rule(drgg):
    r = drgg.lib.router_gemm_fp32_bf16x3_ws
    ws_status = {int(s) for s in range(0, 12) if "workspace" in drgg.status_string(s)}
    assert r(0, A16, 16, 256, 16, A16, None, 0, None) == 1
    assert r(A16, A16, 16, 256, 12, A16, None, 0, None) == 3
    assert r(A16, A16, 16, 256, 2 ** 22 + 8, A16, None, 0, None) == 2
    assert r(A16, A16, 2048, 256, 4096, A16, None, 0, None) in ws_status      # 7 slices need 14 MiB
    assert r(A16, A16, 2048, 256, 4096, A16, A16 + 4, 7 * 2048 * 256 * 4, None) == 3
    # the program: single pass (ks = 0) once its 128x128 tiles fill 256
    # workgroups; else slices so that ceil(M/256) * ceil(N/256) * ks reaches
    # 256, at most 8, none shorter than 256 values, whole 32-value pairs
    assert drgg.router_split(16384, 256, 4096) == (0, 4096)
    assert drgg.router_split(65536, 256, 4096) == (0, 4096)
    assert drgg.router_split(16, 256, 2 ** 21 + 8) == (0, 2 ** 21 + 8)
    assert drgg.router_split(8192, 256, 4096) == (8, 512)
    assert drgg.router_split(2048, 256, 4096) == (8, 512)
    assert drgg.router_split(300, 256, 520) == (2, 288)
    assert drgg.router_split(128, 128, 64) == (1, 64)
    assert drgg.router_workspace_size(2048, 256, 4096) == 7 * 2048 * 256 * 4
    assert drgg.router_workspace_size(16384, 256, 4096) == 0
    rng = np.random.default_rng(3)
    for _ in range(300):
        M, N, K = int(rng.integers(1, 1 << 17)), 4 * int(rng.integers(1, 300)), 8 * int(rng.integers(1, 2048))
        ks, kq = drgg.router_split(M, N, K)
        if ks == 0:
            assert kq == K and -(-M // 128) * -(-N // 128) >= 256
            continue
        assert -(-M // 128) * -(-N // 128) < 256
        assert 1 <= ks <= 8 and kq % 32 == 0 and (ks - 1) * kq < K <= ks * kq
        assert ks == 1 or kq >= 256


def test_knob_checks(drgg):
    assert drgg.lib.drgg_set_knob(99, 1) == 1
    assert drgg.lib.drgg_set_knob(drgg.KNOB_TILE, 42) == 1
    assert drgg.lib.drgg_set_knob(drgg.KNOB_TILE, 0) == 0
    for knob in (drgg.KNOB_CHECK_OFFSETS, drgg.KNOB_CHECK_WORKSPACE):
        assert drgg.lib.drgg_set_knob(knob, 1) == 0
        assert drgg.lib.drgg_set_knob(knob, 0) == 0


# ---- the tail-split rule ---------------------------------------------------------

def test_tailsplit_units_pages_tuples(drgg):
    """flashinfer PR #7516, #7632 commit body: the row M 6889, N 12288 has
    27 x 48 = 1296 tiles of 256 x 256 on SM pairs; on 148 SMs (74 pairs) the
    38-tile tail does not fit as 76 half units, so every tile stays whole; on
    152 SMs (76 pairs) the 4-tile tail becomes 8 half units."""
    def units(m, n, sm_count):
        return drgg.tailsplit_units(-(-m // 256) * -(-n // 256), sm_count // 2)
    assert units(6889, 12288, 148) == (1296, 1296, 1296, 1)
    assert units(6889, 12288, 152) == (1296, 1300, 1292, 2)


def test_tailsplit_units_closed_form(drgg):
    rng = np.random.default_rng(3)
    for _ in range(500):
        tiles, workers = int(rng.integers(0, 5000)), int(rng.integers(1, 600))
        t, units, full, split = drgg.tailsplit_units(tiles, workers)
        tail = tiles % workers
        assert t == tiles
        if tail and 2 * tail <= workers:
            # the full waves whole, the tail in halves: one more wave of units
            assert (units, full, split) == (tiles + tail, tiles - tail, 2)
            assert (units - full) <= workers
        else:
            assert (units, full, split) == (tiles, tiles, 1)
    assert drgg.tailsplit_units(256, 256) == (256, 256, 256, 1)      # no tail
    assert drgg.tailsplit_units(384, 256) == (384, 512, 256, 2)      # gate_up: 128 tail tiles in halves
    assert drgg.tailsplit_units(0, 256) == (0, 0, 0, 1)
    with pytest.raises(drgg.DrggError):
        drgg.tailsplit_units(10, 0)


# ---- planner -------------------------------------------------------------------

WORKLOADS = {
    "gate_up": (8, 131072, 1536, 2048),
    "down": (32, 131072, 2048, 768),
    "square": (1, 16384, 4096, 4096),
    "dense48": (1, 16384, 48, 4096),
    "dense1024": (1, 16384, 1024, 4096),
    "tiny": (4, 512, 512, 256),
}


def test_chunk_rule_values(drgg):
    cm = {k: drgg.plan(drgg.OP_WGRAD, *v, drgg.FP32, True)["chunk_max"] for k, v in WORKLOADS.items()}
    assert cm["gate_up"] == 12288 and drgg.wgrad_chunking(16384, cm["gate_up"]) == (8192, 2)
    # down: the balanced expert (4096 tokens) stays whole, so the long experts
    # are cut into chunks of at least one reference CU's share (131072 * 24 / 256)
    assert cm["down"] == 12288 and drgg.wgrad_chunking(42987, cm["down"]) == (10752, 4)
    assert cm["square"] == 16384 and drgg.wgrad_chunking(16384, cm["square"]) == (16384, 1)
    assert drgg.wgrad_chunking(128, cm["tiny"]) == (128, 1)
    # skinny dense: 16 equal chunks, 16 tiles x 16 chunks = one full wave of 256 items
    for n in (48, 64):
        c = drgg.plan(drgg.OP_WGRAD, 1, 16384, n, 4096, drgg.FP32, True)["chunk_max"]
        assert c == 1024 and drgg.wgrad_chunking(16384, c) == (1024, 16)
    for n, want in ((512, 2048), (1024, 4096)):
        assert drgg.plan(drgg.OP_WGRAD, 1, 16384, n, 4096, drgg.FP32, True)["chunk_max"] == want


def test_chunk_rule_share_clamp(drgg):
    """Whenever the rule leaves a balanced expert (ceil(M/E) tokens) whole,
    its chunk length is at least one reference CU's share of the token-tile
    work, ceil(M * P0 / 256) rounded up to 64; when it cuts the balanced
    expert, the chunk count it picked is kept."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        E = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
        M = int(rng.integers(1, 1 << 18))
        N = int(rng.choice([48, 64, 512, 768, 1536, 2048, 4096]))
        K = int(rng.choice([256, 768, 1024, 2048, 4096]))
        cm = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True)["chunk_max"]
        p0 = -(-N // 256) * -(-K // 256)
        share = -(-(-(-M * p0 // 256)) // 64) * 64
        tb = -(-M // E)
        assert cm % 64 == 0 and cm >= 512
        if drgg.wgrad_chunking(tb, cm)[1] <= 1:
            assert cm >= share, (E, M, N, K, cm, share)


@pytest.mark.parametrize("chunk_max", [512, 1152, 6144, 12288, 16384])
def test_chunking_properties(drgg, chunk_max):
    for T in list(range(0, 300)) + list(np.random.default_rng(1).integers(1, 200000, 300)):
        T = int(T)
        ln, n = drgg.wgrad_chunking(T, chunk_max)
        if T == 0:
            assert (ln, n) == (0, 0)
            continue
        assert ln % 64 == 0 and ln > 0
        assert n * ln >= T and (n - 1) * ln < T                  # chunks tile [0, T)
        assert n <= -(-T // chunk_max)                            # no more than ceil(T/chunk_max)
        assert ln <= -(-chunk_max // 64) * 64 or n == 1
        if T <= chunk_max:
            assert n == 1


ARITH = ("tile_m", "tile_n", "tile_k", "mfma_m", "mfma_n", "mfma_k", "chunk_max", "max_partials",
         "workspace_bytes")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_det_plan_arithmetic_does_not_depend_on_cu_count(drgg, name):
    """Only the persistent grid may follow the CU count; the tile, MFMA shape,
    chunk rule and workspace are fixed by the problem."""
    for op in (drgg.OP_FWD, drgg.OP_DGRAD, drgg.OP_WGRAD):
        plans = [drgg.plan(op, *WORKLOADS[name], drgg.BF16, True, cu) for cu in (1, 64, 80, 256, 304)]
        assert all({k: p[k] for k in ARITH} == {k: plans[0][k] for k in ARITH} for p in plans)
        assert plans[0]["grid"] <= plans[-1]["grid"]


def _distributions(E, M, rng):
    yield np.full(E, M // E) + (np.arange(E) < M % E)            # balanced
    c = np.zeros(E, dtype=np.int64); c[0] = M; yield c            # all on one expert
    c = np.zeros(E, dtype=np.int64); c[-1] = M; yield c
    for _ in range(20):
        p = rng.dirichlet(np.full(E, 0.3))
        yield rng.multinomial(M, p)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_grid_and_slot_bounds_cover_every_distribution(drgg, name):
    E, M, N, K = WORKLOADS[name]
    rng = np.random.default_rng(7)
    for tile in (0, 1, 2, 3, 4, 5):
        drgg.set_knob(drgg.KNOB_TILE, tile)
        try:
            pw = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True)
            pf = drgg.plan(drgg.OP_FWD, E, M, N, K, drgg.FP32, True)
            pd = drgg.plan(drgg.OP_DGRAD, E, M, N, K, drgg.FP32, True)
        finally:
            drgg.set_knob(drgg.KNOB_TILE, 0)
        P = -(-N // pw["tile_m"]) * -(-K // pw["tile_n"])
        bound_w = P * (M // pw["chunk_max"] + E)
        for counts in _distributions(E, M, rng):
            assert counts.sum() == M
            chunks = np.array([drgg.wgrad_chunking(int(t), pw["chunk_max"])[1] for t in counts])
            assert P * chunks.sum() <= bound_w                  # the grid's cap is a true bound
            assert chunks[chunks > 1].sum() <= pw["max_partials"]
            for p, cols in ((pf, N), (pd, K)):
                items = sum(-(-int(t) // p["tile_m"]) for t in counts) * -(-cols // p["tile_n"])
                assert items <= (M // p["tile_m"] + E) * -(-cols // p["tile_n"])
        for p in (pw, pf, pd):
            assert 1 <= p["grid"] <= 256 * 2


def test_nondet_plan_uses_the_cu_count_and_unit(drgg):
    drgg.set_knob(drgg.KNOB_NONDET, 1)   # the split program
    try:
        p = drgg.plan(drgg.OP_WGRAD, 32, 131072, 2048, 768, drgg.FP32, False, 256)
        assert p["grid"] == 256 and p["unit"] == 512            # one 256x256 workgroup per CU
        P = (2048 // 256) * (768 // 256)
        assert p["workspace_bytes"] >= 32 * P * 256 * 256 * 4 + 32 * P * 4
        assert drgg.plan(drgg.OP_WGRAD, 32, 131072, 2048, 768, drgg.FP32, False, 80)["grid"] == 80
    finally:
        drgg.set_knob(drgg.KNOB_NONDET, 0)


def test_nondet_routes_to_the_det_program_by_default(drgg):
    # the default route runs the deterministic program: its plan and
    # workspace; the split program only with the knob
    for E, M, N, K in ((32, 131072, 2048, 768), (8, 131072, 1536, 2048), (1, 16384, 48, 4096)):
        det = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True, 256)
        nd = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, False, 256)
        assert nd == det
        assert drgg.workspace_size(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, False) == \
            drgg.workspace_size(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True)
        drgg.set_knob(drgg.KNOB_NONDET, 1)
        try:
            assert drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, False, 256)["unit"] == 512
        finally:
            drgg.set_knob(drgg.KNOB_NONDET, 0)
    drgg.set_knob(drgg.KNOB_GRID, 7)
    try:
        assert drgg.plan(drgg.OP_WGRAD, 32, 131072, 2048, 768, drgg.FP32, False, 256)["grid"] == 7
    finally:
        drgg.set_knob(drgg.KNOB_GRID, 0)


# ---- the deterministic weight gradient's tail-only plan ----------------------------

def _offs(counts):
    import synth
    return synth.offsets_from_counts(np.asarray(counts))


def test_tail_plan_choices(drgg):
    """The plan the kernel picks for the measured workloads: balanced gate_up
    runs 4 of its 6 row bands as whole tiles (256 whole tiles, one full wave
    on 256 reference workgroups, and 128 tail tiles in 2 chunks); the
    Zipf-routed down workload, the dense and the square shapes keep the
    all-split plan."""
    import synth
    tail, row0 = drgg.wgrad_tail_plan(_offs(np.full(8, 16384)), 1536, 2048)
    assert tail and row0.tolist() == [1024] * 8
    tail, row0 = drgg.wgrad_tail_plan(_offs(synth.zipf_counts(4004, 131072, 32, 2)), 2048, 768)
    assert not tail and not row0.any()
    for n in (48, 64, 512, 1024, 4096):
        assert drgg.wgrad_tail_plan(_offs([16384]), n, 4096)[0] is False
    tail, row0 = drgg.wgrad_tail_plan(_offs(np.full(32, 768)), 768, 1024)
    assert tail and row0.tolist() == [512] * 32


def test_tail_plan_properties(drgg):
    rng = np.random.default_rng(11)
    for _ in range(60):
        E = int(rng.choice([1, 2, 4, 8, 16, 32]))
        M = int(rng.choice([4096, 32768, 131072]))
        N = int(rng.choice([64, 512, 768, 1536, 2048]))
        K = int(rng.choice([256, 768, 1024, 2048]))
        w = rng.lognormal(0, float(rng.choice([0.0, 0.1, 0.35, 1.0])), E)
        counts = rng.multinomial(M, w / w.sum())
        tail, row0 = drgg.wgrad_tail_plan(_offs(counts), N, K)
        cm = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True)["chunk_max"]
        for e in range(E):
            chunks = drgg.wgrad_chunking(int(counts[e]), cm)[1]
            if not tail or chunks <= 1:
                assert row0[e] == 0
            else:
                assert row0[e] % 256 == 0 or row0[e] == N
                assert 0 <= row0[e] <= N
        if tail:
            assert row0.any()
    # more experts than the tail-only walk has positions for: always all-split
    assert drgg.wgrad_tail_plan(_offs(np.full(600, 2048)), 4096, 4096)[0] is False
    assert drgg.wgrad_tail_plan(_offs(np.full(512, 2048)), 4096, 4096)[0] in (True, False)
    with pytest.raises(drgg.DrggError):
        drgg.wgrad_tail_plan([0], 64, 64)


# ---- the split program's tail: whole on the least-loaded workgroups or chunked -----

# E=64 skewed experts, 4096 tokens, N=1536, K=256: the tail (18 tiles of the
# two longest experts) fits whole on the least-loaded workgroups
SLACK_COUNTS = [30, 6, 0, 96, 126, 18, 28, 16, 288, 1, 2, 72, 7, 1, 1, 332, 25, 0, 7, 871, 12, 8, 23, 14, 1, 16, 15, 9, 2, 2, 5, 4,
              0, 59, 791, 0, 48, 1, 7, 5, 18, 4, 138, 53, 17, 4, 7, 9, 5, 1, 0, 12, 0, 104, 22, 626, 4, 30, 13, 2, 8, 63, 1, 6]
SLACK_CASE = (SLACK_COUNTS, 1536, 256)


def test_split_plan_decisions(drgg):
    import synth
    slack, tail = drgg.wgrad_split_plan(_offs(np.full(8, 16384)), 1536, 2048)
    assert (slack, tail) == (False, 128)          # balanced: no workgroup has room for a whole tail tile
    slack, tail = drgg.wgrad_split_plan(_offs(synth.zipf_counts(4004, 131072, 32, 2)), 2048, 768)
    assert not slack and tail > 0
    assert drgg.wgrad_split_plan(_offs([16384]), 512, 4096) == (False, 32)
    counts, n, k = SLACK_CASE
    assert drgg.wgrad_split_plan(_offs(counts), n, k, banded=True) == (True, 18, True)
    # more tail tiles than workgroups, or a grid beyond the ranking's limit: chunked
    assert drgg.wgrad_split_plan(_offs(counts), n, k, grid=1)[0] is False
    assert drgg.wgrad_split_plan(_offs(counts), n, k, grid=2000)[0] is False
    # a few idle workgroups: the all-split walk is faster than placing whole
    # tail tiles, even where they would fit
    small = [498, 482, 432, 689, 505, 699, 350, 441]
    assert drgg.wgrad_split_plan(_offs(small), 256, 256, banded=True) == (False, 2, False)
    # balanced gate_up: the banded walk with its tail in chunks
    assert drgg.wgrad_split_plan(_offs(np.full(8, 16384)), 1536, 2048, banded=True) == (False, 128, True)


def test_split_plan_slack_only_with_room(drgg):
    """Slack placement is taken only with at most one tail tile per
    workgroup, and only on the banded walk."""
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(600):
        E = int(rng.choice([8, 16, 32, 64]))
        M = int(rng.choice([4096, 8192, 16384]))
        N, K = int(rng.choice([256, 512, 768, 1536])), int(rng.choice([256, 512]))
        w = rng.lognormal(0, 2.0, E)
        counts = rng.multinomial(M, w / w.sum())
        slack, tail, banded = drgg.wgrad_split_plan(_offs(counts), N, K, banded=True)
        if slack:
            checked += 1
            assert banded and 0 < tail <= 256
    assert checked >= 5


def test_plans_give_experts_without_tokens_no_items(drgg):
    """An expert without tokens has no work items in either plan (a whole
    tile of zero tokens would be a tile with no reduction steps)."""
    for pos in (0, 15, 31):
        counts = [768] * 32
        counts[pos] = 0
        assert drgg.wgrad_tail_plan(_offs(counts), 768, 1024)[0] is True
        # 4 tail tiles (one 256-row band of 4 tiles) for each of the 31 experts with tokens
        assert drgg.wgrad_split_plan(_offs(counts), 768, 1024, banded=True) == (False, 31 * 4, True)


def test_dgrad_transposes_w_only_from_3072_tokens_per_expert(drgg):
    """The data gradient's W^T workspace (and with it the transpose) is
    planned only when the experts average at least 3072 tokens; the test
    knob forces it at any size."""
    cases = [((4, 512, 512, 256), 0), ((8, 16384, 1024, 1024), 0), ((3, 9215, 64, 64), 0),
             ((3, 9216, 64, 64), 3 * 64 * 64 * 2), ((8, 131072, 1536, 2048), 8 * 1536 * 2048 * 2),
             ((1, 16384, 4096, 4096), 4096 * 4096 * 2), ((5, 20000, 72, 136), 5 * 72 * 136 * 2)]
    for (E, M, N, K), want in cases:
        got = drgg.workspace_size(drgg.OP_DGRAD, E, M, N, K, drgg.BF16, True)
        assert got == -(-want // 256) * 256, (E, M, N, K, got)
    drgg.set_knob(drgg.KNOB_DGRAD_WT, 1)
    try:
        assert drgg.workspace_size(drgg.OP_DGRAD, 4, 512, 512, 256, drgg.BF16, True) == 4 * 512 * 256 * 2
    finally:
        drgg.set_knob(drgg.KNOB_DGRAD_WT, 0)


def test_small_forward_and_data_gradient_take_128_tiles(drgg):
    """A forward or data gradient whose 256x256 tiles could fill at most half
    of 256 CUs (ceil(M/256) * ceil(cols/256) <= 128, cols = N forward, K data
    gradient) is planned on 128x128 tiles; larger calls and every weight
    gradient keep their tiles."""
    def tile(op, E, M, N, K):
        p = drgg.plan(op, E, M, N, K)
        return p["tile_m"], p["tile_n"]
    F, D, W = drgg.OP_FWD, drgg.OP_DGRAD, drgg.OP_WGRAD
    assert tile(F, 4, 512, 512, 256) == (128, 128)            # 2 x 2 tiles
    assert tile(D, 4, 512, 512, 256) == (128, 128)
    assert tile(F, 1, 32768, 256, 4096) == (128, 128)         # 128 x 1: exactly half
    assert tile(F, 1, 32769, 256, 4096) == (256, 256)         # 129 x 1
    assert tile(D, 1, 32769, 4096, 256) == (256, 256)         # data gradient counts K's columns
    assert tile(D, 1, 32768, 4096, 256) == (128, 128)
    assert tile(F, 1, 32768, 4096, 256) == (256, 256)         # 128 x 16
    assert tile(F, 8, 131072, 1536, 2048) == (256, 256)
    assert tile(D, 32, 8192, 2048, 768) == (128, 128)         # 32 x 3
    assert tile(F, 32, 8192, 2048, 768) == (256, 256)         # 32 x 8
    assert tile(W, 8, 131072, 1536, 2048) == (256, 256)       # experts cut into chunks, many items
    assert tile(F, 64, 5515, 4096, 1024) == (128, 128)        # lo 352, but under 128 tokens per group
    assert tile(F, 64, 8192, 4096, 1024) == (256, 256)        # 128 tokens per group on average
    assert tile(W, 1, 16384, 48, 4096) == (64, 256)


def test_one_to_one_and_a_half_waves_take_128x256_tiles(drgg):
    """Between one and one and a half waves of 256x256 tiles (more than 256
    even with every group's rows packed, at most 384 even with one partial
    row tile per group), a forward or a data gradient on W^T runs 128x256
    tiles; a data gradient that reads W transposed keeps 256x256."""
    def tile(op, E, M, N, K):
        p = drgg.plan(op, E, M, N, K)
        return p["tile_m"], p["tile_n"]
    F, D = drgg.OP_FWD, drgg.OP_DGRAD
    assert tile(F, 8, 12288, 1536, 2048) == (128, 256)        # 288 .. 330 tiles
    assert tile(F, 1, 5120, 4096, 4096) == (128, 256)         # 320
    assert tile(D, 1, 5120, 4096, 4096) == (128, 256)         # W^T: 5120 tokens per expert
    assert tile(D, 1, 6144, 4096, 4096) == (128, 256)         # 384
    assert tile(F, 1, 6400, 4096, 4096) == (256, 256)         # 400
    assert tile(F, 1, 4096, 4096, 4096) == (256, 256)         # 256: one full wave
    assert tile(D, 8, 12288, 2048, 1536) == (256, 256)        # 1536 tokens per expert: W read transposed
    assert tile(D, 8, 12288, 1536, 2048) == (256, 256)        # 384 packed, up to 440
    assert tile(F, 64, 16384 + 64, 1536, 2048) == (256, 256)  # 390 packed: beyond the band
    assert tile(F, 40, 11264, 1536, 2048) == (256, 256)       # 264 packed, up to 498 with partial tiles
    drgg.set_knob(drgg.KNOB_DGRAD_WT, 1)
    try:
        assert tile(D, 8, 12288, 2048, 1536) == (128, 256)    # on W^T: 288 .. 330 tiles
    finally:
        drgg.set_knob(drgg.KNOB_DGRAD_WT, 0)


def test_wgrad_without_chunks_needs_no_workspace(drgg):
    """A deterministic weight gradient whose experts can never be cut into
    chunks (M at most chunk_max) writes no partials and runs no fold: its
    workspace size is 0, so the call takes a null workspace."""
    for E, M, N, K in ((4, 512, 512, 256), (1, 512, 2048, 2048), (8, 256, 1024, 1024)):
        p = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True)
        assert p["chunk_max"] >= M and p["max_partials"] == 0 and p["workspace_bytes"] == 0, (E, M, N, K, p)
        assert drgg.workspace_size(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True) == 0
    p = drgg.plan(drgg.OP_WGRAD, 8, 1024, 1024, 1024, drgg.FP32, True)
    assert p["chunk_max"] < 1024 and p["max_partials"] > 0 and p["workspace_bytes"] > 0


def test_weight_gradients_with_few_items_take_smaller_tiles(drgg):
    """A deterministic weight gradient none of whose experts can be cut into
    chunks (M <= chunk_max) spreads its E * ceil(N/256) * ceil(K/256) output
    tiles: at most 32 take 128x128, at most 128 take 128x256 (rows over N);
    a chunked one with at most 128 items (bound U) takes 128x128; the split
    program keeps 256x256."""
    def tile(E, M, N, K, det=True):
        p = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, det)
        return p["tile_m"], p["tile_n"]
    assert tile(4, 512, 512, 256) == (128, 128)       # 8 tiles
    assert tile(1, 384, 768, 768) == (128, 128)       # 9
    assert tile(2, 512, 1024, 512) == (128, 128)      # 16
    assert tile(1, 512, 2048, 2048) == (128, 256)     # 64
    assert tile(8, 512, 1024, 1024) == (128, 256)     # 128
    assert tile(64, 512, 512, 512) == (256, 256)      # 256
    assert tile(1, 4096, 4096, 4096) == (256, 256)    # 256
    # chunked: U = ceil(N/256) * ceil(K/256) * (E + M // chunk_max) items at most
    assert tile(4, 1024, 512, 512) == (128, 128)      # U = 4 * (4 + 2) = 24
    assert tile(1, 8192, 256, 1024) == (128, 128)     # U = 4 * (1 + 16) = 68
    assert tile(4, 8192, 512, 512) == (128, 128)      # U = 4 * (4 + 16) = 80
    assert tile(1, 16384, 256, 1024) == (256, 256)    # U = 4 * (1 + 32) = 132
    assert tile(2, 4096, 1024, 1024) == (256, 256)    # U = 16 * (2 + 8) = 160
    drgg.set_knob(drgg.KNOB_NONDET, 1)
    try:
        assert tile(4, 512, 512, 256, det=False) == (256, 256)
    finally:
        drgg.set_knob(drgg.KNOB_NONDET, 0)


def test_measured_workloads_tiles(drgg):
    """The tiles the planner gives the measured workloads (a change here
    changes what bench.py measures)."""
    def tile(op, E, M, N, K):
        p = drgg.plan(op, E, M, N, K)
        return p["tile_m"], p["tile_n"]
    F, D, W = drgg.OP_FWD, drgg.OP_DGRAD, drgg.OP_WGRAD
    # tiny MoE: E=4, 512 tokens, N=512, K=256
    assert [tile(op, 4, 512, 512, 256) for op in (F, D, W)] == [(128, 128)] * 3
    # dense projection weight gradients, 16384 tokens, K=4096
    assert tile(W, 1, 16384, 48, 4096) == (64, 256)
    assert tile(W, 1, 16384, 64, 4096) == (64, 256)
    assert tile(W, 1, 16384, 512, 4096) == (256, 256)
    assert tile(W, 1, 16384, 1024, 4096) == (256, 256)
    # MoE gate_up (the headline), Zipf down weight gradient, square dense
    assert [tile(op, 8, 131072, 1536, 2048) for op in (F, D, W)] == [(256, 256)] * 3
    assert tile(W, 32, 131072, 2048, 768) == (256, 256)
    assert [tile(op, 1, 16384, 4096, 4096) for op in (F, D, W)] == [(256, 256)] * 3
