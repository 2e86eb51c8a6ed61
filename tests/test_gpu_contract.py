"""GPU tests of the variants' contracts and of the boundary's behaviour.

* deterministic variant: bitwise identical over 20 runs, across output tile
  shapes, across the order the work items are walked in, on streams
  restricted to 16, 64 and 128 of the CUs (fewer CUs, same bits), and next to
  a kernel that holds 8, 16 or 32 CUs;
* non-deterministic variant: the tile sums and tickets are zero again after
  every call; every stream-K partition (grid sizes from 1 to more workgroups
  than units) matches the oracle;
* the router's BF16x3 split against both oracles;
* edge cases: no tokens, one token per expert, 1024 experts, the smallest N
  and K, all tokens on one expert;
* error paths: misaligned pointers, a short workspace, bad dtypes; the
  debug checks of the group offsets and of the split program's workspace;
* a split-program call on a stream other than the current one.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.test_gpu_parity import dev_inputs, ragged_problem, run_program

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def drgg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_ragged_grouped_amd as d
    # non-deterministic calls in these tests exercise the split program
    # (by default the library routes them to the deterministic one)
    d.set_knob(d.KNOB_NONDET, 1)
    return d


def bits(t):
    return parity.from_dev(t).view(np.uint16 if t.dtype == torch.bfloat16 else np.uint32).copy()


DET_CASE = (301, 4, 3000, 264, 520, (1,))   # multi-chunk wgrad, ragged, an empty expert


@pytest.mark.parametrize("program", ["fwd", "dgrad", "wgrad"])
def test_deterministic_20_runs_bitwise(drgg, program):
    prob = ragged_problem(*DET_CASE)
    dv = dev_inputs(prob)
    for out_dtype in (torch.float32, torch.bfloat16):
        ref = bits(run_program(drgg, program, dv, out_dtype, True))
        for i in range(19):
            got = bits(run_program(drgg, program, dv, out_dtype, True))
            assert np.array_equal(got, ref), f"run {i + 2} differs"


def test_nondet_default_route_runs_the_det_program(drgg):
    """With the library's default route a non-deterministic weight gradient
    runs the deterministic program: bitwise the deterministic result."""
    prob = ragged_problem(*DET_CASE)
    dv = dev_inputs(prob)
    for out_dtype in (torch.float32, torch.bfloat16):
        det = bits(run_program(drgg, "wgrad", dv, out_dtype, True))
        drgg.set_knob(drgg.KNOB_NONDET, 0)
        try:
            nd = bits(run_program(drgg, "wgrad", dv, out_dtype, False))
        finally:
            drgg.set_knob(drgg.KNOB_NONDET, 1)
        assert np.array_equal(nd, det)


@pytest.mark.parametrize("program", ["fwd", "dgrad", "wgrad"])
def test_deterministic_across_tile_shapes_and_walk_order(drgg, program):
    """The tile shape and the order of the work items are free choices of the
    deterministic variant: they must not change a bit."""
    prob = ragged_problem(*DET_CASE)
    dv = dev_inputs(prob)
    tiles = [1, 2, 3, 4] + ([5] if program == "wgrad" else [])
    for out_dtype in (torch.float32, torch.bfloat16):
        ref = bits(run_program(drgg, program, dv, out_dtype, True))
        try:
            for tile in tiles:
                for rev in (0, 1):
                    drgg.set_knob(drgg.KNOB_TILE, tile)
                    drgg.set_knob(drgg.KNOB_REVERSE, rev)
                    got = bits(run_program(drgg, program, dv, out_dtype, True))
                    assert np.array_equal(got, ref), f"tile {tile} reverse {rev} changed the bits"
        finally:
            drgg.set_knob(drgg.KNOB_TILE, 0)
            drgg.set_knob(drgg.KNOB_REVERSE, 0)
    parity.compare(prob, program, parity.from_dev(run_program(drgg, program, dv, torch.float32, True)), False)


@pytest.mark.parametrize("program", ["fwd", "dgrad", "wgrad"])
def test_deterministic_across_grid_sizes(drgg, program):
    """The number of workgroups (what the CU count sets) decides which
    workgroup takes which work item, and for the weight gradient the snake
    walk over the longest-first order: it must not change a bit.  Many
    experts of very different lengths, a few equal, some empty."""
    counts = np.array([900, 40, 2500, 0, 40, 1300, 700, 3100, 40, 0, 260, 1800, 900, 120, 5000, 600],
                      dtype=np.int64)
    prob = synth.make_problem("ragged_grid", 305, counts, N=264, K=520, w_std=0.02)
    dv = dev_inputs(prob)
    ref = bits(run_program(drgg, program, dv, torch.float32, True))
    try:
        for grid in (1, 3, 17, 64, 255):
            drgg.set_knob(drgg.KNOB_GRID, grid)
            got = bits(run_program(drgg, program, dv, torch.float32, True))
            assert np.array_equal(got, ref), f"grid {grid} changed the bits"
    finally:
        drgg.set_knob(drgg.KNOB_GRID, 0)
    parity.compare(prob, program, parity.from_dev(run_program(drgg, program, dv, torch.float32, True)), False,
                   what=f"ragged grid {program}")


def _hip():
    # torch's own HIP runtime: torch loads it under this name, so the dynamic
    # loader returns the copy already in the process
    return ctypes.CDLL("libamdhip64.so")


def _cu_mask_stream(hip, n):
    """A stream restricted to the CUs of the first n bits of the CU mask.  The
    mask's bits go round the XCDs (bit i on XCD i mod 8), so the first n bits
    leave n/8 CUs on every XCD; a mask that leaves an XCD without CUs is
    refused (the runtime returns hipErrorOutOfMemory for it)."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    words = (ncu + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for cu in range(n):
        mask[cu // 32] |= 1 << (cu % 32)
    stream = ctypes.c_void_p()
    hip.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(stream), ctypes.c_uint32(words), mask)
    if rc != 0:
        hip.hipGetLastError()      # clear the error so that later calls do not report it
        return None, rc
    return stream, 0


FEWER_CU_CASES = [DET_CASE, (306, 3, 4000, 264, 520, (1,))]


@pytest.mark.parametrize("n_cus", [16, 64, 128])
def test_deterministic_on_fewer_cus(drgg, n_cus):
    """Run on a stream whose CU mask enables n_cus of the CUs, with the
    default persistent grid (sized for the whole device, so workgroups queue
    for the CUs left) and with a grid of n_cus workgroups: the deterministic
    results must equal those on the full device."""
    hip = _hip()
    stream, rc = _cu_mask_stream(hip, n_cus)
    if stream is None:
        pytest.skip(f"hipExtStreamCreateWithCUMask({n_cus} CUs) returned {rc}: CU masks unavailable here")
    try:
        ext = torch.cuda.ExternalStream(stream.value)
        for case in FEWER_CU_CASES:
            prob = ragged_problem(*case)
            dv = dev_inputs(prob)
            for program in ("fwd", "dgrad", "wgrad"):
                print(f"fewer CUs: {n_cus} CUs, case {case[0]}, {program}", flush=True)
                ref = bits(run_program(drgg, program, dv, torch.bfloat16, True))
                torch.cuda.synchronize()
                for grid in (0, n_cus):
                    drgg.set_knob(drgg.KNOB_GRID, grid)
                    try:
                        with torch.cuda.stream(ext):
                            out = run_program(drgg, program, dv, torch.bfloat16, True)
                        ext.synchronize()
                    finally:
                        drgg.set_knob(drgg.KNOB_GRID, 0)
                    assert np.array_equal(bits(out), ref), f"{program}: {n_cus} CUs (grid {grid}) changed the bits"
        # the router's sliced program (8 reduction slices here) and its fold
        X, Wr = synth.router_inputs(1024, 256, 2048, cfg_seed=11)
        Xd, Wd = parity.to_dev(X), parity.to_dev(Wr)
        assert drgg.router_split(1024, 256, 2048)[0] == 8
        ref = drgg.router_gemm_fp32_bf16x3(Xd, Wd).view(torch.int32).cpu()
        print(f"fewer CUs: {n_cus} CUs, router", flush=True)
        ws = torch.empty(drgg.router_workspace_size(1024, 256, 2048), dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(ext):
            out = drgg.router_gemm_fp32_bf16x3(Xd, Wd, workspace=ws)
        ext.synchronize()
        assert torch.equal(out.view(torch.int32).cpu(), ref), f"router: {n_cus} CUs changed the bits"
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(stream)


@pytest.mark.parametrize("held", [8, 16, 32])
def test_deterministic_next_to_cu_holder(drgg, held):
    """A kernel on another stream holds `held` CUs while the programs run
    (their persistent workgroups then share the device unevenly): the
    deterministic results must not change."""
    other = torch.cuda.Stream()
    for case in FEWER_CU_CASES:
        prob = ragged_problem(*case)
        dv = dev_inputs(prob)
        for program in ("fwd", "dgrad", "wgrad"):
            ref = bits(run_program(drgg, program, dv, torch.bfloat16, True))
            torch.cuda.synchronize()
            drgg.hold_cus(held, 3000, stream=other)
            out = run_program(drgg, program, dv, torch.bfloat16, True)
            torch.cuda.synchronize()
            assert np.array_equal(bits(out), ref), f"{program}: holding {held} CUs changed the bits"


def _nondet_ws(drgg, prob, out_code):
    n = drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, out_code, False)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("grid", [0, 1, 3, 7, 100, 1000, 5000])
def test_nondet_stream_k_partitions(drgg, grid):
    prob = ragged_problem(311, 3, 2500, 136, 392, (2,))
    dv = dev_inputs(prob)
    drgg.set_knob(drgg.KNOB_GRID, grid)
    try:
        for out_dtype, code in ((torch.float32, drgg.FP32), (torch.bfloat16, drgg.BF16)):
            ws = _nondet_ws(drgg, prob, code)
            out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=out_dtype,
                                          deterministic=False, workspace=ws)
            torch.cuda.synchronize()
            assert int(torch.count_nonzero(ws)) == 0, "tile sums / tickets not cleared"
            parity.compare(prob, "wgrad", parity.from_dev(out), out_dtype == torch.bfloat16,
                           what=f"stream-K grid {grid}")
    finally:
        drgg.set_knob(drgg.KNOB_GRID, 0)


def test_nondet_repeated_calls_keep_workspace_zero(drgg):
    prob = ragged_problem(312, 4, 3000, 256, 256, ())
    dv = dev_inputs(prob)
    ws = _nondet_ws(drgg, prob, drgg.FP32)
    det = parity.from_dev(run_program(drgg, "wgrad", dv, torch.float32, True)).astype(np.float64)
    for _ in range(10):
        out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32,
                                      deterministic=False, workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0
        g = parity.from_dev(out).astype(np.float64)
        assert np.linalg.norm(g - det) <= 1e-6 * np.linalg.norm(det)


def test_nondet_integer_inputs_match_det_bitwise(drgg):
    prob = ragged_problem(313, 4, 3000, 256, 256, (3,), integer=True)
    dv = dev_inputs(prob)
    det = bits(run_program(drgg, "wgrad", dv, torch.float32, True))
    ws = _nondet_ws(drgg, prob, drgg.FP32)
    for grid in (0, 5, 300):
        drgg.set_knob(drgg.KNOB_GRID, grid)
        try:
            out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32,
                                          deterministic=False, workspace=ws)
        finally:
            drgg.set_knob(drgg.KNOB_GRID, 0)
        assert np.array_equal(bits(out), det)


# ---- router ------------------------------------------------------------------

ROUTER_SHAPES = [(300, 256, 520), (128, 128, 64), (1000, 40, 264), (1, 8, 8), (777, 256, 4104), (513, 300, 1032)]


@pytest.mark.parametrize("sliced", [True, False], ids=["sliced", "single_pass"])
@pytest.mark.parametrize("shape", ROUTER_SHAPES)
def test_router_bf16x3(drgg, shape, sliced):
    """Both router programs against the step-by-step emulation and the exact
    product; the sliced program's reduction slices (several of them, the last
    one shorter, on the last two shapes) and masked tile rows and columns."""
    M, N, K = shape
    X, Wr = synth.router_inputs(M, N, K, cfg_seed=7)
    print(f"router {shape} sliced={sliced} split={drgg.router_split(M, N, K)}", flush=True)
    ws = None if sliced else False
    out = parity.from_dev(drgg.router_gemm_fp32_bf16x3(parity.to_dev(X), parity.to_dev(Wr), workspace=ws))
    out = out.astype(np.float64)
    emul = oracle.router_bf16x3(X, Wr)
    exact = oracle.router_exact(X, Wr)
    # against the step-by-step emulation: only the FP32 accumulation order differs
    assert np.linalg.norm(out - emul) <= 1e-6 * np.linalg.norm(emul)
    # against the exact product: the FP32-output tolerance
    kred = np.full(out.size, K)
    ax = np.abs(X).max(axis=1)[:, None] * np.ones((1, N))
    aw = np.ones((M, 1)) * np.abs(Wr).max(axis=1)[None, :]
    parity.check_fp32(out, exact, kred, ax, aw, what=f"router {shape}")


@pytest.mark.parametrize("sliced", [True, False], ids=["sliced", "single_pass"])
def test_router_bf16_representable_inputs_exact(drgg, sliced):
    """Inputs with at most 8 significant bits make lo = 0; with small integers
    every sum is exact too, so the router equals the exact product bit for bit
    (in the sliced program: 4 slices of 256)."""
    rng = np.random.default_rng(5)
    X = rng.integers(-4, 5, size=(256, 1024)).astype(np.float32)
    Wr = rng.integers(-4, 5, size=(256, 1024)).astype(np.float32)
    assert drgg.router_split(256, 256, 1024) == (4, 256)
    out = parity.from_dev(drgg.router_gemm_fp32_bf16x3(parity.to_dev(X), parity.to_dev(Wr),
                                                       workspace=None if sliced else False))
    assert np.array_equal(out, oracle.round_f32(oracle.router_exact(X, Wr)))


def test_router_sliced_is_reproducible_and_checks_its_workspace(drgg):
    """The sliced program gives the same bits on every call (its slices are
    added in a fixed order), with a caller-owned workspace too, and refuses a
    workspace that is too small."""
    X, Wr = synth.router_inputs(2048, 256, 4096, cfg_seed=9)
    Xd, Wd = parity.to_dev(X), parity.to_dev(Wr)
    ks, kq = drgg.router_split(2048, 256, 4096)
    assert ks == 8 and kq == 512
    nbytes = drgg.router_workspace_size(2048, 256, 4096)
    assert nbytes == (ks - 1) * 2048 * 256 * 4
    a = parity.from_dev(drgg.router_gemm_fp32_bf16x3(Xd, Wd))
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")   # stale contents do not matter
    b = parity.from_dev(drgg.router_gemm_fp32_bf16x3(Xd, Wd, workspace=ws))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    with pytest.raises(drgg.DrggError):
        drgg.router_gemm_fp32_bf16x3(Xd, Wd, workspace=ws[: nbytes - 16])


# ---- edge cases --------------------------------------------------------------

def test_no_tokens(drgg):
    E, N, K = 3, 64, 72
    offs = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    X = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    G = torch.zeros((0, N), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((E, N, K), dtype=torch.bfloat16, device="cuda")
    assert drgg.grouped_gemm_fwd(X, W, offs).shape == (0, N)
    assert drgg.grouped_gemm_dgrad(G, W, offs).shape == (0, K)
    for det in (True, False):
        for dt in (torch.float32, torch.bfloat16):
            dW = torch.full((E, N, K), 7.0, dtype=dt, device="cuda")
            drgg.grouped_gemm_wgrad(X, G, offs, out_dtype=dt, deterministic=det, out=dW)
            torch.cuda.synchronize()
            assert not np.any(bits(dW)), "experts without tokens must get +0"


@pytest.mark.parametrize("det", [True, False])
def test_tiny_experts_and_many_groups(drgg, det):
    # 1024 experts, most with 0..3 tokens; smallest N and K
    rng = np.random.default_rng(9)
    counts = rng.integers(0, 4, size=1024)
    prob = synth.make_problem("many", 91, counts, N=8, K=8)
    dv = dev_inputs(prob)
    for program in ("fwd", "dgrad", "wgrad"):
        out = run_program(drgg, program, dv, torch.float32, det)
        torch.cuda.synchronize()
        parity.compare(prob, program, parity.from_dev(out), False, what=f"many {program}")


@pytest.mark.parametrize("det", [True, False])
def test_one_hot_routing_equals_dense_call(drgg, det):
    prob = ragged_problem(321, 4, 1500, 200, 136, (0, 1, 3))   # all tokens on expert 2
    dense = synth.Problem("dense", 1, prob.M, prob.N, prob.K, np.array([0, prob.M], dtype=np.int32),
                          prob.X, prob.W[2:3].copy(), prob.G)
    dv, dd = dev_inputs(prob), dev_inputs(dense)
    for program in ("fwd", "dgrad", "wgrad"):
        g = bits(run_program(drgg, program, dv, torch.float32, True))
        d = bits(run_program(drgg, program, dd, torch.float32, True))
        if program == "wgrad":
            g = g.reshape(4, prob.N, prob.K)
            assert np.array_equal(g[2], d.reshape(prob.N, prob.K))
            assert not np.any(g[[0, 1, 3]])
        else:
            assert np.array_equal(g, d)


# ---- errors ------------------------------------------------------------------

def _raw_call(drgg, program, dv, prob, out, ws=None, det=1, code=None):
    """A call straight through the C ABI (no Python-side checks)."""
    code = drgg.FP32 if code is None else code
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_bytes = ws.numel() if ws is not None else 0
    s = torch.cuda.current_stream().cuda_stream
    f = {"fwd": drgg.lib.grouped_gemm_fwd, "dgrad": drgg.lib.grouped_gemm_dgrad,
         "wgrad": drgg.lib.grouped_gemm_wgrad}[program]
    a, b = {"fwd": ("X", "W"), "dgrad": ("G", "W"), "wgrad": ("X", "G")}[program]
    return f(dv[a].data_ptr(), dv[b].data_ptr(), dv["offs"].data_ptr(), prob.E, prob.M, prob.N, prob.K, code,
             det, out.data_ptr(), ws_ptr, ws_bytes, s)


def test_offsets_debug_check(drgg):
    """With the offsets check on, offsets that do not start at 0, decrease or
    do not end at M are refused with DRGG_ESHAPE and nothing is written;
    valid offsets still run."""
    prob = ragged_problem(332, 4, 900, 64, 72, (2,))
    dv = dev_inputs(prob)
    good = prob.offs.copy()
    bad_sets = []
    b = good.copy(); b[0] = 5; bad_sets.append(b)                      # o[0] != 0
    b = good.copy(); b[2] = b[1] - 1; bad_sets.append(b)               # decreasing
    b = good.copy(); b[-1] = prob.M - 8; bad_sets.append(b)            # o[E] != M
    shapes = {"fwd": (prob.M, prob.N), "dgrad": (prob.M, prob.K), "wgrad": (prob.E, prob.N, prob.K)}
    ws = torch.zeros(drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True),
                     dtype=torch.uint8, device="cuda")
    drgg.set_knob(drgg.KNOB_CHECK_OFFSETS, 1)
    try:
        for program in ("fwd", "dgrad", "wgrad"):
            for bad in bad_sets:
                d = dict(dv, offs=parity.to_dev(bad))
                out = torch.full(shapes[program], 7.0, dtype=torch.float32, device="cuda")
                st = _raw_call(drgg, program, d, prob, out, ws)
                torch.cuda.synchronize()
                assert st == 2, f"{program}: bad offsets {bad.tolist()} gave status {st}"
                assert bool(torch.all(out == 7.0)), f"{program}: a refused call wrote its output"
            out = torch.empty(shapes[program], dtype=torch.float32, device="cuda")
            assert _raw_call(drgg, program, dv, prob, out, ws) == 0
            torch.cuda.synchronize()
            parity.compare(prob, program, parity.from_dev(out), False, what=f"checked offsets {program}")
    finally:
        drgg.set_knob(drgg.KNOB_CHECK_OFFSETS, 0)


def test_split_workspace_debug_check(drgg):
    """With the workspace check on, a split-program call whose workspace
    still holds a deterministic call's partials is refused with
    DRGG_EWORKSPACE; after drgg_workspace_init it runs and leaves the
    workspace zero."""
    prob = ragged_problem(333, 3, 3000, 256, 264, ())
    dv = dev_inputs(prob)
    n_det = drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)
    n_split = drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, False)
    ws = torch.zeros(max(n_det, n_split), dtype=torch.uint8, device="cuda")
    out = torch.empty((prob.E, prob.N, prob.K), dtype=torch.float32, device="cuda")
    assert _raw_call(drgg, "wgrad", dv, prob, out, ws, det=1) == 0     # leaves partials behind
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:n_split])) > 0
    drgg.set_knob(drgg.KNOB_CHECK_WORKSPACE, 1)
    try:
        out.fill_(7.0)
        assert _raw_call(drgg, "wgrad", dv, prob, out, ws, det=0) == 5
        torch.cuda.synchronize()
        assert bool(torch.all(out == 7.0))
        drgg.workspace_init(ws)
        assert _raw_call(drgg, "wgrad", dv, prob, out, ws, det=0) == 0
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0
        parity.compare(prob, "wgrad", parity.from_dev(out), False, what="split after workspace check")
    finally:
        drgg.set_knob(drgg.KNOB_CHECK_WORKSPACE, 0)


def test_split_program_on_another_stream(drgg):
    """The split program with the default workspace on a stream that is not
    the current one: the workspace is allocated and zeroed on that stream and
    the result matches the oracle, twice in a row (the second call reuses the
    buffer, which the first left zero)."""
    prob = ragged_problem(334, 4, 3000, 264, 392, (1,))
    dv = dev_inputs(prob)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32, deterministic=False,
                                      stream=side)
        side.synchronize()
        parity.compare(prob, "wgrad", parity.from_dev(out), False, what="split program on a side stream")

def test_error_paths(drgg):
    prob = ragged_problem(331, 2, 100, 64, 64, ())
    dv = dev_inputs(prob)
    with pytest.raises(TypeError):
        drgg.grouped_gemm_fwd(dv["X"].float(), dv["W"], dv["offs"])
    # a pointer that is not 16-byte aligned: reaches the C ABI, which refuses
    x_off = torch.empty(prob.M * prob.K + 8, dtype=torch.bfloat16, device="cuda")[1:1 + prob.M * prob.K]
    x_off = x_off.view(prob.M, prob.K)
    with pytest.raises(drgg.DrggError) as ei:
        drgg.grouped_gemm_fwd(x_off, dv["W"], dv["offs"])
    assert ei.value.status == 3
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(drgg.DrggError) as ei:
        drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], deterministic=False, workspace=small)
    assert ei.value.status == 5
    # outputs of the wrong shape are refused before anything is launched
    with pytest.raises(ValueError):
        drgg.grouped_gemm_fwd(dv["X"], dv["W"], dv["offs"], out=torch.empty(prob.M - 1, prob.N, dtype=torch.bfloat16,
                                                                              device="cuda"))
    Xr = torch.zeros(40, 64, device="cuda")
    Wr = torch.zeros(24, 64, device="cuda")
    with pytest.raises(ValueError):
        drgg.router_gemm_fp32_bf16x3(Xr, Wr, out=torch.empty(39, 24, device="cuda"))
    with pytest.raises(ValueError):
        drgg.router_gemm_fp32_bf16x3(Xr, Wr, out=torch.empty(24, 40, device="cuda"))


# ---- the deterministic weight gradient's tail-only plan ------------------------

def _tail_problem(integer=False):
    """32 equal experts of 768 tokens, N = 768, K = 1024: the kernel runs the
    first two 256-row bands of every expert as whole tiles and cuts only the
    third band into chunks."""
    return synth.make_problem("tail_plan", 341, np.full(32, 768), N=768, K=1024, w_std=0.02, integer=integer)


def _fold_table(drgg, prob, ws):
    p = drgg.plan(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)
    off = p["max_partials"] * prob.N * prob.K * 4
    return ws[off:off + 16 * prob.E].view(torch.int32).reshape(prob.E, 4).cpu().numpy()


@pytest.mark.parametrize("case", ["tail", "tail_empty", "zipf_small", "dense"])
def test_wgrad_plan_on_device_matches_host_rule(drgg, case):
    """The chunk kernel writes, for the fold, each expert's token count,
    chunk count and first folded row; that row must be the one the host
    mirror of the plan rule gives (tail-only: the whole bands' end; all-split:
    0), and the result must match the oracle."""
    if case == "tail":
        prob = _tail_problem()
    elif case == "tail_empty":   # the tail-only plan with an expert without tokens
        counts = np.full(32, 768)
        counts[15] = 0
        prob = synth.make_problem("tail_empty", 344, counts, N=768, K=1024, w_std=0.02)
    elif case == "zipf_small":
        prob = synth.make_problem("zipf_small", 342, synth.zipf_counts(342, 24576, 16, 2), N=768, K=1024,
                                  w_std=0.02)
    else:
        prob = synth.make_problem("dense_plan", 343, np.array([8192]), N=512, K=1024, w_std=0.02)
    dv = dev_inputs(prob)
    n = drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32, deterministic=True,
                                  workspace=ws)
    torch.cuda.synchronize()
    tail, row0 = drgg.wgrad_tail_plan(prob.offs, prob.N, prob.K)
    assert tail == case.startswith("tail")
    table = _fold_table(drgg, prob, ws)
    cm = drgg.plan(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)["chunk_max"]
    assert table[:, 0].tolist() == prob.counts.tolist()
    assert table[:, 1].tolist() == [drgg.wgrad_chunking(int(t), cm)[1] for t in prob.counts]
    assert table[:, 3].tolist() == row0.tolist()
    idx = np.union1d(parity.sample_indices(prob, "wgrad"), parity.tile_indices(prob, "wgrad"))
    parity.compare(prob, "wgrad", parity.from_dev(out), False, idx=idx, what=f"plan {case}")


@pytest.mark.parametrize("integer", [False, True])
def test_tail_plan_bitwise_across_tiles_grids_and_order(drgg, integer):
    """In the tail-only plan the whole bands are 256-row bands whatever the
    kernel's tile: every tile shape, grid size and walk order gives the same
    bits (and, on integer inputs, the oracle's)."""
    prob = _tail_problem(integer=integer)
    dv = dev_inputs(prob)
    for out_dtype in (torch.float32, torch.bfloat16):
        ref = bits(run_program(drgg, "wgrad", dv, out_dtype, True))
        try:
            for tile in (1, 2, 3, 4, 5):
                drgg.set_knob(drgg.KNOB_TILE, tile)
                for grid, rev in ((0, 0), (0, 1), (17, 0), (255, 1)):
                    drgg.set_knob(drgg.KNOB_GRID, grid)
                    drgg.set_knob(drgg.KNOB_REVERSE, rev)
                    got = bits(run_program(drgg, "wgrad", dv, out_dtype, True))
                    assert np.array_equal(got, ref), f"tile {tile} grid {grid} reverse {rev} changed the bits"
        finally:
            drgg.set_knob(drgg.KNOB_TILE, 0)
            drgg.set_knob(drgg.KNOB_GRID, 0)
            drgg.set_knob(drgg.KNOB_REVERSE, 0)
        out = run_program(drgg, "wgrad", dv, out_dtype, True)
        torch.cuda.synchronize()
        idx = np.union1d(parity.sample_indices(prob, "wgrad"), parity.tile_indices(prob, "wgrad"))
        parity.compare(prob, "wgrad", parity.from_dev(out), out_dtype == torch.bfloat16, idx=idx,
                       integer=integer, what=f"tail plan integer={integer}")


# ---- the split program's tail: slack placement, chunked tails, arrival orders -----

# 64 skewed experts, 4096 tokens: the tail (18 tiles) fits whole on the
# least-loaded workgroups, and that walk is the faster one
SLACK_COUNTS = np.array([30, 6, 0, 96, 126, 18, 28, 16, 288, 1, 2, 72, 7, 1, 1, 332, 25, 0, 7, 871, 12, 8, 23, 14, 1, 16, 15, 9, 2, 2, 5, 4,
              0, 59, 791, 0, 48, 1, 7, 5, 18, 4, 138, 53, 17, 4, 7, 9, 5, 1, 0, 12, 0, 104, 22, 626, 4, 30, 13, 2, 8, 63, 1, 6])


def _report(drgg):
    rep = torch.zeros(4, dtype=torch.int32, device="cuda")
    drgg.set_knob(drgg.KNOB_SPLIT_REPORT, rep.data_ptr())
    return rep


@pytest.mark.parametrize("integer", [False, True])
def test_split_slack_placement(drgg, integer):
    """A ragged problem whose tail tiles fit whole on the least-loaded
    workgroups: the kernel reports the slack placement the host rule
    predicts, the tail runs with no tile sums (the workspace stays zero), and
    the result is the oracle's (bit for bit on integer inputs, like the
    deterministic program)."""
    prob = synth.make_problem("slack", 351, SLACK_COUNTS, N=1536, K=256, w_std=0.02, integer=integer)
    dv = dev_inputs(prob)
    slack, tail = drgg.wgrad_split_plan(prob.offs, prob.N, prob.K)
    assert slack and tail == 18
    ws = _nondet_ws(drgg, prob, drgg.FP32)
    rep = _report(drgg)
    try:
        out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32, deterministic=False,
                                      workspace=ws)
        torch.cuda.synchronize()
    finally:
        drgg.set_knob(drgg.KNOB_SPLIT_REPORT, 0)
    r = rep.cpu().tolist()
    assert r[0] == 1 and r[1] == tail and r[2] == 1, r
    assert int(torch.count_nonzero(ws)) == 0
    parity.compare(prob, "wgrad", parity.from_dev(out), False, integer=integer, what="slack placement")
    if integer:
        assert np.array_equal(bits(out), bits(run_program(drgg, "wgrad", dv, torch.float32, True)))


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_split_tail_arrival_orders(drgg, seed):
    """The chunked tail of a problem whose tail does not fit whole, with
    seeded delays before each piece adds its partial (other arrival orders
    at the tickets): always the oracle's result (bit for bit on integer
    inputs), the workspace zero again after every call, and the reported
    decision the host rule's."""
    for integer in (False, True):
        prob = synth.make_problem("chunked_tail", 352, np.full(8, 2048), N=1536, K=2048, w_std=0.02,
                                  integer=integer)
        dv = dev_inputs(prob)
        slack, tail, banded = drgg.wgrad_split_plan(prob.offs, prob.N, prob.K, banded=True)
        assert not slack and tail > 0 and banded
        ws = _nondet_ws(drgg, prob, drgg.FP32)
        rep = _report(drgg)
        drgg.set_knob(drgg.KNOB_DELAY_SEED, seed)
        try:
            out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32,
                                          deterministic=False, workspace=ws)
            torch.cuda.synchronize()
        finally:
            drgg.set_knob(drgg.KNOB_DELAY_SEED, 0)
            drgg.set_knob(drgg.KNOB_SPLIT_REPORT, 0)
        r = rep.cpu().tolist()
        assert r[0] == 0 and r[1] == tail and r[2] == 1, r
        assert int(torch.count_nonzero(ws)) == 0
        idx = np.union1d(parity.sample_indices(prob, "wgrad"), parity.tile_indices(prob, "wgrad"))
        parity.compare(prob, "wgrad", parity.from_dev(out), False, idx=idx, integer=integer,
                       what=f"arrival orders seed {seed}")


def test_split_program_with_an_expert_without_tokens(drgg):
    """The split program's walk on a problem with an empty expert (the walk
    has two positions per expert): the empty expert gets no items and a zero
    gradient, the others the oracle's result, bit for bit on integers."""
    counts = np.full(32, 768)
    counts[15] = 0
    for integer in (False, True):
        prob = synth.make_problem("split_empty", 345, counts, N=768, K=1024, w_std=0.02, integer=integer)
        dv = dev_inputs(prob)
        ws = _nondet_ws(drgg, prob, drgg.FP32)
        print(f"split program with an empty expert, integer={integer}", flush=True)
        out = drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=torch.float32, deterministic=False,
                                      workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0
        assert not np.any(bits(out).reshape(prob.E, prob.N, prob.K)[15])
        idx = np.union1d(parity.sample_indices(prob, "wgrad"), parity.tile_indices(prob, "wgrad"))
        parity.compare(prob, "wgrad", parity.from_dev(out), False, idx=idx, integer=integer,
                       what=f"split program, empty expert, integer={integer}")


# ---- HIP graph capture ---------------------------------------------------------------

def test_graph_replays_match_eager(drgg):
    """The deterministic forward, data gradient (W^T workspace), weight
    gradient and the weight gradient that allocates nothing, captured into one
    HIP graph: each of three replays, with eager work and synchronisations
    between them, gives the eager results bit for bit.  The split program in
    its own graph: every replay matches the oracle and leaves its workspace
    zero."""
    drgg.set_knob(drgg.KNOB_DGRAD_WT, 1)   # W^T at these 768 tokens per expert too
    try:
        _graph_replays(drgg)
    finally:
        drgg.set_knob(drgg.KNOB_DGRAD_WT, 0)


def _graph_replays(drgg):
    prob = _tail_problem()
    dv = dev_inputs(prob)
    small = ragged_problem(*DET_CASE)   # within the fixed array of the call that allocates nothing
    dvs = dev_inputs(small)
    f32 = torch.float32
    Y = torch.empty((prob.M, prob.N), dtype=f32, device="cuda")
    dX = torch.empty((prob.M, prob.K), dtype=f32, device="cuda")
    dW = torch.empty((prob.E, prob.N, prob.K), dtype=f32, device="cuda")
    dW2 = torch.empty((small.E, small.N, small.K), dtype=f32, device="cuda")
    dW3 = torch.empty_like(dW2)
    wsd = torch.zeros(drgg.workspace_size(drgg.OP_DGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True),
                      dtype=torch.uint8, device="cuda")
    wsw = torch.zeros(drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True),
                      dtype=torch.uint8, device="cuda")

    def programs():
        drgg.grouped_gemm_fwd(dv["X"], dv["W"], dv["offs"], out_dtype=f32, out=Y)
        drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=f32, out=dX, workspace=wsd)
        drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=f32, deterministic=True, out=dW,
                                workspace=wsw)
        drgg.grouped_gemm_wgrad_noalloc(dvs["X"], dvs["G"], dvs["offs"], dW2, deterministic=True)

    programs()
    torch.cuda.synchronize()
    refs = [bits(t) for t in (Y, dX, dW, dW2)]
    drgg.grouped_gemm_wgrad(dvs["X"], dvs["G"], dvs["offs"], out_dtype=f32, deterministic=True, out=dW3)
    torch.cuda.synchronize()
    assert np.array_equal(refs[3], bits(dW3))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        programs()
    other = ragged_problem(*DET_CASE)
    dvo = dev_inputs(other)
    for i in range(3):
        for t in (Y, dX, dW, dW2):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t, ref in zip((Y, dX, dW, dW2), refs):
            assert np.array_equal(bits(t), ref), f"replay {i} differs from the eager result"
        # eager work between the replays
        run_program(drgg, "wgrad", dvo, f32, True)
        torch.cuda.synchronize()
    # the split program (atomic tile sums) in a graph
    ws = _nondet_ws(drgg, prob, drgg.FP32)
    out = torch.empty_like(dW)
    drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=f32, deterministic=False, out=out, workspace=ws)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=f32, deterministic=False, out=out,
                                workspace=ws)
    idx = np.union1d(parity.sample_indices(prob, "wgrad"), parity.tile_indices(prob, "wgrad"))
    for i in range(3):
        out.fill_(float("nan"))
        g2.replay()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0
        parity.compare(prob, "wgrad", parity.from_dev(out), False, idx=idx, what=f"split program replay {i}")
        run_program(drgg, "fwd", dvo, f32, True)
        torch.cuda.synchronize()
