"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small and medium shapes are compared element by element on every output;
they span several tiles, ragged expert boundaries, empty experts, reduction
tails that are not multiples of the 64-wide step and partial output tiles.
Integer-valued inputs are compared bit for bit in every mode.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

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


def dev_inputs(prob):
    d = {"offs": parity.to_dev(prob.offs)}
    for name in ("X", "W", "G"):
        a = getattr(prob, name)
        if a is not None:
            d[name] = parity.to_dev_bf16(a)
    return d


def run_program(drgg, program, dv, out_dtype, det):
    if program == "fwd":
        return drgg.grouped_gemm_fwd(dv["X"], dv["W"], dv["offs"], out_dtype=out_dtype, deterministic=det)
    if program == "dgrad":
        return drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=out_dtype, deterministic=det)
    return drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=out_dtype, deterministic=det)


def ragged_problem(seed, E, M, N, K, empty=(), integer=False, w_std=0.02):
    counts = synth.ragged_counts(seed, M, E, empty)
    return synth.make_problem(f"ragged_s{seed}", seed, counts, N=N, K=K, w_std=w_std, integer=integer)


PROGRAMS = ["fwd", "dgrad", "wgrad"]


@pytest.mark.parametrize("forced_empty", [False, True])
@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("program", PROGRAMS)
def test_tiny_moe_fp32(drgg, program, det, forced_empty):
    """Workload 1: E=4, 512 tokens, FP32 outputs, both variants."""
    prob = synth.config1(forced_empty=forced_empty)
    print(f"tiny moe {program} det={det} counts={prob.counts.tolist()}", flush=True)
    dv = dev_inputs(prob)
    out = run_program(drgg, program, dv, torch.float32, det)
    torch.cuda.synchronize()
    parity.compare(prob, program, parity.from_dev(out), False, what=f"tiny {program}")


MEDIUM = [
    # seed, E, M, N, K, empty
    (101, 3, 1000, 520, 392, (1,)),
    (102, 5, 777, 264, 200, (0, 4)),
    (103, 1, 600, 312, 648, ()),
    (104, 2, 300, 8, 40, ()),
    (105, 2, 4000, 64, 256, ()),
]


@pytest.mark.parametrize("out_bf16", [False, True])
@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("program", PROGRAMS)
@pytest.mark.parametrize("case", MEDIUM, ids=lambda c: f"s{c[0]}_E{c[1]}_M{c[2]}_N{c[3]}_K{c[4]}")
def test_medium_ragged(drgg, case, program, det, out_bf16):
    seed, E, M, N, K, empty = case
    prob = ragged_problem(seed, E, M, N, K, empty)
    print(f"medium {case} {program} det={det} bf16={out_bf16}", flush=True)
    dv = dev_inputs(prob)
    out = run_program(drgg, program, dv, torch.bfloat16 if out_bf16 else torch.float32, det)
    torch.cuda.synchronize()
    parity.compare(prob, program, parity.from_dev(out), out_bf16, what=f"{case} {program}")


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("program", PROGRAMS)
def test_integer_inputs_bitwise(drgg, program, det, tile):
    """Integer-valued inputs: exact partial sums, so bit-for-bit equality in
    every variant and at every tile shape."""
    prob = ragged_problem(201, 4, 1500, 136, 328, (2,), integer=True)
    dv = dev_inputs(prob)
    drgg.set_knob(drgg.KNOB_TILE, tile)
    try:
        print(f"integer {program} det={det} tile={tile}", flush=True)
        for out_dtype in (torch.float32, torch.bfloat16):
            out = run_program(drgg, program, dv, out_dtype, det)
            torch.cuda.synchronize()
            parity.compare(prob, program, parity.from_dev(out), out_dtype == torch.bfloat16, integer=True,
                           what=f"integer {program} tile {tile}")
    finally:
        drgg.set_knob(drgg.KNOB_TILE, 0)


# expert lengths covering the remainders of the 512-token unit: 0, 1, one
# step minus and plus one, half a unit (256: the "k256 tail"), 257, 300, 511
UNIT_REMAINDERS = [512 * a + r for a, r in ((2, 0), (2, 1), (3, 31), (2, 32), (2, 33), (2, 255), (3, 256),
                                            (2, 257), (2, 300), (2, 511))]


@pytest.mark.parametrize("det", [True, False])
def test_wgrad_unit_remainders_bitwise(drgg, det):
    """Weight gradients of experts whose lengths leave remainders 0, 1, 31,
    32, 33, 255, 256, 257, 300 and 511 modulo the 512-token unit, each cut
    into several chunks (in the split program whole units, the last one the
    remainder): integer inputs, so both programs match the oracle bit for
    bit."""
    prob = synth.make_problem("unit_remainders", 301, UNIT_REMAINDERS, N=264, K=200, integer=True)
    plan = drgg.plan(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)
    chunks = [drgg.wgrad_chunking(int(t), plan["chunk_max"]) for t in UNIT_REMAINDERS]
    assert all(n > 1 for _, n in chunks), chunks
    print(f"unit remainders det={det} chunks={chunks}", flush=True)
    dv = dev_inputs(prob)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = run_program(drgg, "wgrad", dv, out_dtype, det)
        torch.cuda.synchronize()
        parity.compare(prob, "wgrad", parity.from_dev(out), out_dtype == torch.bfloat16, integer=True,
                       what=f"unit remainders det={det}")


@pytest.mark.parametrize("E", [63, 64, 65])
def test_expert_count_around_one_wave_bitwise(drgg, E):
    """Up to 63 experts (64 offsets) the kernels build their schedule, the
    weight gradient its per-expert table, ranking and walk prefixes on one
    wave; from 64 on with the workgroup-wide scans.  Skewed (Zipf) routing
    with three empty experts and some experts cut into chunks, integer
    inputs: all three programs and both weight-gradient programs match the
    oracle bit for bit on either side of the boundary."""
    counts = synth.zipf_counts(500 + E, 10000, E, 3, 1.0)
    prob = synth.make_problem(f"wave_boundary_E{E}", 500 + E, counts, N=264, K=200, integer=True)
    plan = drgg.plan(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)
    chunks = [drgg.wgrad_chunking(int(t), plan["chunk_max"])[1] for t in counts]
    assert max(chunks) > 1 and int((counts == 0).sum()) == 3, (chunks, counts.tolist())
    dv = dev_inputs(prob)
    for program in PROGRAMS:
        for det in ((True, False) if program == "wgrad" else (True,)):
            print(f"wave boundary E={E} {program} det={det}", flush=True)
            out = run_program(drgg, program, dv, torch.float32, det)
            torch.cuda.synchronize()
            parity.compare(prob, program, parity.from_dev(out), False, integer=True,
                           what=f"wave boundary E={E} {program} det={det}")


def test_forward_and_data_gradient_same_bits_across_one_wave_boundary(drgg):
    """The same 63 experts as a 63-expert call (one-wave schedule) and as a
    64-expert call whose last expert is empty (workgroup-wide schedule):
    the forward and data gradient compute the same tiles the same way, so
    their outputs are equal bit for bit (random inputs, FP32 and BF16)."""
    counts = np.append(synth.zipf_counts(640, 9000, 63, 2, 1.0), 0)
    prob = synth.make_problem("wave_boundary_pair", 640, counts, N=200, K=328)
    dv = dev_inputs(prob)
    offs63 = dv["offs"][:64].clone()
    W63 = dv["W"][:63].contiguous()
    for out_dtype in (torch.float32, torch.bfloat16):
        y64 = drgg.grouped_gemm_fwd(dv["X"], dv["W"], dv["offs"], out_dtype=out_dtype)
        y63 = drgg.grouped_gemm_fwd(dv["X"], W63, offs63, out_dtype=out_dtype)
        g64 = drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=out_dtype)
        g63 = drgg.grouped_gemm_dgrad(dv["G"], W63, offs63, out_dtype=out_dtype)
        torch.cuda.synchronize()
        iv = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(y64.view(iv), y63.view(iv)), f"forward {out_dtype}"
        assert torch.equal(g64.view(iv), g63.view(iv)), f"data gradient {out_dtype}"
    parity.compare(prob, "fwd", parity.from_dev(y64), True, what="wave boundary pair forward")


PLANNER_TILE_CASES = [
    # program, seed, E, M, N, K, the planner's tile
    ("fwd", 650, 2, 8448, 2304, 264, (128, 256)),     # 297 .. 306 tiles of 256x256
    ("dgrad", 651, 1, 5120, 264, 4096, (128, 256)),   # on W^T, 320 tiles
    ("fwd", 652, 2, 700, 2304, 264, (128, 128)),      # 27 tiles
    ("dgrad", 653, 2, 8448, 2304, 264, (128, 128)),   # 66 tiles
]


@pytest.mark.parametrize("case", PLANNER_TILE_CASES, ids=lambda c: f"{c[0]}_M{c[3]}_N{c[4]}_K{c[5]}")
def test_planner_tiles_match_256_tiles_bitwise(drgg, case):
    """Calls the planner puts on 128x256 tiles (between one and one and a
    half waves of 256x256 tiles) or 128x128 tiles (at most half a wave) give
    the bits of the 256x256 tile; the oracle checks a sample."""
    program, seed, E, M, N, K, want = case
    prob = synth.make_problem(f"planner_tile_{seed}", seed, synth.ragged_counts(seed, M, E), N=N, K=K)
    plan = drgg.plan(drgg.OP_FWD if program == "fwd" else drgg.OP_DGRAD, E, M, N, K)
    print(f"planner tile {program} E={E} M={M} N={N} K={K}: {plan['tile_m']}x{plan['tile_n']}", flush=True)
    assert (plan["tile_m"], plan["tile_n"]) == want
    dv = dev_inputs(prob)
    for out_dtype in (torch.float32, torch.bfloat16):
        got = run_program(drgg, program, dv, out_dtype, True)
        drgg.set_knob(drgg.KNOB_TILE, 1)
        try:
            ref = run_program(drgg, program, dv, out_dtype, True)
        finally:
            drgg.set_knob(drgg.KNOB_TILE, 0)
        torch.cuda.synchronize()
        iv = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(got.view(iv), ref.view(iv)), f"{program} {out_dtype}"
    parity.compare(prob, program, parity.from_dev(got), True, idx=parity.sample_indices(prob, program),
                   what=f"planner tile {program} M={M}")


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_wgrad_without_fold_zeroes_empty_experts(drgg, out_dtype):
    """When no expert can be cut into chunks (chunk_max >= M) the
    deterministic weight gradient runs without its fold kernel, and the
    chunk kernel itself writes the zero output of experts without tokens:
    here 8 of 16 experts are empty and the output buffer starts as NaN;
    integer inputs, so every expert matches the oracle bit for bit."""
    counts = np.zeros(16, dtype=np.int64)
    counts[[0, 2, 3, 7, 8, 11, 13, 15]] = [61, 5, 77, 1, 40, 99, 18, 63]
    prob = synth.make_problem("no_fold_empty", 660, counts, N=72, K=136, integer=True)
    plan = drgg.plan(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)
    assert plan["chunk_max"] >= prob.M, plan
    dv = dev_inputs(prob)
    dt = torch.float32 if out_dtype == "fp32" else torch.bfloat16
    dW = torch.full((prob.E, prob.N, prob.K), float("nan"), dtype=dt, device="cuda")
    drgg.set_knob(drgg.KNOB_TIMING, 1)
    try:
        drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=dt, deterministic=True, out=dW)
        kernels = [name for name, _ in drgg.last_call_kernel_times()]
    finally:
        drgg.set_knob(drgg.KNOB_TIMING, 0)
    torch.cuda.synchronize()
    assert kernels == ["gg_wgrad_det_kernel"], kernels
    parity.compare(prob, "wgrad", parity.from_dev(dW), out_dtype == "bf16", integer=True,
                   what=f"no fold, empty experts, {out_dtype}")


def test_wgrad_share_clamp_skewed_bitwise(drgg):
    """A skewed routing where the chunk rule raises the chunk length to one
    reference CU's share (64 Zipf-routed experts, 4 of them empty: the
    balanced expert stays whole, the long ones are cut into chunks of at
    least 768 tokens); integer inputs, every element of both programs bit for
    bit (one oracle evaluation for both)."""
    counts = synth.zipf_counts(4321, 24576, 64, 4, 1.2)
    prob = synth.make_problem("share_clamp", 302, counts, N=512, K=1024, integer=True)
    cm = drgg.plan(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K, drgg.FP32, True)["chunk_max"]
    assert cm == 768 and drgg.wgrad_chunking(int(counts.max()), cm)[1] > 1
    dv = dev_inputs(prob)
    want = oracle.round_f32(parity.oracle_program(prob, "wgrad", None)[0]).view(np.uint32)
    for det in (True, False):
        print(f"share clamp det={det} chunk_max={cm} max T={counts.max()}", flush=True)
        out = run_program(drgg, "wgrad", dv, torch.float32, det)
        torch.cuda.synchronize()
        got = parity.from_dev(out).astype(np.float32).view(np.uint32)
        assert np.array_equal(got.ravel(), want.ravel()), f"share clamp det={det}: integer inputs must match bit for bit"


SPLIT_CASE = (106, 3, 4000, 264, 520, (1,))   # two experts of about 2000 tokens: cut into chunks
MEDIUM_SPLIT = [SPLIT_CASE, (107, 1, 9000, 64, 392, ())]


def test_wgrad_det_split_cases_are_split(drgg):
    """The cases below really exercise the chunked (partials + ordered fold)
    path: some expert is cut into more than one chunk."""
    for seed, E, M, N, K, empty in MEDIUM_SPLIT:
        plan = drgg.plan(drgg.OP_WGRAD, E, M, N, K, drgg.FP32, True)
        counts = synth.ragged_counts(seed, M, E, empty)
        chunks = [drgg.wgrad_chunking(int(t), plan["chunk_max"])[1] for t in counts]
        assert max(chunks) > 1, (seed, plan["chunk_max"], counts.tolist(), chunks)


@pytest.mark.parametrize("out_bf16", [False, True])
@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("case", MEDIUM_SPLIT, ids=lambda c: f"s{c[0]}_E{c[1]}_M{c[2]}_N{c[3]}_K{c[4]}")
def test_medium_split_wgrad(drgg, case, det, out_bf16):
    """Every element of weight gradients whose experts are cut into several
    chunks (deterministic: partials and ordered fold; split program: atomic
    tile sums and tickets)."""
    seed, E, M, N, K, empty = case
    prob = ragged_problem(seed, E, M, N, K, empty)
    print(f"medium split {case} det={det} bf16={out_bf16}", flush=True)
    dv = dev_inputs(prob)
    out = run_program(drgg, "wgrad", dv, torch.bfloat16 if out_bf16 else torch.float32, det)
    torch.cuda.synchronize()
    parity.compare(prob, "wgrad", parity.from_dev(out), out_bf16, what=f"split {case}")


@pytest.mark.parametrize("shape", [(302, 3, 1000, 264, 520, (1,)), (303, 8, 4096, 1536, 2048, ()),
                                   (304, 1, 700, 72, 136, ())])
def test_dgrad_transposed_w_matches_direct_bitwise(drgg, shape):
    """The data gradient with a workspace (W transposed into it first) and
    without (W read transposed by the kernel) multiply the same values in the
    same order: bitwise equal outputs; the direct one also against the
    oracle."""
    prob = ragged_problem(*shape)
    print(f"dgrad W^T vs direct shape={shape}", flush=True)
    dv = dev_inputs(prob)
    for out_dtype, view in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        # these experts average fewer tokens than the transpose needs to pay:
        # force it, to compare the two programs
        drgg.set_knob(drgg.KNOB_DGRAD_WT, 1)
        try:
            via_wt = drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=out_dtype)
        finally:
            drgg.set_knob(drgg.KNOB_DGRAD_WT, 0)
        direct = drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=out_dtype, workspace=False)
        torch.cuda.synchronize()
        assert torch.equal(via_wt.view(view), direct.view(view))
        if out_dtype == torch.float32:
            parity.compare(prob, "dgrad", parity.from_dev(direct), False, what=f"dgrad direct {shape}")
