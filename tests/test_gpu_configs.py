"""GPU parity at the full sizes of the five measured workloads, in the launch
configuration the benchmark times.

Every output element at these sizes would take the CPU oracle minutes, so
each program is checked on the elements the oracle computes one by one:
every element of four whole 256x256 output blocks (the first, the last, one
across an expert boundary -- for the weight gradient one of the longest
expert -- and a random one) plus scattered samples (random elements, every
expert's and every 256-row tile's first and last row, the last column, every
expert's output corners), at the tolerances of tests/parity.py.  Integer-valued inputs of the same shapes are compared bit
for bit on the same samples, empty experts are checked in full, and the
deterministic variant is re-run and compared bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.test_gpu_parity import dev_inputs, run_program

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


def sampled_check(prob, program, out, out_bf16, integer=False, what=""):
    idx = np.union1d(parity.sample_indices(prob, program), parity.tile_indices(prob, program))
    n = parity.compare(prob, program, parity.from_dev(out), out_bf16, idx=idx, integer=integer, what=what)
    worst = f"; worst {parity.check_bf16.last_worst_ulp:.2f} ulp" if out_bf16 and not integer else ""
    print(f"{what}: {idx.size} elements (4 whole tiles + samples) ok; {n} needed the FP32-accumulation "
          f"floor{worst}", flush=True)


def empty_experts_zero(prob, out):
    v = bits(out).reshape(prob.E, prob.N, prob.K)
    for e in np.flatnonzero(prob.counts == 0):
        assert not np.any(v[e]), f"expert {e} has no tokens but a non-zero gradient"


# ---- workload 2: dense projection weight gradient, one group -----------------

@pytest.mark.parametrize("d_out", [48, 64, 512, 1024])
def test_dense_wgrad(drgg, d_out):
    for integer in (False, True):
        prob = synth.config2(d_out, integer=integer)
        dv = dev_inputs(prob)
        print(f"dense wgrad d_out={d_out} integer={integer}", flush=True)
        det = run_program(drgg, "wgrad", dv, torch.float32, True)
        sampled_check(prob, "wgrad", det, False, integer, f"dense {d_out} det")
        again = run_program(drgg, "wgrad", dv, torch.float32, True)
        assert np.array_equal(bits(again), bits(det))
        nd = run_program(drgg, "wgrad", dv, torch.float32, False)
        sampled_check(prob, "wgrad", nd, False, integer, f"dense {d_out} split")
        if integer:
            assert np.array_equal(bits(nd), bits(det))


# ---- workload 3: MoE gate_up, E=8 balanced -------------------------------------

@pytest.fixture(scope="module")
def moe_gate_up():
    return synth.config3()


@pytest.mark.parametrize("program", ["fwd", "dgrad", "wgrad"])
def test_moe_gate_up_bf16(drgg, moe_gate_up, program):
    prob = moe_gate_up
    dv = dev_inputs(prob)
    out = run_program(drgg, program, dv, torch.bfloat16, True)
    sampled_check(prob, program, out, True, what=f"gate_up {program} det")
    assert np.array_equal(bits(run_program(drgg, program, dv, torch.bfloat16, True)), bits(out))
    if program == "wgrad":
        nd = run_program(drgg, program, dv, torch.bfloat16, False)
        sampled_check(prob, program, nd, True, what=f"gate_up {program} split")


@pytest.mark.parametrize("program", ["fwd", "dgrad", "wgrad"])
def test_moe_gate_up_integer_bitwise(drgg, program):
    prob = synth.config3(integer=True)
    dv = dev_inputs(prob)
    for det in (True, False) if program == "wgrad" else (True,):
        out = run_program(drgg, program, dv, torch.bfloat16, det)
        sampled_check(prob, program, out, True, integer=True, what=f"gate_up integer {program} det={det}")


def test_moe_gate_up_dgrad_direct_bitwise(drgg):
    """The data gradient without a workspace (W read transposed, its loads
    spread over the steps and across tile boundaries) at a size with 16
    tiles per workgroup: bitwise equal to the W^T program, and exact against
    the oracle on integer inputs."""
    prob = synth.config3(integer=True)
    dv = dev_inputs(prob)
    via_wt = drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=torch.bfloat16)
    direct = drgg.grouped_gemm_dgrad(dv["G"], dv["W"], dv["offs"], out_dtype=torch.bfloat16, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(via_wt.view(torch.int16), direct.view(torch.int16))
    sampled_check(prob, "dgrad", direct, True, integer=True, what="gate_up integer dgrad direct")


# ---- workload 4: MoE down, Zipf-skewed, 2 empty experts --------------------------

@pytest.mark.parametrize("integer", [False, True])
def test_moe_down_skewed_wgrad(drgg, integer):
    prob = synth.config4(integer=integer)
    assert np.sum(prob.counts == 0) == 2
    dv = dev_inputs(prob)
    det = run_program(drgg, "wgrad", dv, torch.float32, True)
    sampled_check(prob, "wgrad", det, False, integer, f"down det integer={integer}")
    empty_experts_zero(prob, det)
    assert np.array_equal(bits(run_program(drgg, "wgrad", dv, torch.float32, True)), bits(det))
    nd = run_program(drgg, "wgrad", dv, torch.float32, False)
    sampled_check(prob, "wgrad", nd, False, integer, f"down split integer={integer}")
    empty_experts_zero(prob, nd)
    a = parity.from_dev(det).astype(np.float64)
    b = parity.from_dev(nd).astype(np.float64)
    assert np.linalg.norm(a - b) <= 1e-6 * np.linalg.norm(a)
    if integer:
        assert np.array_equal(bits(nd), bits(det))


# ---- workload 5: square dense projection + FP32 router -------------------------

@pytest.mark.parametrize("program", ["fwd", "dgrad", "wgrad"])
def test_dense_square_bf16(drgg, program):
    prob = synth.config5(need=("X", "W") if program == "fwd" else ("G", "W") if program == "dgrad" else ("X", "G"))
    dv = dev_inputs(prob)
    out = run_program(drgg, program, dv, torch.bfloat16, True)
    sampled_check(prob, program, out, True, what=f"square {program}")
    assert np.array_equal(bits(run_program(drgg, program, dv, torch.bfloat16, True)), bits(out))


@pytest.mark.parametrize("rows", [16384, 8192])
def test_router_full_size(drgg, rows):
    """The router workload (16384 tokens: the single-pass program) and its
    first 8192 tokens (the sliced program, 8 reduction slices)."""
    X, Wr = synth.router_inputs()
    X = np.ascontiguousarray(X[:rows])
    print(f"router {rows} tokens: program {drgg.router_split(rows, Wr.shape[0], X.shape[1])}", flush=True)
    out = drgg.router_gemm_fp32_bf16x3(parity.to_dev(X), parity.to_dev(Wr))
    o = parity.from_dev(out).ravel().astype(np.float64)
    rng = np.random.default_rng(0)
    M, N = out.shape
    # every element of three whole 128 x 128 output tiles (first, last, one
    # random) plus scattered samples
    blocks = []
    for r0, c0 in ((0, 0), (M - 128, N - 128), (int(rng.integers(0, M // 128)) * 128, 128)):
        r = np.arange(r0, r0 + 128)
        c = np.arange(c0, c0 + 128)
        blocks.append((r[:, None] * N + c[None, :]).ravel())
    idx = np.unique(np.concatenate([rng.integers(0, o.size, 4000), [0, o.size - 1], *blocks]))
    emul = oracle.router_bf16x3(X, Wr, idx)
    exact = oracle.router_exact(X, Wr, idx)
    assert np.linalg.norm(o[idx] - emul) <= 1e-6 * np.linalg.norm(emul)
    ax = np.abs(X).max(axis=1)[idx // N]
    aw = np.abs(Wr).max(axis=1)[idx % N]
    parity.check_fp32(o[idx], exact, np.full(idx.size, X.shape[1]), ax, aw, what="router full size")
    rel = np.linalg.norm(o[idx] - exact) / np.linalg.norm(exact)
    print(f"router: relative Frobenius error vs exact FP32 product {rel:.2e}", flush=True)
