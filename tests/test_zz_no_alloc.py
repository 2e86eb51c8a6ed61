"""GPU test of grouped_gemm_wgrad_noalloc, the weight gradient whose
workspace is the library's fixed per-device array (the entry point for
callers that cannot allocate).  Called through the C ABI and checked against
grouped_gemm_wgrad with its own workspace: bitwise for the deterministic
program, within the FP32/BF16 tolerances (and bitwise on integer inputs) for
the split program; two calls in a row, the second on a smaller problem; a
split-program call right after a deterministic one (the array then holds
partials, which the call must clear); a problem too large for the array is
refused with nothing written."""
import numpy as np
import pytest

from tests import parity
from tests.test_gpu_parity import dev_inputs, ragged_problem

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def drgg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_ragged_grouped_amd as d
    return d


def bits(t):
    return parity.from_dev(t).view(np.uint16 if t.dtype == torch.bfloat16 else np.uint32).copy()


def noalloc(drgg, prob, dv, out, det):
    code = drgg.BF16 if out.dtype == torch.bfloat16 else drgg.FP32
    return drgg.lib.grouped_gemm_wgrad_noalloc(dv["X"].data_ptr(), dv["G"].data_ptr(), dv["offs"].data_ptr(),
                                               prob.E, prob.M, prob.N, prob.K, code, int(det), out.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)


def reference(drgg, prob, dv, dtype, det):
    ws = torch.zeros(drgg.workspace_size(drgg.OP_WGRAD, prob.E, prob.M, prob.N, prob.K,
                                         drgg.BF16 if dtype == torch.bfloat16 else drgg.FP32, det) + 256,
                     dtype=torch.uint8, device="cuda")
    return drgg.grouped_gemm_wgrad(dv["X"], dv["G"], dv["offs"], out_dtype=dtype, deterministic=det, workspace=ws)


CASES = [(401, 4, 6000, 264, 392, (1,)), (402, 3, 2000, 136, 200, ())]   # the second one smaller


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_deterministic_bitwise(drgg, dtype):
    for case in CASES:
        print(f"noalloc det {case} {dtype}", flush=True)
        prob = ragged_problem(*case)
        dv = dev_inputs(prob)
        ref = reference(drgg, prob, dv, dtype, True)
        out = torch.full((prob.E, prob.N, prob.K), 7.0, dtype=dtype, device="cuda")
        assert noalloc(drgg, prob, dv, out, True) == 0
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(ref)), f"{case}: differs from grouped_gemm_wgrad"
        parity.compare(prob, "wgrad", parity.from_dev(out), dtype == torch.bfloat16, what=f"noalloc det {case}")


@pytest.mark.parametrize("integer", [False, True])
def test_noalloc_split_program(drgg, integer):
    drgg.set_knob(drgg.KNOB_NONDET, 1)
    try:
        for case in CASES:
            print(f"noalloc split {case} integer={integer}", flush=True)
            prob = ragged_problem(*case, integer=integer)
            dv = dev_inputs(prob)
            # a deterministic call first leaves partials in the array
            det_out = torch.empty((prob.E, prob.N, prob.K), dtype=torch.float32, device="cuda")
            assert noalloc(drgg, prob, dv, det_out, True) == 0
            out = torch.full((prob.E, prob.N, prob.K), 7.0, dtype=torch.float32, device="cuda")
            assert noalloc(drgg, prob, dv, out, False) == 0
            torch.cuda.synchronize()
            ref = reference(drgg, prob, dv, torch.float32, False)
            torch.cuda.synchronize()
            if integer:
                assert np.array_equal(bits(out), bits(ref))
                assert np.array_equal(bits(out), bits(det_out))
            else:
                a = parity.from_dev(out).astype(np.float64)
                b = parity.from_dev(ref).astype(np.float64)
                assert np.linalg.norm(a - b) <= 1e-6 * np.linalg.norm(b)
            parity.compare(prob, "wgrad", parity.from_dev(out), False, integer=integer,
                           what=f"noalloc split {case}")
    finally:
        drgg.set_knob(drgg.KNOB_NONDET, 0)


def test_noalloc_refuses_a_problem_beyond_the_array(drgg):
    """The gate_up shape needs more workspace than the fixed array: refused
    with DRGG_EWORKSPACE before anything is launched."""
    E, M, N, K = 8, 131072, 1536, 2048
    assert drgg.workspace_size(drgg.OP_WGRAD, E, M, N, K, drgg.BF16, True) > 64 << 20
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    G = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    offs = torch.arange(0, M + 1, M // E, dtype=torch.int32, device="cuda")
    out = torch.full((E, N, K), 3.0, dtype=torch.bfloat16, device="cuda")
    st = drgg.lib.grouped_gemm_wgrad_noalloc(X.data_ptr(), G.data_ptr(), offs.data_ptr(), E, M, N, K, drgg.BF16, 1,
                                             out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 5
    assert bool(torch.all(out == 3.0))
    with pytest.raises(drgg.DrggError):
        drgg.grouped_gemm_wgrad_noalloc(X, G, offs, out)
