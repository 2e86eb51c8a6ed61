"""The autograd wrapper on the GPU: the layer's forward and backward are the
library's programs (bitwise), they match the oracle, and a non-reentrant
checkpoint recomputes the forward kernel only with early stop off."""
import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def drgg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_ragged_grouped_amd as d
    import dense_ragged_grouped_amd.autograd  # noqa: F401
    # the library's default route (other modules' fixtures select the split
    # program): a non-deterministic weight gradient at these points is then
    # bitwise reproducible, which the comparisons below rely on
    d.set_knob(d.KNOB_NONDET, 0)
    yield d
    d.set_knob(d.KNOB_NONDET, 0)


def problem(seed=401, E=4, M=1500, N=136, K=328, empty=(2,)):
    counts = synth.ragged_counts(seed, M, E, empty)
    return synth.make_problem(f"autograd_s{seed}", seed, counts, N=N, K=K, w_std=0.02)


def leaves(prob):
    X = parity.to_dev_bf16(prob.X).requires_grad_(True)
    W = parity.to_dev_bf16(prob.W).requires_grad_(True)
    G = parity.to_dev_bf16(prob.G)
    return X, W, G, parity.to_dev(prob.offs)


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_layer_is_the_library_programs_and_matches_the_oracle(drgg):
    from dense_ragged_grouped_amd.autograd import grouped_linear
    prob = problem()
    X, W, G, offs = leaves(prob)
    print("autograd layer", prob.counts.tolist(), flush=True)
    Y = grouped_linear(X, W, offs)
    dX, dW = torch.autograd.grad(Y, (X, W), G)
    torch.cuda.synchronize()
    with torch.no_grad():
        assert same_bits(Y, drgg.grouped_gemm_fwd(X, W, offs))
        assert same_bits(dX, drgg.grouped_gemm_dgrad(G, W, offs))
        assert same_bits(dW, drgg.grouped_gemm_wgrad(X, G, offs, out_dtype=torch.bfloat16))
    for program, out in (("fwd", Y), ("dgrad", dX), ("wgrad", dW)):
        parity.compare(prob, program, parity.from_dev(out.detach()), True, what=f"autograd {program}")
    # empty expert: no tokens, zero gradient
    e = int(np.flatnonzero(prob.counts == 0)[0])
    assert not torch.any(dW[e].view(torch.int16))


def test_noncontiguous_output_gradient(drgg):
    """A gradient arriving as a strided view is made contiguous first."""
    from dense_ragged_grouped_amd.autograd import grouped_linear
    prob = problem(402, 3, 700, 64, 136, ())
    X, W, G, offs = leaves(prob)
    Y = grouped_linear(X, W, offs)
    Gt = G.t().contiguous().t()   # same values, column-major strides
    assert not Gt.is_contiguous()
    dX, dW = torch.autograd.grad(Y, (X, W), Gt)
    dX0, dW0 = torch.autograd.grad(grouped_linear(X, W, offs), (X, W), G)
    assert same_bits(dX, dX0) and same_bits(dW, dW0)


@pytest.mark.parametrize("deterministic", [True, False])
def test_checkpoint_recomputes_the_forward_only_without_early_stop(drgg, monkeypatch, deterministic):
    import dense_ragged_grouped_amd.autograd as ag
    prob = problem(403, 4, 2000, 200, 264, ())
    X, W, G, offs = leaves(prob)
    calls = {"n": 0}
    fwd = ag.grouped_gemm_fwd

    def counting_fwd(*args, **kwargs):
        calls["n"] += 1
        return fwd(*args, **kwargs)

    monkeypatch.setattr(ag, "grouped_gemm_fwd", counting_fwd)
    ref = torch.autograd.grad(ag.grouped_linear(X, W, offs, deterministic), (X, W), G)
    for early_stop, launches in ((False, 2), (True, 1)):
        calls["n"] = 0
        Y = ag.checkpointed_grouped_linear(X, W, offs, deterministic, early_stop=early_stop)
        got = torch.autograd.grad(Y, (X, W), G)
        torch.cuda.synchronize()
        print(f"checkpoint early_stop={early_stop}: {calls['n']} forward launches", flush=True)
        assert calls["n"] == launches
        # the library routes the non-deterministic weight gradient to the
        # deterministic program by default: bitwise equal either way
        assert same_bits(got[0], ref[0]) and same_bits(got[1], ref[1])
