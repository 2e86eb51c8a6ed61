"""Host logic of the autograd wrapper: recording the backward's tensors
before the forward computation (what lets a checkpoint recompute with early
stop end before the forward kernel).  Runs on the CPU with a stand-in
Function whose forward is a CPU matmul; the GPU tests run the real one."""
import pytest

torch = pytest.importorskip("torch")
from torch.utils.checkpoint import checkpoint, set_checkpoint_early_stop

from dense_ragged_grouped_amd.autograd import save_before_compute, saved

CALLS = {"forward": 0}


class StandIn(torch.autograd.Function):
    """Y = X W^T with the wrapper's save order (save, then compute)."""

    @staticmethod
    def forward(ctx, x, w):
        save_before_compute(ctx, x, w)
        CALLS["forward"] += 1
        return x @ w.t()

    @staticmethod
    def backward(ctx, g):
        x, w = saved(ctx)
        return g @ w, g.t() @ x


def grads(fn, x, w):
    CALLS["forward"] = 0
    y = fn(x, w)
    g = torch.autograd.grad(y.sum(), (x, w))
    return CALLS["forward"], g


@pytest.fixture
def xw():
    gen = torch.Generator().manual_seed(5)
    x = torch.randn(16, 8, generator=gen, dtype=torch.float64, requires_grad=True)
    w = torch.randn(4, 8, generator=gen, dtype=torch.float64, requires_grad=True)
    return x, w


def test_plain_and_checkpointed_gradients_and_forward_counts(xw):
    x, w = xw
    ref = torch.autograd.grad((x @ w.t()).sum(), (x, w))
    n, g = grads(StandIn.apply, x, w)
    assert n == 1 and all(torch.equal(a, b) for a, b in zip(g, ref))
    with set_checkpoint_early_stop(False):
        n, g = grads(lambda a, b: checkpoint(StandIn.apply, a, b, use_reentrant=False), x, w)
    assert n == 2, "without early stop the backward recomputes the forward"
    assert all(torch.equal(a, b) for a, b in zip(g, ref))
    with set_checkpoint_early_stop(True):
        n, g = grads(lambda a, b: checkpoint(StandIn.apply, a, b, use_reentrant=False), x, w)
    assert n == 1, "with early stop the recompute ends before the forward computation"
    assert all(torch.equal(a, b) for a, b in zip(g, ref))


def test_early_stop_still_computes_what_a_later_op_needs(xw):
    """A later op of the checkpointed region saves Y: the recompute must run
    the forward, and the gradients stay exact."""
    x, w = xw
    region = lambda a, b: torch.tanh(StandIn.apply(a, b))
    ref = torch.autograd.grad(torch.tanh(x @ w.t()).sum(), (x, w))
    with set_checkpoint_early_stop(True):
        n, g = grads(lambda a, b: checkpoint(region, a, b, use_reentrant=False), x, w)
    assert n == 2
    assert all(torch.allclose(a, b, rtol=1e-12, atol=1e-12) for a, b in zip(g, ref))


def test_other_saved_tensor_hooks_see_the_tensors(xw):
    """Under a user's saved-tensor hooks the tensors go through them."""
    x, w = xw
    seen = []

    def pack(t):
        seen.append(t.shape)
        return t.clone()

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        n, g = grads(StandIn.apply, x, w)
    ref = torch.autograd.grad((x @ w.t()).sum(), (x, w))
    assert seen[:2] == [x.shape, w.shape]
    assert all(torch.equal(a, b) for a, b in zip(g, ref))
