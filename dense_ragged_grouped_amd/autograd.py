"""Autograd over the grouped GEMM: the per-expert linear layer of a
mixture-of-experts block, Y[t] = X[t] W[e(t)]^T for the tokens of each
expert's contiguous range, with the backward dX = G W and dW = G^T X.

Every product runs in the library's kernels (forward, data gradient, weight
gradient); this module only wires them into torch.autograd.  It is the layer
behind the checkpointed training step that PR #8258 times ("Operations and
shapes", its ckpt and ckpt ES rows): the layer wrapped in activation
checkpointing without re-entry, run forward and backward, once with the
early-stop option of the checkpoint disabled and once enabled.

Checkpoint early stop.  A custom autograd Function saves its tensors only
after its forward has returned, so a non-reentrant checkpoint recomputing it
would run the forward kernel even when early stop could end the recompute
as soon as the saved tensors are back, and those are just the inputs X, W
and the offsets (the same PR page notes that skipping this recompute is what
makes "ckpt ES" faster).  GroupedLinearFunction therefore hands its tensors to
the active saved-tensor hooks itself, before the forward kernel: inside a
checkpoint recompute with early stop the hook ends the recompute there, and
the kernel is not launched; with early stop off, or when a later operation of
the checkpointed region needs Y, the forward runs as usual.  Outside any hook
it uses save_for_backward.
"""
import warnings

import torch

from . import grouped_gemm_dgrad, grouped_gemm_fwd, grouped_gemm_wgrad

# torch's accessor for the innermost active saved-tensor hooks (internal API)
_TOP_HOOKS = getattr(torch._C._autograd, "_top_saved_tensors_default_hooks", None)
if _TOP_HOOKS is None:
    warnings.warn("torch has no _top_saved_tensors_default_hooks: grouped_linear saves its tensors after the "
                  "forward kernel, so a checkpoint with early stop still recomputes the forward", RuntimeWarning)


def save_before_compute(ctx, *tensors):
    """Record `tensors` for the backward now, through the innermost
    saved-tensor hooks if any are active (a checkpoint, CPU offloading), else
    with save_for_backward.  Without torch's accessor for those hooks (warned
    at import) the tensors are saved with save_for_backward, which is
    correct but lets an early-stopping checkpoint run the forward kernel."""
    hooks = _TOP_HOOKS(False) if _TOP_HOOKS is not None else None
    if hooks is None:
        ctx.packed = None
        ctx.save_for_backward(*tensors)
    else:
        pack, unpack = hooks
        ctx.packed = (unpack, [pack(t) for t in tensors])


def saved(ctx):
    """The tensors recorded by save_before_compute, in order."""
    if ctx.packed is None:
        return ctx.saved_tensors
    unpack, handles = ctx.packed
    return tuple(unpack(h) for h in handles)


class GroupedLinearFunction(torch.autograd.Function):
    """Y = grouped_gemm_fwd(X, W, offsets); backward: dX = grouped_gemm_dgrad(G,
    W, offsets), dW = grouped_gemm_wgrad(X, G, offsets) in W's dtype, the
    weight gradient deterministic (bitwise reproducible) unless
    `deterministic` is False."""

    @staticmethod
    def forward(ctx, X, W, group_offsets, deterministic):
        save_before_compute(ctx, X, W, group_offsets)
        ctx.deterministic = bool(deterministic)
        return grouped_gemm_fwd(X, W, group_offsets, out_dtype=X.dtype)

    @staticmethod
    def backward(ctx, G):
        X, W, offs = saved(ctx)
        G = G.contiguous()
        dX = dW = None
        if ctx.needs_input_grad[0]:
            dX = grouped_gemm_dgrad(G, W, offs, out_dtype=X.dtype)
        if ctx.needs_input_grad[1]:
            dW = grouped_gemm_wgrad(X, G, offs, out_dtype=W.dtype, deterministic=ctx.deterministic)
        return dX, dW, None, None


def grouped_linear(X, W, group_offsets, deterministic=True):
    """Y[t] = X[t] W[e]^T for the tokens t of expert e (rows group_offsets[e]
    .. group_offsets[e+1]-1), differentiable in X and W.  X [M, K] and W
    [E, N, K] BF16, group_offsets int32 [E+1] on the device."""
    return GroupedLinearFunction.apply(X, W, group_offsets, deterministic)


def checkpointed_grouped_linear(X, W, group_offsets, deterministic=True, early_stop=True):
    """grouped_linear inside a non-reentrant activation checkpoint: the
    forward keeps no activations, and the backward recomputes what it needs;
    with early_stop (torch's default) that recompute ends before the forward
    kernel, so a step costs one forward and the backward, else two forwards
    and the backward."""
    from torch.utils.checkpoint import checkpoint, set_checkpoint_early_stop
    with set_checkpoint_early_stop(early_stop):
        return checkpoint(grouped_linear, X, W, group_offsets, deterministic, use_reentrant=False)
