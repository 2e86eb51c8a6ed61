"""Batched projection GEMM on the GPU: B independent products of one shape
through the grouped kernels with uniform groups and strided token-major
buffers.  Bitwise equal to the grouped call on contiguous rows, a
head-interleaved layout ([T, H, K] used in place) gives the same bits, and
the results match the oracle."""
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
    return d


def problem(seed, B, T, N, K):
    counts = np.full(B, T, dtype=np.int64)
    return synth.make_problem(f"batched_s{seed}", seed, counts, N=N, K=K, w_std=0.02)


def dev(prob, B, T):
    X = parity.to_dev_bf16(prob.X).view(B, T, prob.K)
    G = parity.to_dev_bf16(prob.G).view(B, T, prob.N)
    W = parity.to_dev_bf16(prob.W)
    return X, W, G, parity.to_dev(prob.offs)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_batched_equals_grouped_with_uniform_groups(drgg, out_dtype):
    B, T, N, K = 5, 300, 136, 200
    prob = problem(501, B, T, N, K)
    X, W, G, offs = dev(prob, B, T)
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    print(f"batched vs grouped B={B} T={T} N={N} K={K} {out_dtype}", flush=True)
    y = drgg.batched_gemm_fwd(X, W, out_dtype=dt)
    dx = drgg.batched_gemm_dgrad(G, W, out_dtype=dt)
    dw = drgg.batched_gemm_wgrad(X, G, out_dtype=dt)
    y0 = drgg.grouped_gemm_fwd(X.reshape(B * T, K), W, offs, out_dtype=dt)
    dx0 = drgg.grouped_gemm_dgrad(G.reshape(B * T, N), W, offs, out_dtype=dt)
    dw0 = drgg.grouped_gemm_wgrad(X.reshape(B * T, K), G.reshape(B * T, N), offs, out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(bits(y.reshape(B * T, N)), bits(y0))
    assert torch.equal(bits(dx.reshape(B * T, K)), bits(dx0))
    assert torch.equal(bits(dw), bits(dw0))
    bf = out_dtype == "bf16"
    parity.compare(prob, "fwd", parity.from_dev(y.reshape(B * T, N)), bf, what="batched fwd")
    parity.compare(prob, "dgrad", parity.from_dev(dx.reshape(B * T, K)), bf, what="batched dgrad")
    parity.compare(prob, "wgrad", parity.from_dev(dw), bf, what="batched wgrad")


def test_head_interleaved_layout_in_place(drgg):
    """Activations [T, H, K] and gradients [T, H, N] with batch = head, read
    and written in place through their strides: the same bits as the
    contiguous [H, T, .] copies."""
    H, T, N, K = 8, 520, 64, 128
    gen = torch.Generator(device="cuda").manual_seed(7)
    Xi = torch.randn(T, H, K, device="cuda", generator=gen).to(torch.bfloat16)
    Gi = torch.randn(T, H, N, device="cuda", generator=gen).to(torch.bfloat16)
    W = (0.02 * torch.randn(H, N, K, device="cuda", generator=gen)).to(torch.bfloat16)
    Xv, Gv = Xi.transpose(0, 1), Gi.transpose(0, 1)          # [H, T, .] views, strided
    assert not Xv.is_contiguous() and Xv.stride() == (K, H * K, 1)
    Xc, Gc = Xv.contiguous(), Gv.contiguous()
    print(f"head-interleaved H={H} T={T} N={N} K={K}", flush=True)
    Yi = torch.empty(T, H, N, dtype=torch.bfloat16, device="cuda")
    drgg.batched_gemm_fwd(Xv, W, out=Yi.transpose(0, 1))
    dXi = torch.empty(T, H, K, dtype=torch.float32, device="cuda")
    drgg.batched_gemm_dgrad(Gv, W, out_dtype=torch.float32, out=dXi.transpose(0, 1))
    dW = drgg.batched_gemm_wgrad(Xv, Gv, out_dtype=torch.float32)
    y = drgg.batched_gemm_fwd(Xc, W)
    dx = drgg.batched_gemm_dgrad(Gc, W, out_dtype=torch.float32)
    dw = drgg.batched_gemm_wgrad(Xc, Gc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(bits(Yi.transpose(0, 1).contiguous()), bits(y))
    assert torch.equal(bits(dXi.transpose(0, 1).contiguous()), bits(dx))
    assert torch.equal(bits(dW), bits(dw))
    # against a plain float64 product per head on a few heads
    for h in (0, H - 1):
        ref = Xc[h].double() @ W[h].double().t()
        err = (y[h].double() - ref).abs().max().item()
        assert err <= 2 ** -6 * ref.abs().max().item() + 1e-3, (h, err)


def test_no_tokens(drgg):
    B, N, K = 3, 64, 64
    X = torch.empty(B, 0, K, dtype=torch.bfloat16, device="cuda")
    G = torch.empty(B, 0, N, dtype=torch.bfloat16, device="cuda")
    W = torch.ones(B, N, K, dtype=torch.bfloat16, device="cuda")
    assert drgg.batched_gemm_fwd(X, W).shape == (B, 0, N)
    dw = drgg.batched_gemm_wgrad(X, G, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not torch.any(bits(dw))
