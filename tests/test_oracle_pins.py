"""Pins of the CPU oracle against facts that do not come from the oracle.

Every oracle function is pinned here (CPU only):

* integer-valued inputs: fwd/dgrad/wgrad equal numpy int64 matrix products
  per expert slice, exactly (a library routine on a special case where
  every sum is exact);
* general inputs: within 1e-12 of numpy float64 matmul (another summation
  order);
* closed forms: identity weights, one-hot routing = the dense call, empty
  experts give +0 weight gradients, grouped = a loop of dense calls;
* finite differences: dgrad and wgrad are the exact gradients of
  <R, fwd(X, W)> (linear, so the central difference is exact on integer
  inputs);
* the hand-worked example in tests/golden/;
* rounding: ties to even, no double rounding, overflow, NaN, agreement with
  torch's float32 -> bfloat16 conversion and numpy's float64 -> float32;
* the router: BF16-representable inputs make the emulation exact, the
  split-algebra closed form for a single product, and the error bound of
  the dropped terms.

A plausible mistake anywhere in the oracle (a dropped term, a wrong sign or
index, a transposed operand, an off-by-one expert boundary, double rounding)
fails at least one of these.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(a):
    """Exact float -> BF16 bits for values that are BF16-representable."""
    b = synth.to_bf16_bits(np.asarray(a, dtype=np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(b), np.asarray(a, dtype=np.float32))
    return b


def f64(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def ragged_case(seed, E, M, N, K, empty=(), integer=True):
    counts = synth.ragged_counts(seed, M, E, empty)
    offs = synth.offsets_from_counts(counts)
    X = synth.bf16_tensor(seed * 10 + 1, (M, K), 1.0, integer)
    W = synth.bf16_tensor(seed * 10 + 2, (E, N, K), 0.02, integer)
    G = synth.bf16_tensor(seed * 10 + 3, (M, N), 1.0, integer)
    return offs, X, W, G


def per_expert(offs):
    return [(int(offs[e]), int(offs[e + 1])) for e in range(len(offs) - 1)]


CASES = [
    # seed, E, M, N, K, empty experts
    (1, 1, 37, 9, 13, ()),
    (2, 3, 61, 8, 16, (1,)),
    (3, 4, 97, 24, 17, (0, 3)),
    (4, 4, 5, 1, 1, ()),
    (5, 3, 0, 4, 8, ()),
    (6, 5, 130, 16, 24, (2,)),
]


@pytest.mark.parametrize("seed,E,M,N,K,empty", CASES)
def test_integer_inputs_equal_int64_matmul(seed, E, M, N, K, empty):
    offs, X, W, G = ragged_case(seed, E, M, N, K, empty)
    xi, wi, gi = (f64(a).astype(np.int64) for a in (X, W, G))
    y, _ = oracle.fwd(X, W, offs)
    dx, _ = oracle.dgrad(G, W, offs)
    dw, _ = oracle.wgrad(X, G, offs)
    for e, (a, b) in enumerate(per_expert(offs)):
        assert np.array_equal(y[a:b], (xi[a:b] @ wi[e].T).astype(np.float64))
        assert np.array_equal(dx[a:b], (gi[a:b] @ wi[e]).astype(np.float64))
        assert np.array_equal(dw[e], (gi[a:b].T @ xi[a:b]).astype(np.float64))


@pytest.mark.parametrize("seed,E,M,N,K,empty", CASES)
def test_float_inputs_match_float64_matmul(seed, E, M, N, K, empty):
    offs, X, W, G = ragged_case(seed, E, M, N, K, empty, integer=False)
    x, w, g = f64(X), f64(W), f64(G)
    y, _ = oracle.fwd(X, W, offs)
    dx, _ = oracle.dgrad(G, W, offs)
    dw, _ = oracle.wgrad(X, G, offs)
    for e, (a, b) in enumerate(per_expert(offs)):
        np.testing.assert_allclose(y[a:b], x[a:b] @ w[e].T, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dx[a:b], g[a:b] @ w[e], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dw[e], g[a:b].T @ x[a:b], rtol=1e-12, atol=1e-13)


def test_sumsq_scale_matches_library():
    offs, X, W, G = ragged_case(7, 3, 50, 12, 20, (1,))
    x, w, g = f64(X), f64(W), f64(G)
    _, qy = oracle.fwd(X, W, offs)
    _, qx = oracle.dgrad(G, W, offs)
    _, qw = oracle.wgrad(X, G, offs)
    for e, (a, b) in enumerate(per_expert(offs)):
        assert np.array_equal(qy[a:b], np.sqrt((x[a:b] ** 2) @ (w[e] ** 2).T))
        assert np.array_equal(qx[a:b], np.sqrt((g[a:b] ** 2) @ (w[e] ** 2)))
        assert np.array_equal(qw[e], np.sqrt((g[a:b] ** 2).T @ (x[a:b] ** 2)))


def test_identity_weights_return_inputs():
    E, M, D = 3, 40, 16
    counts = synth.ragged_counts(11, M, E)
    offs = synth.offsets_from_counts(counts)
    X = synth.bf16_tensor(111, (M, D), 1.0)
    G = synth.bf16_tensor(113, (M, D), 1.0)
    W = np.broadcast_to(bf(np.eye(D, dtype=np.float32)), (E, D, D)).copy()
    y, qy = oracle.fwd(X, W, offs)
    dx, _ = oracle.dgrad(G, W, offs)
    assert np.array_equal(y, f64(X))
    assert np.array_equal(dx, f64(G))
    assert np.array_equal(qy, np.abs(f64(X)))


def test_one_hot_routing_equals_dense_call():
    M, N, K = 33, 10, 14
    X = synth.bf16_tensor(21, (M, K), 1.0)
    W = synth.bf16_tensor(22, (3, N, K), 0.02)
    G = synth.bf16_tensor(23, (M, N), 1.0)
    grouped = np.array([0, 0, M, M], dtype=np.int32)     # every token on expert 1
    dense = np.array([0, M], dtype=np.int32)
    assert np.array_equal(oracle.fwd(X, W, grouped)[0], oracle.fwd(X, W[1:2], dense)[0])
    assert np.array_equal(oracle.dgrad(G, W, grouped)[0], oracle.dgrad(G, W[1:2], dense)[0])
    dw = oracle.wgrad(X, G, grouped)[0]
    assert np.array_equal(dw[1], oracle.wgrad(X, G, dense)[0][0])
    assert not np.any(dw[0]) and not np.any(dw[2])


def test_empty_experts_give_positive_zero_weight_gradient():
    offs, X, W, G = ragged_case(31, 4, 50, 8, 8, empty=(1, 3), integer=False)
    dw, q = oracle.wgrad(X, G, offs)
    for e in (1, 3):
        assert offs[e] == offs[e + 1]
        assert np.all(dw[e] == 0.0) and not np.any(np.signbit(dw[e]))
        assert np.all(q[e] == 0.0)
    assert np.all(np.abs(dw[0]) > 0) or dw[0].size == 0


def test_grouped_equals_loop_of_dense_calls():
    offs, X, W, G = ragged_case(41, 4, 77, 12, 9, empty=(2,), integer=False)
    y = oracle.fwd(X, W, offs)[0]
    dx = oracle.dgrad(G, W, offs)[0]
    dw = oracle.wgrad(X, G, offs)[0]
    for e, (a, b) in enumerate(per_expert(offs)):
        d = np.array([0, b - a], dtype=np.int32)
        assert np.array_equal(y[a:b], oracle.fwd(X[a:b], W[e:e + 1], d)[0])
        assert np.array_equal(dx[a:b], oracle.dgrad(G[a:b], W[e:e + 1], d)[0])
        assert np.array_equal(dw[e], oracle.wgrad(X[a:b], G[a:b], d)[0][0])


@pytest.mark.parametrize("seed", [51, 52])
def test_finite_differences_of_forward(seed):
    """L(X, W) = <R, fwd(X, W)> is linear in X and in W, so on integer inputs
    the central difference is exact: it must equal <dgrad(R, W), D> and
    <wgrad(X, R), D>."""
    offs, X, W, R = ragged_case(seed, 3, 45, 7, 11, empty=(1,))
    rng = np.random.default_rng(seed)
    r = f64(R)

    def loss(Xb, Wb):
        return float(np.sum(r * oracle.fwd(Xb, Wb, offs)[0]))

    D = rng.integers(-2, 3, size=X.shape).astype(np.float32)
    x = synth.bf16_bits_to_f32(X)
    fd = (loss(bf(x + D), W) - loss(bf(x - D), W)) / 2.0
    assert fd == float(np.sum(oracle.dgrad(R, W, offs)[0] * D))

    DW = rng.integers(-2, 3, size=W.shape).astype(np.float32)
    w = synth.bf16_bits_to_f32(W)
    fd = (loss(X, bf(w + DW)) - loss(X, bf(w - DW))) / 2.0
    assert fd == float(np.sum(oracle.wgrad(X, R, offs)[0] * DW))


def test_hand_worked_golden_example():
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example_e2_m3.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *nums = line.split()
                vals[key] = np.array([float(v) for v in nums])
    offs = vals["offsets"].astype(np.int32)
    X = bf(vals["X"].reshape(3, 2))
    W = bf(vals["W"].reshape(2, 2, 2))
    G = bf(vals["G"].reshape(3, 2))
    assert np.array_equal(oracle.fwd(X, W, offs)[0].ravel(), vals["Y"])
    assert np.array_equal(oracle.dgrad(G, W, offs)[0].ravel(), vals["dX"])
    assert np.array_equal(oracle.wgrad(X, G, offs)[0].ravel(), vals["dW"])


def test_sampled_elements_equal_full_result():
    offs, X, W, G = ragged_case(61, 4, 70, 12, 10, empty=(2,), integer=False)
    rng = np.random.default_rng(61)
    for fn, a, b, shape in ((oracle.fwd, X, W, (70, 12)), (oracle.dgrad, G, W, (70, 10)),
                            (oracle.wgrad, X, G, (4, 12, 10))):
        full, qf = fn(a, b, offs)
        idx = rng.integers(0, full.size, size=40)
        v, q = fn(a, b, offs, idx=idx)
        assert np.array_equal(v, full.ravel()[idx]) and np.array_equal(q, qf.ravel()[idx])


def test_bad_offsets_are_rejected():
    X = synth.bf16_tensor(1, (10, 4), 1.0)
    W = synth.bf16_tensor(2, (2, 3, 4), 1.0)
    for bad in ([0, 6, 5], [1, 5, 10], [0, 5, 9], [0, 11, 10]):
        with pytest.raises(ValueError):
            oracle.fwd(X, W, np.array(bad, dtype=np.int32))


# ---- rounding -------------------------------------------------------------

def bits_to_f32(u16):
    return synth.bf16_bits_to_f32(np.asarray(u16, dtype=np.uint16))


def test_bf16_rounding_closed_forms():
    cases = [
        (1.0, 1.0),
        (1.0 + 2.0 ** -8, 1.0),                        # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),        # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -7),  # above the tie: no double rounding
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), -(1.0 + 2.0 ** -7)),
        (1.0 + 2.0 ** -9, 1.0),
        (3.0 * 2.0 ** -133, 3.0 * 2.0 ** -133),        # subnormal, exact
        (2.5 * 2.0 ** -133, 2.0 * 2.0 ** -133),        # subnormal tie -> even
        (2.0 ** -134, 0.0),                            # half the smallest subnormal: tie -> 0
        (2.0 ** -134 * 1.5, 2.0 ** -133),
        ((2 - 2.0 ** -8) * 2.0 ** 127, np.inf),        # rounds up past the largest finite
        ((2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),
        (-1e300, -np.inf),
        (np.inf, np.inf),
    ]
    src = np.array([c[0] for c in cases], dtype=np.float64)
    got = bits_to_f32(oracle.round_bf16(src)).astype(np.float64)
    want = np.array([c[1] for c in cases], dtype=np.float64)
    assert np.array_equal(got, want), (got, want)
    assert np.isnan(bits_to_f32(oracle.round_bf16(np.array([np.nan])))[0])
    assert np.signbit(bits_to_f32(oracle.round_bf16(np.array([-0.0])))[0])


def test_bf16_rounding_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.round_bf16(f.astype(np.float64))
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_f32_rounding_matches_numpy():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(100000) * np.exp(rng.uniform(-80, 80, 100000))
    assert np.array_equal(oracle.round_f32(v), v.astype(np.float32))


# ---- router ---------------------------------------------------------------

def test_router_bf16_representable_inputs_make_emulation_exact():
    rng = np.random.default_rng(8)
    X = synth.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((9, 64), dtype=np.float32)))
    Wr = synth.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((5, 64), dtype=np.float32)))
    assert np.array_equal(oracle.router_bf16x3(X, Wr), oracle.router_exact(X, Wr))
    np.testing.assert_allclose(oracle.router_exact(X, Wr), X.astype(np.float64) @ Wr.T.astype(np.float64),
                               rtol=1e-13, atol=1e-13)


def test_router_split_algebra_single_product():
    # x = 1 + 2^-8 + 2^-12: hi = 1 + 2^-7, lo = -(2^-8 - 2^-12) (both exact);
    # x*x - emulation = lo*lo exactly (the dropped term).
    x = np.float32(1.0 + 2.0 ** -8 + 2.0 ** -12)
    lo = -(2.0 ** -8 - 2.0 ** -12)
    X = np.array([[x]], dtype=np.float32)
    ex = oracle.router_exact(X, X)[0, 0]
    em = oracle.router_bf16x3(X, X)[0, 0]
    assert ex - em == lo * lo
    one = np.array([[1.0]], dtype=np.float32)
    assert oracle.router_bf16x3(X, one)[0, 0] == float(x)


def test_router_emulation_error_bound():
    """x = hi + lo + r with |r| <= 2^-16 |x|: dropping lo*lo and the residuals
    leaves |x w - emulation| <= 2^-14 |x w| per product."""
    rng = np.random.default_rng(9)
    X = rng.standard_normal((16, 256), dtype=np.float32)
    Wr = rng.standard_normal((8, 256), dtype=np.float32)
    ex = oracle.router_exact(X, Wr)
    em = oracle.router_bf16x3(X, Wr)
    absdot = np.abs(X.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T
    err = np.abs(ex - em)
    assert np.all(err <= 2.0 ** -14 * absdot)
    assert np.any(err > 0)                      # the emulation really is an approximation
    rel = np.linalg.norm(ex - em) / np.linalg.norm(ex)
    assert rel < 1e-5
