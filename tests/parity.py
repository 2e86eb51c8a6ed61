"""Parity helpers for the GPU tests: move seeded inputs to the device and
compare GPU outputs with the CPU oracle.

Tolerances (written here, used by every parity test):

* FP32 outputs: relative Frobenius error <= 1e-5 AND per element
  |gpu - ref| <= 1e-4 * sqrt(K_red) * max|a| * max|b|, where K_red is the
  reduction length of that element (K for the forward, N for the data
  gradient, T_e for the weight gradient) and max|a|, max|b| are taken over the
  two operand slices that feed that element.
* BF16 outputs: per element |gpu - bf16(ref)| <= 2 BF16 ulps of ref, OR
  |gpu - ref| <= ulp(ref)/2 + 8 * 2^-24 * sqrt(K_red) * q, with
  q = sqrt(sum of squared products) from the oracle.  The second clause is
  the floor for outputs that nearly cancel: FP32 accumulation (which the
  method prescribes) has an error of order 2^-24 sqrt(K_red) q that no
  rounding of the result can undo, so a pure ulp bound cannot hold where
  |ref| is far below that.  The elements that needed the floor must be rare.
  An element needs it when |ref| is within a few hundred times its
  accumulation error of zero; relative to the spread of the outputs that
  error grows like sqrt(K_red), and so does the chance.  The bound is
  1 per million times sqrt(K_red) per element checked, plus 3 (so that a
  sample of a few thousand elements is not failed by one near-zero output):
  128 per million at K_red = 16384, where the kernels measured 23-30, and
  45 per million at K_red = 2048.  The worst error in BF16 ulps of the
  elements that passed the ulp clause is reported.
* Integer-valued inputs: every partial sum is exact in FP32, so the GPU must
  equal the oracle bit for bit, in every mode.
"""
from __future__ import annotations

import numpy as np

import oracle


def to_dev_bf16(u16, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev(arr, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def from_dev(t):
    """Device tensor -> numpy (BF16 as uint16 bits, FP32 as float32)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_ulp(x):
    """Spacing of BF16 values at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def check_fp32(gpu, ref, kred, amax_a, amax_b, what=""):
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    err = np.abs(gpu - ref)
    bound = 1e-4 * np.sqrt(np.asarray(kred, dtype=np.float64).ravel()) * \
        np.asarray(amax_a, dtype=np.float64).ravel() * np.asarray(amax_b, dtype=np.float64).ravel()
    bad = err > bound
    assert not np.any(bad), (f"{what}: {bad.sum()} of {bad.size} elements beyond the per-element bound; "
                             f"first at {np.flatnonzero(bad)[:5]}: gpu {gpu[bad][:5]} ref {ref[bad][:5]}")
    nref = np.linalg.norm(ref)
    if nref > 0:
        rel = np.linalg.norm(gpu - ref) / nref
        assert rel <= 1e-5, f"{what}: relative Frobenius error {rel:.3e} > 1e-5"
    else:
        assert np.all(gpu == 0), f"{what}: reference is zero but the GPU result is not"


FLOOR_PPM_PER_SQRT_K = 1.0   # elements allowed to need the floor, per million, times sqrt(K_red)
FLOOR_SLACK = 3              # ... plus this many


def check_bf16(gpu_u16, ref, q, kred, what=""):
    """Returns the number of elements that needed the accumulation floor
    (bounded by FLOOR_PPM_PER_SQRT_K per million times sqrt(K_red), summed
    over the elements, + FLOOR_SLACK)."""
    g = bf16_to_f64(np.asarray(gpu_u16).ravel())
    ref = np.asarray(ref, dtype=np.float64).ravel()
    q = np.asarray(q, dtype=np.float64).ravel()
    kred = np.asarray(kred, dtype=np.float64).ravel()
    r16 = bf16_to_f64(oracle.round_bf16(ref))
    ulp = bf16_ulp(ref)
    ok_ulp = np.abs(g - r16) <= 2 * ulp
    floor = 0.5 * ulp + 8.0 * 2.0 ** -24 * np.sqrt(kred) * q
    ok_floor = np.abs(g - ref) <= floor
    bad = ~(ok_ulp | ok_floor)
    assert not np.any(bad), (f"{what}: {bad.sum()} of {bad.size} BF16 elements out of tolerance; "
                             f"first at {np.flatnonzero(bad)[:5]}: gpu {g[bad][:5]} ref {ref[bad][:5]}")
    n_floor = int(np.sum(~ok_ulp))
    limit = FLOOR_PPM_PER_SQRT_K * 1e-6 * float(np.sum(np.sqrt(kred))) + FLOOR_SLACK
    assert n_floor <= limit, (f"{what}: {n_floor} of {g.size} elements needed the FP32-accumulation floor "
                              f"(limit {limit:.1f})")
    if g.size:
        worst = float(np.max(np.where(ok_ulp, np.abs(g - r16) / ulp, 0.0)))
        check_bf16.last_worst_ulp = worst
    return n_floor


check_bf16.last_worst_ulp = 0.0


def expert_of_rows(offs, M):
    return np.searchsorted(np.asarray(offs[1:], dtype=np.int64), np.arange(M), side="right")


def _mag(u16):
    """|value| ordering of BF16 bit patterns as integers (finite inputs)."""
    return np.asarray(u16, dtype=np.uint16) & np.uint16(0x7FFF)


def _mag_to_f64(m):
    return bf16_to_f64(np.asarray(m, dtype=np.uint16))


def operand_scales(prob, program, idx=None):
    """(kred, amax_a, amax_b) per output element (flat row-major index array
    idx, or all elements) for the FP32 per-element bound.  Maxima are taken
    on the BF16 bit patterns (magnitude order = integer order), so no
    full-size float copy of an operand is made."""
    offs = prob.offs.astype(np.int64)
    E, M, N, K = prob.E, prob.M, prob.N, prob.K
    if program == "fwd":
        idx = np.arange(M * N) if idx is None else np.asarray(idx)
        t, n = idx // N, idx % N
        e = expert_of_rows(offs, M)[t]
        ax = _mag_to_f64(_mag(prob.X).max(axis=1))
        aw = _mag_to_f64(_mag(prob.W).max(axis=2))               # [E, N]
        return np.full(idx.size, K), ax[t], aw[e, n]
    if program == "dgrad":
        idx = np.arange(M * K) if idx is None else np.asarray(idx)
        t, k = idx // K, idx % K
        e = expert_of_rows(offs, M)[t]
        ag = _mag_to_f64(_mag(prob.G).max(axis=1))
        aw = _mag_to_f64(_mag(prob.W).max(axis=1))               # [E, K]
        return np.full(idx.size, N), ag[t], aw[e, k]
    if program == "wgrad":
        idx = np.arange(E * N * K) if idx is None else np.asarray(idx)
        e, r = idx // (N * K), idx % (N * K)
        n, k = r // K, r % K
        ag = np.zeros((E, N))
        ax = np.zeros((E, K))
        for ee in np.unique(e):
            a, b = offs[ee], offs[ee + 1]
            if b > a:
                ag[ee] = _mag_to_f64(_mag(prob.G[a:b]).max(axis=0))
                ax[ee] = _mag_to_f64(_mag(prob.X[a:b]).max(axis=0))
        return (offs[e + 1] - offs[e]), ag[e, n], ax[e, k]
    raise ValueError(program)


def sample_indices(prob, program, n_random=3000, seed=0):
    """Flat output indices for sampled parity at full size: random elements
    plus the first and last row of every expert's range (and of every 256-row
    tile inside it for the forward and data gradient), the last column, and
    for the weight gradient the corners of every expert's output."""
    rng = np.random.default_rng(seed)
    offs = prob.offs.astype(np.int64)
    E, M, N, K = prob.E, prob.M, prob.N, prob.K
    if program in ("fwd", "dgrad"):
        cols = N if program == "fwd" else K
        size = M * cols
        rows = []
        for e in range(E):
            a, b = offs[e], offs[e + 1]
            for r0 in range(a, b, 256):
                rows += [r0, min(r0 + 255, b - 1)]
        rows = np.unique(np.array(rows, dtype=np.int64)) if rows else np.zeros(0, np.int64)
        c = np.concatenate([[0, cols - 1], rng.integers(0, cols, 2)])
        struct = (rows[:, None] * cols + c[None, :]).ravel()
    else:
        size = E * N * K
        struct = []
        for e in range(E):
            base = e * N * K
            struct += [base, base + K - 1, base + (N - 1) * K, base + N * K - 1]
        struct = np.array(struct, dtype=np.int64)
    if size == 0:
        return np.zeros(0, dtype=np.int64)
    rand = rng.integers(0, size, n_random)
    return np.unique(np.concatenate([struct, rand]).astype(np.int64))


def tile_indices(prob, program, tile=256, seed=0):
    """Flat output indices of four whole tile x tile output blocks (every
    element of each, clipped to the output): the first block, the last one,
    one that straddles an expert boundary (forward and data gradient: rows
    across the start of the second non-empty expert; weight gradient: a block
    of the expert with the most tokens) and a random one."""
    rng = np.random.default_rng(seed + 17)
    offs = prob.offs.astype(np.int64)
    E, M, N, K = prob.E, prob.M, prob.N, prob.K
    blocks = []   # (expert or -1, row0, col0)
    if program in ("fwd", "dgrad"):
        cols = N if program == "fwd" else K
        rows = M
        nonempty = [e for e in range(E) if offs[e + 1] > offs[e]]
        boundary = offs[nonempty[1]] - tile // 2 if len(nonempty) > 1 else rows // 2
        starts = [(0, 0), (max(rows - tile, 0), max(cols - tile, 0)),
                  (min(max(boundary, 0), max(rows - tile, 0)), int(rng.integers(0, max(cols - tile, 0) + 1))),
                  (int(rng.integers(0, max(rows - tile, 0) + 1)), int(rng.integers(0, max(cols - tile, 0) + 1)))]
        idx = []
        for r0, c0 in starts:
            r = np.arange(r0, min(r0 + tile, rows))
            c = np.arange(c0, min(c0 + tile, cols))
            idx.append((r[:, None] * cols + c[None, :]).ravel())
        return np.unique(np.concatenate(idx)).astype(np.int64)
    counts = offs[1:] - offs[:-1]
    nonempty = np.flatnonzero(counts > 0)
    if nonempty.size == 0:
        return np.zeros(0, dtype=np.int64)
    big = int(np.argmax(counts))
    re = int(rng.choice(nonempty))
    starts = [(int(nonempty[0]), 0, 0),
              (int(nonempty[-1]), max(N - tile, 0), max(K - tile, 0)),
              (big, int(rng.integers(0, max(N - tile, 0) + 1)), int(rng.integers(0, max(K - tile, 0) + 1))),
              (re, int(rng.integers(0, max(N - tile, 0) + 1)), int(rng.integers(0, max(K - tile, 0) + 1)))]
    idx = []
    for e, r0, c0 in starts:
        r = np.arange(r0, min(r0 + tile, N))
        c = np.arange(c0, min(c0 + tile, K))
        idx.append((e * N * K + r[:, None] * K + c[None, :]).ravel())
    return np.unique(np.concatenate(idx)).astype(np.int64)


def oracle_program(prob, program, idx=None):
    if program == "fwd":
        return oracle.fwd(prob.X, prob.W, prob.offs, idx)
    if program == "dgrad":
        return oracle.dgrad(prob.G, prob.W, prob.offs, idx)
    return oracle.wgrad(prob.X, prob.G, prob.offs, idx)


def compare(prob, program, gpu, out_bf16, idx=None, integer=False, what=""):
    """Compare a GPU output (numpy, full array) with the oracle on all
    elements (idx None) or on the flat indices idx.  Returns the number of
    BF16 elements that needed the floor (0 for FP32 outputs)."""
    ref, q = oracle_program(prob, program, idx)
    g = np.asarray(gpu).ravel() if idx is None else np.asarray(gpu).ravel()[np.asarray(idx)]
    ref = ref.ravel()
    if integer:
        want = oracle.round_bf16(ref) if out_bf16 else oracle.round_f32(ref)
        if out_bf16:
            assert np.array_equal(g.astype(np.uint16), want), f"{what}: integer inputs must match bit for bit"
        else:
            assert np.array_equal(g.astype(np.float32).view(np.uint32), want.view(np.uint32)), \
                f"{what}: integer inputs must match bit for bit"
        return 0
    kred, aa, ab = operand_scales(prob, program, idx)
    if out_bf16:
        return check_bf16(g, ref, q, kred, what)
    check_fp32(g, ref, kred, aa, ab, what)
    return 0
