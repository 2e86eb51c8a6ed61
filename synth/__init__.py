"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no arithmetic of the GEMM itself: it only draws random
numbers, stores them as BF16 (or FP32) bit patterns and builds group offsets.
Both the GPU path and the CPU oracle are fed from here.

Workloads (the shapes and distributions of the five workloads the grouped GEMM
is measured on; the pages time only synthetic shapes -- flashinfer PR #8258,
"Operations and shapes"; PR #8363, the dense K1 tables):

1. tiny MoE: E=4, 512 tokens, multinomial counts; X [512,256] N(0,1),
   W [4,512,256] N(0,0.02), G [512,512] N(0,1); a forced-empty variant puts
   probability 0 on expert 2.
2. dense projection weight gradient (one group): T=16384, X [16384,4096]
   N(0,1), G [16384,d_out] N(0,0.1), d_out in {48,64,512,1024}.
3. MoE gate_up: E=8 balanced (16384 tokens each), d_model 2048, N=1536;
   X N(0,1), W N(0,0.02), G N(0,1).
4. MoE down, skewed: E=32, 131072 tokens; rank shares p_r ~ r^-1.2 over 30
   ranks, multinomial counts, ranks mapped to expert ids by a seeded
   permutation, the 2 left-over ids empty; K=768, N=2048.
5. square dense 16384 x 4096 x 4096 plus the FP32 router
   [16384,4096] x [256,4096]^T with N(0,1) inputs.

Seeds: ``numpy.random.default_rng(1000*cfg + tensor_id)`` with tensor ids
X=1, W=2, G=3, counts=4, router weights=5 (the router's X uses id 6).
Values are drawn as float32 normals, scaled, then stored as BF16 with round
to nearest even.  ``integer=True`` draws integers in [-4, 4] instead: they
are exact in BF16 and every FP32 partial sum of their products stays exact,
so integer runs can be compared bit for bit.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TID_X, TID_W, TID_G, TID_COUNTS, TID_WR, TID_XR = 1, 2, 3, 4, 5, 6


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest, ties to even.
    The inputs drawn here are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24                      # draw in slices to bound host memory
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        v = rng.standard_normal(n, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[s:s + n] = to_bf16_bits(v)
    return out


def _int_bf16(seed: int, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, hi + 1, size=shape, dtype=np.int8).astype(np.float32)
    return to_bf16_bits(v)


def bf16_tensor(seed: int, shape, std: float = 1.0, integer: bool = False) -> np.ndarray:
    return _int_bf16(seed, shape) if integer else _normal_bf16(seed, shape, std)


def offsets_from_counts(counts) -> np.ndarray:
    c = np.asarray(counts, dtype=np.int64)
    o = np.zeros(c.size + 1, dtype=np.int32)
    o[1:] = np.cumsum(c)
    return o


def multinomial_counts(seed: int, total: int, probs) -> np.ndarray:
    rng = np.random.default_rng(seed)
    p = np.asarray(probs, dtype=np.float64)
    return rng.multinomial(total, p / p.sum())


def zipf_counts(seed: int, total: int, experts: int, empty: int, s: float = 1.2) -> np.ndarray:
    """Rank shares p_r ~ r^-s over the (experts - empty) non-empty ranks,
    multinomial counts, ranks placed on expert ids by a seeded permutation;
    the left-over ids get no tokens."""
    rng = np.random.default_rng(seed)
    ranks = experts - empty
    p = np.arange(1, ranks + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    rank_counts = rng.multinomial(total, p)
    perm = rng.permutation(experts)
    counts = np.zeros(experts, dtype=np.int64)
    counts[perm[:ranks]] = rank_counts
    return counts


def ragged_counts(seed: int, total: int, experts: int, empty=()) -> np.ndarray:
    """Uneven counts for small parity cases: multinomial over random shares,
    with the listed experts forced empty."""
    rng = np.random.default_rng(seed)
    p = rng.uniform(0.2, 1.0, size=experts)
    for e in empty:
        p[e] = 0.0
    if p.sum() == 0:
        return np.zeros(experts, dtype=np.int64)
    return rng.multinomial(total, p / p.sum())


@dataclass
class Problem:
    """Host copies of one grouped-GEMM problem (BF16 as uint16 bits)."""
    name: str
    E: int
    M: int
    N: int
    K: int
    offs: np.ndarray
    X: np.ndarray | None = None   # [M, K]
    W: np.ndarray | None = None   # [E, N, K]
    G: np.ndarray | None = None   # [M, N]
    extra: dict = field(default_factory=dict)

    @property
    def counts(self):
        return np.diff(self.offs.astype(np.int64))


def make_problem(name, cfg_seed, counts, N, K, x_std=1.0, w_std=0.02, g_std=1.0,
                 need=("X", "W", "G"), integer=False) -> Problem:
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    M = int(counts.sum())
    offs = offsets_from_counts(counts)
    base = 1000 * cfg_seed
    p = Problem(name=name, E=E, M=M, N=N, K=K, offs=offs)
    if "X" in need:
        p.X = bf16_tensor(base + TID_X, (M, K), x_std, integer)
    if "W" in need:
        p.W = bf16_tensor(base + TID_W, (E, N, K), w_std, integer)
    if "G" in need:
        p.G = bf16_tensor(base + TID_G, (M, N), g_std, integer)
    return p


# ---- the five workloads --------------------------------------------------

def config1(forced_empty: bool = False, integer: bool = False) -> Problem:
    probs = [1 / 3, 1 / 3, 0.0, 1 / 3] if forced_empty else [0.25] * 4
    counts = multinomial_counts(1000 * 1 + TID_COUNTS, 512, probs)
    return make_problem("tiny_moe_e4_t512" + ("_empty2" if forced_empty else ""), 1, counts,
                        N=512, K=256, integer=integer)


def config2(d_out: int, integer: bool = False, need=("X", "G")) -> Problem:
    return make_problem(f"dense_wgrad_t16384_k4096_n{d_out}", 2, [16384], N=d_out, K=4096,
                        g_std=0.1, need=need, integer=integer)


def config3(integer: bool = False, need=("X", "W", "G")) -> Problem:
    return make_problem("moe_gate_up_e8_t131072_k2048_n1536", 3, [16384] * 8, N=1536, K=2048,
                        need=need, integer=integer)


def config4_counts() -> np.ndarray:
    return zipf_counts(1000 * 4 + TID_COUNTS, 131072, 32, 2, 1.2)


def config4(integer: bool = False, need=("X", "G")) -> Problem:
    return make_problem("moe_down_e32_zipf1.2_t131072_k768_n2048", 4, config4_counts(),
                        N=2048, K=768, need=need, integer=integer)


def config5(integer: bool = False, need=("X", "W", "G")) -> Problem:
    return make_problem("dense_square_t16384_k4096_n4096", 5, [16384], N=4096, K=4096,
                        need=need, integer=integer)


def router_inputs(M=16384, N=256, K=4096, cfg_seed=5):
    """FP32 router operands: X [M,K], Wr [N,K], both N(0,1)."""
    rx = np.random.default_rng(1000 * cfg_seed + TID_XR)
    rw = np.random.default_rng(1000 * cfg_seed + TID_WR)
    X = rx.standard_normal((M, K), dtype=np.float32)
    Wr = rw.standard_normal((N, K), dtype=np.float32)
    return X, Wr
