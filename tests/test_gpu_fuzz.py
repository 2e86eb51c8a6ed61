"""GPU parity on seeded random problems: expert counts from 1 to 1024, token
counts from zero to about 24000, N and K any multiple of 8, routings from
balanced to one expert holding every token, FP32 and BF16 outputs, the
planner's tile or a forced one.  Every program (forward, data gradient,
deterministic and split weight gradient) is compared element by element
with the CPU oracle; integer-valued inputs bit for bit.  Each case prints
its parameters before it runs."""
import numpy as np
import pytest

import synth
from tests import parity
from tests.test_gpu_parity import dev_inputs, run_program

torch = pytest.importorskip("torch")

N_CASES = 96
MAX_W_ELEMS = 12_000_000      # E * N * K, keeps W and dW small
MAX_MNK = 2_000_000_000       # M * N * K, keeps the oracle to about a second per program


@pytest.fixture(scope="module")
def drgg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_ragged_grouped_amd as d
    d.set_knob(d.KNOB_NONDET, 1)      # det=False runs the split program
    return d


def _mult8(rng, lo, hi):
    """A multiple of 8 in [lo, hi], log-uniform."""
    v = int(np.exp(rng.uniform(np.log(lo), np.log(hi))))
    return max(8, v // 8 * 8)


def fuzz_case(seed):
    """(E, counts, N, K, integer, out_bf16) of case `seed`."""
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.choice([1, 2, 3, 5, 8, 16, 31, 64, 65, 130, 257, 1024]))
    M = 0 if seed % 11 == 5 else int(np.exp(rng.uniform(np.log(1), np.log(24000))))
    kind = seed % 4
    if kind == 0:          # uneven shares, some experts empty
        p = rng.uniform(0.0, 1.0, E) * (rng.uniform(size=E) > 0.2)
        p = p if p.sum() > 0 else np.ones(E)
        counts = rng.multinomial(M, p / p.sum())
    elif kind == 1:        # Zipf over the experts
        counts = synth.zipf_counts(8000 + seed, M, E, int(rng.integers(0, max(1, E // 4) + 1)) if E > 1 else 0,
                                   float(rng.uniform(0.8, 1.6)))
    elif kind == 2:        # one expert holds every token
        counts = np.zeros(E, dtype=np.int64)
        counts[int(rng.integers(0, E))] = M
    else:                  # tiny experts: one token each where possible, the rest on one expert
        counts = np.zeros(E, dtype=np.int64)
        ones = min(E, M)
        counts[:ones] = 1
        counts[int(rng.integers(0, E))] += M - ones
    N = _mult8(rng, 8, 800)
    K = _mult8(rng, 8, 800)
    while E * N * K > MAX_W_ELEMS or max(M, 1) * N * K > MAX_MNK:
        N, K = max(8, N // 2 // 8 * 8), max(8, K // 2 // 8 * 8)
    return E, np.asarray(counts, dtype=np.int64), N, K, bool(seed % 2), bool((seed // 2) % 2)


def test_fuzz_cases_are_valid_and_varied():
    cases = [fuzz_case(s) for s in range(N_CASES)]
    for E, counts, N, K, _, _ in cases:
        assert counts.size == E and counts.min() >= 0 and N % 8 == 0 and K % 8 == 0 and N >= 8 and K >= 8
        assert E * N * K <= MAX_W_ELEMS and counts.sum() * N * K <= MAX_MNK
    assert any(c.sum() == 0 for _, c, *_ in cases)
    assert any(E >= 257 for E, *_ in cases)
    assert any(c.sum() > 3000 for _, c, *_ in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_problem_all_programs(drgg, seed):
    E, counts, N, K, integer, out_bf16 = fuzz_case(seed)
    prob = synth.make_problem(f"fuzz_{seed}", 7000 + seed, counts, N=N, K=K, integer=integer)
    print(f"fuzz seed={seed} E={E} M={prob.M} N={N} K={K} integer={integer} bf16={out_bf16} "
          f"max_count={int(counts.max())} empty={int((counts == 0).sum())} tile={seed % 6}", flush=True)
    dv = dev_inputs(prob)
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    tile = seed % 6           # 0: the planner's tile; 5 (64x256) applies to the weight gradient only
    drgg.set_knob(drgg.KNOB_TILE, tile)
    try:
        for program, det in (("fwd", True), ("dgrad", True), ("wgrad", True), ("wgrad", False)):
            out = run_program(drgg, program, dv, out_dtype, det)
            torch.cuda.synchronize()
            parity.compare(prob, program, parity.from_dev(out), out_bf16, integer=integer,
                           what=f"fuzz {seed} {program} det={det} tile={tile}")
    finally:
        drgg.set_knob(drgg.KNOB_TILE, 0)
