"""The route rule for non-deterministic weight-gradient calls: which program
(the deterministic one, or the split program with atomic tile sums) a
problem point runs.

The rule is the one PR #8363 applies to its planner (Summary, and the
#8438 commit body, which restates it as three conditions): a point keeps the
split program only if

  (a) at the op level the split program was faster than the deterministic
      one in every run -- a one-sided paired sign test at p < 0.05 -- with a
      median time ratio (split / deterministic) below 0.99, in eager
      launches and in graph replays;
  (b) next to a kernel that holds 8, 16 or 32 compute units on another
      stream it was at most 3 % slower than the deterministic program, in
      both launch orders;
  (c) the whole backward (data + weight gradient) and the checkpointed step
      (2 x forward + backward) were at most 1.3 % slower than with the
      deterministic program, as the ratio of the medians over the runs, in
      eager launches and in graph replays;

and otherwise runs the deterministic program.  The thresholds are the
pages'; on this hardware "compute unit" stands for their SM.

Everything here is plain Python on measured times (no GPU): the decision
functions take the per-run timings that calibrate.py collects.
"""
from math import comb
from statistics import median

SIGN_TEST_ALPHA = 0.05
OP_RATIO_MAX = 0.99        # (a) median split / det
CORUN_SLOWDOWN_MAX = 1.03  # (b) split / det next to a CU-holding kernel
STEP_SLOWDOWN_MAX = 1.013  # (c) backward and checkpointed step
HOLDER_CUS = (8, 16, 32)   # (b)


def sign_test_p(wins, n):
    """One-sided paired sign test: the probability of at least `wins`
    successes in `n` fair coin flips (ties already dropped)."""
    if not 0 <= wins <= n:
        raise ValueError("need 0 <= wins <= n")
    return sum(comb(n, k) for k in range(wins, n + 1)) / 2.0 ** n


def op_level_keeps_split(det_runs, split_runs):
    """Condition (a) for one launch mode: paired per-run times (same run
    index = same group).  Returns (kept, details)."""
    if len(det_runs) != len(split_runs) or not det_runs:
        raise ValueError("paired runs of equal, non-zero length")
    wins = sum(s < d for d, s in zip(det_runs, split_runs))
    ties = sum(s == d for d, s in zip(det_runs, split_runs))
    n = len(det_runs) - ties
    p = sign_test_p(wins, n) if n > 0 else 1.0
    ratio = median(split_runs) / median(det_runs)
    every = wins == len(det_runs)
    kept = every and p < SIGN_TEST_ALPHA and ratio < OP_RATIO_MAX
    return kept, {"wins": wins, "runs": len(det_runs), "p": p, "median_ratio": ratio}


def corun_keeps_split(corun):
    """Condition (b): corun maps (holder CUs, launch order) to (det runs,
    split runs); every entry must have split at most 3 % slower (ratio of
    medians)."""
    details, kept = {}, True
    for key, (det, split) in corun.items():
        r = median(split) / median(det)
        details[str(key)] = r
        kept = kept and r <= CORUN_SLOWDOWN_MAX
    return kept, details


def steps_keep_split(steps):
    """Condition (c): steps maps (step name, mode) to (det runs, split runs)
    for the backward and the checkpointed step; each ratio of medians must
    be at most 1.013."""
    details, kept = {}, True
    for key, (det, split) in steps.items():
        r = median(split) / median(det)
        details[str(key)] = r
        kept = kept and r <= STEP_SLOWDOWN_MAX
    return kept, details


def choose_program(op_runs, corun, steps):
    """The route of one point.  op_runs maps a launch mode ("eager",
    "graph") to (det runs, split runs); corun and steps as above.  Returns
    ("split" or "det", details); a point with any condition unmet, or
    without measurements for a condition, runs the deterministic program."""
    details = {}
    ok = bool(op_runs) and bool(corun) and bool(steps)
    for mode, (det, split) in op_runs.items():
        k, d = op_level_keeps_split(det, split)
        details[f"op_{mode}"] = d
        ok = ok and k
    k, d = corun_keeps_split(corun)
    details["corun"] = d
    ok = ok and k
    k, d = steps_keep_split(steps)
    details["steps"] = d
    ok = ok and k
    return ("split" if ok else "det"), details
