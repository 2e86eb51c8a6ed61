"""Calibrate the route table of the non-deterministic weight gradient on the
device at hand: measure the deterministic and the split program at each
problem point, apply the selection rule (route.py) and write the table that
`load_routes` installs.

    python -m dense_ragged_grouped_amd.calibrate --out routes.json [--runs 5] [--reps 10]
                                                 [--points gate_up,down,dense48,...]

Per point, with seeded normal BF16 inputs of the point's shape (balanced
routing unless the point gives token counts):

  (a) op level: `runs` paired groups; in each, both programs are timed over
      `reps` calls, in alternating order, as eager launches and as replays
      of a captured graph of one call;
  (b) co-run: each call next to drgg_hold_cus holding 8, 16 and 32 compute
      units on another stream for half a deterministic call, launched just
      before the call or just after it;
  (c) steps: the backward (data gradient + weight gradient) and the
      checkpointed step (2 x forward + backward: the kernel sequence of the
      checkpointed autograd layer without early stop), eager and replayed.

Times come from events on the launch stream.  The rule keeps the split
program only where every condition holds; the table lists every point with
its program and the measured ratios.
"""
import argparse
import json
import statistics
import sys

import numpy as np


def _points():
    """The weight-gradient points of the measured workloads (name -> E, M,
    N, K, output type, token counts or None for balanced)."""
    pts = {
        "gate_up": (8, 131072, 1536, 2048, "bf16", None),
        "down": (32, 131072, 2048, 768, "fp32", "zipf"),
        "tiny": (4, 512, 512, 256, "fp32", None),
    }
    for d in (48, 64, 512, 1024):
        pts[f"dense{d}"] = (1, 16384, d, 4096, "fp32", None)
    return pts


def _counts(E, M, kind):
    if kind == "zipf":   # the Zipf(1.2) routing of the measured down workload
        try:
            import synth
        except ImportError as exc:
            raise SystemExit("the Zipf-routed point needs the repository's seeded input generators "
                             "(package `synth`): run from the repository root") from exc
        return np.asarray(synth.config4_counts(), dtype=np.int64)
    c = np.full(E, M // E, dtype=np.int64)
    c[: M - int(c.sum())] += 1
    return c


def _time(torch, fn, reps, stream):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def _graph(torch, fn):
    fn()   # allocations (workspaces) before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g.replay


def measure_point(torch, drgg, route, E, M, N, K, out, kind, runs, reps, log=print):
    """Timings of both programs at one point and the rule's decision."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(1000 + E * 7 + N)
    X = torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16)
    G = torch.randn(M, N, device=dev, generator=gen).to(torch.bfloat16)
    W = (0.02 * torch.randn(E, N, K, device=dev, generator=gen)).to(torch.bfloat16)
    counts = _counts(E, M, kind)
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    code = drgg.BF16 if out == "bf16" else drgg.FP32
    dW = torch.empty(E, N, K, dtype=odt, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    ws = {"det": drgg.Workspace(dev), "split": drgg.Workspace(dev)}
    wsd = drgg.Workspace(dev)
    drgg.route_split(E, M, N, K, code)   # deterministic=False now runs the split program
    try:
        wg = {p: (lambda p=p: drgg.grouped_gemm_wgrad(X, G, offs, out_dtype=odt, deterministic=p == "det",
                                                      out=dW, workspace=ws[p])) for p in ("det", "split")}
        fwd = lambda: drgg.grouped_gemm_fwd(X, W, offs, out=Y)
        dgrad = lambda: drgg.grouped_gemm_dgrad(G, W, offs, out=dX, workspace=wsd)
        steps = {}
        for p in ("det", "split"):
            steps[("bwd", p)] = lambda p=p: (dgrad(), wg[p]())
            steps[("ckpt", p)] = lambda p=p: (fwd(), fwd(), dgrad(), wg[p]())
        graphs = {p: _graph(torch, wg[p]) for p in wg}
        step_graphs = {k: _graph(torch, f) for k, f in steps.items()}
        stream = torch.cuda.current_stream()
        other = torch.cuda.Stream()
        op = {"eager": ([], []), "graph": ([], [])}
        corun = {}
        st = {}
        for r in range(runs):
            order = ("det", "split") if r % 2 == 0 else ("split", "det")
            for mode, fns in (("eager", wg), ("graph", graphs)):
                t = {p: _time(torch, fns[p], reps, stream) for p in order}
                op[mode][0].append(t["det"])
                op[mode][1].append(t["split"])
            # every call next to a holder that keeps `cus` compute units for
            # half a deterministic call, launched just before or just after it
            hold_us = max(20, int(500 * op["eager"][0][-1]))
            for cus in route.HOLDER_CUS:
                for first in ("holder first", "calls first"):
                    t = {}
                    for p in order:
                        torch.cuda.synchronize()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for _ in range(reps):
                            if first == "holder first":
                                drgg.hold_cus(cus, hold_us, other)
                            wg[p]()
                            if first == "calls first":
                                drgg.hold_cus(cus, hold_us, other)
                        e1.record(stream)
                        torch.cuda.synchronize()
                        t[p] = e0.elapsed_time(e1) / reps
                    d, s = corun.setdefault((cus, first), ([], []))
                    d.append(t["det"])
                    s.append(t["split"])
            for name in ("bwd", "ckpt"):
                for mode, fns in (("eager", steps), ("graph", step_graphs)):
                    t = {p: _time(torch, fns[(name, p)], max(1, reps // 2), stream) for p in order}
                    d, s = st.setdefault((name, mode), ([], []))
                    d.append(t["det"])
                    s.append(t["split"])
        program, details = route.choose_program(op, corun, st)
        details["median_ms"] = {f"{m}_{p}": statistics.median(v[i]) for m, v in op.items()
                                for i, p in enumerate(("det", "split"))}
        log(f"E={E} M={M} N={N} K={K} {out}: {program}; op eager ratio "
            f"{details['op_eager']['median_ratio']:.3f}, graph {details['op_graph']['median_ratio']:.3f}")
        return program, details
    finally:
        drgg.route_clear()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", required=True, help="route table to write (JSON)")
    ap.add_argument("--runs", type=int, default=5)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--points", default="", help="comma list of point names (default: all)")
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("calibration needs the GPU", file=sys.stderr)
        return 2
    import dense_ragged_grouped_amd as drgg
    from dense_ragged_grouped_amd import route
    pts = _points()
    names = [p for p in args.points.split(",") if p] or list(pts)
    if drgg.route_count():
        print("the route table is not empty; calibrating from a cleared table", file=sys.stderr)
        drgg.route_clear()
    props = torch.cuda.get_device_properties(0)
    table = {"device": props.name, "compute_units": props.multi_processor_count, "runs": args.runs,
             "reps": args.reps, "rule": "PR #8363 selection rule (route.py)", "points": []}
    for name in names:
        E, M, N, K, out, kind = pts[name]
        program, details = measure_point(torch, drgg, route, E, M, N, K, out, kind, args.runs, args.reps,
                                         log=lambda s, n=name: print(f"{n}: {s}", flush=True))
        table["points"].append({"name": name, "E": E, "M": M, "N": N, "K": K,
                                "out_dtype": drgg.BF16 if out == "bf16" else drgg.FP32, "program": program,
                                "details": json.loads(json.dumps(details, default=str))})
    with open(args.out, "w") as f:
        json.dump(table, f, indent=1)
    print(f"wrote {args.out}: {sum(p['program'] == 'split' for p in table['points'])} of "
          f"{len(table['points'])} points keep the split program", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
