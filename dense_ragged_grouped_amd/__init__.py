"""Python binding of libdrgg.so, the MI355X (gfx950) ragged BF16 grouped GEMM.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/drgg.h).  PyTorch supplies device memory
and the current stream.  If the library is missing the import fails loudly:
there is no fallback of any kind.

Programs (flashinfer PR #8258, opening summary paragraph), shapes row-major:

    grouped_gemm_fwd(X [M,K], W [E,N,K], offsets [E+1])   -> Y  [M,N]    = X W_e^T
    grouped_gemm_dgrad(G [M,N], W [E,N,K], offsets)       -> dX [M,K]    = G W_e
    grouped_gemm_wgrad(X [M,K], G [M,N], offsets)         -> dW [E,N,K]  = G_e^T X_e
    router_gemm_fp32_bf16x3(X [M,K] fp32, Wr [N,K] fp32)  -> out [M,N] fp32

``offsets`` is an int32 CUDA tensor: offsets[0] = 0, non-decreasing,
offsets[E] = M; expert e owns tokens offsets[e] .. offsets[e+1]-1.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdrgg.so")

BF16, FP32 = 0, 1
OP_FWD, OP_DGRAD, OP_WGRAD = 0, 1, 2
KNOB_TILE, KNOB_GRID, KNOB_REVERSE, KNOB_TIMING, KNOB_NONDET = 1, 2, 3, 4, 5
KNOB_CHECK_OFFSETS, KNOB_CHECK_WORKSPACE, KNOB_DELAY_SEED, KNOB_SPLIT_REPORT = 6, 7, 8, 9
KNOB_DGRAD_WT = 10
TILE_AUTO, TILE_256x256, TILE_128x128, TILE_256x128, TILE_128x256, TILE_64x256 = range(6)

# the symbols include/drgg.h declares
EXPORTS = (
    "grouped_gemm_fwd", "grouped_gemm_dgrad", "grouped_gemm_wgrad", "router_gemm_fp32_bf16x3",
    "router_gemm_fp32_bf16x3_ws", "router_workspace_size", "drgg_router_split",
    "batched_gemm_fwd", "batched_gemm_dgrad", "batched_gemm_wgrad",
    "drgg_route_split", "drgg_route_clear", "drgg_route_count", "drgg_hold_cus",
    "grouped_gemm_workspace_size", "drgg_workspace_init", "drgg_plan", "drgg_wgrad_chunking",
    "drgg_tailsplit_units", "drgg_wgrad_tail_plan", "drgg_wgrad_split_plan", "grouped_gemm_wgrad_noalloc",
    "drgg_set_knob", "drgg_timing_count", "drgg_timing_read", "drgg_status_string", "drgg_abi_version",
)


class DrggError(RuntimeError):
    """A non-zero status from the C ABI; the message is drgg_status_string."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("mfma_m", ctypes.c_int32), ("mfma_n", ctypes.c_int32), ("mfma_k", ctypes.c_int32),
        ("grid", ctypes.c_int64), ("chunk_max", ctypes.c_int64), ("unit", ctypes.c_int64),
        ("max_partials", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class Batched(ctypes.Structure):
    """drgg_batched: shape and element strides of a batched call."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("a_row", ctypes.c_int64), ("a_batch", ctypes.c_int64),
        ("b_row", ctypes.c_int64), ("b_batch", ctypes.c_int64),
        ("o_row", ctypes.c_int64), ("o_batch", ctypes.c_int64),
    ]


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m dense_ragged_grouped_amd.build` "
            "(the grouped GEMM has no fallback path)")
    # One HIP runtime per process: libdrgg.so needs libamdhip64.so.7, which
    # resolves to the runtime already loaded under that name.  torch bundles
    # its own; loaded first, it serves both.  Loaded after this library (whose
    # runpath finds the system runtime), torch would bring a second HIP/HSA
    # runtime, and the one initialised last finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, c_int = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    gemm = [vp, vp, vp, i32, i64, i64, i64, c_int, c_int, vp, vp, sz, vp]
    for name in ("grouped_gemm_fwd", "grouped_gemm_dgrad", "grouped_gemm_wgrad"):
        getattr(lib, name).argtypes = gemm
        getattr(lib, name).restype = c_int
    lib.grouped_gemm_wgrad_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, i64, c_int, c_int, vp, vp]
    lib.grouped_gemm_wgrad_noalloc.restype = c_int
    pb = ctypes.POINTER(Batched)
    lib.batched_gemm_fwd.argtypes = [vp, vp, pb, c_int, vp, vp]
    lib.batched_gemm_dgrad.argtypes = [vp, vp, pb, c_int, vp, vp, sz, vp]
    lib.batched_gemm_wgrad.argtypes = [vp, vp, pb, c_int, c_int, vp, vp, sz, vp]
    for name in ("batched_gemm_fwd", "batched_gemm_dgrad", "batched_gemm_wgrad"):
        getattr(lib, name).restype = c_int
    lib.router_gemm_fp32_bf16x3.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    lib.router_gemm_fp32_bf16x3.restype = c_int
    lib.router_gemm_fp32_bf16x3_ws.argtypes = [vp, vp, i64, i64, i64, vp, vp, sz, vp]
    lib.router_gemm_fp32_bf16x3_ws.restype = c_int
    lib.router_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
    lib.router_workspace_size.restype = c_int
    lib.drgg_router_split.argtypes = [i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.drgg_router_split.restype = c_int
    lib.grouped_gemm_workspace_size.argtypes = [c_int, i32, i64, i64, i64, c_int, c_int, c_int,
                                                ctypes.POINTER(sz)]
    lib.grouped_gemm_workspace_size.restype = c_int
    lib.drgg_workspace_init.argtypes = [vp, sz, vp]
    lib.drgg_workspace_init.restype = c_int
    lib.drgg_plan.argtypes = [c_int, i32, i64, i64, i64, c_int, c_int, c_int, ctypes.POINTER(PlanInfo)]
    lib.drgg_plan.restype = c_int
    lib.drgg_wgrad_chunking.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.drgg_wgrad_chunking.restype = c_int
    lib.drgg_wgrad_tail_plan.argtypes = [vp, i32, i64, i64, ctypes.POINTER(c_int), vp]
    lib.drgg_wgrad_tail_plan.restype = c_int
    lib.drgg_wgrad_split_plan.argtypes = [vp, i32, i64, i64, c_int, i64, ctypes.POINTER(c_int), ctypes.POINTER(i64),
                                          ctypes.POINTER(c_int)]
    lib.drgg_wgrad_split_plan.restype = c_int
    lib.drgg_tailsplit_units.argtypes = [i64, i64, ctypes.POINTER(i64)]
    lib.drgg_tailsplit_units.restype = c_int
    lib.drgg_route_split.argtypes = [i32, i64, i64, i64, c_int]
    lib.drgg_route_split.restype = c_int
    lib.drgg_hold_cus.argtypes = [c_int, i64, vp]
    lib.drgg_hold_cus.restype = c_int
    lib.drgg_route_clear.argtypes = []
    lib.drgg_route_clear.restype = c_int
    lib.drgg_route_count.argtypes = []
    lib.drgg_route_count.restype = c_int
    lib.drgg_set_knob.argtypes = [c_int, i64]
    lib.drgg_set_knob.restype = c_int
    lib.drgg_timing_count.argtypes = []
    lib.drgg_timing_count.restype = c_int
    lib.drgg_timing_read.argtypes = [c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
    lib.drgg_timing_read.restype = c_int
    lib.drgg_status_string.argtypes = [c_int]
    lib.drgg_status_string.restype = ctypes.c_char_p
    lib.drgg_abi_version.argtypes = []
    lib.drgg_abi_version.restype = c_int
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.drgg_status_string(status).decode()


def abi_version() -> int:
    return lib.drgg_abi_version()


def _check(status: int, where: str):
    if status != 0:
        raise DrggError(status, where)


# ---- host-only queries ------------------------------------------------------

def plan(op: int, E: int, M: int, N: int, K: int, out_dtype: int = BF16, deterministic: bool = True,
         cu_count: int = 256) -> dict:
    """The plan a call would use (no GPU needed when cu_count > 0)."""
    info = PlanInfo()
    _check(lib.drgg_plan(op, E, M, N, K, out_dtype, int(bool(deterministic)), cu_count, ctypes.byref(info)),
           "drgg_plan")
    return info.as_dict()


def wgrad_chunking(T: int, chunk_max: int):
    """(chunk length, chunk count) of an expert with T tokens."""
    ln, n = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.drgg_wgrad_chunking(T, chunk_max, ctypes.byref(ln), ctypes.byref(n)), "drgg_wgrad_chunking")
    return ln.value, n.value


def tailsplit_units(tiles: int, workers: int):
    """(tiles, units, full, split) of the tail-split rule: `tiles` equal
    tiles on `workers` persistent workers; a partial last wave of
    tail = tiles mod workers tiles is cut into 2 * tail half units when that
    fits one wave, else every tile stays whole."""
    out = (ctypes.c_int64 * 4)()
    _check(lib.drgg_tailsplit_units(int(tiles), int(workers), out), "drgg_tailsplit_units")
    return tuple(int(v) for v in out)


def wgrad_tail_plan(offsets, N: int, K: int):
    """(tail_only, row0) of the deterministic weight gradient's plan for host
    group offsets (a sequence of E + 1 ints): whether the kernel runs the
    tail-only plan, and per expert the first dW row that comes from folded
    partials (the rows above it are whole tiles, stored directly)."""
    import numpy as np
    o = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    E = o.size - 1
    tail = ctypes.c_int()
    row0 = np.zeros(max(E, 1), dtype=np.int32)
    _check(lib.drgg_wgrad_tail_plan(o.ctypes.data, E, N, K, ctypes.byref(tail), row0.ctypes.data),
           "drgg_wgrad_tail_plan")
    return bool(tail.value), row0[:E]


def wgrad_split_plan(offsets, N: int, K: int, grid: int = 256, tile: int = 0, banded: bool = False):
    """(slack, tail_tiles) of the split program's walk for host group offsets
    on `grid` workgroups: whether its tail tiles run whole on the
    least-loaded workgroups (slack placement), and how many tail tiles the
    banded walk has; with banded=True also whether the banded walk runs."""
    import numpy as np
    o = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    slack, tail, band = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
    _check(lib.drgg_wgrad_split_plan(o.ctypes.data, o.size - 1, N, K, tile, grid, ctypes.byref(slack),
                                     ctypes.byref(tail), ctypes.byref(band)), "drgg_wgrad_split_plan")
    if banded:
        return bool(slack.value), int(tail.value), bool(band.value)
    return bool(slack.value), int(tail.value)


def wgrad_runs_deterministic(E: int, M: int, N: int, K: int, out_dtype: int = BF16,
                             deterministic: bool = True) -> bool:
    """Whether a weight-gradient call runs the deterministic program: always
    for deterministic=True; for deterministic=False unless the route table
    (or KNOB_NONDET) sends the point to the split program."""
    if deterministic:
        return True
    return plan(OP_WGRAD, E, M, N, K, out_dtype, False, 1)["unit"] == 0


def route_split(E: int, M: int, N: int, K: int, out_dtype: int = BF16):
    """Send non-deterministic weight-gradient calls at this exact point to the
    split program (see load_routes)."""
    _check(lib.drgg_route_split(E, M, N, K, out_dtype), "drgg_route_split")


def hold_cus(cus: int, microseconds: int, stream=None):
    """Calibration aid: occupy `cus` compute units for `microseconds` on
    `stream` (default: the current stream)."""
    torch = _torch()
    _check(lib.drgg_hold_cus(int(cus), int(microseconds), _stream(torch.device("cuda"), stream)), "drgg_hold_cus")


def route_clear():
    _check(lib.drgg_route_clear(), "drgg_route_clear")


def route_count() -> int:
    return lib.drgg_route_count()


DEFAULT_ROUTES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "routes_mi355x.json")


def load_default_routes() -> int:
    """Install the route table measured on MI355X (256 CUs) that ships with
    the package (done at import unless DRGG_NO_ROUTES=1)."""
    return load_routes(DEFAULT_ROUTES) if os.path.exists(DEFAULT_ROUTES) else 0


def load_routes(path: str) -> int:
    """Install the split points of a route table written by
    `python -m dense_ragged_grouped_amd.calibrate` (JSON); returns how many.
    The table applies to the kind of device it was measured on."""
    import json
    with open(path) as f:
        table = json.load(f)
    n = 0
    for pt in table.get("points", []):
        if pt.get("program") == "split":
            route_split(pt["E"], pt["M"], pt["N"], pt["K"], pt.get("out_dtype", BF16))
            n += 1
    return n


def set_knob(knob: int, value: int):
    """Test knobs (tile shape, persistent grid, reverse walk, timing, split
    program for non-deterministic weight gradients, the debug checks of the
    offsets and of the split program's workspace); 0 restores the default."""
    _check(lib.drgg_set_knob(knob, int(value)), "drgg_set_knob")


def last_call_kernel_times():
    """With KNOB_TIMING on: [(kernel name, milliseconds)] of the most recent
    call's kernel launches, timed by HIP events on the launch stream."""
    out = []
    for i in range(lib.drgg_timing_count()):
        name, ms = ctypes.c_char_p(), ctypes.c_float()
        _check(lib.drgg_timing_read(i, ctypes.byref(name), ctypes.byref(ms)), "drgg_timing_read")
        out.append((name.value.decode(), ms.value))
    return out


def workspace_size(op: int, E: int, M: int, N: int, K: int, out_dtype: int = BF16,
                   deterministic: bool = True, cu_count: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib.grouped_gemm_workspace_size(op, E, M, N, K, out_dtype, int(bool(deterministic)), cu_count,
                                           ctypes.byref(n)), "grouped_gemm_workspace_size")
    return n.value


# ---- torch marshalling ---------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt in (torch.bfloat16, BF16, "bf16"):
        return BF16
    if dt in (torch.float32, FP32, "fp32"):
        return FP32
    raise ValueError(f"unsupported output dtype {dt!r}")


def _torch_dtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def _need(t, dtype, name, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _on_one_device(stream, *tensors):
    """Check that the tensors of one call (None entries skipped) and the
    stream, if given, are on one device, and return a context that makes
    that device current for the launch (the library plans for, and launches
    on, the current device)."""
    torch = _torch()
    dev = tensors[0].device
    for t in tensors[1:]:
        if t is not None and t.device != dev:
            raise ValueError(f"the tensors of one call must be on one device ({dev} and {t.device})")
    if stream is not None and stream.device != dev:
        raise ValueError(f"the stream is on {stream.device}, the tensors on {dev}")
    return torch.cuda.device(dev)


class Workspace:
    """Device workspace for the weight gradient, grown on demand.

    Allocated and zeroed on the stream of the call that needs it (so the
    zeroing is ordered before that call's kernels, and torch's allocator
    ties the memory to that stream); used on another stream, the buffer is
    recorded on it, so that a buffer replaced by a larger one is not handed
    out again before the calls using it have finished.  The split program
    leaves its tile sums and tickets zero after every call, so the buffer
    stays valid for later calls.  One Workspace must not serve two calls in
    flight on different streams at once.
    """

    def __init__(self, device=None):
        torch = _torch()
        self.device = torch.device(device if device is not None else "cuda")
        self.buf = None
        self.home = None

    def get(self, nbytes: int, stream=None):
        torch = _torch()
        if nbytes == 0:
            return None
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        if self.buf is None or self.buf.numel() < nbytes:
            with torch.cuda.stream(s):
                self.buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=self.device)
            self.home = s
        elif s != self.home:
            self.buf.record_stream(s)
        return self.buf


# Default workspaces, one per (device, stream, program): a deterministic call
# leaves its FP32 partials in the buffer, while the split program needs its
# tile sums and tickets to be zero, so the two never share a buffer; calls on
# different streams may run at the same time, so they never share one either.
_default_ws = {}


def _workspace(device, nbytes, workspace, deterministic, kind="wgrad", stream=None):
    torch = _torch()
    if workspace is False:   # explicitly none (the data gradient's direct program)
        return None, 0
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if workspace is not None:
        buf = workspace.get(nbytes, s) if isinstance(workspace, Workspace) else workspace
        if buf is not None and buf.device != device:
            raise ValueError(f"the workspace is on {buf.device}, the operands on {device}")
    else:
        # keyed by the program that runs (`deterministic` here: whether the
        # deterministic program runs): a non-deterministic call routed to it
        # shares its buffer of partials, the split program has its own,
        # zeroed one; the data gradient's W^T and the router's reduction
        # slices have their own
        prog = kind if kind in ("dgrad", "router") else bool(deterministic)
        key = (str(device), s.cuda_stream, prog)
        if key not in _default_ws:
            _default_ws[key] = Workspace(device)
        buf = _default_ws[key].get(nbytes, s)
    if buf is None:
        return None, 0
    return ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size()


def _offsets(offsets):
    torch = _torch()
    _need(offsets, torch.int32, "group_offsets", 1)
    return offsets.numel() - 1


def grouped_gemm_fwd(X, W, group_offsets, out_dtype=None, deterministic=True, out=None, stream=None):
    """Y[t] = X[t] W[e(t)]^T with FP32 accumulation; out_dtype bf16 (default) or fp32."""
    torch = _torch()
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 3)
    E = _offsets(group_offsets)
    M, K = X.shape
    En, N, Kw = W.shape
    if En != E or Kw != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, E={E}")
    code = _dtype_code(out_dtype if out_dtype is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=_torch_dtype(code), device=X.device)
    else:
        _need(out, _torch_dtype(code), "out", 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    with _on_one_device(stream, X, W, group_offsets, out):
        st = lib.grouped_gemm_fwd(X.data_ptr(), W.data_ptr(), group_offsets.data_ptr(), E, M, N, K, code,
                                  int(bool(deterministic)), out.data_ptr(), None, 0, _stream(X.device, stream))
    _check(st, "grouped_gemm_fwd")
    return out


def grouped_gemm_dgrad(G, W, group_offsets, out_dtype=None, deterministic=True, out=None, workspace=None,
                       stream=None):
    """dX[t] = G[t] W[e(t)] with FP32 accumulation.  `workspace` (a Workspace,
    a device tensor, None for the default buffer, or False for none) holds
    W^T, which makes the product faster when the experts average at least
    3072 tokens (below that no W^T is made and the default buffer is not
    allocated); the result is bitwise the same either way."""
    torch = _torch()
    _need(G, torch.bfloat16, "G", 2)
    _need(W, torch.bfloat16, "W", 3)
    E = _offsets(group_offsets)
    M, N = G.shape
    En, Nw, K = W.shape
    if En != E or Nw != N:
        raise ValueError(f"shape mismatch: G {tuple(G.shape)}, W {tuple(W.shape)}, E={E}")
    code = _dtype_code(out_dtype if out_dtype is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((M, K), dtype=_torch_dtype(code), device=G.device)
    else:
        _need(out, _torch_dtype(code), "out", 2)
        if tuple(out.shape) != (M, K):
            raise ValueError("out has the wrong shape")
    nbytes = workspace_size(OP_DGRAD, E, M, N, K, code, deterministic)
    with _on_one_device(stream, G, W, group_offsets, out):
        ws_ptr, ws_bytes = _workspace(G.device, nbytes, workspace, deterministic, kind="dgrad", stream=stream)
        st = lib.grouped_gemm_dgrad(G.data_ptr(), W.data_ptr(), group_offsets.data_ptr(), E, M, N, K, code,
                                    int(bool(deterministic)), out.data_ptr(), ws_ptr, ws_bytes,
                                    _stream(G.device, stream))
    _check(st, "grouped_gemm_dgrad")
    return out


def grouped_gemm_wgrad(X, G, group_offsets, out_dtype=None, deterministic=True, out=None, workspace=None,
                       stream=None):
    """dW[e] = G_e^T X_e over each expert's tokens (+0 for experts without tokens)."""
    torch = _torch()
    _need(X, torch.bfloat16, "X", 2)
    _need(G, torch.bfloat16, "G", 2)
    E = _offsets(group_offsets)
    M, K = X.shape
    Mg, N = G.shape
    if Mg != M:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, G {tuple(G.shape)}")
    code = _dtype_code(out_dtype if out_dtype is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((E, N, K), dtype=_torch_dtype(code), device=X.device)
    else:
        _need(out, _torch_dtype(code), "out", 3)
        if tuple(out.shape) != (E, N, K):
            raise ValueError("out has the wrong shape")
    nbytes = workspace_size(OP_WGRAD, E, M, N, K, code, deterministic)
    with _on_one_device(stream, X, G, group_offsets, out):
        ws_ptr, ws_bytes = _workspace(X.device, nbytes, workspace,
                                      wgrad_runs_deterministic(E, M, N, K, code, deterministic), stream=stream)
        st = lib.grouped_gemm_wgrad(X.data_ptr(), G.data_ptr(), group_offsets.data_ptr(), E, M, N, K, code,
                                    int(bool(deterministic)), out.data_ptr(), ws_ptr, ws_bytes,
                                    _stream(X.device, stream))
    _check(st, "grouped_gemm_wgrad")
    return out


def grouped_gemm_wgrad_noalloc(X, G, group_offsets, out, deterministic=True, stream=None):
    """grouped_gemm_wgrad into a caller-given `out` [E, N, K] (BF16 or FP32)
    with the library's fixed per-device workspace: the call allocates
    nothing (for code that must not, e.g. under graph capture).  Problems
    whose workspace exceeds that array (64 MiB) are refused; calls that
    overlap on one device race on it."""
    torch = _torch()
    _need(X, torch.bfloat16, "X", 2)
    _need(G, torch.bfloat16, "G", 2)
    E = _offsets(group_offsets)
    M, K = X.shape
    Mg, N = G.shape
    if Mg != M:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, G {tuple(G.shape)}")
    code = _dtype_code(out.dtype)
    _need(out, _torch_dtype(code), "out", 3)
    if tuple(out.shape) != (E, N, K):
        raise ValueError("out has the wrong shape")
    with _on_one_device(stream, X, G, group_offsets, out):
        st = lib.grouped_gemm_wgrad_noalloc(X.data_ptr(), G.data_ptr(), group_offsets.data_ptr(), E, M, N, K, code,
                                            int(bool(deterministic)), out.data_ptr(), _stream(X.device, stream))
    _check(st, "grouped_gemm_wgrad_noalloc")
    return out


# ---- batched calls: [B, T, row] views with any batch and row strides -----------

def _need_rows(t, name, shape=None):
    """A BF16 CUDA tensor [B, T, row] whose rows are contiguous (any batch
    and row strides, e.g. a transposed head-interleaved [T, B, row])."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be a 3-d tensor with contiguous rows")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _out_rows(out, shape, code, device, name="out"):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=_torch_dtype(code), device=device)
    if out.dtype != _torch_dtype(code):
        raise TypeError(f"{name} must be {_torch_dtype(code)}")
    _need_rows(out, name, shape)
    return out


def batched_gemm_fwd(X, W, out_dtype=None, out=None, stream=None):
    """Y[b] = X[b] W[b]^T for b < B: X [B, T, K] (rows contiguous, any
    strides, e.g. a head-interleaved [T, H, K] activation passed as
    X.transpose(0, 1)), W [B, N, K] contiguous; Y [B, T, N] (new and
    contiguous, or `out` with contiguous rows)."""
    torch = _torch()
    _need_rows(X, "X")
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    _need(W, torch.bfloat16, "W", 3)
    B, T, K = X.shape
    if W.shape[0] != B or W.shape[2] != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}")
    N = W.shape[1]
    code = _dtype_code(out_dtype if out_dtype is not None else torch.bfloat16)
    out = _out_rows(out, (B, T, N), code, X.device)
    b = Batched(B, T, N, K, X.stride(1), X.stride(0), 0, 0, out.stride(1), out.stride(0))
    with _on_one_device(stream, X, W, out):
        st = lib.batched_gemm_fwd(X.data_ptr(), W.data_ptr(), ctypes.byref(b), code, out.data_ptr(),
                                  _stream(X.device, stream))
    _check(st, "batched_gemm_fwd")
    return out


def batched_gemm_dgrad(G, W, out_dtype=None, out=None, workspace=None, stream=None):
    """dX[b] = G[b] W[b]: G [B, T, N] (rows contiguous), W [B, N, K]
    contiguous; dX [B, T, K].  `workspace` as for grouped_gemm_dgrad."""
    torch = _torch()
    _need_rows(G, "G")
    if G.dtype != torch.bfloat16:
        raise TypeError("G must be bfloat16")
    _need(W, torch.bfloat16, "W", 3)
    B, T, N = G.shape
    if W.shape[0] != B or W.shape[1] != N:
        raise ValueError(f"shape mismatch: G {tuple(G.shape)}, W {tuple(W.shape)}")
    K = W.shape[2]
    code = _dtype_code(out_dtype if out_dtype is not None else torch.bfloat16)
    out = _out_rows(out, (B, T, K), code, G.device)
    nbytes = workspace_size(OP_DGRAD, B, B * T, N, K, code, True)
    b = Batched(B, T, N, K, G.stride(1), G.stride(0), 0, 0, out.stride(1), out.stride(0))
    with _on_one_device(stream, G, W, out):
        ws_ptr, ws_bytes = _workspace(G.device, nbytes, workspace, True, kind="dgrad", stream=stream)
        st = lib.batched_gemm_dgrad(G.data_ptr(), W.data_ptr(), ctypes.byref(b), code, out.data_ptr(), ws_ptr,
                                    ws_bytes, _stream(G.device, stream))
    _check(st, "batched_gemm_dgrad")
    return out


def batched_gemm_wgrad(X, G, out_dtype=None, deterministic=True, out=None, workspace=None, stream=None):
    """dW[b] = G[b]^T X[b]: X [B, T, K], G [B, T, N] (rows contiguous, any
    strides); dW [B, N, K] contiguous.  Workspace as for grouped_gemm_wgrad
    with E = B, M = B*T."""
    torch = _torch()
    _need_rows(X, "X")
    _need_rows(G, "G")
    if X.dtype != torch.bfloat16 or G.dtype != torch.bfloat16:
        raise TypeError("X and G must be bfloat16")
    B, T, K = X.shape
    if G.shape[0] != B or G.shape[1] != T:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, G {tuple(G.shape)}")
    N = G.shape[2]
    code = _dtype_code(out_dtype if out_dtype is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((B, N, K), dtype=_torch_dtype(code), device=X.device)
    else:
        _need(out, _torch_dtype(code), "out", 3)
        if tuple(out.shape) != (B, N, K):
            raise ValueError("out has the wrong shape")
    nbytes = workspace_size(OP_WGRAD, B, B * T, N, K, code, deterministic)
    b = Batched(B, T, N, K, X.stride(1), X.stride(0), G.stride(1), G.stride(0), 0, 0)
    with _on_one_device(stream, X, G, out):
        ws_ptr, ws_bytes = _workspace(X.device, nbytes, workspace,
                                      wgrad_runs_deterministic(B, B * T, N, K, code, deterministic), stream=stream)
        st = lib.batched_gemm_wgrad(X.data_ptr(), G.data_ptr(), ctypes.byref(b), code, int(bool(deterministic)),
                                    out.data_ptr(), ws_ptr, ws_bytes, _stream(X.device, stream))
    _check(st, "batched_gemm_wgrad")
    return out


def router_split(M: int, N: int, K: int):
    """(slices, values per slice) of the router call: (0, K) for the
    single-pass program."""
    ks, kq = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.drgg_router_split(M, N, K, ctypes.byref(ks), ctypes.byref(kq)), "drgg_router_split")
    return ks.value, kq.value


def router_workspace_size(M: int, N: int, K: int) -> int:
    n = ctypes.c_size_t()
    _check(lib.router_workspace_size(M, N, K, ctypes.byref(n)), "router_workspace_size")
    return n.value


def router_gemm_fp32_bf16x3(X, Wr, out=None, stream=None, workspace=None):
    """FP32 router GEMM out = X Wr^T on BF16 MFMA via the BF16x3 split, in
    the program router_split(M, N, K) names (single pass, or reduction slices
    added in a fixed order).  `workspace` (a Workspace, a device tensor, or
    None for the default buffer) holds the slices; False always runs the
    single-pass program (no workspace)."""
    torch = _torch()
    _need(X, torch.float32, "X", 2)
    _need(Wr, torch.float32, "Wr", 2)
    M, K = X.shape
    N, Kw = Wr.shape
    if Kw != K:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        _need(out, torch.float32, "out", 2)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    with _on_one_device(stream, X, Wr, out):
        if workspace is False:
            st = lib.router_gemm_fp32_bf16x3(X.data_ptr(), Wr.data_ptr(), M, N, K, out.data_ptr(),
                                             _stream(X.device, stream))
            _check(st, "router_gemm_fp32_bf16x3")
            return out
        nbytes = router_workspace_size(M, N, K)
        ws_ptr, ws_bytes = _workspace(X.device, nbytes, workspace, True, kind="router", stream=stream)
        st = lib.router_gemm_fp32_bf16x3_ws(X.data_ptr(), Wr.data_ptr(), M, N, K, out.data_ptr(), ws_ptr, ws_bytes,
                                            _stream(X.device, stream))
    _check(st, "router_gemm_fp32_bf16x3_ws")
    return out


def workspace_init(buf, stream=None):
    """Zero a workspace tensor with the library's fill kernel."""
    _check(lib.drgg_workspace_init(buf.data_ptr(), buf.numel() * buf.element_size(),
                                   _stream(buf.device, stream)), "drgg_workspace_init")


if os.environ.get("DRGG_NO_ROUTES", "0") in ("", "0"):
    load_default_routes()
