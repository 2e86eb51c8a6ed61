// api.cpp -- the C ABI of libdrgg.so (declared in include/drgg.h).
//
// Host-side argument checks in checked 64-bit arithmetic, planning (plan.hpp)
// and kernel launches (kernels.hip) on the caller's stream.  Nothing here
// allocates device memory, and nothing synchronises except the two opt-in
// debug checks (group offsets, split-program workspace).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/drgg.h"
#include "internal.hpp"
#include "plan.hpp"

namespace drgg {

namespace {

std::atomic<int64_t> g_knob_tile{0}, g_knob_grid{0}, g_knob_reverse{0}, g_knob_nondet{0};
// Debug checks (DRGG_KNOB_CHECK_OFFSETS / DRGG_KNOB_CHECK_WORKSPACE): 1 = on,
// 0 = the environment's setting (DRGG_CHECK_OFFSETS / DRGG_CHECK_WORKSPACE
// set to anything but "0"), off when unset.
std::atomic<int64_t> g_knob_check_offsets{0}, g_knob_check_ws{0};
// Split-program test aids: seeded delays before tail arrivals, and a device
// address (4 int32) where the kernel reports its tail decision.
std::atomic<int64_t> g_knob_delay{0}, g_knob_report{0};
// DRGG_KNOB_DGRAD_WT: 1 = the data gradient uses a W^T workspace whatever its token count
std::atomic<int64_t> g_knob_dgrad_wt{0};

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}
bool checks_offsets() { return g_knob_check_offsets.load() != 0 || env_flag("DRGG_CHECK_OFFSETS"); }
bool checks_workspace() { return g_knob_check_ws.load() != 0 || env_flag("DRGG_CHECK_WORKSPACE"); }

constexpr int64_t kMaxBytes = (int64_t)1 << 62;
constexpr int kMaxDevices = 64;

// checked a * b for non-negative operands
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > kMaxBytes / a) return false;
    *out = a * b;
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The HIP error behind this thread's most recent DRGG_EDEVICE (its text is
// appended to drgg_status_string(DRGG_EDEVICE)).
thread_local hipError_t g_last_hip_error = hipSuccess;

drgg_status device_error(hipError_t e) {
    g_last_hip_error = e;
    return DRGG_EDEVICE;
}

// CU count of the current device, cached per device.
drgg_status current_cu_count(int* cus) {
    static std::mutex mu;
    static int cache[kMaxDevices] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error(e);
    if (dev < 0 || dev >= kMaxDevices) return DRGG_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return device_error(e);
        if (n <= 0) return DRGG_EUNSUPPORTED;
        cache[dev] = n;
    }
    *cus = cache[dev];
    return DRGG_OK;
}

// Shape checks shared by the three programs.
drgg_status check_problem(int32_t E, int64_t M, int64_t N, int64_t K, drgg_dtype dt) {
    if (E < 1 || E > kMaxExperts) return DRGG_EINVAL;
    if (dt != DRGG_BF16 && dt != DRGG_FP32) return DRGG_EINVAL;
    if (M < 0 || N < 8 || K < 8) return DRGG_ESHAPE;
    // N, K <= 2^22 keep every per-lane byte offset inside a tile below 2^31
    if (M > INT32_MAX || N > (1 << 22) || K > (1 << 22)) return DRGG_ESHAPE;
    if (N % 8 != 0 || K % 8 != 0) return DRGG_EALIGN;
    int64_t t;
    // every buffer: X [M,K], G [M,N], W/dW [E,N,K] (x4 bytes for FP32)
    if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t)) return DRGG_EOVERFLOW;
    if (!mul_ok(M, N, &t) || !mul_ok(t, 4, &t)) return DRGG_EOVERFLOW;
    if (!mul_ok(N, K, &t) || !mul_ok(t, E, &t) || !mul_ok(t, 4, &t)) return DRGG_EOVERFLOW;
    return DRGG_OK;
}

// Element strides of the token-major buffers (see GemmArgs).
struct Layout {
    int64_t a_rs, a_gs, b_rs, b_gs, o_rs, o_gs, T;
};
// grouped calls: rows of one buffer are contiguous, one after the other
Layout grouped_layout(drgg_op op, int64_t N, int64_t K) {
    if (op == DRGG_OP_FWD) return Layout{K, 0, 0, 0, N, 0, 0};
    if (op == DRGG_OP_DGRAD) return Layout{N, 0, 0, 0, K, 0, 0};
    return Layout{N, 0, K, 0, 0, 0, 0};   // weight gradient: A = G rows, B = X rows
}
void set_layout(GemmArgs& a, const Layout& L) {
    a.a_rs = L.a_rs; a.a_gs = L.a_gs; a.b_rs = L.b_rs; a.b_gs = L.b_gs;
    a.o_rs = L.o_rs; a.o_gs = L.o_gs; a.T = L.T;
}

// A batched buffer of B batches x T rows of `row` elements at element
// strides (rs, bs): strides are multiples of 8 (16-byte rows), a row fits
// in its stride, per-lane offsets inside a tile stay below 2^31 (rs <=
// 2^22) and the last element's index fits in 62 bits.  With `output`, no
// two rows may overlap: the batches are either stacked (bs covers T rows)
// or interleaved (rs covers B rows).
drgg_status check_strides(int64_t rs, int64_t bs, int32_t B, int64_t T, int64_t row, bool output) {
    if (rs < row || bs < 0 || rs > (int64_t(1) << 22)) return DRGG_ESHAPE;
    if (rs % 8 != 0 || bs % 8 != 0) return DRGG_EALIGN;
    int64_t a, b;
    if (!mul_ok(T > 0 ? T - 1 : 0, rs, &a) || !mul_ok(B - 1, bs, &b) || a > kMaxBytes - b - row)
        return DRGG_EOVERFLOW;
    if (output && B > 1 && T > 0) {
        const bool stacked = bs >= a + row;
        int64_t c;
        const bool interleaved = bs >= row && mul_ok(B - 1, bs, &c) && rs >= c + row;
        if (!stacked && !interleaved) return DRGG_ESHAPE;
    }
    return DRGG_OK;
}

// Route table of the non-deterministic weight gradient: the problem points
// (E, M, N, K, output type) that run the split program; every other point
// runs the deterministic one.  Filled by the caller from a calibration
// (see drgg_route_split); small and looked up on the host.
constexpr int kMaxRoutes = 256;
struct Route {
    int32_t E;
    int64_t M, N, K;
    int dt;
};
struct RouteTable {
    std::mutex mu;
    Route r[kMaxRoutes];
    int n = 0;
} g_routes;

bool routed_to_split(int32_t E, int64_t M, int64_t N, int64_t K, int dt) {
    std::lock_guard<std::mutex> lock(g_routes.mu);
    for (int i = 0; i < g_routes.n; ++i) {
        const Route& q = g_routes.r[i];
        if (q.E == E && q.M == M && q.N == N && q.K == K && q.dt == dt) return true;
    }
    return false;
}

struct Plan {
    int tile;
    TileShape ts;
    int64_t grid;
    int64_t chunk_max;
    int64_t max_partials;
    size_t ws_bytes;
    int det;   // weight gradient: the program that runs (1 = deterministic)
};

// ws layout, det weight gradient: [partial slots: max_partials*N*K fp32][fold table: E int32x4]
// ws layout, non-det weight gradient: [tile sums: E*P*BM*BN fp32][tickets: E*P u32]
drgg_status make_plan(drgg_op op, int32_t E, int64_t M, int64_t N, int64_t K, int det, int cu_count,
                      Plan* p, int dt = DRGG_BF16) {
    std::memset(p, 0, sizeof *p);
    // The non-deterministic weight gradient runs the deterministic program
    // (chunk partials + ordered fold; its result is a valid
    // non-deterministic result) unless the route table sends the point to
    // the split program; on gfx950 the deterministic program was the faster
    // one at every measured point, because the split program's atomic tile
    // sums are performed beyond the XCDs' L2s.  DRGG_KNOB_NONDET = 1 runs
    // the split program at every point.
    if (op == DRGG_OP_WGRAD && !det && g_knob_nondet.load() == 0 && !routed_to_split(E, M, N, K, dt)) det = 1;
    p->det = det;
    int tile = (int)g_knob_tile.load();
    if (tile < kTileAuto || tile > kTile64x256) tile = kTileAuto;
    if (tile == kTile64x256 && op != DRGG_OP_WGRAD) tile = kTileAuto;
    // the data gradient reads W^T (its workspace) when the experts average
    // enough tokens, or when the test knob asks for it
    const bool dgrad_wt = op == DRGG_OP_DGRAD && (g_knob_dgrad_wt.load() != 0 || dgrad_transposes_w(E, M));
    if (tile == kTileAuto) tile = default_tile((int)op, E, M, N, K, op == DRGG_OP_FWD || dgrad_wt, det != 0);
    p->tile = tile;
    p->ts = tile_shape(tile);
    const int64_t bm = p->ts.bm, bn = p->ts.bn;
    // persistent grid: as many workgroups as fit on the device at once, never
    // more than there are work items (a bound that holds for any offsets)
    const int64_t g_knob = g_knob_grid.load();
    const bool fd = op == DRGG_OP_FWD || op == DRGG_OP_DGRAD;
    const int64_t resident = (int64_t)cu_count * wgs_per_cu(p->ts, fd, !fd && det);
    auto grid_for = [&](int64_t items_max) {
        int64_t g = g_knob > 0 ? g_knob : (resident < items_max ? resident : items_max);
        return g < 1 ? (int64_t)1 : g;
    };
    if (op == DRGG_OP_FWD || op == DRGG_OP_DGRAD) {
        const int64_t ncols = op == DRGG_OP_FWD ? N : K;
        p->grid = grid_for((M / bm + E) * ceil_div(ncols, bn));
        if (op == DRGG_OP_DGRAD) {   // optional: room for W^T
            int64_t b;
            if (!mul_ok((int64_t)E * N, K, &b) || !mul_ok(b, 2, &b)) return DRGG_EOVERFLOW;
            p->ws_bytes = dgrad_wt ? (size_t)round_up(b, 256) : 0;
        }
        return p->grid > INT32_MAX ? DRGG_ESHAPE : DRGG_OK;
    }
    const int64_t P = ceil_div(N, bm) * ceil_div(K, bn);
    if (det) {
        p->chunk_max = wgrad_chunk_max(E, M, N, K);
        p->max_partials = wgrad_max_partials(M, p->chunk_max);
        // chunks_e <= ceil(T_e / chunk_max) <= T_e / chunk_max + 1
        p->grid = grid_for(P * (M / p->chunk_max + E));
        int64_t b;
        if (!mul_ok(p->max_partials, N * K, &b) || !mul_ok(b, 4, &b)) return DRGG_EOVERFLOW;
        // followed by the per-expert fold table: E x {T_e, chunks_e, slot base, 0} int32
        p->ws_bytes = b > 0 ? (size_t)(b + round_up((int64_t)E * 16, 256)) : 0;
    } else {
        p->grid = g_knob > 0 ? g_knob : resident;
        int64_t sums, tk;
        if (!mul_ok(P * E, bm * bn, &sums) || !mul_ok(sums, 4, &sums)) return DRGG_EOVERFLOW;
        tk = P * E * 4;
        p->ws_bytes = (size_t)(round_up(sums, 256) + round_up(tk, 256));
    }
    if (p->grid > INT32_MAX) return DRGG_ESHAPE;
    return DRGG_OK;
}

drgg_status launch_status(hipError_t e) { return e == hipSuccess ? DRGG_OK : device_error(e); }

// Debug check of the group offsets (DRGG_CHECK_OFFSETS): a synchronous copy
// to the host, then o[0] = 0, non-decreasing, o[E] = M, else DRGG_ESHAPE.
// Nothing of the computation has been enqueued when it fails.
drgg_status check_offsets_sync(const int32_t* offs, int32_t E, int64_t M, hipStream_t s) {
    std::vector<int32_t> h((size_t)E + 1);
    hipError_t e = hipMemcpyAsync(h.data(), offs, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return device_error(e);
    if (h[0] != 0 || (int64_t)h[(size_t)E] != M) return DRGG_ESHAPE;
    for (int32_t i = 0; i < E; ++i)
        if (h[(size_t)i + 1] < h[(size_t)i]) return DRGG_ESHAPE;
    return DRGG_OK;
}

// Debug check of the split program's workspace (DRGG_CHECK_WORKSPACE): its
// tile sums and tickets must be zero before a call (a buffer that served a
// deterministic call holds partials); a synchronous copy to the host,
// DRGG_EWORKSPACE if any byte is set.
drgg_status check_workspace_zero(const void* ws, size_t bytes, hipStream_t s) {
    std::vector<uint8_t> h(bytes);
    hipError_t e = hipMemcpyAsync(h.data(), ws, bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return device_error(e);
    for (size_t i = 0; i < bytes; ++i)
        if (h[i] != 0) return DRGG_EWORKSPACE;
    return DRGG_OK;
}

// ---- timing marks (DRGG_KNOB_TIMING) ----------------------------------------
constexpr int kMaxMarks = 8;
std::atomic<int> g_timing_on{0};
struct TimingMarks {
    std::mutex mu;
    hipEvent_t ev[kMaxMarks + 1] = {};
    const char* name[kMaxMarks] = {};
    int n = 0;          // kernels marked in the current call
    bool ended = false;
    int dev = -1;
} g_marks;

}  // namespace

void timing_mark(const char* kernel, hipStream_t s) {
    if (!g_timing_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_marks.mu);
    if (g_marks.ended) { g_marks.n = 0; g_marks.ended = false; }
    if (g_marks.n >= kMaxMarks) return;
    hipEvent_t& e = g_marks.ev[g_marks.n];
    if (!e && hipEventCreate(&e) != hipSuccess) return;
    if (hipEventRecord(e, s) != hipSuccess) return;
    g_marks.name[g_marks.n++] = kernel;
}

void timing_end(hipStream_t s) {
    if (!g_timing_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_marks.mu);
    hipEvent_t& e = g_marks.ev[g_marks.n];
    if (!e && hipEventCreate(&e) != hipSuccess) return;
    if (hipEventRecord(e, s) == hipSuccess) g_marks.ended = true;
}

namespace {

// WT: for the data gradient, a workspace of at least E*N*K*2 bytes to hold
// W^T (then W is transposed into it and the data gradient runs with both
// operands reduction-contiguous), or null (W read transposed in the kernel).
drgg_status run_fwd_dgrad(drgg_op op, const void* A, const void* W, const int32_t* offs, int32_t E,
                          int64_t M, int64_t N, int64_t K, drgg_dtype dt, void* out, hipStream_t s,
                          void* WT, const Layout& L) {
    drgg_status st = check_problem(E, M, N, K, dt);
    if (st != DRGG_OK) return st;
    // with no tokens the token-indexed buffers may be empty (null); a
    // batched call (L.T > 0 or M == 0 with uniform groups) has no offsets
    if (!W || (!offs && L.T == 0 && M > 0) || (M > 0 && (!A || !out))) return DRGG_EINVAL;
    if (!aligned16(A) || !aligned16(W) || !aligned16(out) || (reinterpret_cast<uintptr_t>(offs) & 3u))
        return DRGG_EALIGN;
    if (offs && checks_offsets()) {
        st = check_offsets_sync(offs, E, M, s);
        if (st != DRGG_OK) return st;
    }
    if (M == 0) return DRGG_OK;   // no rows to write
    int cus = 0;
    st = current_cu_count(&cus);
    if (st != DRGG_OK) return st;
    Plan p;
    st = make_plan(op, E, M, N, K, 1, cus, &p);
    if (st != DRGG_OK) return st;
    GemmArgs a{};
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(W);
    a.offs = offs;
    a.out = out;
    a.M = M; a.N = N; a.K = K; a.E = E;
    set_layout(a, L);
    a.items_max = p.grid;
    a.reverse = (int32_t)(g_knob_reverse.load() != 0);
    if (op == DRGG_OP_DGRAD && WT) {
        hipError_t e = launch_transpose_w(a.B, static_cast<uint16_t*>(WT), E, N, K, s);
        if (e != hipSuccess) return device_error(e);
        a.B = static_cast<const uint16_t*>(WT);
        return launch_status(launch_fwd_dgrad(2, p.tile, a, dt == DRGG_BF16, s));
    }
    return launch_status(launch_fwd_dgrad((int)op, p.tile, a, dt == DRGG_BF16, s));
}

// validate_only: run the argument checks (and the offsets debug check) and
// stop before the first launch; the split program's workspace check is left
// to the call that follows.
drgg_status run_wgrad(const void* X, const void* G, const int32_t* group_offsets, int32_t E, int64_t M, int64_t N,
                      int64_t K, drgg_dtype out_dtype, int deterministic, void* dW, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, const Layout& L, bool validate_only = false) {
    drgg_status st = check_problem(E, M, N, K, out_dtype);
    if (st != DRGG_OK) return st;
    if (!dW || (M > 0 && (!X || !G))) return DRGG_EINVAL;
    if (!aligned16(X) || !aligned16(G) || !aligned16(dW) ||
        (reinterpret_cast<uintptr_t>(group_offsets) & 3u))
        return DRGG_EALIGN;
    // the workspace size does not depend on the CU count: check it before
    // touching the device
    Plan p;
    st = make_plan(DRGG_OP_WGRAD, E, M, N, K, deterministic, 1, &p, out_dtype);
    if (st != DRGG_OK) return st;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return DRGG_EWORKSPACE;
        if (!aligned16(workspace)) return DRGG_EALIGN;
    }
    int cus = 0;
    st = current_cu_count(&cus);
    if (st != DRGG_OK) return st;
    const size_t checked = p.ws_bytes;
    const int checked_det = p.det;
    st = make_plan(DRGG_OP_WGRAD, E, M, N, K, deterministic, cus, &p, out_dtype);
    if (st != DRGG_OK) return st;
    // the route table changed in between: the workspace was checked (and
    // may have been prepared) for the other program
    if (p.ws_bytes != checked || p.det != checked_det) return DRGG_EWORKSPACE;
    if (group_offsets && checks_offsets()) {
        st = check_offsets_sync(group_offsets, E, M, stream);
        if (st != DRGG_OK) return st;
    }
    if (!p.det && p.ws_bytes > 0 && checks_workspace() && !validate_only) {
        st = check_workspace_zero(workspace, p.ws_bytes, stream);
        if (st != DRGG_OK) return st;
    }
    if (validate_only) return DRGG_OK;
    GemmArgs a{};
    a.A = static_cast<const uint16_t*>(G);   // A rows: output rows n of dW (from G)
    a.B = static_cast<const uint16_t*>(X);   // B rows: output cols k of dW (from X)
    a.offs = group_offsets;
    a.out = dW;
    a.M = M; a.N = N; a.K = K; a.E = E;
    set_layout(a, L);
    a.reverse = (int32_t)(g_knob_reverse.load() != 0);
    const bool bf16 = out_dtype == DRGG_BF16;
    if (p.det) {
        a.partial = static_cast<float*>(workspace);
        a.fold_info = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.max_partials * N * K * 4);
        a.chunk_max = p.chunk_max;
        a.items_max = M > 0 ? p.grid : 0;
        // an expert has at most M tokens: with chunk_max >= M none is cut
        // into chunks, and the fold would only zero the empty experts
        a.zero_empty = M > 0 && p.chunk_max >= M;
        return launch_status(launch_wgrad_det(p.tile, a, bf16, stream));
    }
    const int64_t P = ceil_div(N, p.ts.bm) * ceil_div(K, p.ts.bn);
    const int64_t sums = round_up(P * E * p.ts.bm * p.ts.bn * 4, 256);
    a.chunk_max = wgrad_chunk_max(E, M, N, K);   // chunks in whole 512-token units on the device
    a.tilesum = static_cast<float*>(workspace);
    a.delay_seed = (int32_t)g_knob_delay.load();
    a.report = reinterpret_cast<int32_t*>(g_knob_report.load());
    a.tickets = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + sums);
    return launch_status(launch_wgrad_atomic(p.tile, a, p.grid, bf16, stream));
}

// The data gradient: with a large enough workspace, W^T goes there (the
// faster program; the results are bitwise the same either way).
drgg_status run_dgrad(const void* G, const void* W, const int32_t* offs, int32_t E, int64_t M, int64_t N,
                      int64_t K, drgg_dtype out_dtype, void* dX, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, const Layout& L) {
    drgg_status st = check_problem(E, M, N, K, out_dtype);
    if (st != DRGG_OK) return st;
    Plan p;
    st = make_plan(DRGG_OP_DGRAD, E, M, N, K, 1, 1, &p);
    if (st != DRGG_OK) return st;
    void* WT = nullptr;
    if (workspace && workspace_bytes >= p.ws_bytes && p.ws_bytes > 0) {
        if (!aligned16(workspace)) return DRGG_EALIGN;
        WT = workspace;
    }
    return run_fwd_dgrad(DRGG_OP_DGRAD, G, W, offs, E, M, N, K, out_dtype, dX, stream, WT, L);
}

// Checks shared by the batched calls; fills E, M and the layout.
drgg_status batched_setup(drgg_op op, const drgg_batched* b, int32_t* E, int64_t* M, Layout* L) {
    if (!b) return DRGG_EINVAL;
    if (b->B < 1 || b->B > kMaxExperts) return DRGG_EINVAL;
    if (b->T < 0 || b->N < 8 || b->K < 8) return DRGG_ESHAPE;
    int64_t m;
    if (!mul_ok(b->B, b->T, &m) || m > INT32_MAX) return DRGG_ESHAPE;
    const int64_t alen = op == DRGG_OP_DGRAD ? b->N : b->K;   // A: dgrad G, else X
    const int64_t olen = op == DRGG_OP_FWD ? b->N : b->K;     // out: Y or dX
    drgg_status st = check_strides(b->a_row, b->a_batch, b->B, b->T, alen, false);
    if (st != DRGG_OK) return st;
    if (op == DRGG_OP_WGRAD) {
        st = check_strides(b->b_row, b->b_batch, b->B, b->T, b->N, false);
        if (st != DRGG_OK) return st;
        // kernel operands: A = G rows (b_*), B = X rows (a_*)
        *L = Layout{b->b_row, b->b_batch - b->T * b->b_row, b->a_row, b->a_batch - b->T * b->a_row, 0, 0, b->T};
    } else {
        st = check_strides(b->o_row, b->o_batch, b->B, b->T, olen, true);
        if (st != DRGG_OK) return st;
        *L = Layout{b->a_row, b->a_batch - b->T * b->a_row, 0, 0, b->o_row, b->o_batch - b->T * b->o_row, b->T};
    }
    *E = b->B;
    *M = m;
    return DRGG_OK;
}

}  // namespace
}  // namespace drgg

using namespace drgg;

extern "C" {

drgg_status grouped_gemm_fwd(const void* X, const void* W, const int32_t* group_offsets, int32_t E,
                             int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype, int deterministic,
                             void* Y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    (void)deterministic; (void)workspace; (void)workspace_bytes;   // one program for both variants
    if (!group_offsets) return DRGG_EINVAL;
    return run_fwd_dgrad(DRGG_OP_FWD, X, W, group_offsets, E, M, N, K, out_dtype, Y, stream, nullptr,
                         grouped_layout(DRGG_OP_FWD, N, K));
}

drgg_status grouped_gemm_dgrad(const void* G, const void* W, const int32_t* group_offsets, int32_t E,
                               int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype, int deterministic,
                               void* dX, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    (void)deterministic;
    if (!group_offsets) return DRGG_EINVAL;
    return run_dgrad(G, W, group_offsets, E, M, N, K, out_dtype, dX, workspace, workspace_bytes, stream,
                     grouped_layout(DRGG_OP_DGRAD, N, K));
}

drgg_status grouped_gemm_wgrad(const void* X, const void* G, const int32_t* group_offsets, int32_t E,
                               int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype, int deterministic,
                               void* dW, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!group_offsets) return DRGG_EINVAL;
    return run_wgrad(X, G, group_offsets, E, M, N, K, out_dtype, deterministic, dW, workspace, workspace_bytes,
                     stream, grouped_layout(DRGG_OP_WGRAD, N, K));
}

drgg_status grouped_gemm_wgrad_noalloc(const void* X, const void* G, const int32_t* group_offsets, int32_t E,
                                       int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype, int deterministic,
                                       void* dW, hipStream_t stream) {
    if (!group_offsets) return DRGG_EINVAL;
    drgg_status st = check_problem(E, M, N, K, out_dtype);
    if (st != DRGG_OK) return st;
    Plan p;   // the workspace size does not depend on the CU count
    st = make_plan(DRGG_OP_WGRAD, E, M, N, K, deterministic, 1, &p, out_dtype);
    if (st != DRGG_OK) return st;
    if (p.ws_bytes > kScratchBytes) return DRGG_EWORKSPACE;
    void* ws = nullptr;
    if (p.ws_bytes > 0) {
        hipError_t e = scratch_buffer(&ws);
        if (e != hipSuccess) return device_error(e);
    }
    // The split program needs zero tile sums and tickets; the array may
    // hold a deterministic call's partials, so clear that much first (a fill
    // kernel on the stream: capturable, allocates nothing).  The plain
    // argument checks of run_wgrad come first, so nothing is enqueued for a
    // call they refuse.
    if (!p.det && p.ws_bytes > 0) {
        st = run_wgrad(X, G, group_offsets, E, M, N, K, out_dtype, deterministic, dW, ws, kScratchBytes, stream,
                       grouped_layout(DRGG_OP_WGRAD, N, K), /*validate_only=*/true);
        if (st != DRGG_OK) return st;
        hipError_t e = launch_zero(ws, p.ws_bytes, stream);
        if (e != hipSuccess) return device_error(e);
    }
    return run_wgrad(X, G, group_offsets, E, M, N, K, out_dtype, deterministic, dW, ws, ws ? kScratchBytes : 0,
                     stream, grouped_layout(DRGG_OP_WGRAD, N, K));
}

drgg_status batched_gemm_fwd(const void* X, const void* W, const drgg_batched* shape, drgg_dtype out_dtype,
                             void* Y, hipStream_t stream) {
    int32_t E;
    int64_t M;
    Layout L;
    drgg_status st = batched_setup(DRGG_OP_FWD, shape, &E, &M, &L);
    if (st != DRGG_OK) return st;
    return run_fwd_dgrad(DRGG_OP_FWD, X, W, nullptr, E, M, shape->N, shape->K, out_dtype, Y, stream, nullptr, L);
}

drgg_status batched_gemm_dgrad(const void* G, const void* W, const drgg_batched* shape, drgg_dtype out_dtype,
                               void* dX, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int32_t E;
    int64_t M;
    Layout L;
    drgg_status st = batched_setup(DRGG_OP_DGRAD, shape, &E, &M, &L);
    if (st != DRGG_OK) return st;
    return run_dgrad(G, W, nullptr, E, M, shape->N, shape->K, out_dtype, dX, workspace, workspace_bytes, stream, L);
}

drgg_status batched_gemm_wgrad(const void* X, const void* G, const drgg_batched* shape, drgg_dtype out_dtype,
                               int deterministic, void* dW, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    int32_t E;
    int64_t M;
    Layout L;
    drgg_status st = batched_setup(DRGG_OP_WGRAD, shape, &E, &M, &L);
    if (st != DRGG_OK) return st;
    return run_wgrad(X, G, nullptr, E, M, shape->N, shape->K, out_dtype, deterministic, dW, workspace,
                     workspace_bytes, stream, L);
}

// Router argument checks shared by both entry points and the size query.
static drgg_status check_router(int64_t M, int64_t N, int64_t K) {
    // N, K <= 2^22 keep every per-lane byte offset inside a 128-row block of
    // the operands (the single-pass program; the sliced one, with 256-row
    // blocks, runs only for K <= 2^21) and of the output below 2^31
    if (M < 0 || N < 1 || K < 8 || M > INT32_MAX || N > (int64_t(1) << 22) || K > (int64_t(1) << 22))
        return DRGG_ESHAPE;
    if (K % 8 != 0 || N % 4 != 0) return DRGG_EALIGN;
    int64_t t;
    if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t) || !mul_ok(M, N, &t) || !mul_ok(t, 32, &t) ||
        !mul_ok(N, K, &t) || !mul_ok(t, 4, &t))
        return DRGG_EOVERFLOW;
    // one workgroup per 128x128 tile (the single-pass program; the sliced
    // one has at most as many): the grid must fit its 32-bit size
    if (ceil_div(M, 128) * ceil_div(N, 128) > INT32_MAX) return DRGG_ESHAPE;
    return DRGG_OK;
}



drgg_status router_gemm_fp32_bf16x3(const float* X, const float* Wr, int64_t M, int64_t N, int64_t K,
                                    float* out, hipStream_t stream) {
    if (!X || !Wr || !out) return DRGG_EINVAL;
    drgg_status st = check_router(M, N, K);
    if (st != DRGG_OK) return st;
    if (!aligned16(X) || !aligned16(Wr) || !aligned16(out)) return DRGG_EALIGN;
    if (M == 0) return DRGG_OK;
    return launch_status(launch_router(X, Wr, out, M, N, K, stream));
}

drgg_status router_workspace_size(int64_t M, int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return DRGG_EINVAL;
    drgg_status st = check_router(M, N, K);
    if (st != DRGG_OK) return st;
    const RouterSplit r = router_split(M, N, K);
    *bytes = r.ks > 1 ? (size_t)((r.ks - 1) * M * N * 4) : 0;
    return DRGG_OK;
}

drgg_status drgg_router_split(int64_t M, int64_t N, int64_t K, int64_t* ks, int64_t* kq) {
    if (!ks || !kq) return DRGG_EINVAL;
    drgg_status st = check_router(M, N, K);
    if (st != DRGG_OK) return st;
    const RouterSplit r = router_split(M, N, K);
    *ks = r.ks;
    *kq = r.kq;
    return DRGG_OK;
}

drgg_status router_gemm_fp32_bf16x3_ws(const float* X, const float* Wr, int64_t M, int64_t N, int64_t K,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    if (!X || !Wr || !out) return DRGG_EINVAL;
    drgg_status st = check_router(M, N, K);
    if (st != DRGG_OK) return st;
    if (!aligned16(X) || !aligned16(Wr) || !aligned16(out)) return DRGG_EALIGN;
    const RouterSplit r = router_split(M, N, K);
    const size_t need = r.ks > 1 ? (size_t)((r.ks - 1) * M * N * 4) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return DRGG_EWORKSPACE;
    if (need > 0 && !aligned16(workspace)) return DRGG_EALIGN;
    if (M == 0) return DRGG_OK;
    if (r.ks == 0) return launch_status(launch_router(X, Wr, out, M, N, K, stream));
    return launch_status(
        launch_router_ks(X, Wr, out, static_cast<float*>(workspace), M, N, K, r.ks, r.kq, stream));
}

drgg_status grouped_gemm_workspace_size(drgg_op op, int32_t E, int64_t M, int64_t N, int64_t K,
                                        drgg_dtype out_dtype, int deterministic, int cu_count,
                                        size_t* bytes) {
    if (!bytes) return DRGG_EINVAL;
    if (op != DRGG_OP_FWD && op != DRGG_OP_DGRAD && op != DRGG_OP_WGRAD) return DRGG_EINVAL;
    drgg_status st = check_problem(E, M, N, K, out_dtype);
    if (st != DRGG_OK) return st;
    Plan p;   // the workspace size does not depend on the CU count
    st = make_plan(op, E, M, N, K, deterministic, cu_count > 0 ? cu_count : 1, &p, out_dtype);
    if (st != DRGG_OK) return st;
    *bytes = p.ws_bytes;
    return DRGG_OK;
}

drgg_status drgg_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (workspace_bytes == 0) return DRGG_OK;
    if (!workspace) return DRGG_EINVAL;
    return launch_status(launch_zero(workspace, workspace_bytes, stream));
}

drgg_status drgg_plan(drgg_op op, int32_t E, int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype,
                      int deterministic, int cu_count, drgg_plan_info* out) {
    if (!out) return DRGG_EINVAL;
    if (op != DRGG_OP_FWD && op != DRGG_OP_DGRAD && op != DRGG_OP_WGRAD) return DRGG_EINVAL;
    drgg_status st = check_problem(E, M, N, K, out_dtype);
    if (st != DRGG_OK) return st;
    if (cu_count <= 0) {
        st = current_cu_count(&cu_count);
        if (st != DRGG_OK) return st;
    }
    Plan p;
    st = make_plan(op, E, M, N, K, deterministic, cu_count, &p, out_dtype);
    if (st != DRGG_OK) return st;
    std::memset(out, 0, sizeof *out);
    out->tile_m = p.ts.bm;
    out->tile_n = p.ts.bn;
    out->tile_k = kStageK;
    out->mfma_m = kMfmaM;
    out->mfma_n = kMfmaN;
    out->mfma_k = kMfmaK;
    out->grid = p.grid;
    out->chunk_max = p.chunk_max;
    out->unit = (op == DRGG_OP_WGRAD && !p.det) ? kStreamKUnit : 0;
    out->max_partials = p.max_partials;
    out->workspace_bytes = p.ws_bytes;
    return DRGG_OK;
}

drgg_status drgg_wgrad_chunking(int64_t T, int64_t chunk_max, int64_t* chunk_len, int64_t* chunks) {
    if (!chunk_len || !chunks || chunk_max < kTileK || chunk_max % kTileK != 0 || T < 0 || T > INT32_MAX)
        return DRGG_EINVAL;
    wgrad_chunking(T, chunk_max, chunk_len, chunks);
    return DRGG_OK;
}

drgg_status drgg_wgrad_tail_plan(const int32_t* group_offsets, int32_t E, int64_t N, int64_t K, int* tail_only,
                                 int32_t* row0) {
    if (!group_offsets || !tail_only || E < 1 || E > kMaxExperts || N < 8 || K < 8 || N > (1 << 22) ||
        K > (1 << 22))
        return DRGG_EINVAL;
    *tail_only = wgrad_tail_plan(group_offsets, E, N, K, row0) ? 1 : 0;
    return DRGG_OK;
}

drgg_status drgg_wgrad_split_plan(const int32_t* group_offsets, int32_t E, int64_t N, int64_t K, int tile,
                                  int64_t grid, int* slack, int64_t* tail_tiles, int* banded_walk) {
    if (!group_offsets || !slack || !tail_tiles || E < 1 || E > kMaxExperts || N < 8 || K < 8 || grid < 1 ||
        tile < kTileAuto || tile > kTile64x256)
        return DRGG_EINVAL;
    const TileShape ts = tile_shape(tile == kTileAuto ? default_tile(DRGG_OP_WGRAD, E, 0, N, K, false, false) : tile);
    int64_t out[2];
    *slack = wgrad_split_plan(group_offsets, E, N, K, ts.bm, ts.bn, grid, out) ? 1 : 0;
    *tail_tiles = out[0];
    if (banded_walk) *banded_walk = (int)out[1];
    return DRGG_OK;
}

drgg_status drgg_tailsplit_units(int64_t tiles, int64_t workers, int64_t* out) {
    if (!out || tiles < 0 || workers < 1) return DRGG_EINVAL;
    const TailSplit t = tailsplit_units(tiles, workers);
    out[0] = t.tiles;
    out[1] = t.units;
    out[2] = t.full;
    out[3] = t.split;
    return DRGG_OK;
}

drgg_status drgg_route_split(int32_t E, int64_t M, int64_t N, int64_t K, drgg_dtype out_dtype) {
    drgg_status st = check_problem(E, M, N, K, out_dtype);
    if (st != DRGG_OK) return st;
    std::lock_guard<std::mutex> lock(g_routes.mu);
    for (int i = 0; i < g_routes.n; ++i) {
        const Route& q = g_routes.r[i];
        if (q.E == E && q.M == M && q.N == N && q.K == K && q.dt == (int)out_dtype) return DRGG_OK;
    }
    if (g_routes.n >= kMaxRoutes) return DRGG_EUNSUPPORTED;
    g_routes.r[g_routes.n++] = Route{E, M, N, K, (int)out_dtype};
    return DRGG_OK;
}

drgg_status drgg_hold_cus(int cus, int64_t microseconds, hipStream_t stream) {
    if (cus < 1 || cus > 4096 || microseconds < 0 || microseconds > 1000000) return DRGG_EINVAL;
    return launch_status(launch_hold_cus(cus, (uint64_t)microseconds * 100, stream));
}

drgg_status drgg_route_clear(void) {
    std::lock_guard<std::mutex> lock(g_routes.mu);
    g_routes.n = 0;
    return DRGG_OK;
}

int drgg_route_count(void) {
    std::lock_guard<std::mutex> lock(g_routes.mu);
    return g_routes.n;
}

drgg_status drgg_set_knob(int knob, int64_t value) {
    switch (knob) {
        case DRGG_KNOB_TILE:
            if (value < 0 || value > kTile64x256) return DRGG_EINVAL;
            g_knob_tile.store(value);
            return DRGG_OK;
        case DRGG_KNOB_GRID:
            if (value < 0 || value > INT32_MAX) return DRGG_EINVAL;
            g_knob_grid.store(value);
            return DRGG_OK;
        case DRGG_KNOB_REVERSE:
            g_knob_reverse.store(value != 0);
            return DRGG_OK;
        case DRGG_KNOB_TIMING:
            g_timing_on.store(value != 0);
            return DRGG_OK;
        case DRGG_KNOB_NONDET:
            g_knob_nondet.store(value != 0);
            return DRGG_OK;
        case DRGG_KNOB_CHECK_OFFSETS:
            g_knob_check_offsets.store(value != 0);
            return DRGG_OK;
        case DRGG_KNOB_CHECK_WORKSPACE:
            g_knob_check_ws.store(value != 0);
            return DRGG_OK;
        case DRGG_KNOB_DELAY_SEED:
            if (value < 0 || value > INT32_MAX) return DRGG_EINVAL;
            g_knob_delay.store(value);
            return DRGG_OK;
        case DRGG_KNOB_SPLIT_REPORT:
            if (value < 0 || (value & 15) != 0) return DRGG_EINVAL;
            g_knob_report.store(value);
            return DRGG_OK;
        case DRGG_KNOB_DGRAD_WT:
            g_knob_dgrad_wt.store(value != 0);
            return DRGG_OK;
        default:
            return DRGG_EINVAL;
    }
}

int drgg_timing_count(void) {
    std::lock_guard<std::mutex> lock(g_marks.mu);
    return g_marks.ended ? g_marks.n : 0;
}

drgg_status drgg_timing_read(int i, const char** kernel, float* ms) {
    if (!kernel || !ms) return DRGG_EINVAL;
    std::lock_guard<std::mutex> lock(g_marks.mu);
    if (!g_marks.ended || i < 0 || i >= g_marks.n) return DRGG_EINVAL;
    if (hipEventSynchronize(g_marks.ev[i + 1]) != hipSuccess) return DRGG_EDEVICE;
    if (hipEventElapsedTime(ms, g_marks.ev[i], g_marks.ev[i + 1]) != hipSuccess) return DRGG_EDEVICE;
    *kernel = g_marks.name[i];
    return DRGG_OK;
}

const char* drgg_status_string(drgg_status s) {
    switch (s) {
        case DRGG_OK: return "ok";
        case DRGG_EINVAL: return "invalid argument (null pointer, bad enum value or E outside 1..1024)";
        case DRGG_ESHAPE: return "invalid shape (negative or too large dimension, or group offsets that fail the debug check)";
        case DRGG_EALIGN: return "misaligned (pointers must be 16-byte aligned, N and K multiples of 8)";
        case DRGG_EOVERFLOW: return "size overflow in 64-bit arithmetic";
        case DRGG_EWORKSPACE: return "workspace missing or too small (or, with the debug check on, not zero for the split program)";
        case DRGG_EUNSUPPORTED: return "unsupported on this device or combination";
        case DRGG_EDEVICE: {
            thread_local char msg[256];
            snprintf(msg, sizeof msg, "HIP error while querying the device or launching (%s: %s)",
                     hipGetErrorName(g_last_hip_error), hipGetErrorString(g_last_hip_error));
            return msg;
        }
    }
    return "unknown status";
}

int drgg_abi_version(void) { return DRGG_ABI_VERSION; }

}  // extern "C"
