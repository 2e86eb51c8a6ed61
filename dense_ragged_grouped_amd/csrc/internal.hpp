// internal.hpp -- declarations shared by the C ABI (api.cpp) and the kernel
// launchers (kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace drgg {

// Arguments of the grouped-GEMM kernels, passed by value.
struct GemmArgs {
    const uint16_t* A;     // fwd: X   dgrad: G   wgrad: G  (BF16 bits)
    const uint16_t* B;     // fwd: W   dgrad: W   wgrad: X
    const int32_t* offs;   // group offsets [E+1], device (null: uniform groups of T rows)
    void* out;             // Y / dX / dW
    float* partial;        // det wgrad: chunk partial slots [slot][N][K]
    int32_t* fold_info;    // det wgrad: [E][4] = T_e, chunks_e, first slot, 0 (chunk kernel -> fold)
    float* tilesum;        // non-det wgrad: FP32 tile sums [E*P][BM*BN]
    uint32_t* tickets;     // non-det wgrad: [E*P]
    int64_t M, N, K;
    // Token-major operands and the fwd/dgrad output: row r (its index in the
    // offsets' row space) of group e starts at element base + r * rs + e * gs.
    // Grouped calls: rs = the row length, gs = 0.  Batched calls (offs null,
    // groups of T rows): rs = the row stride, gs = batch stride - T * rs.
    int64_t a_rs, a_gs;    // A: fwd X, dgrad G, wgrad G
    int64_t b_rs, b_gs;    // wgrad B: X
    int64_t o_rs, o_gs;    // fwd Y, dgrad dX
    int64_t T;             // offs null: group e is rows e*T .. e*T+T-1
    int64_t chunk_max;     // det wgrad: longest chunk
    int64_t items_max;     // workgroups launched (fwd/dgrad/det wgrad)
    int32_t E;
    int32_t reverse;       // walk work items in reverse (test knob)
    int32_t delay_seed;    // split program: seeded delays before tail arrivals (test knob; 0 = off)
    int32_t* report;       // split program: if set, workgroup 0 writes its tail decision here (test aid)
    int32_t zero_empty;    // det wgrad: no expert can have two chunks, so no fold runs and the chunk
                           // kernel writes the zero output of experts without tokens itself
};

// op 0: forward; 1: data gradient; 2: data gradient with a.B = W^T [E][K][N]
hipError_t launch_fwd_dgrad(int op, int tile, const GemmArgs& a, bool bf16, hipStream_t s);
hipError_t launch_transpose_w(const uint16_t* W, uint16_t* WT, int32_t E, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_wgrad_det(int tile, const GemmArgs& a, bool bf16, hipStream_t s);
hipError_t launch_wgrad_atomic(int tile, const GemmArgs& a, int64_t grid_n, bool bf16, hipStream_t s);
hipError_t launch_router(const float* X, const float* Wr, float* out, int64_t M, int64_t N, int64_t K,
                         hipStream_t s);
hipError_t launch_router_ks(const float* X, const float* Wr, float* out, float* part, int64_t M, int64_t N,
                            int64_t K, int64_t ks, int64_t kq, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// The fixed device workspace of grouped_gemm_wgrad_noalloc: its size, and the
// device address of the current device's copy (looked up once per device).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_buffer(void** ptr);
hipError_t launch_hold_cus(int n, uint64_t ticks, hipStream_t s);

// Per-launch timing marks (a measurement knob, off by default): when on, an
// event is recorded on the stream before every kernel launch of a call and
// once after the last one, so each kernel's duration can be read back.
void timing_mark(const char* kernel, hipStream_t s);   // before a launch
void timing_end(hipStream_t s);                         // after the last launch

}  // namespace drgg
