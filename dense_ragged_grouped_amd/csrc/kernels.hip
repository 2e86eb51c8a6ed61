// kernels.hip -- gfx950 (CDNA4) kernels of the ragged BF16 grouped GEMM.
//
// Programs (flashinfer PR #8258, "run the split k512 wgrad tail whole on the
// least-loaded clusters on sm_107a", opening summary paragraph):
//   forward          Y[t,n]    = sum_k X[t,k]   W[e(t),n,k]
//   data gradient    dX[t,k]   = sum_n G[t,n]   W[e(t),n,k]
//   weight gradient  dW[e,n,k] = sum_{t of e} G[t,n] X[t,k]
// with FP32 accumulation on v_mfma_f32_32x32x16_bf16 and one rounding.
//
// One workgroup computes one BMxBN output tile at a time and walks a list of
// tiles (persistent).  The 256x256 forward, data-gradient and deterministic
// weight-gradient kernels run 8 waves (two per SIMD) in a 4x2 wave grid, each
// wave a 64x128 block; every other kernel runs 4 waves (one per SIMD) in a
// 2x2 grid, each wave a (BM/2)x(BN/2) block.  A wave's block is made of
// 32x32 MFMA tiles whose FP32 accumulators stay in registers for the whole
// reduction.
//
// Operand staging.  The reduction runs in stages of 32 values through four
// LDS stage slots per operand, filled straight from HBM by 16-byte buffer
// loads with an LDS destination (no registers in between), three steps
// ahead of their use.  Operands whose reduction index is contiguous in
// memory ("K-major": X and W in the forward, G in the data gradient) are
// loaded two stages at a time as whole 128-byte rows; operands whose
// reduction index is strided ("MN-major": W in the data gradient, G and X in
// the weight gradient, reduced over tokens) one 32-row stage at a time and
// read back transposed by ds_read_b64_tr_b16.  Both layouts are XOR-swizzled
// so that the MFMA operand reads are free of bank conflicts.
//
// Ragged groups.  Every workgroup reads the group offsets, clamps them into
// [0, M] and builds the per-expert prefix of work items in LDS; a work index
// is then mapped to (expert, tile, chunk) by binary search.  Rows, columns
// and reduction positions outside an operand's valid range are never read:
// their loads carry an out-of-range offset and write zeros to LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "internal.hpp"
#include "plan.hpp"

namespace drgg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;       // fold / zero / router kernels
// Grouped-GEMM kernels run 4 waves (one per SIMD) or, for the 256x256
// forward and data-gradient tiles, 8 (two per SIMD, each on half the
// accumulators): a second wave per SIMD covers the stalls of the first.
constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kMaxGemmThreads = 512;

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    // round to nearest, ties to even; NaN stays a (quiet) NaN
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// ---------------------------------------------------------------------------
// ragged work decode

// LDS pointers keep their address space in the type, so that every access
// compiles to ds_* instructions (a generic pointer would become a flat access
// that also waits for outstanding global loads).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_t;

struct Sched {
    int32_t offs[kMaxExperts + 1];    // clamped, non-decreasing offsets
    int32_t prefix[kMaxExperts + 1];  // exclusive prefix of work per expert
    int32_t scan[kMaxGemmThreads];
};

// Exclusive scan of v over the workgroup's threads (in thread order), with
// the sum (MAX = false) or the maximum (MAX = true, identity 0: the values
// are non-negative); *total gets the reduction over all threads.  Inclusive
// scans within each wave by lane shuffles, then one pass over the (at most
// 8) wave results in `tmp` (LDS, one word per wave plus one).  A serial pass
// over every thread's value, or a barrier per doubling step, costs
// microseconds at kernel start; this costs a few hundred cycles.  Must be
// called by all threads; ends with a barrier.
template <bool MAX = false, class Ptr>
__device__ int32_t block_exclusive_scan(int32_t v, Ptr tmp, int32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x = MAX ? max(x, y) : x + y;
    }
    const int32_t excl_in_wave = MAX ? __shfl_up(x, 1, 64) : x - v;
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t acc = 0;
        for (int w = 0; w < nw; ++w) {
            const int32_t t = tmp[w];
            tmp[w] = acc;
            acc = MAX ? max(acc, t) : acc + t;
        }
        tmp[nw] = acc;
    }
    __syncthreads();
    const int32_t before = tmp[wave];
    const int32_t r = MAX ? max(before, lane > 0 ? excl_in_wave : 0) : before + excl_in_wave;
    *total = tmp[nw];
    __syncthreads();
    return r;
}

// Lanes of one wave exchanging data through LDS: the fences order each
// lane's accesses before and after this point for the compiler (no
// instruction is emitted; the wave's DS instructions execute in order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive scans (maximum, sum) over the 64 lanes of a wave.  With fewer
// than kWaveExperts experts the prologue steps below run on wave 0 alone:
// shuffles instead of the workgroup scans, one barrier instead of three or
// more per step (each costs a few hundred cycles at kernel start).
constexpr int kWaveExperts = 64;
__device__ __forceinline__ int32_t wave_incl_max(int32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x = max(x, y);
    }
    return x;
}
__device__ __forceinline__ int32_t wave_incl_sum(int32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

// Fills s.offs[0..E] with the offsets clamped into [0, M] (and made
// non-decreasing), and s.prefix[0..E] with the exclusive prefix of
// work(e, T_e).  With no offsets array (a batched call) the groups are
// uniform: offs[e] = e * T.  With fewer than kWaveExperts experts wave 0
// does it all (offsets on lanes 0..E, shuffle scans).  Must be called by all
// threads; ends with a barrier.
template <class WorkFn>
__device__ void build_schedule(Sched& s, const int32_t* __restrict__ offs, int E, int64_t M, int64_t T,
                               WorkFn work) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    if (E < kWaveExperts) {
        // lane e of wave 0 holds offset e (e <= E)
        if (tid < 64) {
            int64_t v = 0;
            if (tid <= E) v = offs ? (int64_t)offs[tid] : tid * T;
            v = v < 0 ? 0 : (v > M ? M : v);
            const int32_t o = wave_incl_max(tid <= E ? (int32_t)v : 0);
            const int32_t o1 = __shfl_down(o, 1, 64);
            const int32_t wk = tid < E ? work(tid, o1 - o) : 0;
            const int32_t incl = wave_incl_sum(wk);
            if (tid <= E) {
                s.offs[tid] = o;
                s.prefix[tid] = incl - wk;
            }
        }
        __syncthreads();
        return;
    }
    int32_t* tmp = s.scan;   // free until the prefix is written
    for (int e = tid; e <= E; e += nthr) {
        int64_t v = offs ? (int64_t)offs[e] : e * T;
        v = v < 0 ? 0 : (v > M ? M : v);
        s.offs[e] = (int32_t)v;
    }
    __syncthreads();
    // make non-decreasing (a running max); E <= 1024, one run per thread
    const int per = (E + nthr) / nthr;   // covers indices 0..E
    const int lo = min(tid * per, E + 1);
    const int hi = min(lo + per, E + 1);
    int32_t run = 0;
    for (int i = lo; i < hi; ++i) run = max(run, s.offs[i]);
    int32_t total;
    int32_t carry = block_exclusive_scan<true>(run, tmp, &total);
    for (int i = lo; i < hi; ++i) {
        carry = max(carry, s.offs[i]);
        s.offs[i] = carry;
    }
    __syncthreads();
    // work counts and their exclusive prefix
    int32_t local = 0;
    for (int e = lo; e < hi && e < E; ++e) local += work(e, s.offs[e + 1] - s.offs[e]);
    int32_t acc = block_exclusive_scan(local, tmp, &total);
    for (int e = lo; e < hi; ++e) {
        s.prefix[e] = acc;
        if (e < E) acc += work(e, s.offs[e + 1] - s.offs[e]);
    }
    __syncthreads();
}

// Weight-gradient work order: longest token chunks first.  Items of one
// expert all cost about the same (a tile over one chunk of its tokens), so
// the experts are put in decreasing order of chunk length (ties: expert
// index) and, for the persistent walk below, the rounds alternate direction
// ("snake"): the longest items of round r and the shortest of round r+1 land
// on the same workgroup.  On the Zipf-routed E=32 workload that balances the
// workgroups to 96 % of the mean load, against 81 % in expert order.
//
// rank_experts writes that order as 16-bit expert ids over s.scan (which
// build_schedule no longer needs): expert_at(s, p) is the expert at position
// p.  position_prefix then rebuilds s.prefix[0..npos] as the exclusive
// prefix of work(p) over positions p < npos (a plan may give an expert more
// than one position: the tail-only plan of the deterministic weight
// gradient has its whole tiles at p and its chunks at E + p).  `scr` is
// 4 KB of LDS that is free until the first stage load; `clen(e)` is expert
// e's chunk length.  Both must be called by all threads and end with a
// barrier; rank_experts after build_schedule.
static_assert(kMaxExperts <= 2 * kMaxGemmThreads && kMaxExperts <= 32767, "16-bit expert order in Sched::scan");
__device__ __forceinline__ int expert_at(const Sched& s, int p) {
    return reinterpret_cast<const int16_t*>(s.scan)[p];
}
template <class LenFn>
__device__ void rank_experts(Sched& s, lds_t* scr, int E, LenFn clen) {
    static_assert(kMaxExperts <= 4 * kGemmThreads, "at most four experts per thread");
    const int tid = threadIdx.x, nthr = blockDim.x;
    auto* key = reinterpret_cast<__attribute__((address_space(3))) int32_t*>(scr);
    if (E < kWaveExperts) {   // wave 0: lane e ranks expert e (keys exchanged through LDS)
        if (tid < 64) {
            const int32_t k0 = tid < E ? clen(tid) : 0;
            if (tid < E) key[tid] = k0;
            wave_lds_sync();
            int32_t r = 0;
            for (int f = 0; f < E; ++f) {
                const int32_t kf = key[f];
                r += kf > k0 || (kf == k0 && f < tid);
            }
            if (tid < E) reinterpret_cast<int16_t*>(s.scan)[r] = (int16_t)tid;
        }
        __syncthreads();
        return;
    }
    for (int e = tid; e < E; e += nthr) key[e] = clen(e);
    __syncthreads();
    // rank of expert e: experts with a longer chunk, or as long and a lower
    // index, go first; each thread ranks its (up to four) experts in one
    // pass over the keys
    int32_t k4[4], r4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = tid + u * nthr;
        k4[u] = e < E ? key[e] : 0;
        r4[u] = 0;
    }
    if (E <= nthr) {
        // one expert per thread; waves without an expert skip the pass
        if ((tid & ~63) < E)
            for (int f = 0; f < E; ++f) {
                const int32_t kf = key[f];
                r4[0] += kf > k4[0] || (kf == k4[0] && f < tid);
            }
    } else {
        for (int f = 0; f < E; ++f) {
            const int32_t kf = key[f];
#pragma unroll
            for (int u = 0; u < 4; ++u) r4[u] += kf > k4[u] || (kf == k4[u] && f < tid + u * nthr);
        }
    }
    __syncthreads();   // the keys are read; s.scan may be overwritten
    int16_t* perm = reinterpret_cast<int16_t*>(s.scan);
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (tid + u * nthr < E) perm[r4[u]] = (int16_t)(tid + u * nthr);
    __syncthreads();
}
template <class WorkFn>
__device__ void position_prefix(Sched& s, lds_t* scr, int npos, WorkFn work) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    if (npos <= 2 * kWaveExperts) {   // wave 0: lane l holds positions 2l and 2l+1
        if (tid < 64) {
            const int q0 = 2 * tid, q1 = q0 + 1;
            const int32_t w0 = q0 < npos ? work(q0) : 0, w1 = q1 < npos ? work(q1) : 0;
            const int32_t incl = wave_incl_sum(w0 + w1);
            if (q0 < npos) s.prefix[q0] = incl - w0 - w1;
            if (q1 < npos) s.prefix[q1] = incl - w1;
            if (tid == 63) s.prefix[npos] = incl;
        }
        __syncthreads();
        return;
    }
    // per-thread runs of positions, then a scan of the run sums
    const int per = (npos + nthr - 1) / nthr;
    const int lo = min(tid * per, npos), hi = min(lo + per, npos);
    int32_t run = 0;
    for (int q = lo; q < hi; ++q) run += work(q);
    int32_t total;
    int32_t acc = block_exclusive_scan(run, reinterpret_cast<__attribute__((address_space(3))) int32_t*>(scr), &total);
    for (int q = lo; q < hi; ++q) {
        s.prefix[q] = acc;
        acc += work(q);
    }
    if (tid == 0) s.prefix[npos] = total;
    __syncthreads();
}

// Work item of round r for the workgroup at (XCD-remapped) index wb of G:
// rounds alternate direction.
__device__ __forceinline__ int64_t snake_item(int64_t r, int64_t wb, int64_t G) {
    return r * G + ((r & 1) ? G - 1 - wb : wb);
}

// Values read from LDS arrive in vector registers even when every lane reads
// the same address; the tile decode is wave-uniform, so it is moved to scalar
// registers (keeps the per-tile state out of the VGPR budget).
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Largest e < n with prefix[e] <= w (so that prefix[e] <= w < prefix[e+1]
// when w < prefix[n]); n is the number of experts, or of positions of a
// plan's walk.
__device__ __forceinline__ int find_expert(const Sched& s, int n, int32_t w) {
    int lo = 0, hi = n;   // answer in [0, n)
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s.prefix[mid] <= w) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// The deterministic weight gradient's chunk rule (device side of
// wgrad_chunking in plan.hpp), in 32-bit unsigned arithmetic: T < 2^31, and a
// chunk_max of T or more gives one chunk, so it is clamped to T first.  (A
// 64-bit division is a long integer sequence on this GPU; the prologues
// evaluate these per expert and the walk per tile.)
__device__ __forceinline__ int32_t chunk_len_dev(int32_t T, int64_t chunk_max) {
    if (T <= 0) return 0;
    const uint32_t t = (uint32_t)T;
    const uint32_t cm = chunk_max < (int64_t)t ? (uint32_t)chunk_max : t;
    const uint32_t s = (t + cm - 1) / cm;
    const uint32_t l = (t + s - 1) / s;
    return (int32_t)(((l + kTileK - 1) / kTileK) * kTileK);
}
__device__ __forceinline__ int32_t chunks_dev(int32_t T, int64_t chunk_max) {
    const int32_t l = chunk_len_dev(T, chunk_max);
    return l ? (int32_t)(((uint32_t)T + (uint32_t)l - 1) / (uint32_t)l) : 0;
}

// Maximum / minimum of a 64-bit value over the lanes of a wave (butterfly
// shuffles).  An LDS atomic issued by every lane is expanded by the compiler
// into a loop over the active lanes, 64 dependent steps per wave; reducing
// first leaves one atomic per wave.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const uint64_t o = __shfl_xor((unsigned long long)v, m, 64);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const uint64_t o = __shfl_xor((unsigned long long)v, m, 64);
        v = o < v ? o : v;
    }
    return v;
}

// Estimated time of a planned walk on `workers` workgroups: the items
// 0 .. prefix[npos]-1 handed out in snake rounds, as the persistent kernels
// hand them out, each costing len(its position) plus kItemOverheadTokens
// tokens; returns the largest per-workgroup load.  The deterministic weight
// gradient chooses between its two plans with it on kRuleCUs reference
// workgroups (a function of the plan only, never of the device); the split
// program on its live grid.  `red` is an LDS word; `tab` is LDS scratch for
// npos words (the lengths, read once per position).  A workgroup's items
// have increasing indices, so their positions are found by advancing one
// pointer.  Must be called by all threads; ends with a barrier.
template <class LenFn>
__device__ uint64_t walk_makespan(const Sched& s, int npos, LenFn len, unsigned long long* red,
                                  __attribute__((address_space(3))) uint32_t* tab, int64_t workers = kRuleCUs) {
    if (threadIdx.x == 0) *red = 0;
    for (int q = threadIdx.x; q < npos; q += blockDim.x) tab[q] = (uint32_t)len(q);
    __syncthreads();
    const int64_t total = s.prefix[npos];
    uint64_t worst = 0;
    for (int64_t b = threadIdx.x; b < workers; b += blockDim.x) {
        uint64_t load = 0;
        int q = 0;
        for (int64_t r = 0;; ++r) {
            const int64_t i = snake_item(r, b, workers);
            if (i >= total) break;   // later rounds hold only larger indices
            while (s.prefix[q + 1] <= i) ++q;   // stops below npos: i < prefix[npos]
            load += (uint64_t)tab[q] + (uint64_t)kItemOverheadTokens;
        }
        worst = load > worst ? load : worst;
    }
    worst = wave_max_u64(worst);
    if ((threadIdx.x & 63) == 0) atomicMax(red, (unsigned long long)worst);
    __syncthreads();
    const uint64_t m = *red;
    __syncthreads();
    return m;
}

// Workgroup b of G -> logical work index.  Workgroups are dispatched to the
// 8 XCDs round-robin (b % 8); this gives each XCD a contiguous run of work
// items so that tiles sharing operand panels share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t G) {
    const int64_t x = b & 7, i = b >> 3;
    const int64_t q = G >> 3, r = G & 7;
    return x * q + (x < r ? x : r) + i;
}

// ---------------------------------------------------------------------------
// operand tiles

// A view of one operand of a tile: element (i, kk) with i in [0, nvalid) the
// output index inside the tile and kk the reduction index from the start of
// the reduction range [0, klen).
//   K-major:  base[i * ld + kk]   (reduction index contiguous)
//   MN-major: base[kk * ld + i]   (output index contiguous; nvalid % 8 == 0)
// Everything outside reads as zero.
struct Operand {
    const uint16_t* base;
    int64_t ld;
    int32_t nvalid;
    int32_t klen;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// Buffer descriptor over [base, base + 2 GB): raw (stride 0) addressing with
// range checking.  A lane whose offset is kOOB lies past the range, and its
// load writes zeros to LDS; this is how every mask below is applied.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFF0, 0x00020000);
}
constexpr uint32_t kOOB = 0xFFFFFFF0u;
// Cache-policy operand of a buffer store: the non-temporal (nt) hint, for
// output that this kernel never reads back, so that it is evicted before the
// operand panels that the workgroups of an XCD share through L2.
constexpr int kCpolNT = 2;

// ---------------------------------------------------------------------------
// main-loop pipeline
//
// The reduction runs in stages of kStageK = 32 values.  Each operand has
// kStages = 4 LDS buffers; stage s lives in buffer s % 4.  A step computes
// one stage in two MFMA sub-steps of 16 and is cut in half by the one
// workgroup barrier of the step:
//
//   sub-step 0   MFMAs of sub-step 0 (fragments already in registers),
//                LDS reads of the sub-step 1 fragments
//   barrier      after this wave's loads of stage s+1 have landed and its
//                LDS reads of stage s have returned
//   sub-step 1   MFMAs of sub-step 1, LDS reads of the next stage's sub-step
//                0 fragments, and the global loads of stage s+4 into the
//                buffer stage s has just freed
//
// so a load has three steps between its issue and its first use, and the
// MFMA pipe is fed from registers while the barrier and the next stage's
// first reads resolve.  Global loads go straight from HBM to LDS (16-byte
// buffer loads with an LDS destination), and the MFMAs, LDS reads and
// global loads of a sub-step are interleaved one by one.
//
// The stage stream runs through consecutive tiles of a workgroup without a
// break: the loads of the last three steps of a tile fetch the first stages
// of the next tile.  Every tile runs a multiple of four steps (padding steps
// compute nothing) so that each tile starts in buffer 0 and every buffer
// index is a compile-time constant; the eight buffers are distinct
// __shared__ arrays, so the compiler sees that a read of one buffer does not
// alias the loads in flight into another and never waits for those.

constexpr int kSubSteps = kStageK / kMfmaK;   // 2
static_assert(kSubSteps == 2, "the step schedule assumes two MFMA sub-steps per stage");

// s_waitcnt with vmcnt(N) and lgkmcnt(0) (expcnt left free).  GFX9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without a memory fence: the waits above are the only
// synchronisation the pipeline needs, and a fence would drain every load in
// flight.  The "memory" clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Scheduling groups (masks of __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

// Interleave NM MFMAs with NR LDS reads and NL global loads of the same
// region: the reads spread over the first half of the MFMAs (they feed the
// next sub-step), the loads over all of them.  Used when both operands are
// K-major; with transposed (MN-major) reads the compiler's own order is
// faster, as measured.
template <int NM, int NR, int NL, int T>
__device__ __forceinline__ void sched_slot() {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    constexpr int H = NM / 2;   // the reads go out during the first half
    constexpr int r = T < H ? NR * (T + 1) / H - NR * T / H : 0;
    constexpr int l = NL * (T + 1) / NM - NL * T / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, r, 0);
    if constexpr (l > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, l, 0);
}
template <int NM, int NR, int NL, int... T>
__device__ __forceinline__ void sched_interleave_impl(std::integer_sequence<int, T...>) {
    (sched_slot<NM, NR, NL, T>(), ...);
}
template <int NM, int NR, int NL>
__device__ __forceinline__ void sched_interleave() {
    sched_interleave_impl<NM, NR, NL>(std::make_integer_sequence<int, NM>{});
}

// LDS layouts:
//   K-major operands (reduction index contiguous in memory) are staged in
//   pairs of stages: a pair buffer holds ROWS rows of 64 reduction values
//   (128 B = 8 chunks of 16 B), stage 2p in the first four chunks of each
//   row and stage 2p+1 in the last four.  Loading a pair moves whole 128-byte
//   lines (a 32-value stage alone would be half a line per row, twice the
//   memory requests and address translations per byte).  Chunk c of row r
//   sits at c ^ swzK(r), which puts the 16 rows an MFMA operand read covers
//   per pass (one chunk each) on 16 distinct 16-byte bank groups, and any 8
//   consecutive rows on 8.
//   MN-major operands: one buffer per stage, 32 rows (reduction index) of
//   ROWS output indices (ROWS*2 B = CPR chunks), already whole lines in
//   memory; chunk c of row r sits at c ^ swzMN(r).  A transposed read has
//   each group of 32 lanes read 4 rows at the same 4 chunks (c0 .. c0+3, c0
//   a multiple of 4), each group of 16 lanes 2 of those chunks.  The XOR
//   values 0, 10, 12, 6 for r % 4 = 0..3 send the 4 rows to 4 different
//   64-byte bank groups of a 256-byte window (bits 2-3 of the chunk index
//   all differ) and, for the 16-lane halves, to 4 different 32-byte groups of
//   a 128-byte window (bits 1-2 all differ): no bank conflicts with either
//   32 or 64 banks.
__device__ __forceinline__ int swzK(int row) { return (row & 7) ^ ((row >> 3) & 1); }
template <int CPR>
__device__ __forceinline__ int swzMN(int row) {
    return ((0x6CA0 >> (4 * (row & 3))) & 15) & (CPR - 1);
}

// Loads stages of an operand from HBM into LDS with 16-byte buffer loads (no
// registers in between): a K-major operand two stages (one pair buffer) at a
// time, an MN-major operand one stage at a time.  Either way one load is
// ROWS*64*SPAN bytes = ROWS*SPAN/16 wave instructions of 1 KB, of which each
// of the 4 waves issues a quarter.  Lane l of instruction g writes LDS bytes
// [g*1024 + 16*l, +16); the swizzle is applied by choosing which global
// chunk the lane fetches.
template <int ROWS, bool KMAJ, int WAVES>
struct StageLoader {
    static constexpr int kSpan = KMAJ ? 2 : 1;   // stages per load
    static constexpr int kPerWave = ROWS * kStageK * 2 * kSpan / 1024 / WAVES;
    static_assert(kPerWave >= 1, "every wave issues at least one load per stage");
    static constexpr int kRowBytes = KMAJ ? 2 * kStageK * 2 : ROWS * 2;
    static constexpr int kCPR = kRowBytes / 16;
    static_assert(ROWS % 64 == 0, "tile rows must be a multiple of 64");
    uint32_t off[kPerWave];   // byte offset of this lane's 16 bytes from the load base (kOOB if masked)
    int32_t kp[kPerWave];     // reduction position of those 16 bytes from the first stage loaded
    int64_t step_bytes;       // byte distance between consecutive stages
    const char* base;
    int32_t klen;

    __device__ __forceinline__ void init(const Operand& op) {
        // opaque lane index: keeps the lane-dependent offset arithmetic here
        // instead of hoisted (and held in registers) across the tile loop
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        base = reinterpret_cast<const char*>(op.base);
        klen = op.klen;
        step_bytes = KMAJ ? kStageK * 2 : (int64_t)kStageK * op.ld * 2;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int b = (wave * kPerWave + i) * 1024 + lane * 16;
            const int row = b / kRowBytes, phys = (b % kRowBytes) / 16;
            if constexpr (KMAJ) {
                const int logical = phys ^ swzK(row);
                off[i] = row < op.nvalid ? (uint32_t)(row * op.ld * 2 + logical * 16) : kOOB;
                kp[i] = logical * 8;
            } else {
                const int col = (phys ^ swzMN<kCPR>(row)) * 8;
                off[i] = col < op.nvalid ? (uint32_t)(row * op.ld * 2 + col * 2) : kOOB;
                kp[i] = row;
            }
        }
    }

    // Issue the load of stage L (stages L, L+1 for a K-major operand) into
    // `buf`; reduction positions at or past klen read as zero, and so does
    // everything when !valid (or when L lies past the last stage): such a
    // load accesses no memory.
    __device__ __forceinline__ void issue(lds_t* buf, int L, bool valid) const {
        issue_part<0, kPerWave>(buf, L, valid);
    }
    // instructions J0 .. J1-1 of that load (a load may be spread over steps)
    template <int J0, int J1>
    __device__ __forceinline__ void issue_part(lds_t* buf, int L, bool valid) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base + L * step_bytes);
        const int rem = valid ? klen - L * kStageK : 0;
#pragma unroll
        for (int i = J0; i < J1; ++i) {
            const uint32_t o = kp[i] < rem ? off[i] : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void_t*)(buf + (wave * kPerWave + i) * 1024), 16, o, 0, 0, 0);
        }
    }
};

// MFMA operand fragment: lane l gets the 8 reduction values 16*s + 8*(l/32)
// .. +7 of tile row rb + (l & 31) from the stage in `buf` (for a K-major pair
// buffer, the stage in half h).
template <int ROWS, bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const lds_t* buf, int h, int rb, int s, int l) {
    if constexpr (KMAJ) {
        const int row = rb + (l & 31), c = 4 * h + 2 * s + (l >> 5);
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            buf + row * (4 * kStageK) + ((c ^ swzK(row)) << 4));
    } else {
        // ds_read_b64_tr_b16: in a group of 16 lanes, lane 4j+q addresses
        // 4 values of row kbase+j at column col0+4q; lane i receives column
        // col0+i of rows kbase..kbase+3.
        constexpr int CPR = ROWS * 2 / 16;
        const int g = l >> 4, j = (l >> 2) & 3, q = l & 3;
        const int col = rb + 16 * (g & 1) + 4 * q;
        const int chunk = col >> 3, within = (col & 7) * 2;
        const int r0 = 16 * s + 8 * (g >> 1) + j, r1 = r0 + 4;
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(buf + r0 * ROWS * 2 + ((chunk ^ swzMN<CPR>(r0)) << 4) + within));
        v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(buf + r1 * ROWS * 2 + ((chunk ^ swzMN<CPR>(r1)) << 4) + within));
        v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
}

// One tile of work for the persistent driver: the two operand views and the
// kernel's own output coordinates.
struct TileInfo {
    Operand A, B;
    int64_t o0, o1;      // output row / column base (kernel specific)
    int32_t rows, cols;  // valid output rows / columns of the tile
    int32_t e, aux, aux2;  // expert and kernel-specific tags
};

// The LDS buffers of a kernel, indexed by stage % 4: for a K-major operand
// entries 2p and 2p+1 name the same pair buffer p, for an MN-major operand
// each entry is its own buffer.  Every buffer is a distinct __shared__ array
// (see above).
struct Stages {
    lds_t* a[kStages];
    lds_t* b[kStages];
};

#define DRGG_STAGE_BUFS(ROWS, KMAJ, name)                                                        \
    __shared__ __attribute__((aligned(256))) char name##0[(KMAJ ? 2 : 1) * (ROWS) * kStageK * 2]; \
    __shared__ __attribute__((aligned(256))) char name##1[(KMAJ ? 2 : 1) * (ROWS) * kStageK * 2]; \
    __shared__ __attribute__((aligned(256))) char name##2[(KMAJ ? 0 : 1) * (ROWS) * kStageK * 2 + 16]; \
    __shared__ __attribute__((aligned(256))) char name##3[(KMAJ ? 0 : 1) * (ROWS) * kStageK * 2 + 16]

#define DRGG_STAGE_PTRS(KMAJ, name)                                                              \
    KMAJ ? (lds_t*)name##0 : (lds_t*)name##0, KMAJ ? (lds_t*)name##0 : (lds_t*)name##1,          \
    KMAJ ? (lds_t*)name##1 : (lds_t*)name##2, KMAJ ? (lds_t*)name##1 : (lds_t*)name##3

#define DRGG_STAGES(BM, BN, AK, BK, name)                                                        \
    DRGG_STAGE_BUFS(BM, AK, name##_a);                                                           \
    DRGG_STAGE_BUFS(BN, BK, name##_b);                                                           \
    const Stages name{{DRGG_STAGE_PTRS(AK, name##_a)}, {DRGG_STAGE_PTRS(BK, name##_b)}}

// The accumulators and operand fragments of one BMxBN tile on 4 waves (one
// per SIMD, a 2x2 wave grid) or 8 waves (two per SIMD, a 4x2 grid for
// 256-row tiles): each wave owns a block of 32x32 MFMA tiles whose FP32
// accumulators stay in registers.  The MFMA takes the B-side fragment as its first operand,
// so that the accumulator of lane l holds tile row l%32 and, in registers
// 4q..4q+3, four consecutive tile columns 8q + 4*(l/32) .. +3: a lane's
// outputs leave as 8- or 16-byte stores.
template <int BM, int BN, bool AK, bool BK, int WAVES = kGemmWaves>
struct TileMma {
    // wave grid: kWGM waves along the tile rows, kWGN along its columns
    static constexpr int kWGM = (WAVES == 8 && BM >= 256) ? 4 : 2;
    static constexpr int kWGN = WAVES / kWGM;
    static constexpr int WM = BM / kWGM, WN = BN / kWGN;
    __device__ static __forceinline__ int wave_row(int wave) { return (wave / kWGN) * WM; }
    __device__ static __forceinline__ int wave_col(int wave) { return (wave % kWGN) * WN; }
    static constexpr int kBI = WM / 32, kBJ = WN / 32;
    static_assert(kBI >= 1 && kBJ >= 1, "tile too small for the 2x2 wave grid");
    // LDS reads per sub-step: one per 32-row block (K-major), two (MN-major)
    static constexpr int kReads = kBI * (AK ? 1 : 2) + kBJ * (BK ? 1 : 2);
    static constexpr int kMfmas = kBI * kBJ;
    f32x16 acc[kBI][kBJ];
    bf16x8 fa[2][kBI], fb[2][kBJ];   // fragments of sub-step 0 and 1

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    // fragments of sub-step s of stage ST (its buffers in st) into set F
    template <int F, int ST>
    __device__ __forceinline__ void read(const Stages& st, int s) {
        const int l = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int ra = wave_row(wave), rb = wave_col(wave);
        // in the order the MFMAs consume them
        fa[F][0] = read_frag<BM, AK>(st.a[ST], ST & 1, ra, s, l);
#pragma unroll
        for (int j = 0; j < kBJ; ++j) fb[F][j] = read_frag<BN, BK>(st.b[ST], ST & 1, rb + 32 * j, s, l);
#pragma unroll
        for (int i = 1; i < kBI; ++i) fa[F][i] = read_frag<BM, AK>(st.a[ST], ST & 1, ra + 32 * i, s, l);
    }

    // FIRST: the tile's first products, accumulated onto zero (this is what
    // clears the accumulators between tiles)
    template <int F, bool FIRST = false>
    __device__ __forceinline__ void mfma() {
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[F][j], fa[F][i], FIRST ? f32x16{} : acc[i][j],
                                                                    0, 0, 0);
    }
};

// Write a finished tile: out[row * ld + col] = tile[row][col] rounded once to
// the output type, for row < rows and col < cols (cols a multiple of 4).
// Each lane stores its four consecutive columns as one 8- or 16-byte buffer
// store; lanes outside the valid region get an out-of-range offset, and
// their stores are dropped by the hardware range check, so the epilogue has
// no branches.  Each 32-row block gets its own descriptor, which keeps the
// per-lane offsets below 2^31 for ld <= 2^22.
template <bool OUT_BF16, class Mma>
__device__ __forceinline__ void store_tile(const Mma& mma, void* out, int64_t ld, int rows, int cols) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int ES = OUT_BF16 ? 2 : 4;
    // opaque lane index: the offsets do not depend on the tile and would
    // otherwise be hoisted out of the tile loop and held in registers
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ra = Mma::wave_row(wave), rb = Mma::wave_col(wave);
    const int r = lane & 31;
#pragma unroll
    for (int i = 0; i < Mma::kBI; ++i) {
        const int r0 = ra + 32 * i;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<char*>(out) + (int64_t)r0 * ld * ES);
        const bool rok = r0 + r < rows;
#pragma unroll
        for (int j = 0; j < Mma::kBJ; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = rb + 32 * j + 8 * q + 4 * (lane >> 5);
                const uint32_t o = rok && c < cols ? (uint32_t)((r * ld + c) * ES) : kOOB;
                const f32x16& a = mma.acc[i][j];
                if constexpr (OUT_BF16) {
                    const bf16x2 lo = __builtin_convertvector((f32x2{a[4 * q], a[4 * q + 1]}), bf16x2);
                    const bf16x2 hi = __builtin_convertvector((f32x2{a[4 * q + 2], a[4 * q + 3]}), bf16x2);
                    const u32x2 d = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                    __builtin_amdgcn_raw_buffer_store_b64(d, rs, o, 0, 0);
                } else {
                    const u32x4 d = {__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]),
                                     __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3])};
                    __builtin_amdgcn_raw_buffer_store_b128(d, rs, o, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Write a finished tile like store_tile, but so that every global store
// instruction writes whole 128-byte lines (R = ep_rows of the tile, from
// plan.hpp, which sizes the LDS for it), with the non-temporal hint.  In the
// accumulator layout a lane owns one row of each 32x32 block, so a direct
// store touches 32 rows (32 lines, 16 or 32 bytes each) per instruction;
// written back-to-back by every workgroup at a tile boundary, those partial
// lines cost more than the rest of the epilogue.  Here each wave moves its
// blocks through its own R x 128-byte LDS scratch `scr`: a 128-byte row
// segment (64 BF16 or 32 FP32 columns, i.e. two or one 32-column blocks) of R
// rows at a time, written by the lanes that own those rows and read back as
// 16-byte chunks, eight lanes per row, then stored with 16-byte buffer stores
// (R/8 rows of whole lines per instruction).  Chunk c of scratch row rr sits
// at 16 * (c ^ (rr & 7)), so the read-back is free of bank conflicts.  Masking
// as in store_tile; cols must be a multiple of 8 (BF16) or 4 (FP32).  The
// scratch is private to the wave, so a wave-level sync between the phases is
// all it needs.  CPOL is the stores' cache policy: non-temporal for outputs;
// 0 for data read back soon (the weight gradient's chunk partials, which the
// fold then finds in the last-level cache).
template <bool OUT_BF16, int R, int CPOL = kCpolNT, class Mma>
__device__ __forceinline__ void store_tile_lines(const Mma& mma, lds_t* scr, void* out, int64_t ld, int rows,
                                                 int cols) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int ES = OUT_BF16 ? 2 : 4;
    constexpr int SEG = 128 / ES;   // columns per 128-byte segment
    constexpr int BPS = SEG / 32;   // 32-column blocks per segment
    constexpr int CPL = R / 8;      // read-back chunks per lane and round
    static_assert(R == 8 || R == 16, "rounds of 8 or 16 rows");
    static_assert(Mma::kBJ % BPS == 0, "whole segments per wave");
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ra = Mma::wave_row(wave), rb = Mma::wave_col(wave);
    lds_t* sw = scr + wave * (R * 128);
    const int r = lane & 31, h = lane >> 5;
    const int rr = r % R;   // this lane's scratch row in the round that owns it
    const int sx = rr & 7;
#pragma unroll
    for (int i = 0; i < Mma::kBI; ++i) {
        const int r0 = ra + 32 * i;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<char*>(out) + (int64_t)r0 * ld * ES);
#pragma unroll
        for (int g = 0; g < Mma::kBJ / BPS; ++g) {
            const int c0 = rb + g * SEG;
#pragma unroll
            for (int s = 0; s < 32 / R; ++s) {
                if (r / R == s) {
#pragma unroll
                    for (int b = 0; b < BPS; ++b) {
                        const f32x16& a = mma.acc[i][g * BPS + b];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if constexpr (OUT_BF16) {
                                // columns 32b + 8q + 4h .. +3: chunk 4b + q, its half h
                                const bf16x2 lo = __builtin_convertvector((f32x2{a[4 * q], a[4 * q + 1]}), bf16x2);
                                const bf16x2 hi = __builtin_convertvector((f32x2{a[4 * q + 2], a[4 * q + 3]}), bf16x2);
                                *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                                    sw + rr * 128 + (((4 * b + q) ^ sx) << 4) + 8 * h) =
                                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                            } else {
                                // columns 8q + 4h .. +3: chunk 2q + h
                                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                                    sw + rr * 128 + (((2 * q + h) ^ sx) << 4)) =
                                    u32x4{__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]),
                                          __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3])};
                            }
                        }
                    }
                }
                wave_lds_sync();   // the round's rows are in the scratch
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const int idx = lane + 64 * k, row = idx >> 3, c = idx & 7;
                    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                        sw + row * 128 + ((c ^ (row & 7)) << 4));
                    const int rowb = s * R + row;            // row within the 32-row block
                    const int col = c0 + c * (16 / ES);
                    const uint32_t o = r0 + rowb < rows && col < cols ? (uint32_t)((rowb * ld + col) * ES) : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(v, rs, o, 0, CPOL);
                }
                wave_lds_sync();   // read back before the next round overwrites it
            }
        }
    }
}

// A split tile's FP32 sum lives in the workspace in the accumulators' own
// order: element (wave w, block (i, j), register r, lane l) at
// ((((w * kBI + i) * kBJ + j) * 16 + r) * 64 + l), so each atomic or load
// instruction covers 64 consecutive floats (two cache lines).  Positions
// outside the tile's valid rows and columns hold zeros (their operands were
// zero-filled) and need no masking.
template <class Mma>
__device__ __forceinline__ uint32_t tile_sum_offset(int wave, int i, int j, int r, int lane) {
    return (uint32_t)(((((wave * Mma::kBI + i) * Mma::kBJ + j) * 16 + r) * 64 + lane) * 4);
}

// Add a finished tile into its FP32 tile sum with device-coherent atomic
// adds (performed in L2).
template <class Mma>
__device__ __forceinline__ void atomic_add_tile(const Mma& mma, float* ts) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(ts);
#pragma unroll
    for (int i = 0; i < Mma::kBI; ++i)
#pragma unroll
        for (int j = 0; j < Mma::kBJ; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(mma.acc[i][j][r], rs,
                                                                 tile_sum_offset<Mma>(wave, i, j, r, lane), 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
}

// The last piece of a split tile: out[row * ld + col] = the tile sum (+ this
// piece's own partial when ADD_OWN), rounded once, for row < rows and
// col < cols; the tile sum is cleared back to zero for the next call.  The
// caller has made the other pieces' atomic adds visible.
template <bool OUT_BF16, bool ADD_OWN, class Mma>
__device__ __forceinline__ void drain_tile_sum(const Mma& mma, float* ts, void* out, int64_t ld, int rows,
                                               int cols) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int ES = OUT_BF16 ? 2 : 4;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ra = Mma::wave_row(wave), rb = Mma::wave_col(wave);
    const int r = lane & 31;
    const __amdgpu_buffer_rsrc_t rsum = make_rsrc(ts);
#pragma unroll
    for (int i = 0; i < Mma::kBI; ++i) {
        const int r0 = ra + 32 * i;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<char*>(out) + (int64_t)r0 * ld * ES);
        const bool rok = r0 + r < rows;
#pragma unroll
        for (int j = 0; j < Mma::kBJ; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = rb + 32 * j + 8 * q + 4 * (lane >> 5);
                const uint32_t o = rok && c < cols ? (uint32_t)((r * ld + c) * ES) : kOOB;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rsum, tile_sum_offset<Mma>(wave, i, j, 4 * q + e, lane), 0, 0));
                    if constexpr (ADD_OWN) {
                        float own = mma.acc[i][j][4 * q + e];
                        // With a BF16 output the compiler otherwise copies
                        // every accumulator out of the AGPRs up front, which
                        // needs more VGPRs than there are: read each one here.
                        if constexpr (OUT_BF16)
                            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(own) : "a"(mma.acc[i][j][4 * q + e]));
                        v[e] += own;
                    }
                }
                if constexpr (OUT_BF16) {
                    const bf16x2 lo = __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2);
                    const bf16x2 hi = __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2);
                    const u32x2 d = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                    __builtin_amdgcn_raw_buffer_store_b64(d, rs, o, 0, 0);
                } else {
                    const u32x4 d = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                     __float_as_uint(v[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(d, rs, o, 0, 0);
                }
                // issued after the store above, whose data needed the loads:
                // the clear cannot overtake the read
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(0u, rsum, tile_sum_offset<Mma>(wave, i, j, 4 * q + e, lane),
                                                          0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Issue schedule of the stage loads of a 4-wave runner (steps t of the
// global step sequence; the prologue acts as steps -4 .. -1).  A K-major operand loads stages t+3
// and t+4 at odd steps (into the pair buffer whose two stages t-1 and t were
// read by then), an MN-major operand stage t+4 at every step; within a step
// A goes before B.  The pipeline waits, at the barrier of step s, until
// stage s+1 of both operands has landed: with buffer loads returning in
// issue order, that is "at most N pending", N the number of loads issued
// after the last one of stage s+1.
template <bool AK, bool BK, int CA, int CB>
struct IssuePlan {
    static constexpr int loads_at(int t, int op) {
        const bool k = op == 0 ? AK : BK;
        const int c = op == 0 ? CA : CB;
        return k ? ((t & 1) ? c : 0) : c;
    }
    static constexpr int issue_step(bool k, int X) { return k ? ((X & 1) ? X - 4 : X - 3) : X - 4; }
    // loads issued after those of stage X, up to and including step `upto`
    static constexpr int after(int X, int upto) {
        const int ta = issue_step(AK, X), tb = issue_step(BK, X);
        const int last = 2 * ta > 2 * tb + 1 ? 2 * ta : 2 * tb + 1;
        int n = 0;
        for (int t = (ta < tb ? ta : tb); t <= upto; ++t)
            for (int op = 0; op < 2; ++op)
                if (2 * t + op > last) n += loads_at(t, op);
        return n;
    }
    static constexpr int at_barrier(int s) { return after(s + 1, s - 1); }   // wait at step s
    static constexpr int prologue = after(0, -1);                              // wait for stage 0
};

// Persistent tile loop over the stage pipeline.  `more()` tells whether this
// workgroup has another tile and `next(t)` decodes it; `finish(t, mma)`
// writes a finished tile from the accumulators.  Every step has the same
// shape (up to the parity that decides whether a K-major pair is loaded):
// it runs both MFMA sub-steps and issues its loads.  Stages past the end of a
// tile (the padding up to a multiple of four, or past the last tile) are
// "loaded" with every lane masked, which writes zeros to LDS without
// touching memory, so the MFMAs of a padding step add zeros and no branch is
// taken around the accumulators.  The next tile is decoded at the start of
// step nk4-4, whose loads fetch its first stage.  Must be called by all
// threads.
template <int BM, int BN, bool AK, bool BK, int WAVES = kGemmWaves>
struct TileRunner {
    using Mma = TileMma<BM, BN, AK, BK, WAVES>;
    using LA = StageLoader<BM, AK, WAVES>;
    using LB = StageLoader<BN, BK, WAVES>;
    using Plan = IssuePlan<AK, BK, LA::kPerWave, LB::kPerWave>;
    Mma mma;
    LA la;
    LB lb;
    Stages st;
    TileInfo cur, nxt;
    int nk, nk4, nk_nxt;
    bool has_next;

    // The first step group of a tile accumulates onto zero instead of
    // clearing the accumulators first.  Only with 8 waves, whose accumulators
    // live in VGPRs: with 4 waves they sit in AGPRs, and the extra copy of
    // the group makes the compiler move them out and spill.
    static constexpr bool kPeel = WAVES == 8;

    static __device__ __forceinline__ int stages_of(const TileInfo& t) {
        return (t.A.klen + kStageK - 1) / kStageK;
    }
    // steps run for a tile of n stages: whole groups of kStages (the stages
    // past n load zeros), at least the peeled group.  The next tile is
    // decoded inside a group's steps, so every tile must have at least one
    // reduction value: a tile of none would never hand over to the next one
    // (the callers' walks hold no item of zero length).  Forcing a group
    // here instead makes the compiler spill the 4-wave kernels' accumulators.
    static __device__ __forceinline__ int round4(int n) {
        const int r = (n + kStages - 1) & ~(kStages - 1);
        return kPeel && r < kStages ? kStages : r;
    }

    // With 8 waves the workgroup barrier is passed at odd steps only: the
    // two waves of a SIMD stop issuing MFMAs at a barrier, and with two of
    // them per SIMD that stall is the larger cost.  The loads then belong to
    // the odd steps: step t loads stages t+3 and t+4 into the buffers of
    // stages t-1 and t, which every wave has finished reading at its
    // barrier, and that barrier waits for all loads in flight: those of
    // stages t+1 and t+2, which steps t and t+1 read.
    static constexpr bool kBar2 = WAVES == 8;

    // With kBar2 the loads of an odd step t (stages t+3 and t+4: kNLT wave
    // instructions per wave, A's before B's) may be spread over three
    // sub-steps: instructions [0, kS1) go out in sub-step 1 of step t,
    // [kS1, kS2) in sub-step 0 of step t+1 and [kS2, kNLT) in its sub-step 1,
    // interleaved with their MFMAs.  All of them still land before the
    // barrier of step t+2, which waits for every load in flight.  The last
    // odd step of a tile fetches the next tile's stages 2 and 3, and that
    // tile's first step issues the rest; the prologue issues the first
    // tile's stages 0 and 1 and part of 2 and 3 in the same way.  As
    // measured, spreading pays with a transposed (MN-major) B operand, read
    // back with two LDS instructions per fragment: 3/3/2 of the 8 gained 4 %
    // on the data gradient without W^T and 1 % on the weight gradient (8 of
    // 8 at the odd step and the other splits tried were slower); with both
    // operands K-major it gained nothing or lost, so they issue everything
    // at the odd step.
    static constexpr int kNLT = (AK ? 1 : 2) * LA::kPerWave + (BK ? 1 : 2) * LB::kPerWave;
    static constexpr int kS1 = kBar2 && !BK && kNLT == 8 ? 3 : kNLT;
    static constexpr int kS2 = kBar2 && !BK && kNLT == 8 ? 6 : kNLT;
    // the step that switches the loaders to the next tile: the first one
    // whose loads fetch from it
    static constexpr int kReinitST = kBar2 ? 1 : 0;

    // Instructions [I0, I1) of the loads of odd step kt_odd (STO = kt_odd % 4).
    template <int STO, int I0, int I1, int Q>
    __device__ __forceinline__ void issue_odd_entry(int kt_odd) {
        // entry Q: a load of A for Q < nA, else of B; a K-major operand has
        // one (the pair t+3, t+4), an MN-major one two (t+3, then t+4)
        constexpr int nA = AK ? 1 : 2;
        constexpr bool isA = Q < nA;
        constexpr int P = isA ? LA::kPerWave : LB::kPerWave;
        constexpr int start = isA ? Q * LA::kPerWave : nA * LA::kPerWave + (Q - nA) * LB::kPerWave;
        constexpr int j0 = I0 - start < 0 ? 0 : I0 - start > P ? P : I0 - start;
        constexpr int j1 = I1 - start < 0 ? 0 : I1 - start > P ? P : I1 - start;
        if constexpr (j0 < j1) {
            constexpr int d = 3 + (isA ? Q : Q - nA);
            const int L = kt_odd + d;
            const int Ls = L < nk4 ? L : L - nk4;
            if constexpr (isA) la.template issue_part<j0, j1>(st.a[(STO + d) % kStages], Ls, L < nk4 || has_next);
            else lb.template issue_part<j0, j1>(st.b[(STO + d) % kStages], Ls, L < nk4 || has_next);
        }
    }
    template <int STO, int I0, int I1, int... Q>
    __device__ __forceinline__ void issue_odd_entries(int kt_odd, std::integer_sequence<int, Q...>) {
        (issue_odd_entry<STO, I0, I1, Q>(kt_odd), ...);
    }
    template <int STO, int I0, int I1>
    __device__ __forceinline__ void issue_odd(int kt_odd) {
        if constexpr (I0 < I1)
            issue_odd_entries<STO, I0, I1>(kt_odd, std::make_integer_sequence<int, (AK ? 1 : 2) + (BK ? 1 : 2)>{});
    }

    // Without kBar2, the loads of step t (t % 4 == ST) for operand loader
    // `ld`: stage t+4, or for a K-major operand at odd t the pair t+3, t+4,
    // of this tile or, past nk4, of the next one (the loaders then point at
    // the next tile).
    template <int ST, bool K, class Ld>
    __device__ __forceinline__ void issue(Ld& ld, lds_t* const* bufs, int kt) {
        static_assert(!kBar2, "with kBar2 the loads go through issue_odd");
        if constexpr (!K || (ST & 1)) {
            const int L = kt + (K ? 3 : 4);
            const int Ls = L < nk4 ? L : L - nk4;
            ld.issue(bufs[(ST + (K ? 3 : 4)) % kStages], Ls, L < nk4 || has_next);
        }
    }

    // Sub-step 1 of odd step kt with kBar2: its MFMAs, the loads [0, N) of
    // the step, the sub-step 0 fragments of stage kt+1.
    template <int ST, int N>
    __device__ __forceinline__ void odd_substep1(int kt) {
        issue_odd<ST, 0, N>(kt);
        mma.template read<0, (ST + 1) % kStages>(st, 0);
        mma.template mfma<1>();
        if constexpr (AK && BK) sched_interleave<Mma::kMfmas, Mma::kReads, N>();
    }

    // Step kt of the current tile; ST = kt % 4; FIRST for step 0.
    template <int ST, bool FIRST = false, class Next>
    __device__ __forceinline__ void step(int kt, Next& next) {
        constexpr int NX = (ST + 1) % kStages;
        constexpr int STO = (ST + kStages - 1) % kStages;
        // with kBar2 an even step issues the deferred loads of step kt-1 (for
        // a tile's first step, those of the previous tile's last step or of
        // the prologue: its stages 2 and 3)
        constexpr bool DEF = kBar2 && !(ST & 1);
        // loads issued in this step without kBar2 (the schedule hints place them)
        constexpr int NL = (AK && !(ST & 1) ? 0 : LA::kPerWave) + (BK && !(ST & 1) ? 0 : LB::kPerWave);
        if constexpr (ST == kReinitST) {
            if (kt - ST + kStages == nk4 && has_next) {
                next(nxt);
                nk_nxt = stages_of(nxt);
                la.init(nxt.A);
                lb.init(nxt.B);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 0: its MFMAs; the sub-step 1 fragments
        mma.template read<1, ST>(st, 1);
        if constexpr (DEF) issue_odd<STO, kS1, kS2>(kt - 1);
        mma.template mfma<0, FIRST>();
        if constexpr (AK && BK) sched_interleave<Mma::kMfmas, Mma::kReads, DEF ? kS2 - kS1 : 0>();
        __builtin_amdgcn_sched_barrier(0);
        // stage kt+1 has landed for every wave, and every wave is done
        // reading stage kt
        if constexpr (!kBar2 || (ST & 1)) {
            wait_vm_lgkm<kBar2 ? 0 : Plan::at_barrier(4 + ST)>();
            barrier_nofence();
        }
        // sub-step 1: its MFMAs; the loads into the buffers just freed; the
        // sub-step 0 fragments of stage kt+1
        if constexpr (kBar2 && (ST & 1)) {
            odd_substep1<ST, kS1>(kt);
        } else if constexpr (kBar2) {
            if constexpr (DEF) issue_odd<STO, kS2, kNLT>(kt - 1);
            mma.template read<0, NX>(st, 0);
            mma.template mfma<1>();
            if constexpr (AK && BK) sched_interleave<Mma::kMfmas, Mma::kReads, DEF ? kNLT - kS2 : 0>();
        } else {
            issue<ST, AK>(la, st.a, kt);
            issue<ST, BK>(lb, st.b, kt);
            mma.template read<0, NX>(st, 0);
            mma.template mfma<1>();
            if constexpr (AK && BK) sched_interleave<Mma::kMfmas, Mma::kReads, NL>();
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    template <class More, class Next, class Finish>
    __device__ __forceinline__ void run(More more, Next next, Finish finish) {
        if (!more()) return;
        next(cur);
        nk = stages_of(cur);
        nk4 = round4(nk);
        has_next = false;
        la.init(cur.A);
        lb.init(cur.B);
        if constexpr (kBar2) {
            // prologue: stages 0, 1 and the first part of 2, 3, as odd
            // steps -3 and -1 would issue them; then wait for stages 0 and 1
            // (step 0 reads both)
            issue_odd<1, 0, kNLT>(-3);
            issue_odd<3, 0, kS1>(-1);
            wait_vm_lgkm<kS1>();
        } else {
            // prologue: stages 0..3 (zeros past nk) in the order of steps -4..-1
#pragma unroll
            for (int t = -4; t < 0; ++t) {
#pragma unroll
                for (int op = 0; op < 2; ++op) {
                    const bool k = op == 0 ? AK : BK;
                    if (k && !(t & 1)) continue;
                    const int L = t + (k ? 3 : 4);
                    if (op == 0) la.issue(st.a[L], L, true);
                    else lb.issue(st.b[L], L, true);
                }
            }
            // stage 0 landed
            wait_vm_lgkm<Plan::prologue>();
        }
        barrier_nofence();
        mma.template read<0, 0>(st, 0);
        for (;;) {
            has_next = more();
            nk_nxt = 0;
            int kt0 = 0;
            if constexpr (kPeel) {
                step<0, true>(0, next);
                step<1>(1, next);
                step<2>(2, next);
                step<3>(3, next);
                kt0 = kStages;
            } else {
                mma.zero();
            }
            for (int kt = kt0; kt < nk4; kt += kStages) {
                step<0>(kt, next);
                step<1>(kt + 1, next);
                step<2>(kt + 2, next);
                step<3>(kt + 3, next);
            }
            finish(cur, mma);
            if (!has_next) break;
            cur = nxt;
            nk = nk_nxt;
            nk4 = round4(nk);
        }
        // the masked loads past the last tile are still in flight
        __builtin_amdgcn_s_waitcnt(0);
    }
};

template <bool OUT_BF16>
__device__ __forceinline__ void store1(void* out, int64_t idx, float v) {
    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
    else reinterpret_cast<float*>(out)[idx] = v;
}

// out[idx .. idx+3] = v, rounded once to the output type (idx a multiple of 4)
template <bool OUT_BF16>
__device__ __forceinline__ void store4(void* out, int64_t idx, f32x4 v) {
    if constexpr (OUT_BF16) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        u32x2 h;
        h[0] = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        h[1] = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) = h;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = v;
    }
}

// ---------------------------------------------------------------------------
// W^T for the data gradient: WT[e][k][n] = W[e][n][k] (BF16 bits), in 64x64
// tiles through LDS.  Grid (ceil(K/64), ceil(N/64), E), 256 threads; each
// thread reads two 16-byte row pieces of W and writes two of WT, so both
// sides are whole 16-byte, row-contiguous accesses.  N and K are multiples
// of 8, so a 16-byte piece is either inside the matrix or wholly outside.
// The tile is kept in LDS with a row pitch of 66 values, which spreads the
// column reads of the write-out over the banks.
__global__ __launch_bounds__(kThreads) void gg_transpose_w_kernel(const uint16_t* __restrict__ W,
                                                                  uint16_t* __restrict__ WT, int64_t N,
                                                                  int64_t K) {
    constexpr int P = 66;
    __shared__ uint16_t t[64 * P];
    const int64_t e = blockIdx.z, n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
    const uint16_t* src = W + e * N * K;
    uint16_t* dst = WT + e * N * K;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = threadIdx.x + i * kThreads, r = c >> 3, q = c & 7;   // tile row n0+r, columns k0+8q..
        const int64_t n = n0 + r, k = k0 + 8 * q;
        if (n < N && k < K) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + n * K + k);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                t[r * P + 8 * q + 2 * j] = (uint16_t)(v[j] & 0xFFFFu);
                t[r * P + 8 * q + 2 * j + 1] = (uint16_t)(v[j] >> 16);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = threadIdx.x + i * kThreads, r = c >> 3, q = c & 7;   // WT row k0+r, columns n0+8q..
        const int64_t k = k0 + r, n = n0 + 8 * q;
        if (k < K && n < N) {
            u32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = (uint32_t)t[(8 * q + 2 * j) * P + r] | ((uint32_t)t[(8 * q + 2 * j + 1) * P + r] << 16);
            *reinterpret_cast<u32x4*>(dst + k * N + n) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// forward / data gradient (identical in both variants)
//
// Persistent: workgroup b of G takes work items xcd_remap(b) + i*G, so at any
// time the 32 workgroups of one XCD work on 32 consecutive output tiles (the
// tiles of a few 256-row panels), which share operand slabs in that XCD's L2.

template <int OP, int BM, int BN, bool OUT_BF16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gg_fwd_dgrad_kernel(GemmArgs a) {
    // OP 0: forward; 1: data gradient; 2: data gradient with B = W^T
    // ([E][K][N], made by gg_transpose_w_kernel), so that both operands are
    // reduction-contiguous like the forward's
    constexpr bool BK = OP != 1;
    DRGG_STAGES(BM, BN, true, BK, stg);
    __shared__ Sched sch;
    __shared__ __attribute__((aligned(16))) char ep[WAVES * ep_rows(BM, BN) * 128];
    // output columns: N (forward) or K (data gradient)
    const int64_t ncols = OP == 0 ? a.N : a.K;
    const int32_t ntn = (int32_t)((ncols + BN - 1) / BN);
    build_schedule(sch, a.offs, a.E, a.M, a.T,
                   [=](int, int32_t T) { return ((T + BM - 1) / BM) * ntn; });
    const int64_t total = uni(sch.prefix[a.E]);
    const int64_t G = gridDim.x;
    int64_t w = xcd_remap(blockIdx.x, G);
    if (a.reverse) w = G - 1 - w;
    auto more = [&]() { return w < total; };
    auto next = [&](TileInfo& t) {
        const int e = uni(find_expert(sch, a.E, (int32_t)w));
        const int32_t oe = uni(sch.offs[e]), oe1 = uni(sch.offs[e + 1]);
        const int32_t local = (int32_t)w - uni(sch.prefix[e]);
        const int32_t mt = local / ntn, nt = local % ntn;
        const int64_t t0 = oe + (int64_t)mt * BM;
        const int64_t c0 = (int64_t)nt * BN;
        const uint16_t* We = a.B + (int64_t)e * a.N * a.K;
        t.o0 = t0;
        t.o1 = c0;
        t.rows = (int32_t)min<int64_t>(BM, oe1 - t0);
        t.cols = (int32_t)min<int64_t>(BN, ncols - c0);
        t.e = e;
        if constexpr (OP == 0) {   // Y = X W^T: both reduction-contiguous
            t.A = Operand{a.A + t0 * a.a_rs + e * a.a_gs, a.a_rs, t.rows, (int32_t)a.K};
            t.B = Operand{We + c0 * a.K, a.K, t.cols, (int32_t)a.K};
        } else if constexpr (OP == 1) {   // dX = G W: W is [n][k], reduction n strided
            t.A = Operand{a.A + t0 * a.a_rs + e * a.a_gs, a.a_rs, t.rows, (int32_t)a.N};
            t.B = Operand{We + c0, a.K, t.cols, (int32_t)a.N};
        } else {                   // dX = G (W^T)^T: W^T is [k][n], reduction n contiguous
            t.A = Operand{a.A + t0 * a.a_rs + e * a.a_gs, a.a_rs, t.rows, (int32_t)a.N};
            t.B = Operand{We + c0 * a.N, a.N, t.cols, (int32_t)a.N};
        }
        w += G;
    };
    void* out = a.out;
    auto finish = [&](const TileInfo& t, const TileMma<BM, BN, true, BK, WAVES>& mma) {
        const int64_t o = t.o0 * a.o_rs + (int64_t)t.e * a.o_gs + t.o1;
        void* base = OUT_BF16 ? (void*)(reinterpret_cast<uint16_t*>(out) + o) : (void*)(reinterpret_cast<float*>(out) + o);
        store_tile_lines<OUT_BF16, ep_rows(BM, BN)>(mma, (lds_t*)ep, base, a.o_rs, t.rows, t.cols);
    };
    TileRunner<BM, BN, true, BK, WAVES> runner;
    runner.st = stg;
    runner.run(more, next, finish);
}

// ---------------------------------------------------------------------------
// deterministic weight gradient: chunk partials (K3) and ordered fold (K4)

// Waves of the chunk kernel: 8 for the 256x256 tile (two per SIMD, VGPR
// accumulators, the barrier at every second step and the spread loads of
// the runner), 4 for the smaller tiles.  The arithmetic does not depend on it.
template <int BM, int BN>
constexpr int wgrad_det_waves() { return BM == 256 && BN == 256 ? 8 : 4; }

// The deterministic weight gradient's two plans (chunk rule parts 1-3 in
// plan.hpp).  Both cut expert e into S_e chunks of L_e tokens.  The
// all-split plan runs every tile of an expert with S_e > 1 as S_e chunk
// items; the tail-only plan runs the tiles of its first h_e 256-row bands
// (wgrad_whole_rows) as whole items and only the others as chunk items.
// Every workgroup estimates both planned walks on the kRuleCUs reference
// workgroups with the 256x256 reference tile (walk_makespan) and takes the
// tail-only plan when it is not slower: with equal experts its whole tiles
// fill full waves and the plan writes a third of the partials or fewer;
// with ragged experts whole tiles of different lengths balance badly and the
// all-split plan is kept.  The choice depends on the offsets and (E, M, N,
// K) only: not on the CU count, the grid or the kernel's tile shape.
//
// Walk positions: all-split plan, position p < E = the p-th expert of the
// longest-chunk-first order with all its items; tail-only plan, position
// p < E = that expert's whole tiles (none unless S_e > 1) and E + p = its
// chunk items (or, for S_e = 1, its whole tiles, which are as short).
template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__((64 * wgrad_det_waves<BM, BN>())) void gg_wgrad_det_kernel(GemmArgs a) {
    constexpr int WV = wgrad_det_waves<BM, BN>();
    constexpr bool kStaged = wgrad_det_staged(BM, BN);
    DRGG_STAGES(BM, BN, false, false, stg);
    __shared__ Sched sch;
    __shared__ int32_t slot_base[kMaxExperts + 1];
    __shared__ __attribute__((aligned(16))) char ep[kStaged ? WV * ep_rows(BM, BN) * 128 : 16];
    __shared__ unsigned long long s_red;
    const int32_t tn = (int32_t)((a.N + BM - 1) / BM), tk = (int32_t)((a.K + BN - 1) / BN);
    const int32_t P = tn * tk;
    const int32_t tn0 = (int32_t)((a.N + 255) / 256), tk0 = (int32_t)((a.K + 255) / 256);
    const int32_t P0 = tn0 * tk0;   // reference tiles per expert
    const int64_t cmax = a.chunk_max;
    const int E = a.E;
    build_schedule(sch, a.offs, E, a.M, a.T, [=](int, int32_t T) { return P * chunks_dev(T, cmax); });
    // Per-expert table in three stage buffers, which are free until the first
    // stage load: chunk length L_e, chunks S_e and, for S_e > 1, the whole
    // 256-row bands of the tail-only plan (wgrad_whole_rows).  Computed once
    // here, so that the plan estimates below read it instead of deriving it
    // again for every position and item.  Only the prologue reads it.
    typedef __attribute__((address_space(3))) int32_t lds_i32;
    lds_i32* const tL = reinterpret_cast<lds_i32*>(stg.b[1]);
    lds_i32* const tS = reinterpret_cast<lds_i32*>(stg.b[2]);
    lds_i32* const tB = reinterpret_cast<lds_i32*>(stg.b[3]);
    auto* const tab = reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(stg.a[1]);   // walk scratch
    int keeps_whole = 0;
    // ... and the partial slots: experts cut into more than one chunk, in
    // expert order (wave 0 alone with few experts; the ranking below ends
    // with the barrier that publishes both)
    if (E < kWaveExperts) {
        if (threadIdx.x < 64) {
            const int x = threadIdx.x;
            int32_t S = 0;
            if (x < E) {
                const int32_t T = sch.offs[x + 1] - sch.offs[x];
                const int32_t L = chunk_len_dev(T, cmax);
                S = L ? (int32_t)(((uint32_t)T + (uint32_t)L - 1) / (uint32_t)L) : 0;
                const int32_t B = S > 1 ? (int32_t)wgrad_whole_rows(T, a.M, a.N, a.K, S) : 0;
                tL[x] = L;
                tS[x] = S;
                tB[x] = B;
                keeps_whole = S > 1 && B > 0;
            }
            const int32_t sl = S > 1 ? S : 0;
            const int32_t incl = wave_incl_sum(sl);
            if (x < E) slot_base[x] = incl - sl;
            if (x == 63) slot_base[E] = incl;
        }
    } else {
        const int nthr = blockDim.x, per = (E + nthr - 1) / nthr;
        const int lo = min((int)threadIdx.x * per, E), hi = min(lo + per, E);
        int32_t run = 0;
        for (int x = lo; x < hi; ++x) {
            const int32_t T = sch.offs[x + 1] - sch.offs[x];
            const int32_t L = chunk_len_dev(T, cmax);
            const int32_t S = L ? (int32_t)(((uint32_t)T + (uint32_t)L - 1) / (uint32_t)L) : 0;
            const int32_t B = S > 1 ? (int32_t)wgrad_whole_rows(T, a.M, a.N, a.K, S) : 0;
            tL[x] = L;
            tS[x] = S;
            tB[x] = B;
            keeps_whole |= S > 1 && B > 0;
            run += S > 1 ? S : 0;
        }
        int32_t total;
        int32_t acc = block_exclusive_scan(run, reinterpret_cast<lds_i32*>(stg.b[0]), &total);
        for (int x = lo; x < hi; ++x) {
            slot_base[x] = acc;
            acc += tS[x] > 1 ? tS[x] : 0;
        }
        if (threadIdx.x == 0) slot_base[E] = total;
    }
    rank_experts(sch, stg.b[0], E, [&](int e) { return tL[e]; });
    auto e_at = [&](int q) { return expert_at(sch, q); };
    auto T_of = [&](int e) { return sch.offs[e + 1] - sch.offs[e]; };
    // plan choice on the reference tile (only when some split expert keeps
    // whole bands, else the two plans are the same)
    int tail = 0;
    if (E <= kTailPlanMaxExperts && __syncthreads_or(keeps_whole)) {
        position_prefix(sch, stg.b[0], E, [&](int q) { return P0 * tS[e_at(q)]; });
        const uint64_t mk_split = walk_makespan(sch, E, [&](int q) {
            const int e = e_at(q);
            return tS[e] > 1 ? tL[e] : T_of(e);
        }, &s_red, tab);
        position_prefix(sch, stg.b[0], 2 * E, [&](int q) {
            const int e = e_at(q < E ? q : q - E);
            const int32_t S = tS[e];
            if (S == 0) return 0;                // no tokens: no items
            if (S == 1) return q < E ? 0 : P0;
            const int32_t w0 = tB[e] * tk0;      // whole reference tiles
            return q < E ? w0 : (P0 - w0) * S;
        });
        const uint64_t mk_tail = walk_makespan(sch, 2 * E, [&](int q) {
            const int e = e_at(q < E ? q : q - E);
            return q < E || tS[e] <= 1 ? T_of(e) : tL[e];
        }, &s_red, tab);
        tail = mk_tail <= mk_split;
    }
    // the fold kernel's per-expert table (the same values from every
    // workgroup; workgroup 0 writes it): T_e, chunks, first partial slot,
    // first row of the partials (rows above it were stored directly).  With
    // zero_empty no fold runs and the call has no workspace.
    if (blockIdx.x == 0 && !a.zero_empty)
        for (int e = threadIdx.x; e < E; e += blockDim.x) {
            const int32_t S = tS[e];
            const int32_t row0 = tail && S > 1 ? (int32_t)min<int64_t>(a.N, (int64_t)tB[e] * 256) : 0;
            *reinterpret_cast<int4*>(a.fold_info + 4 * e) = int4{T_of(e), S, slot_base[e], row0};
        }
    // whole kernel tiles of an expert with S chunks and B whole bands (a
    // prefix of its row-major tiles)
    auto whole_tiles = [&](int32_t S, int32_t B) {
        return tail && S > 1 ? (int32_t)min<int64_t>(tn, (int64_t)B * (256 / BM)) * tk : 0;
    };
    const int npos = tail ? 2 * E : E;
    position_prefix(sch, stg.b[0], npos, [&](int q) {
        const int e = e_at(q < E ? q : q - E);
        const int32_t S = tS[e];
        if (!tail || S == 0) return P * S;   // (no tokens: no items)
        if (S == 1) return q < E ? 0 : P;
        const int32_t nw = whole_tiles(S, tB[e]);
        return q < E ? nw : (P - nw) * S;
    });
    const int64_t total = uni(sch.prefix[npos]);
    const int64_t G = gridDim.x;
    if (a.zero_empty) {
        // no fold kernel follows: the experts without tokens (which have no
        // items) get their zero output here, spread over all workgroups
        int any = 0;
        for (int e = threadIdx.x; e < E; e += blockDim.x) any |= T_of(e) == 0;
        if (__syncthreads_or(any)) {
            const int64_t nk8 = a.N * a.K / 8;   // K is a multiple of 8
            const int64_t n8 = (int64_t)E * nk8;
            for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += G * blockDim.x) {
                const int e = (int)(i / nk8);
                if (T_of(e) != 0) continue;
                if constexpr (OUT_BF16) {
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + i * 8) = u32x4{0u, 0u, 0u, 0u};
                } else {
                    f32x4* d = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + i * 8);
                    d[0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    d[1] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
    int64_t wb = xcd_remap(blockIdx.x, G), round = 0;
    if (a.reverse) wb = G - 1 - wb;
    int64_t w = snake_item(0, wb, G);
    auto more = [&]() { return w < total; };
    auto next = [&](TileInfo& t) {
        const int pos = uni(find_expert(sch, npos, (int32_t)w));
        const int e = uni(expert_at(sch, pos < E ? pos : pos - E));
        const int32_t oe = uni(sch.offs[e]), oe1 = uni(sch.offs[e + 1]);
        const int32_t T = oe1 - oe;
        const int32_t clen = chunk_len_dev(T, cmax);
        const int32_t nch = (int32_t)(((uint32_t)T + (uint32_t)clen - 1) / (uint32_t)clen);
        const int32_t local = (int32_t)w - uni(sch.prefix[pos]);
        int32_t tile, chunk = 0;
        bool whole;
        if (tail && pos < E) {          // a whole tile of a split expert
            tile = local;
            whole = true;
        } else if (nch > 1) {           // a chunk item: chunk-major, tiles of a chunk adjacent
            const int32_t nw = tail ? whole_tiles(nch, (int32_t)wgrad_whole_rows(T, a.M, a.N, a.K, nch)) : 0;
            const int32_t ps = P - nw;
            chunk = local / ps;
            tile = nw + local % ps;
            whole = false;
        } else {
            tile = local;
            whole = true;
        }
        const int32_t ti = tile / tk, tj = tile % tk;
        const int64_t n0 = (int64_t)ti * BM, k0 = (int64_t)tj * BN;
        const int64_t tb = oe + (whole ? 0 : (int64_t)chunk * clen);
        const int32_t len = whole ? T : (int32_t)min<int64_t>(clen, oe1 - tb);
        t.o0 = n0;
        t.o1 = k0;
        t.rows = (int32_t)min<int64_t>(BM, a.N - n0);
        t.cols = (int32_t)min<int64_t>(BN, a.K - k0);
        t.e = e;
        t.aux = whole ? -1 : uni(slot_base[e]) + chunk;   // -1: store the output directly
        // dW[n][k] = sum_t G[t][n] X[t][k]: both operands token-major (MN-major)
        t.A = Operand{a.A + tb * a.a_rs + e * a.a_gs + n0, a.a_rs, t.rows, len};
        t.B = Operand{a.B + tb * a.b_rs + e * a.b_gs + k0, a.b_rs, t.cols, len};
        w = snake_item(++round, wb, G);
    };
    auto finish = [&](const TileInfo& t, const TileMma<BM, BN, false, false, WV>& mma) {
        const int64_t ld = a.K;
        if (t.aux < 0) {   // a whole tile: round and store the output directly
            const int64_t off = (int64_t)t.e * a.N * a.K + t.o0 * a.K + t.o1;
            void* base = OUT_BF16 ? (void*)(reinterpret_cast<uint16_t*>(a.out) + off)
                                  : (void*)(reinterpret_cast<float*>(a.out) + off);
            if constexpr (kStaged) store_tile_lines<OUT_BF16, ep_rows(BM, BN)>(mma, (lds_t*)ep, base, ld, t.rows, t.cols);
            else store_tile<OUT_BF16>(mma, base, ld, t.rows, t.cols);
        } else {           // a chunk partial of an expert cut into several chunks
            float* dst = a.partial + (int64_t)t.aux * a.N * a.K + t.o0 * a.K + t.o1;
            if constexpr (kStaged) store_tile_lines<false, ep_rows(BM, BN), 0>(mma, (lds_t*)ep, dst, ld, t.rows, t.cols);
            else store_tile<false>(mma, dst, ld, t.rows, t.cols);
        }
    };
    TileRunner<BM, BN, false, false, WV> runner;
    runner.st = stg;
    runner.run(more, next, finish);
}

// Fold the partials of every expert cut into more than one chunk, in chunk
// order, in FP32, then round once (only rows from the expert's first
// partial row on: the rows of its whole tiles were stored directly);
// zero-fill experts without tokens.
// Grid: (ceil(N*K / 2048), E); 256 threads x 8 consecutive elements.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gg_wgrad_fold_kernel(GemmArgs a) {
    const int e = blockIdx.y;
    // T_e, chunks_e and the first partial slot, from the chunk kernel's
    // table; with M = 0 that kernel does not run and every expert is empty
    int32_t Te = 0, ce = 0, sb = 0, row0 = 0;
    if (a.M > 0) {
        const int4 info = *reinterpret_cast<const int4*>(a.fold_info + 4 * e);
        Te = info.x;
        ce = info.y;
        sb = info.z;
        row0 = info.w;
    }
    if (Te > 0 && ce <= 1) return;   // written directly by the chunk kernel
    const int64_t nk = a.N * a.K;
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
    if (i0 >= nk) return;            // nk is a multiple of 8
    if (i0 < (int64_t)row0 * a.K) return;   // a row of whole tiles, written directly
    float s[8];
    if (Te == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] = 0.f;
    } else {
        const float* p = a.partial + (int64_t)sb * nk + i0;
        f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
        f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) { s[j] = x0[j]; s[4 + j] = x1[j]; }
        // chunks 1 .. ce-1, added in chunk order; the loads of up to four
        // chunks are in flight at once
        int c = 1;
        for (; c + 4 <= ce; c += 4) {
            f32x4 y[4][2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float* q = p + (int64_t)(c + u) * nk;
                y[u][0] = *reinterpret_cast<const f32x4*>(q);
                y[u][1] = *reinterpret_cast<const f32x4*>(q + 4);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) { s[j] += y[u][0][j]; s[4 + j] += y[u][1][j]; }
        }
        for (; c < ce; ++c) {
            const float* q = p + (int64_t)c * nk;
            x0 = *reinterpret_cast<const f32x4*>(q);
            x1 = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { s[j] += x0[j]; s[4 + j] += x1[j]; }
        }
    }
    const int64_t o = (int64_t)e * nk + i0;
    if constexpr (OUT_BF16) {
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = (uint32_t)f32_to_bf16(s[2 * q]) | ((uint32_t)f32_to_bf16(s[2 * q + 1]) << 16);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + o) = v;
    } else {
        float* d = reinterpret_cast<float*>(a.out) + o;
        *reinterpret_cast<f32x4*>(d) = f32x4{s[0], s[1], s[2], s[3]};
        *reinterpret_cast<f32x4*>(d + 4) = f32x4{s[4], s[5], s[6], s[7]};
    }
}

// ---------------------------------------------------------------------------
// non-deterministic weight gradient: whole tiles in full waves, the tail
// either placed whole on the least-loaded workgroups or cut into chunks of
// whole 512-token units whose partials are added into an FP32 tile sum by
// atomics, a per-tile ticket picking the last arrival, which writes the tile
// (flashinfer PR #8258, Summary)

// the deterministic chunk length rounded up to whole 512-token units
__device__ __forceinline__ int32_t unit_chunk_len(int32_t T, int64_t chunk_max) {
    const int32_t l = chunk_len_dev(T, chunk_max);
    return (int32_t)(((l + kStreamKUnit - 1) / kStreamKUnit) * kStreamKUnit);
}
__device__ __forceinline__ int32_t unit_chunks(int32_t T, int64_t chunk_max) {
    const int32_t l = unit_chunk_len(T, chunk_max);
    return l ? (T + l - 1) / l : 0;
}

// Test aid (DRGG_KNOB_DELAY_SEED): a bounded sleep, a different length for
// every (seed, workgroup, tile, expert), before a tail piece adds its
// partial (the pieces of a tile run on different workgroups), so that the
// arrivals at a tile's ticket come in other orders.  At most 47 x 16 x 64
// cycles.
__device__ __forceinline__ void arrival_delay(int32_t seed, int32_t tile, int32_t expert) {
    uint32_t h = (uint32_t)seed * 2654435761u ^ (uint32_t)blockIdx.x * 40503u ^ (uint32_t)tile * 977u ^
                 (uint32_t)expert * 131u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    const int n = (int)(h % 48u);
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(16);
}

// Walks (experts in decreasing order of unit chunk length).  Banded walk:
// position p < E holds the whole tiles of the p-th expert (split_whole_rows:
// full waves on its share of the grid; all of an expert not cut into
// chunks), position E + p its tail tiles, whole (slack placement) or as chunk
// items.  All-split walk: position p holds every tile of the p-th expert,
// as chunk items if it is cut into chunks.  Like the deterministic program,
// the kernel estimates both walks (walk_makespan, here on the live grid) and
// runs the banded one when it is not slower: with ragged experts, whole
// tiles of different lengths balance worse than chunk items.  With more
// than kTailPlanMaxExperts experts only the all-split walk exists.
//
// Slack placement: at the start every workgroup computes the load of every
// workgroup from the first pass (the whole tiles, in snake rounds over the
// grid), ranks them and checks whether the i-th tail tile fits whole on the
// i-th least-loaded workgroup within the largest load plus one tail share
// (a chunk of that expert).  All the workgroups reach the same answer; if
// every tail tile fits, the workgroup of rank i runs tail tile i whole after
// its first pass, otherwise the tail runs as chunk items after the first
// pass.  (The pages rank the clusters while the first tiles run; here the
// ranking is recomputed by every workgroup from the plan, so no workgroup
// waits for another.)
template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gg_wgrad_atomic_kernel(GemmArgs a) {
    DRGG_STAGES(BM, BN, false, false, stg);
    __shared__ Sched sch;
    __shared__ int32_t nw_tab[kMaxExperts];   // whole tiles of each expert (the decode reads it)
    __shared__ int32_t s_last;
    __shared__ int32_t s_rank;
    __shared__ unsigned long long s_red, s_min;
    const int32_t tn = (int32_t)((a.N + BM - 1) / BM), tk = (int32_t)((a.K + BN - 1) / BN);
    const int32_t P = tn * tk;
    const int64_t cmax = a.chunk_max;
    const int E = a.E;
    const int64_t G = gridDim.x;
    const int tid = threadIdx.x, nthr = blockDim.x;
    build_schedule(sch, a.offs, E, a.M, a.T, [=](int, int32_t) { return 0; });
    rank_experts(sch, stg.b[0], E, [&](int e) { return unit_chunk_len(sch.offs[e + 1] - sch.offs[e], cmax); });
    auto T_at = [&](int q) { const int e = expert_at(sch, q); return sch.offs[e + 1] - sch.offs[e]; };
    const bool banded = E <= kTailPlanMaxExperts;
    auto* const tab = reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(stg.a[1]);   // walk scratch
    // whole tiles of each expert: a prefix of its row-major tiles (none for
    // an expert without tokens, which has no items at all); computed once,
    // so that the per-tile decode is a table read
    for (int e = tid; e < E; e += nthr) {
        const int32_t T = sch.offs[e + 1] - sch.offs[e], S = unit_chunks(T, cmax);
        int32_t nw = 0;
        if (S == 1) nw = P;
        else if (S > 1 && banded)
            nw = (int32_t)min<int64_t>(tn, split_whole_rows(T, a.M, a.N, a.K, S, G) * (256 / BM)) * tk;
        nw_tab[e] = nw;
    }
    __syncthreads();
    auto nw_at = [&](int q) { return nw_tab[expert_at(sch, q)]; };
    const int64_t wb0 = a.reverse ? G - 1 - xcd_remap(blockIdx.x, G) : xcd_remap(blockIdx.x, G);
    auto S_at = [&](int q) { return unit_chunks(T_at(q), cmax); };
    auto L_at = [&](int q) { return unit_chunk_len(T_at(q), cmax); };
    // the all-split walk: every tile of an expert cut into chunks as chunk
    // items, the others whole (one position per expert)
    auto split_walk = [&] {
        position_prefix(sch, stg.b[0], E, [&](int q) {
            const int32_t S = S_at(q);
            return S > 1 ? P * S : S == 1 ? P : 0;
        });
    };
    // the banded walk with its tail as chunk items
    auto band_walk = [&] {
        position_prefix(sch, stg.b[0], 2 * E, [&](int q) {
            const int qe = q < E ? q : q - E;
            const int32_t T = T_at(qe), nw = nw_at(qe);
            return T == 0 ? 0 : q < E ? nw : (P - nw) * unit_chunks(T, cmax);
        });
    };
    int use_band = 0, slack = 0;
    int64_t total1 = 0, ntail = 0;
    if (banded) {
        // the banded walk's first pass (whole tiles) and its tail tile counts
        position_prefix(sch, stg.b[0], 2 * E, [&](int q) {
            const int qe = q < E ? q : q - E;
            const int32_t T = T_at(qe), nw = nw_at(qe);
            return T == 0 ? 0 : q < E ? nw : P - nw;
        });
        total1 = sch.prefix[E];
        ntail = sch.prefix[2 * E] - total1;
        // with no whole tiles the banded walk is the all-split walk
        if (total1 > 0) {
            // every workgroup's load from the first pass
            const bool rank = ntail > 0 && ntail <= G && G <= kSlackMaxGrid;
            auto* load = reinterpret_cast<__attribute__((address_space(3))) uint64_t*>(stg.b[1]);
            auto* sorted = reinterpret_cast<__attribute__((address_space(3))) uint64_t*>(stg.b[2]);
            if (tid == 0) {
                s_red = 0;
                s_min = ~0ull;
            }
            __syncthreads();
            uint64_t hi = 0, lo = ~0ull;
            for (int64_t b = tid; b < G; b += nthr) {
                uint64_t l = 0;
                for (int64_t r = 0;; ++r) {
                    const int64_t i = snake_item(r, b, G);
                    if (i >= total1) break;   // later rounds hold only larger indices
                    l += (uint64_t)T_at(find_expert(sch, E, (int32_t)i)) + (uint64_t)kItemOverheadTokens;
                }
                if (rank) load[b] = l;
                hi = l > hi ? l : hi;
                lo = l < lo ? l : lo;
            }
            hi = wave_max_u64(hi);
            lo = wave_min_u64(lo);
            if ((tid & 63) == 0) {
                atomicMax(&s_red, (unsigned long long)hi);
                atomicMin(&s_min, (unsigned long long)lo);
            }
            __syncthreads();
            const uint64_t lmax = s_red, lmin = s_min;
            // slack placement needs at least the longest tail tile to fit
            // whole on the least-loaded workgroup; only then rank them all
            const int32_t T0 = ntail > 0 ? T_at(find_expert(sch, 2 * E, (int32_t)total1) - E) : 0;
            if (rank && lmin + (uint64_t)T0 <= lmax + (uint64_t)unit_chunk_len(T0, cmax)) {
                for (int64_t b = tid; b < G; b += nthr) {
                    const uint64_t lb = load[b];
                    int64_t r = 0;
                    for (int64_t c = 0; c < G; ++c) r += load[c] < lb || (load[c] == lb && c < b);
                    sorted[r] = lb;
                    if (b == wb0) s_rank = (int32_t)r;
                }
                __syncthreads();
                int fits = 1;
                uint64_t top = 0;   // the placed tail's largest load
                for (int64_t i = tid; i < ntail; i += nthr) {
                    const int32_t T = T_at(find_expert(sch, 2 * E, (int32_t)(total1 + i)) - E);
                    fits &= sorted[i] + (uint64_t)T <= lmax + (uint64_t)unit_chunk_len(T, cmax);
                    const uint64_t t = sorted[i] + (uint64_t)T + (uint64_t)kItemOverheadTokens;
                    top = t > top ? t : top;
                }
                slack = __syncthreads_and(fits);
                if (slack) {
                    if (tid == 0) s_red = lmax;
                    __syncthreads();
                    top = wave_max_u64(top);
                    if ((tid & 63) == 0) atomicMax(&s_red, (unsigned long long)top);
                    __syncthreads();
                }
            }
            // estimated times of the banded walk (slack placement, or its
            // tail as chunk items) and of the all-split walk; without slack
            // placement and with no expert cut into chunks keeping whole
            // tiles, both walks hold the same items and the all-split one
            // runs
            int keeps = 0;
            for (int q = tid; q < E; q += nthr) keeps |= S_at(q) > 1 && nw_at(q) > 0;
            if (__syncthreads_or(keeps) || slack) {
                uint64_t mk_band;
                if (slack) {
                    mk_band = s_red;
                    __syncthreads();
                } else {
                    band_walk();
                    mk_band = walk_makespan(sch, 2 * E, [&](int q) { return q < E ? T_at(q) : L_at(q - E); }, &s_red,
                                            tab, G);
                }
                split_walk();
                const uint64_t mk_split = walk_makespan(sch, E, [&](int q) {
                    return S_at(q) > 1 ? L_at(q) : T_at(q);
                }, &s_red, tab, G);
                use_band = mk_band <= mk_split;
            }
            slack = slack && use_band;
        }
    }
    if (a.report && blockIdx.x == 0 && tid == 0) {
        a.report[0] = slack;
        a.report[1] = (int32_t)ntail;
        a.report[2] = use_band;
        a.report[3] = (int32_t)G;
    }
    // the walk that runs: first pass and placed tail; first pass and chunked
    // tail; or all split
    int npos = E;
    if (use_band) {
        npos = 2 * E;
        if (slack) {
            position_prefix(sch, stg.b[0], 2 * E, [&](int q) {
                const int qe = q < E ? q : q - E;
                const int32_t T = T_at(qe), nw = nw_at(qe);
                return T == 0 ? 0 : q < E ? nw : P - nw;
            });
        } else {
            band_walk();
        }
    } else {
        split_walk();
    }
    const int64_t total = uni(sch.prefix[npos]);
    const int64_t wb = wb0;
    int64_t round = 0;
    int64_t w = snake_item(0, wb, G);
    // with slack placement the walk ends with this workgroup's tail tile
    slack = uni(slack);
    use_band = uni(use_band);
    total1 = uni((int32_t)total1);
    const int64_t first_end = slack ? total1 : total;
    const int64_t tail_item = slack && uni(s_rank) < total - total1 ? total1 + uni(s_rank) : -1;
    bool tail_done = tail_item < 0;
    auto more = [&]() {
        if (w < first_end) return true;
        if (!tail_done) {
            w = tail_item;
            tail_done = true;
            return true;
        }
        return false;
    };
    auto next = [&](TileInfo& t) {
        const int pos = uni(find_expert(sch, npos, (int32_t)w));
        const int e = uni(expert_at(sch, pos < E ? pos : pos - E));
        const int32_t oe = uni(sch.offs[e]), oe1 = uni(sch.offs[e + 1]);
        const int32_t T = oe1 - oe;
        const int32_t clen = unit_chunk_len(T, cmax);
        const int32_t nch = (T + clen - 1) / clen;
        const int32_t local = (int32_t)w - uni(sch.prefix[pos]);
        int32_t tile, chunk = 0;
        bool whole;
        if (use_band && pos < E) {                // first pass: a whole tile
            tile = local;
            whole = true;
        } else if (use_band && slack) {          // a tail tile placed whole
            tile = uni(nw_tab[e]) + local;
            whole = true;
        } else if (nch > 1) {                    // a chunk item (of the tail, or of every tile)
            const int32_t nw = use_band ? uni(nw_tab[e]) : 0, ps = P - nw;
            chunk = local / ps;
            tile = nw + local % ps;
            whole = false;
        } else {
            tile = local;
            whole = true;
        }
        const int32_t ti = tile / tk, tj = tile % tk;
        const int64_t n0 = (int64_t)ti * BM, k0 = (int64_t)tj * BN;
        const int64_t tb = oe + (whole ? 0 : (int64_t)chunk * clen);
        const int32_t len = whole ? T : (int32_t)min<int64_t>(clen, oe1 - tb);
        t.o0 = n0;
        t.o1 = k0;
        t.rows = (int32_t)min<int64_t>(BM, a.N - n0);
        t.cols = (int32_t)min<int64_t>(BN, a.K - k0);
        t.e = e;
        t.aux = whole ? -1 : tile;   // -1: the whole tile in this item, store directly
        t.aux2 = nch;                // pieces of a split tile
        t.A = Operand{a.A + tb * a.a_rs + e * a.a_gs + n0, a.a_rs, t.rows, len};
        t.B = Operand{a.B + tb * a.b_rs + e * a.b_gs + k0, a.b_rs, t.cols, len};
        w = w < first_end ? snake_item(++round, wb, G) : first_end;
    };
    auto finish = [&](const TileInfo& t, const TileMma<BM, BN, false, false>& mma) {
        const int64_t base = (int64_t)t.e * a.N * a.K + t.o0 * a.K + t.o1;
        void* out = a.out;
        if (t.aux < 0) {   // the whole tile in this workgroup: store directly
            void* ob = OUT_BF16 ? (void*)(reinterpret_cast<uint16_t*>(out) + base)
                                : (void*)(reinterpret_cast<float*>(out) + base);
            store_tile<OUT_BF16>(mma, ob, a.K, t.rows, t.cols);
            return;
        }
        if (a.delay_seed) arrival_delay(a.delay_seed, t.aux, t.e);
        const int64_t slot = (int64_t)t.e * P + t.aux;
        float* ts = a.tilesum + slot * (BM * BN);
        const uint32_t parts = (uint32_t)t.aux2;
        void* ob = OUT_BF16 ? (void*)(reinterpret_cast<uint16_t*>(out) + base)
                            : (void*)(reinterpret_cast<float*>(out) + base);
        // If every other piece of this tile has already added its partial and
        // taken its ticket, this piece is the last one: it adds its own
        // partial from registers and skips the atomic adds (mode 2).
        // Otherwise it adds into the tile sum, takes a ticket, and is the last
        // one (mode 1) if the ticket says so.
        if (threadIdx.x == 0)
            s_last = __hip_atomic_load(a.tickets + slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) + 1 == parts
                         ? 2 : 0;
        __syncthreads();
        int mode = s_last;
        if (mode == 0) {
            atomic_add_tile(mma, ts);
            __threadfence();
            __syncthreads();
            if (threadIdx.x == 0) {
                const uint32_t old = __hip_atomic_fetch_add(a.tickets + slot, 1u, __ATOMIC_ACQ_REL,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                s_last = old + 1 == parts ? 1 : 0;
            }
            __syncthreads();
            mode = s_last;
        }
        if (mode != 0) {   // last piece: write the tile from the sum and clear it
            __threadfence();
            if (mode == 2) drain_tile_sum<OUT_BF16, true>(mma, ts, ob, a.K, t.rows, t.cols);
            else drain_tile_sum<OUT_BF16, false>(mma, ts, ob, a.K, t.rows, t.cols);
            if (threadIdx.x == 0)
                __hip_atomic_store(a.tickets + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    };
    TileRunner<BM, BN, false, false> runner;
    runner.st = stg;
    runner.run(more, next, finish);
    // experts without tokens: dW[e] = +0, shared out over the grid
    const int64_t nk = a.N * a.K;
    const int64_t b = blockIdx.x;
    for (int e = 0; e < E; ++e) {
        if (sch.offs[e + 1] != sch.offs[e]) continue;
        for (int64_t i = (b * kGemmThreads + threadIdx.x) * 8; i < nk; i += (int64_t)gridDim.x * kGemmThreads * 8) {
            const int64_t o = (int64_t)e * nk + i;
            if constexpr (OUT_BF16) {
                *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + o) = u32x4{0, 0, 0, 0};
            } else {
                float* d = reinterpret_cast<float*>(a.out) + o;
                *reinterpret_cast<f32x4*>(d) = f32x4{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4*>(d + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// FP32 router GEMM as a BF16x3 split on MFMA (flashinfer PR #8363, Summary:
// a 256-expert router whose FP32 products are emulated by three BF16 ones).
//   out[m,n] = sum_k X[m,k] Wr[n,k];  v = hi + lo, hi = bf16(v), lo = bf16(v - hi)
//   per 16-step: acc += hi_x hi_w, then hi_x lo_w, then lo_x hi_w.
//
// One workgroup per 128x128 output tile, 4 waves in a 2x2 grid (64x64 each),
// with the grouped GEMM's step schedule.  The FP32 operands go straight from
// HBM into four 32-value LDS stages per operand (rows of 128 bytes, chunk c of
// row r at c ^ swzK(r), conflict-free for the operand reads); each MFMA
// operand fragment is read as 8 FP32 values and split into its BF16 hi and
// lo parts in registers (v - hi is exact in FP32).

constexpr int kRouterBM = 128, kRouterBN = 128;
// Waves per router workgroup: one per SIMD.  Eight (two per SIMD, 64x32 wave
// tiles) give bitwise the same output but ran 168 us against 148-160 us.
constexpr int kRouterWaves = 4;

struct RouterArgs {
    const float* X;
    const float* Wr;
    float* out;
    int64_t M, N, K;
};

// Loads one 32-value stage of ROWS FP32 rows (128 bytes each) into LDS.
template <int ROWS, int WAVES>
struct F32StageLoader {
    static constexpr int kPerWave = ROWS * 128 / 1024 / WAVES;
    static_assert(kPerWave >= 1 && kPerWave * WAVES * 1024 == ROWS * 128, "whole 1 KB loads per wave");
    uint32_t off[kPerWave];   // byte offset of this lane's 16 bytes from the stage base (kOOB if masked)
    int32_t kp[kPerWave];     // reduction position of those 16 bytes within the stage
    const char* base;
    int32_t klen;

    __device__ __forceinline__ void init(const float* b, int64_t ld, int32_t nvalid, int32_t kl) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        base = reinterpret_cast<const char*>(b);
        klen = kl;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int bb = (wave * kPerWave + i) * 1024 + lane * 16;
            const int row = bb / 128, logical = ((bb % 128) / 16) ^ swzK(row);
            off[i] = row < nvalid ? (uint32_t)(row * ld * 4 + logical * 16) : kOOB;
            kp[i] = logical * 4;
        }
    }

    // stage L into `buf`; positions at or past klen read as zero
    __device__ __forceinline__ void issue(lds_t* buf, int L) const {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) issue_one(buf, L, i);
    }

    // load i of this wave's share of stage L
    __device__ __forceinline__ void issue_one(lds_t* buf, int L, int i) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)L * 128);
        const int rem = klen - L * 32;
        const uint32_t o = kp[i] < rem ? off[i] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(buf + (wave * kPerWave + i) * 1024), 16, o, 0,
                                                 0, 0);
    }
};

// Lane l's 8 FP32 values 16*s + 8*(l/32) .. +7 of tile row rb + (l & 31).
struct Raw8 {
    f32x4 x0, x1;
};
__device__ __forceinline__ Raw8 read_raw(const lds_t* buf, int rb, int s, int l) {
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    const int row = rb + (l & 31), c0 = 4 * s + 2 * (l >> 5);
    Raw8 r;
    r.x0 = *reinterpret_cast<const lds_f32x4*>(buf + row * 128 + ((c0 ^ swzK(row)) << 4));
    r.x1 = *reinterpret_cast<const lds_f32x4*>(buf + row * 128 + (((c0 + 1) ^ swzK(row)) << 4));
    return r;
}

// Split values 2p, 2p+1 of a raw fragment into BF16 hi = bf16(v) and
// lo = bf16(v - hi), both rounded to nearest even (v - hi is exact in FP32).
__device__ __forceinline__ void split_pair(const Raw8& r, int p, bf16x8& hi, bf16x8& lo) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const float x0 = p < 2 ? r.x0[2 * p] : r.x1[2 * p - 4], x1 = p < 2 ? r.x0[2 * p + 1] : r.x1[2 * p - 3];
    const bf16x2 h = __builtin_convertvector((f32x2{x0, x1}), bf16x2);
    const bf16x2 d = __builtin_convertvector((f32x2{x0 - (float)h[0], x1 - (float)h[1]}), bf16x2);
    hi[2 * p] = h[0];
    hi[2 * p + 1] = h[1];
    lo[2 * p] = d[0];
    lo[2 * p + 1] = d[1];
}

// Split 8 FP32 values into BF16 hi = bf16(v) and lo = bf16(v - hi), both
// rounded to nearest even (v - hi is exact in FP32).
__device__ __forceinline__ void split8(const Raw8& r, bf16x8& hi, bf16x8& lo) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const float x[8] = {r.x0[0], r.x0[1], r.x0[2], r.x0[3], r.x1[0], r.x1[1], r.x1[2], r.x1[3]};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const bf16x2 h = __builtin_convertvector((f32x2{x[2 * p], x[2 * p + 1]}), bf16x2);
        const bf16x2 d = __builtin_convertvector((f32x2{x[2 * p] - (float)h[0], x[2 * p + 1] - (float)h[1]}), bf16x2);
        hi[2 * p] = h[0];
        hi[2 * p + 1] = h[1];
        lo[2 * p] = d[0];
        lo[2 * p + 1] = d[1];
    }
}

constexpr int kSchedValu = 0x002;

// Router sub-step schedule: the NR LDS reads, the NV vector instructions
// that split the fragments read in the previous sub-step, and the NL global
// loads are spread evenly over the NM MFMAs.
template <int NM, int NR, int NL, int NV, int T>
__device__ __forceinline__ void router_slot() {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    constexpr int r = NR * (T + 1) / NM - NR * T / NM;
    constexpr int v = NV * (T + 1) / NM - NV * T / NM;
    constexpr int l = NL * (T + 1) / NM - NL * T / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, r, 0);
    if constexpr (l > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, l, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(kSchedValu, v, 0);
}
template <int NM, int NR, int NL, int NV, int... T>
__device__ __forceinline__ void router_sched_impl(std::integer_sequence<int, T...>) {
    (router_slot<NM, NR, NL, NV, T>(), ...);
}
template <int NM, int NR, int NL, int NV>
__device__ __forceinline__ void router_sched() {
    router_sched_impl<NM, NR, NL, NV>(std::make_integer_sequence<int, NM>{});
}

template <int BM, int BN, int WAVES>
struct RouterMma {
    static constexpr int kWGM = (WAVES == 8 && BM >= 256) ? 4 : 2;
    static constexpr int kWGN = WAVES / kWGM;
    static constexpr int WM = BM / kWGM, WN = BN / kWGN;
    __device__ static __forceinline__ int wave_row(int wave) { return (wave / kWGN) * WM; }
    __device__ static __forceinline__ int wave_col(int wave) { return (wave % kWGN) * WN; }
    static constexpr int kBI = WM / 32, kBJ = WN / 32;
    static constexpr int kReads = 2 * (kBI + kBJ);
    static constexpr int kMfmas = 3 * kBI * kBJ;
    static constexpr int kSplitValu = 24 * (kBI + kBJ);   // about 24 per 8-value fragment
    f32x16 acc[kBI][kBJ];
    bf16x8 ah[2][kBI], al[2][kBI], bh[2][kBJ], bl[2][kBJ];   // split fragments of sub-step 0 and 1
    Raw8 ra[kBI], rbv[kBJ];                                    // raw fragments waiting to be split

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    // raw fragments of sub-step s of the stage in (sA, sB)
    __device__ __forceinline__ void read(const lds_t* sA, const lds_t* sB, int s) {
        const int l = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int oa = wave_row(wave), ob = wave_col(wave);
#pragma unroll
        for (int i = 0; i < kBI; ++i) ra[i] = read_raw(sA, oa + 32 * i, s, l);
#pragma unroll
        for (int j = 0; j < kBJ; ++j) rbv[j] = read_raw(sB, ob + 32 * j, s, l);
    }

    // split the raw fragments into set F
    template <int F>
    __device__ __forceinline__ void split() {
#pragma unroll
        for (int i = 0; i < kBI; ++i) split8(ra[i], ah[F][i], al[F][i]);
#pragma unroll
        for (int j = 0; j < kBJ; ++j) split8(rbv[j], bh[F][j], bl[F][j]);
    }

    // the raw fragments of one side (H = 0: the A side, 1: the B side) of
    // sub-step s of the stage in buf
    template <int H>
    __device__ __forceinline__ void read_side(const lds_t* buf, int s) {
        const int l = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if constexpr (H == 0) {
            const int oa = wave_row(wave);
#pragma unroll
            for (int i = 0; i < kBI; ++i) ra[i] = read_raw(buf, oa + 32 * i, s, l);
        } else {
            const int ob = wave_col(wave);
#pragma unroll
            for (int j = 0; j < kBJ; ++j) rbv[j] = read_raw(buf, ob + 32 * j, s, l);
        }
    }

    // split the raw fragments of one side into set F
    template <int F, int H>
    __device__ __forceinline__ void split_side() {
        if constexpr (H == 0) {
#pragma unroll
            for (int i = 0; i < kBI; ++i) split8(ra[i], ah[F][i], al[F][i]);
        } else {
#pragma unroll
            for (int j = 0; j < kBJ; ++j) split8(rbv[j], bh[F][j], bl[F][j]);
        }
    }

    // one 16-byte half (hh) of the raw fragment fr of side H
    template <int H, int FR, int HH>
    __device__ __forceinline__ void read_one(const lds_t* buf, int s) {
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        const int l = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int row = (H == 0 ? wave_row(wave) : wave_col(wave)) + 32 * FR + (l & 31);
        const int c = 4 * s + 2 * (l >> 5) + HH;
        const f32x4 v = *reinterpret_cast<const lds_f32x4*>(buf + row * 128 + ((c ^ swzK(row)) << 4));
        Raw8& r = H == 0 ? ra[FR] : rbv[FR];
        if constexpr (HH == 0) r.x0 = v;
        else r.x1 = v;
    }

    // values 2p, 2p+1 of raw fragment fr of side H into set F
    template <int F, int H, int FR, int P>
    __device__ __forceinline__ void split_one() {
        if constexpr (H == 0) split_pair(ra[FR], P, ah[F][FR], al[F][FR]);
        else split_pair(rbv[FR], P, bh[F][FR], bl[F][FR]);
    }

    // product p of mfma<F> (kind p / (kBI*kBJ) on block p % (kBI*kBJ))
    template <int F, int P>
    __device__ __forceinline__ void mfma_one() {
        constexpr int NB = kBI * kBJ, kind = P / NB, i = (P % NB) / kBJ, j = P % kBJ;
        const bf16x8& b = kind == 1 ? bl[F][j] : bh[F][j];
        const bf16x8& a = kind == 2 ? al[F][i] : ah[F][i];
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[i][j], 0, 0, 0);
    }

    // products P0 .. P1-1 of the 3 * kBI * kBJ of mfma<F>, in its order
    // (product p is kind p / (kBI*kBJ) on block p % (kBI*kBJ))
    template <int F, int P0, int P1>
    __device__ __forceinline__ void mfma_range() {
        constexpr int NB = kBI * kBJ;
#pragma unroll
        for (int p = P0; p < P1; ++p) {
            const int kind = p / NB, i = (p % NB) / kBJ, j = p % kBJ;
            const bf16x8& b = kind == 1 ? bl[F][j] : bh[F][j];
            const bf16x8& a = kind == 2 ? al[F][i] : ah[F][i];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[i][j], 0, 0, 0);
        }
    }

    // the three products of one 16-step, each over all blocks before the
    // next, so that dependent MFMAs on one accumulator are kBI*kBJ apart
    template <int F>
    __device__ __forceinline__ void mfma() {
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[F][j], ah[F][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[F][j], ah[F][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[F][j], al[F][i], acc[i][j], 0, 0, 0);
    }
};

// kRouterStages LDS stages per operand: with no other LDS in this kernel, five
// (all 160 KB) fit, one more stage of loads in flight than the grouped GEMM.
constexpr int kRouterStages = 5;

__global__ __launch_bounds__(64 * kRouterWaves) void router_bf16x3_kernel(RouterArgs a) {
    constexpr int BM = kRouterBM, BN = kRouterBN, S = kRouterStages;
    static_assert(S == 5, "the stage buffers below are written out for five stages");
    __shared__ __attribute__((aligned(256))) char sa0[BM * 128], sa1[BM * 128], sa2[BM * 128], sa3[BM * 128],
        sa4[BM * 128];
    __shared__ __attribute__((aligned(256))) char sb0[BN * 128], sb1[BN * 128], sb2[BN * 128], sb3[BN * 128],
        sb4[BN * 128];
    lds_t* const sa[S] = {(lds_t*)sa0, (lds_t*)sa1, (lds_t*)sa2, (lds_t*)sa3, (lds_t*)sa4};
    lds_t* const sb[S] = {(lds_t*)sb0, (lds_t*)sb1, (lds_t*)sb2, (lds_t*)sb3, (lds_t*)sb4};
    using Mma = RouterMma<BM, BN, kRouterWaves>;
    using LA = F32StageLoader<BM, kRouterWaves>;
    using LB = F32StageLoader<BN, kRouterWaves>;
    constexpr int C = LA::kPerWave + LB::kPerWave;   // loads per wave per stage

    const int64_t ntn = (a.N + BN - 1) / BN;
    const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t m0 = (w / ntn) * BM, n0 = (w % ntn) * BN;
    const int32_t rows = (int32_t)min<int64_t>(BM, a.M - m0);
    const int32_t cols = (int32_t)min<int64_t>(BN, a.N - n0);
    LA la;
    LB lb;
    la.init(a.X + m0 * a.K, a.K, rows, (int32_t)a.K);
    lb.init(a.Wr + n0 * a.K, a.K, cols, (int32_t)a.K);
    const int nk = (int)((a.K + 31) / 32);
    const int nkS = ((nk + S - 1) / S) * S;
    Mma mma;
#pragma unroll
    for (int X = 0; X < S; ++X) {
        la.issue(sa[X], X);
        lb.issue(sb[X], X);
    }
    // stages 0 and 1 have landed; the fragments of stage 0 are read (and
    // those of sub-step 0 split) ahead of step 0
    wait_vm_lgkm<(S - 2) * C>();
    barrier_nofence();
    mma.read(sa[0], sb[0], 0);
    mma.template split<0>();
    mma.read(sa[0], sb[0], 1);
    mma.zero();
    // Step kt of stage slot ST, software-pipelined over the two sub-steps:
    //   region 0: MFMAs of (kt, 0); split of the raw (kt, 1); read raw (kt+1, 0)
    //   barrier:  stage kt+2 has landed for every wave (the loads of kt+3 ..
    //             kt+S-1 may still be in flight); stage kt was read in full
    //             during step kt-1, so its slot takes the loads of stage kt+S
    //   region 1: MFMAs of (kt, 1); split of the raw (kt+1, 0); read raw (kt+1, 1)
    // Stages past nk load zeros, which add nothing.
    auto step = [&](auto st_tag, int kt) {
        constexpr int ST = decltype(st_tag)::value, NX = (ST + 1) % S;
        __builtin_amdgcn_sched_barrier(0);
        mma.template mfma<0>();
        mma.template split<1>();
        mma.read(sa[NX], sb[NX], 0);
        router_sched<Mma::kMfmas, Mma::kReads, 0, Mma::kSplitValu>();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm<(S - 3) * C>();
        barrier_nofence();
        la.issue(sa[ST], kt + S);
        lb.issue(sb[ST], kt + S);
        mma.template mfma<1>();
        mma.template split<0>();
        mma.read(sa[NX], sb[NX], 1);
        router_sched<Mma::kMfmas, Mma::kReads, C, Mma::kSplitValu>();
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < nkS; kt += S) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
        step(std::integral_constant<int, 2>{}, kt + 2);
        step(std::integral_constant<int, 3>{}, kt + 3);
        step(std::integral_constant<int, 4>{}, kt + 4);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the masked loads past the end
    store_tile<false>(mma, a.out + m0 * a.N + n0, a.N, rows, cols);
}

// FP32 router with the reduction cut into slices (the same BF16x3 products,
// flashinfer PR #8363, Summary).  One workgroup per 256x256 output tile and
// reduction slice q (ks slices of kq values): 4 waves in a 2x2 grid of
// 128x128 wave tiles, so every split fragment feeds twice as many MFMAs as in
// the 128x128 kernel above, and every byte loaded into LDS twice as many
// products.  Slice 0 writes its FP32 sum to `out`, slice q > 0 to
// part[q - 1] ([M, N] each); router_fold_kernel then adds the slices in order
// q = 1 .. ks-1, so the result is fixed: a function of (M, N, K), never of the
// device.  Workgroups of one slice are adjacent (an XCD's L2 holds that slice
// of Wr); every X value is loaded by one workgroup.
//
// Steps of 16 values; the operands are loaded in pairs of steps (32 values:
// whole 128-byte rows, the layout of the kernel above) into two pair buffers
// of 64 KB.  Each step is cut in two by its one barrier:
//   region 0: the first half of step kt's MFMAs (fragment set kt%2); the B
//             side of step kt+1 is read and its A side (read in region 1 of
//             step kt-1) split into set (kt+1)%2
//   barrier:  every wave has finished reading step kt+1's B side, and (even
//             steps) the pair holding step kt+2 has landed
//   region 1: on even steps the loads of the pair two ahead (steps kt+4,
//             kt+5) into the buffer of steps kt, kt+1; the second half of the
//             MFMAs; the A side of step kt+2 is read and the B side of step
//             kt+1 split
// so the reads and the split of a region are independent (the split always
// consumes reads of the region before).  Within a region each MFMA slot
// carries one product, one pair of the split, and one read or one load, in
// that order, fenced so that the compiler keeps the interleave (left to
// itself it clustered the MFMAs and the split and ran no faster than the
// kernel above).
constexpr int kRksBM = 256, kRksBN = 256;

// fn(integral_constant<int, T>) for T = 0, 1, ... in order
template <class Fn, int... T>
__device__ __forceinline__ void for_each_slot(std::integer_sequence<int, T...>, Fn&& fn) {
    (fn(std::integral_constant<int, T>{}), ...);
}

struct RouterKsArgs {
    const float* X;
    const float* Wr;
    float* out;
    float* part;      // (ks - 1) x [M, N] slice sums, slices 1 .. ks-1
    int64_t M, N, K;
    int64_t kq;       // reduction values per slice (a multiple of 16)
};

__global__ __launch_bounds__(256) void router_ks_kernel(RouterKsArgs a) {
    constexpr int BM = kRksBM, BN = kRksBN, KV = 16;   // 16-value steps in 32-value pairs
    __shared__ __attribute__((aligned(256))) char sa0[BM * 128], sa1[BM * 128];
    __shared__ __attribute__((aligned(256))) char sb0[BN * 128], sb1[BN * 128];
    lds_t* const sa[2] = {(lds_t*)sa0, (lds_t*)sa1};
    lds_t* const sb[2] = {(lds_t*)sb0, (lds_t*)sb1};
    using Mma = RouterMma<BM, BN, 4>;
    using LA = F32StageLoader<BM, 4>;
    using LB = F32StageLoader<BN, 4>;
    constexpr int C2 = LA::kPerWave + LB::kPerWave;   // loads per wave per pair

    const int64_t ntn = (a.N + BN - 1) / BN, tiles = ((a.M + BM - 1) / BM) * ntn;
    const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t q = w / tiles, t = w % tiles;
    const int64_t m0 = (t / ntn) * BM, n0 = (t % ntn) * BN, k0 = q * a.kq;
    const int32_t rows = (int32_t)min<int64_t>(BM, a.M - m0);
    const int32_t cols = (int32_t)min<int64_t>(BN, a.N - n0);
    const int32_t klen = (int32_t)max<int64_t>(0, min<int64_t>(a.kq, a.K - k0));
    LA la;
    LB lb;
    la.init(a.X + m0 * a.K + k0, a.K, rows, klen);
    lb.init(a.Wr + n0 * a.K + k0, a.K, cols, klen);
    const int nk = (klen + KV - 1) / KV;
    const int nkS = ((nk + 3) / 4) * 4;
    Mma mma;
    la.issue(sa[0], 0);
    lb.issue(sb[0], 0);
    la.issue(sa[1], 1);
    lb.issue(sb[1], 1);
    wait_vm_lgkm<C2>();
    barrier_nofence();
    mma.template read_side<0>(sa[0], 0);
    mma.template read_side<1>(sb[0], 0);
    mma.template split_side<0, 0>();
    mma.template split_side<0, 1>();
    mma.template read_side<0>(sa[0], 1);
    mma.zero();
    constexpr int HALF = Mma::kMfmas / 2;
    static_assert(HALF == 24 && Mma::kBI == 4 && Mma::kBJ == 4 && C2 == 16, "the slot plan below");
    auto region = [&](auto f_tag, auto r_tag, auto t_tag, auto h_tag, auto ld_tag, const lds_t* rbuf, lds_t* lda,
                      lds_t* ldb, int lpair) __attribute__((always_inline)) {
        constexpr int F = decltype(f_tag)::value, R = decltype(r_tag)::value, T = decltype(t_tag)::value;
        constexpr int H = decltype(h_tag)::value, LD = decltype(ld_tag)::value;
        constexpr int SPLIT_SIDE = R == 0 ? 0 : 1, READ_SIDE = R == 0 ? 1 : 0;
        mma.template mfma_one<F, R * HALF + T>();
        if constexpr (T < 16) mma.template split_one<F ^ 1, SPLIT_SIDE, T / 4, T % 4>();
        if constexpr (T < 8) mma.template read_one<READ_SIDE, T / 2, T % 2>(rbuf, H);
        if constexpr (R == 1 && LD && T >= 8) {
            if constexpr (T < 16) la.issue_one(lda, lpair, T - 8);
            else lb.issue_one(ldb, lpair, T - 16);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto run_region = [&](auto f_tag, auto r_tag, auto h_tag, auto ld_tag, const lds_t* rbuf, lds_t* lda,
                          lds_t* ldb, int lpair) __attribute__((always_inline)) {
        for_each_slot(std::make_integer_sequence<int, HALF>{}, [&](auto t_tag) __attribute__((always_inline)) {
            region(f_tag, r_tag, t_tag, h_tag, ld_tag, rbuf, lda, ldb, lpair);
        });
    };
    auto step = [&](auto st_tag, int kt) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_tag)::value, F = ST & 1;
        constexpr int P1 = ((ST + 1) / 2) % 2, H1 = (ST + 1) % 2, P2 = ((ST + 2) / 2) % 2, H2 = (ST + 2) % 2;
        constexpr int LD = (ST % 2) == 0, PB = ST / 2;
        __builtin_amdgcn_sched_barrier(0);
        run_region(std::integral_constant<int, F>{}, std::integral_constant<int, 0>{}, std::integral_constant<int, H1>{},
                   std::integral_constant<int, 0>{}, sb[P1], sa[PB], sb[PB], 0);
        if constexpr (LD) wait_vm_lgkm<0>();
        else wait_vm_lgkm<C2>();
        barrier_nofence();
        run_region(std::integral_constant<int, F>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, H2>{},
                   std::integral_constant<int, LD>{}, sa[P2], sa[PB], sb[PB], kt / 2 + 2);
    };
    for (int kt = 0; kt < nkS; kt += 4) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
        step(std::integral_constant<int, 2>{}, kt + 2);
        step(std::integral_constant<int, 3>{}, kt + 3);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the masked loads past the end
    float* dst = q == 0 ? a.out : a.part + (q - 1) * a.M * a.N;
    store_tile<false>(mma, dst + m0 * a.N + n0, a.N, rows, cols);
}

// out += part[0], then += part[1], ... (the reduction slices in order), four
// values per thread; n4 = M * N / 4 (N is a multiple of 4).
__global__ __launch_bounds__(kThreads) void router_fold_kernel(float* out, const float* part, int64_t n4,
                                                               int32_t nparts) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
        f32x4 s = reinterpret_cast<const f32x4*>(out)[i];
        for (int p = 0; p < nparts; ++p) {
            const f32x4 v = reinterpret_cast<const f32x4*>(part)[p * n4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] += v[j];
        }
        reinterpret_cast<f32x4*>(out)[i] = s;
    }
}

// ---------------------------------------------------------------------------
// host launchers (called from api.cpp)

template <int OP, int BM, int BN>
static hipError_t launch_fwd_dgrad_t(const GemmArgs& a, bool bf16, hipStream_t s) {
    // two waves per SIMD for the 256x256 tile, one otherwise
    constexpr int WAVES = (BM == 256 && BN == 256) ? 8 : 4;
    dim3 grid((unsigned)a.items_max), block(64 * WAVES);
    timing_mark(OP == 0 ? "gg_fwd_kernel" : "gg_dgrad_kernel", s);
    if (bf16) hipLaunchKernelGGL((gg_fwd_dgrad_kernel<OP, BM, BN, true, WAVES>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gg_fwd_dgrad_kernel<OP, BM, BN, false, WAVES>), grid, block, 0, s, a);
    timing_end(s);
    return hipGetLastError();
}

template <int OP>
static hipError_t launch_fwd_dgrad_op(int tile, const GemmArgs& a, bool bf16, hipStream_t s) {
    switch (tile) {
        case kTile128x128: return launch_fwd_dgrad_t<OP, 128, 128>(a, bf16, s);
        case kTile256x128: return launch_fwd_dgrad_t<OP, 256, 128>(a, bf16, s);
        case kTile128x256: return launch_fwd_dgrad_t<OP, 128, 256>(a, bf16, s);
        default: return launch_fwd_dgrad_t<OP, 256, 256>(a, bf16, s);
    }
}

hipError_t launch_fwd_dgrad(int op, int tile, const GemmArgs& a, bool bf16, hipStream_t s) {
    if (op == 0) return launch_fwd_dgrad_op<0>(tile, a, bf16, s);
    if (op == 1) return launch_fwd_dgrad_op<1>(tile, a, bf16, s);
    return launch_fwd_dgrad_op<2>(tile, a, bf16, s);
}

hipError_t launch_transpose_w(const uint16_t* W, uint16_t* WT, int32_t E, int64_t N, int64_t K, hipStream_t s) {
    dim3 grid((unsigned)((K + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)E), block(kThreads);
    timing_mark("gg_transpose_w_kernel", s);
    hipLaunchKernelGGL(gg_transpose_w_kernel, grid, block, 0, s, W, WT, N, K);
    return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_wgrad_det_t(const GemmArgs& a, bool bf16, hipStream_t s) {
    if (a.items_max > 0) {
        dim3 grid((unsigned)a.items_max), block(64 * wgrad_det_waves<BM, BN>());
        timing_mark("gg_wgrad_det_kernel", s);
        if (bf16) hipLaunchKernelGGL((gg_wgrad_det_kernel<BM, BN, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gg_wgrad_det_kernel<BM, BN, false>), grid, block, 0, s, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (a.zero_empty && a.items_max > 0) {   // nothing to fold (see zero_empty)
        timing_end(s);
        return hipSuccess;
    }
    const int64_t nk = a.N * a.K;
    dim3 fgrid((unsigned)((nk + kThreads * 8 - 1) / (kThreads * 8)), (unsigned)a.E);
    timing_mark("gg_wgrad_fold_kernel", s);
    if (bf16) hipLaunchKernelGGL(gg_wgrad_fold_kernel<true>, fgrid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(gg_wgrad_fold_kernel<false>, fgrid, dim3(kThreads), 0, s, a);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_wgrad_det(int tile, const GemmArgs& a, bool bf16, hipStream_t s) {
    switch (tile) {
        case kTile128x128: return launch_wgrad_det_t<128, 128>(a, bf16, s);
        case kTile256x128: return launch_wgrad_det_t<256, 128>(a, bf16, s);
        case kTile128x256: return launch_wgrad_det_t<128, 256>(a, bf16, s);
        case kTile64x256: return launch_wgrad_det_t<64, 256>(a, bf16, s);
        default: return launch_wgrad_det_t<256, 256>(a, bf16, s);
    }
}

template <int BM, int BN>
static hipError_t launch_wgrad_atomic_t(const GemmArgs& a, int64_t grid_n, bool bf16, hipStream_t s) {
    dim3 grid((unsigned)grid_n), block(kGemmThreads);
    timing_mark("gg_wgrad_atomic_kernel", s);
    if (bf16) hipLaunchKernelGGL((gg_wgrad_atomic_kernel<BM, BN, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gg_wgrad_atomic_kernel<BM, BN, false>), grid, block, 0, s, a);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_wgrad_atomic(int tile, const GemmArgs& a, int64_t grid_n, bool bf16, hipStream_t s) {
    switch (tile) {
        case kTile128x128: return launch_wgrad_atomic_t<128, 128>(a, grid_n, bf16, s);
        case kTile256x128: return launch_wgrad_atomic_t<256, 128>(a, grid_n, bf16, s);
        case kTile128x256: return launch_wgrad_atomic_t<128, 256>(a, grid_n, bf16, s);
        case kTile64x256: return launch_wgrad_atomic_t<64, 256>(a, grid_n, bf16, s);
        default: return launch_wgrad_atomic_t<256, 256>(a, grid_n, bf16, s);
    }
}

hipError_t launch_router(const float* X, const float* Wr, float* out, int64_t M, int64_t N, int64_t K,
                         hipStream_t s) {
    RouterArgs a{X, Wr, out, M, N, K};
    const int64_t tiles = ((M + kRouterBM - 1) / kRouterBM) * ((N + kRouterBN - 1) / kRouterBN);
    timing_mark("router_bf16x3_kernel", s);
    hipLaunchKernelGGL(router_bf16x3_kernel, dim3((unsigned)tiles), dim3(64 * kRouterWaves), 0, s, a);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_router_ks(const float* X, const float* Wr, float* out, float* part, int64_t M, int64_t N,
                            int64_t K, int64_t ks, int64_t kq, hipStream_t s) {
    RouterKsArgs a{X, Wr, out, part, M, N, K, kq};
    const int64_t tiles = ((M + kRksBM - 1) / kRksBM) * ((N + kRksBN - 1) / kRksBN);
    timing_mark("router_ks_kernel", s);
    hipLaunchKernelGGL(router_ks_kernel, dim3((unsigned)(tiles * ks)), dim3(256), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || ks <= 1) {
        timing_end(s);
        return err;
    }
    const int64_t n4 = M * N / 4;
    const int64_t blocks = std::min<int64_t>((n4 + kThreads - 1) / kThreads, 4096);
    timing_mark("router_fold_kernel", s);
    hipLaunchKernelGGL(router_fold_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, out, part, n4,
                       (int32_t)(ks - 1));
    timing_end(s);
    return hipGetLastError();
}

// Calibration aid: each workgroup takes (almost) all of one CU's LDS, so n
// workgroups hold n CUs, and waits (sleeping) until `ticks` of the 100 MHz
// real-time counter have passed, then exits.
constexpr int kHoldLds = 160 * 1024 - 1024;
__global__ __launch_bounds__(64) void hold_cus_kernel(uint64_t ticks) {
    __shared__ char pad[kHoldLds];
    pad[threadIdx.x] = 0;   // keeps the allocation
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
    if (pad[(threadIdx.x + 1) & 63] != 0) pad[0] = 1;
}

hipError_t launch_hold_cus(int n, uint64_t ticks, hipStream_t s) {
    hipLaunchKernelGGL(hold_cus_kernel, dim3((unsigned)n), dim3(64), 0, s, ticks);
    return hipGetLastError();
}

// Fill kernel for workspace initialisation (a kernel rather than a memset so
// that the call can be captured into a HIP graph and replayed).
__global__ void zero_kernel(uint8_t* p, size_t bytes) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 16;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; i < bytes; i += stride) {
        if (i + 16 <= bytes && (((uintptr_t)(p + i)) & 15) == 0) {
            *reinterpret_cast<u32x4*>(p + i) = u32x4{0, 0, 0, 0};
        } else {
            for (size_t j = i; j < i + 16 && j < bytes; ++j) p[j] = 0;
        }
    }
}

// Workspace of the entry point that allocates nothing
// (grouped_gemm_wgrad_noalloc): a fixed array in device memory, one copy per
// device that runs the library's kernels, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not the device array, so
// it is never passed to a kernel: scratch_buffer looks up the device address
// of the current device's copy once (hipGetSymbolAddress, with that device
// current) and every later use goes through that address.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_buffer(void** ptr) {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static void* addr[kDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    size_t blocks = (bytes + kThreads * 16 - 1) / (kThreads * 16);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, static_cast<uint8_t*>(p), bytes);
    return hipGetLastError();
}

}  // namespace drgg
