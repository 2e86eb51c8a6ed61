// kernels.hip -- gfx950 (CDNA4) kernels of the ragged BF16 grouped GEMM.
//
// Programs (flashinfer PR #8258, "run the split k512 wgrad tail whole on the
// least-loaded clusters on sm_107a", opening summary paragraph):
//   forward          Y[t,n]    = sum_k X[t,k]   W[e(t),n,k]
//   data gradient    dX[t,k]   = sum_n G[t,n]   W[e(t),n,k]
//   weight gradient  dW[e,n,k] = sum_{t of e} G[t,n] X[t,k]
// with FP32 accumulation on v_mfma_f32_32x32x16_bf16 and one rounding.
//
// One workgroup = 4 waves (256 lanes) computes one BMxBN output tile; the
// waves form a 2x2 grid, each wave a (BM/2)x(BN/2) block of 32x32 MFMA tiles
// whose FP32 accumulators stay in registers for the whole reduction.
//
// Operand staging.  The reduction runs in steps of 64.  For each step the
// workgroup loads an A tile (BM x 64) and a B tile (BN x 64) from HBM with
// 16-byte loads into registers, and writes them to LDS in one layout for all
// programs: "K-major" rows of 64 reduction values (128 bytes), whose eight
// 16-byte chunks are XOR-swizzled by the row index so that the MFMA operand
// reads (32 rows, one chunk) and the tile writes hit distinct banks.  Two
// LDS buffers alternate: while the MFMAs consume one step, the next step's
// global loads are in flight and land in the other buffer.
//   * K-major operands (reduction index contiguous in memory: X and W in the
//     forward, G in the data gradient) are copied chunk for chunk.
//   * MN-major operands (reduction index strided: W in the data gradient, G
//     and X in the weight gradient, whose reduction runs over tokens) are
//     loaded as 8x8 blocks -- eight rows of 8 consecutive output indices --
//     and transposed in registers (32 byte permutes) before the LDS write, so
//     the LDS tile is K-major again and the inner loop is the same MFMA code
//     for every program.
//
// Ragged groups.  Every workgroup reads the group offsets, clamps them into
// [0, M] and builds the per-expert prefix of work items in LDS; a work index
// is then mapped to (expert, tile, chunk) by binary search.  Out-of-range
// rows are never loaded from outside the buffers: row indices are clamped to
// the last valid row and reduction positions outside the range are replaced
// by zeros after the load.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"
#include "plan.hpp"

namespace drgg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;       // fold / zero / router kernels
constexpr int kGemmThreads = 512;   // grouped-GEMM kernels: 8 waves

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

// 16-byte chunk swizzle of an LDS row (8 chunks of 8 BF16 per 128-byte row).
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kTileK + ((chunk ^ swz(row)) << 3);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st_lds16(uint16_t* s, int off, u32x4 v) {
    *reinterpret_cast<u32x4*>(s + off) = v;
}

__device__ __forceinline__ bf16x8 ld_lds_frag(const uint16_t* s, int off) {
    return *reinterpret_cast<const bf16x8*>(s + off);
}

// ---------------------------------------------------------------------------
// ragged work decode

struct Sched {
    int32_t offs[kMaxExperts + 1];    // clamped, non-decreasing offsets
    int32_t prefix[kMaxExperts + 1];  // exclusive prefix of work per expert
    int32_t scan[kGemmThreads];
};

// Fills s.offs[0..E] with the offsets clamped into [0, M] (and made
// non-decreasing), and s.prefix[0..E] with the exclusive prefix of
// work(e, T_e).  Must be called by all threads; ends with a barrier.
template <class WorkFn>
__device__ void build_schedule(Sched& s, const int32_t* __restrict__ offs, int E, int64_t M,
                               WorkFn work) {
    const int tid = threadIdx.x;
    for (int e = tid; e <= E; e += kGemmThreads) {
        int64_t v = offs[e];
        v = v < 0 ? 0 : (v > M ? M : v);
        s.offs[e] = (int32_t)v;
    }
    __syncthreads();
    // make non-decreasing (a running max); E <= 1024, one pass per thread chunk
    const int per = (E + kGemmThreads) / kGemmThreads;   // covers indices 0..E
    const int lo = tid * per;
    const int hi = min(lo + per, E + 1);
    int32_t run = 0;
    for (int i = lo; i < hi; ++i) run = max(run, s.offs[i]);
    s.scan[tid] = run;
    __syncthreads();
    for (int d = 1; d < kGemmThreads; d <<= 1) {
        int32_t v = tid >= d ? s.scan[tid - d] : 0;
        __syncthreads();
        s.scan[tid] = max(s.scan[tid], v);
        __syncthreads();
    }
    int32_t carry = tid > 0 ? s.scan[tid - 1] : 0;
    __syncthreads();
    for (int i = lo; i < hi; ++i) {
        carry = max(carry, s.offs[i]);
        s.offs[i] = carry;
    }
    __syncthreads();
    // work counts and their exclusive prefix
    int32_t local = 0;
    for (int e = lo; e < hi && e < E; ++e) local += work(e, s.offs[e + 1] - s.offs[e]);
    s.scan[tid] = local;
    __syncthreads();
    for (int d = 1; d < kGemmThreads; d <<= 1) {
        int32_t v = tid >= d ? s.scan[tid - d] : 0;
        __syncthreads();
        s.scan[tid] += v;
        __syncthreads();
    }
    int32_t acc = tid > 0 ? s.scan[tid - 1] : 0;
    for (int e = lo; e < hi; ++e) {
        s.prefix[e] = acc;
        if (e < E) acc += work(e, s.offs[e + 1] - s.offs[e]);
    }
    __syncthreads();
}

// Values read from LDS arrive in vector registers even when every lane reads
// the same address; the tile decode is wave-uniform, so it is moved to scalar
// registers (keeps the per-tile state out of the VGPR budget).
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Largest e with prefix[e] <= w (so that prefix[e] <= w < prefix[e+1]).
__device__ __forceinline__ int find_expert(const Sched& s, int E, int32_t w) {
    int lo = 0, hi = E;   // answer in [0, E)
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s.prefix[mid] <= w) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// The deterministic weight gradient's chunk rule (device side of
// wgrad_chunking in plan.hpp).
__device__ __forceinline__ int32_t chunk_len_dev(int32_t T, int64_t chunk_max) {
    if (T <= 0) return 0;
    int64_t s = (T + chunk_max - 1) / chunk_max;
    int64_t l = (T + s - 1) / s;
    return (int32_t)(((l + kTileK - 1) / kTileK) * kTileK);
}
__device__ __forceinline__ int32_t chunks_dev(int32_t T, int64_t chunk_max) {
    int32_t l = chunk_len_dev(T, chunk_max);
    return l ? (T + l - 1) / l : 0;
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

// LDS pointers keep their address space in the type, so that every access
// compiles to ds_* instructions (a generic pointer would become a flat access
// that also waits for outstanding global loads).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// Buffer descriptor over [base, base + 2 GB): raw (stride 0) addressing with
// range checking.  A lane whose offset is kOOB lies past the range, and its
// load writes zeros to LDS; this is how every mask below is applied.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFF0, 0x00020000);
}
constexpr uint32_t kOOB = 0xFFFFFFF0u;

// LDS layouts of one 64-wide reduction step ("stage"):
//   K-major:  ROWS rows of 64 reduction values (128 B = 8 chunks of 16 B);
//             chunk c of row r sits at c ^ swzK(r).  The MFMA operand reads
//             (16 lanes = 16 consecutive rows, one chunk) then hit 16
//             distinct 16-byte bank groups.
//   MN-major: 64 rows (reduction index) of ROWS output indices
//             (ROWS*2 B = CPR chunks); chunk c of row r sits at
//             c ^ swzMN(r).  The XOR is even, so the two chunks a group of
//             four lanes reads stay adjacent, and the 16 row segments of one
//             transposed read spread over all banks in two passes.
__device__ __forceinline__ int swzK(int row) { return (row & 7) ^ ((row >> 3) & 1); }
template <int CPR>
__device__ __forceinline__ int swzMN(int row) {
    return (2 * ((row & 3) + 4 * ((row >> 3) & 1))) & (CPR - 2);
}

// Loads one stage of an operand straight from HBM into LDS with 16-byte
// buffer loads (no registers in between).  A stage is ROWS*128 bytes =
// ROWS/8 wave instructions of 1 KB; each of the 8 waves issues ROWS/64 of
// them.  Lane l of instruction g writes LDS bytes [g*1024 + 16*l, +16); the
// swizzle is applied by choosing which global chunk the lane fetches.
template <int ROWS, bool KMAJ>
struct LdsLoader {
    static constexpr int kPerWave = ROWS / 64;
    static constexpr int kRowBytes = KMAJ ? 128 : ROWS * 2;
    static constexpr int kCPR = kRowBytes / 16;
    static_assert(ROWS % 64 == 0, "tile rows must be a multiple of 64");
    uint32_t off[kPerWave];   // byte offset of this lane's 16 bytes from the step base (kOOB if masked)
    int64_t step_bytes;       // byte distance between consecutive steps
    const char* base;
    int32_t klen;

    __device__ __forceinline__ void init(const Operand& op) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        base = reinterpret_cast<const char*>(op.base);
        klen = op.klen;
        step_bytes = KMAJ ? 128 : 64 * op.ld * 2;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int b = (wave * kPerWave + i) * 1024 + lane * 16;
            const int row = b / kRowBytes, phys = (b % kRowBytes) / 16;
            if constexpr (KMAJ) {
                const int logical = phys ^ swzK(row);
                off[i] = row < op.nvalid ? (uint32_t)(row * op.ld * 2 + logical * 16) : kOOB;
            } else {
                const int logical = phys ^ swzMN<kCPR>(row);
                const int col = logical * 8;
                off[i] = col < op.nvalid ? (uint32_t)(row * op.ld * 2 + col * 2) : kOOB;
            }
        }
    }

    // reduction position, within a step, of the 16 bytes instruction i loads
    __device__ __forceinline__ int kpos(int i) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int b = (wave * kPerWave + i) * 1024 + lane * 16;
        const int row = b / kRowBytes, phys = (b % kRowBytes) / 16;
        if constexpr (KMAJ) return (phys ^ swzK(row)) * 8;
        else return row;
    }

    // Issue the loads of reduction step kt into `stage`.  With TAIL, positions
    // at or past klen are masked.
    template <bool TAIL>
    __device__ __forceinline__ void issue(lds_t* stage, int kt) const {
        const int wave = threadIdx.x >> 6;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base + kt * step_bytes);
        const int rem = klen - kt * 64;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            uint32_t o = off[i];
            if constexpr (TAIL) o = kpos(i) < rem ? o : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void_t*)(stage + (wave * kPerWave + i) * 1024), 16, o, 0, 0, 0);
        }
    }
};

// MFMA operand fragment: lane l gets the 8 reduction values 16*s + 8*(l/32)
// .. +7 of tile row rb + (l & 31).
template <int ROWS, bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const lds_t* stage, int rb, int s) {
    const int l = threadIdx.x & 63;
    if constexpr (KMAJ) {
        const int row = rb + (l & 31), c = 2 * s + (l >> 5);
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            stage + row * 128 + ((c ^ swzK(row)) << 4));
    } else {
        // ds_read_b64_tr_b16: in a group of 16 lanes, lane 4j+q addresses
        // 4 values of row kbase+j at column col0+4q; lane i receives column
        // col0+i of rows kbase..kbase+3.
        constexpr int CPR = ROWS * 2 / 16;
        const int g = l >> 4, j = (l >> 2) & 3, q = l & 3;
        const int col = rb + 16 * (g & 1) + 4 * q;
        const int chunk = col >> 3, within = (col & 7) * 2;
        const int k0 = 16 * s + 8 * (g >> 1) + j;
        const int r0 = k0, r1 = k0 + 4;
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(stage + r0 * ROWS * 2 + ((chunk ^ swzMN<CPR>(r0)) << 4) + within));
        v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(stage + r1 * ROWS * 2 + ((chunk ^ swzMN<CPR>(r1)) << 4) + within));
        v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
}

// One BMxBN output tile on 8 waves: the waves form a 2x4 grid, each owning a
// (BM/2)x(BN/4) block of 32x32 MFMA tiles whose accumulators stay in
// registers.  Two LDS stages alternate: after the barrier that ends step
// kt-1, the loads of step kt+1 go out into the free stage while the MFMAs
// consume step kt.
template <int BM, int BN, bool AK, bool BK>
struct TileMma {
    static constexpr int WM = BM / 2, WN = BN / 4;
    static constexpr int kBI = WM / 32, kBJ = WN / 32;
    static constexpr int kStageA = BM * 128, kStageB = BN * 128;
    static constexpr int kLdsBytes = 2 * (kStageA + kStageB);
    static_assert(kBI >= 1 && kBJ >= 1, "tile too small for the 2x4 wave grid");
    f32x16 acc[kBI][kBJ];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    __device__ __forceinline__ void compute(const lds_t* sA, const lds_t* sB) {
        const int wave = threadIdx.x >> 6;
        const int ra = (wave >> 2) * WM, rb = (wave & 3) * WN;
        bf16x8 a[2][kBI], b[2][kBJ];
#pragma unroll
        for (int i = 0; i < kBI; ++i) a[0][i] = read_frag<BM, AK>(sA, ra + 32 * i, 0);
#pragma unroll
        for (int j = 0; j < kBJ; ++j) b[0][j] = read_frag<BN, BK>(sB, rb + 32 * j, 0);
        // The scheduling fences keep this order: the operand reads of step
        // s+1 are issued before the MFMAs of step s, so their LDS latency
        // hides behind those MFMAs instead of stalling each MFMA pair.
#pragma unroll
        for (int s = 0; s < kTileK / kMfmaK; ++s) {
            const int cur = s & 1;
            if (s + 1 < kTileK / kMfmaK) {
#pragma unroll
                for (int i = 0; i < kBI; ++i) a[cur ^ 1][i] = read_frag<BM, AK>(sA, ra + 32 * i, s + 1);
#pragma unroll
                for (int j = 0; j < kBJ; ++j) b[cur ^ 1][j] = read_frag<BN, BK>(sB, rb + 32 * j, s + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kBI; ++i)
#pragma unroll
                for (int j = 0; j < kBJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Visit every accumulator element: f(row, col, value) with (row, col)
    // inside the tile.  For a fixed register, lanes 0..31 hold 32 consecutive
    // columns of one row, so stores from here are 64- or 128-byte runs.
    template <class F>
    __device__ __forceinline__ void for_each(F f) const {
        int lane = threadIdx.x & 63;
        // The (row, col) of each register does not depend on the tile; an
        // opaque copy of the lane index keeps the compiler from hoisting all
        // of them out of the persistent tile loop, where they would occupy
        // registers for its whole length.
        asm volatile("" : "+v"(lane));
        const int wave = threadIdx.x >> 6;
        const int ra = (wave >> 2) * WM, rb = (wave & 3) * WN;
#pragma unroll
        for (int i = 0; i < kBI; ++i)
#pragma unroll
            for (int j = 0; j < kBJ; ++j) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    f(ra + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), rb + 32 * j + (lane & 31),
                      acc[i][j][r]);
                // one block at a time: keeps the store addresses of the
                // other blocks from occupying registers
                __builtin_amdgcn_sched_barrier(0);
            }
    }
};

// One tile of work for the persistent driver: the two operand views and the
// kernel's own output coordinates.
struct TileInfo {
    Operand A, B;
    int64_t o0, o1;      // output row / column base (kernel specific)
    int32_t rows, cols;  // valid output rows / columns of the tile
    int32_t e, aux, aux2;  // expert and kernel-specific tags
};

// Persistent tile loop.  `more()` tells whether this workgroup has another
// tile and `next(t)` decodes it; `finish(t, mma)` writes a finished tile from
// the accumulators.  Reduction steps of consecutive tiles form one stream
// over the two LDS stages: during the last step of a tile the first step of
// the next tile is already loading, so neither the pipeline fill nor the
// epilogue of a tile is exposed.  The next tile is decoded only at that last
// step, so its description does not occupy registers during the loop.  Must
// be called by all threads.
template <int BM, int BN, bool AK, bool BK, class More, class Next, class Finish>
__device__ __forceinline__ void run_tiles(lds_t* lds, More more, Next next, Finish finish) {
    using Mma = TileMma<BM, BN, AK, BK>;
    Mma mma;
    LdsLoader<BM, AK> la;
    LdsLoader<BN, BK> lb;
    lds_t* const sA0 = lds;
    lds_t* const sB0 = lds + 2 * Mma::kStageA;
    if (!more()) return;
    TileInfo cur;
    next(cur);
    la.init(cur.A);
    lb.init(cur.B);
    int stage = 0;
    if (cur.A.klen >= kTileK) {
        la.template issue<false>(sA0, 0);
        lb.template issue<false>(sB0, 0);
    } else {
        la.template issue<true>(sA0, 0);
        lb.template issue<true>(sB0, 0);
    }
    for (;;) {
        const int nk = (cur.A.klen + kTileK - 1) / kTileK;   // >= 1
        const int nfull = cur.A.klen / kTileK;
        const bool has_next = more();
        TileInfo nxt;
        mma.zero();
        for (int kt = 0; kt < nk; ++kt) {
            __builtin_amdgcn_s_waitcnt(0);   // this lane's loads of step kt have landed
            __syncthreads();                 // everyone's; and the other stage is free
            lds_t* const nA = sA0 + (stage ^ 1) * Mma::kStageA;
            lds_t* const nB = sB0 + (stage ^ 1) * Mma::kStageB;
            if (kt + 1 < nfull) {
                la.template issue<false>(nA, kt + 1);
                lb.template issue<false>(nB, kt + 1);
            } else if (kt + 1 < nk) {
                la.template issue<true>(nA, kt + 1);
                lb.template issue<true>(nB, kt + 1);
            } else if (has_next) {
                next(nxt);
                la.init(nxt.A);
                lb.init(nxt.B);
                if (nxt.A.klen >= kTileK) {
                    la.template issue<false>(nA, 0);
                    lb.template issue<false>(nB, 0);
                } else {
                    la.template issue<true>(nA, 0);
                    lb.template issue<true>(nB, 0);
                }
            }
            mma.compute(sA0 + stage * Mma::kStageA, sB0 + stage * Mma::kStageB);
            stage ^= 1;
        }
        finish(cur, mma);
        if (!has_next) break;
        cur = nxt;
    }
}

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
// forward / data gradient (identical in both variants)
//
// Persistent: workgroup b of G takes work items xcd_remap(b) + i*G, so at any
// time the 32 workgroups of one XCD work on 32 consecutive output tiles (the
// tiles of a few 256-row panels), which share operand slabs in that XCD's L2.

template <int OP, int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gg_fwd_dgrad_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[TileMma<BM, BN, true, OP == 0>::kLdsBytes];
    __shared__ Sched sch;
    // output columns: N (forward) or K (data gradient)
    const int64_t ncols = OP == 0 ? a.N : a.K;
    const int32_t ntn = (int32_t)((ncols + BN - 1) / BN);
    build_schedule(sch, a.offs, a.E, a.M,
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
            t.A = Operand{a.A + t0 * a.K, a.K, t.rows, (int32_t)a.K};
            t.B = Operand{We + c0 * a.K, a.K, t.cols, (int32_t)a.K};
        } else {                   // dX = G W: W is [n][k], reduction n strided
            t.A = Operand{a.A + t0 * a.N, a.N, t.rows, (int32_t)a.N};
            t.B = Operand{We + c0, a.K, t.cols, (int32_t)a.N};
        }
        w += G;
    };
    void* out = a.out;
    auto finish = [&](const TileInfo& t, const TileMma<BM, BN, true, OP == 0>& mma) {
        mma.for_each([&](int r, int c, float v) {
            if (r < t.rows && c < t.cols) store1<OUT_BF16>(out, (t.o0 + r) * ncols + t.o1 + c, v);
        });
    };
    run_tiles<BM, BN, true, OP == 0>((lds_t*)lds, more, next, finish);
}

// ---------------------------------------------------------------------------
// deterministic weight gradient: chunk partials (K3) and ordered fold (K4)

template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gg_wgrad_det_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[TileMma<BM, BN, false, false>::kLdsBytes];
    __shared__ Sched sch;
    __shared__ int32_t slot_base[kMaxExperts + 1];
    const int32_t tn = (int32_t)((a.N + BM - 1) / BM), tk = (int32_t)((a.K + BN - 1) / BN);
    const int32_t P = tn * tk;
    const int64_t cmax = a.chunk_max;
    build_schedule(sch, a.offs, a.E, a.M,
                   [=](int, int32_t T) { return P * chunks_dev(T, cmax); });
    // partial slots: experts cut into more than one chunk, in expert order
    if (threadIdx.x == 0) {
        int32_t sb = 0;
        for (int x = 0; x < a.E; ++x) {
            slot_base[x] = sb;
            const int32_t c = chunks_dev(sch.offs[x + 1] - sch.offs[x], cmax);
            if (c > 1) sb += c;
        }
        slot_base[a.E] = sb;
    }
    __syncthreads();
    const int64_t total = uni(sch.prefix[a.E]);
    const int64_t G = gridDim.x;
    int64_t w = xcd_remap(blockIdx.x, G);
    if (a.reverse) w = G - 1 - w;
    auto more = [&]() { return w < total; };
    auto next = [&](TileInfo& t) {
        const int e = uni(find_expert(sch, a.E, (int32_t)w));
        const int32_t oe = uni(sch.offs[e]), oe1 = uni(sch.offs[e + 1]);
        const int32_t T = oe1 - oe;
        const int32_t clen = chunk_len_dev(T, cmax);
        const int32_t nch = (T + clen - 1) / clen;
        const int32_t local = (int32_t)w - uni(sch.prefix[e]);
        const int32_t chunk = local / P, tile = local % P;   // chunk-major: tiles of a chunk adjacent
        const int32_t ti = tile / tk, tj = tile % tk;
        const int64_t n0 = (int64_t)ti * BM, k0 = (int64_t)tj * BN;
        const int64_t tb = oe + (int64_t)chunk * clen;
        const int32_t len = (int32_t)min<int64_t>(clen, oe1 - tb);
        t.o0 = n0;
        t.o1 = k0;
        t.rows = (int32_t)min<int64_t>(BM, a.N - n0);
        t.cols = (int32_t)min<int64_t>(BN, a.K - k0);
        t.e = e;
        t.aux = nch == 1 ? -1 : uni(slot_base[e]) + chunk;   // -1: store the output directly
        // dW[n][k] = sum_t G[t][n] X[t][k]: both operands token-major (MN-major)
        t.A = Operand{a.A + tb * a.N + n0, a.N, t.rows, len};
        t.B = Operand{a.B + tb * a.K + k0, a.K, t.cols, len};
        w += G;
    };
    auto finish = [&](const TileInfo& t, const TileMma<BM, BN, false, false>& mma) {
        if (t.aux < 0) {
            void* out = a.out;
            const int64_t base = (int64_t)t.e * a.N * a.K + t.o0 * a.K + t.o1;
            mma.for_each([&](int r, int c, float v) {
                if (r < t.rows && c < t.cols) store1<OUT_BF16>(out, base + r * a.K + c, v);
            });
        } else {
            float* dst = a.partial + (int64_t)t.aux * a.N * a.K + t.o0 * a.K + t.o1;
            mma.for_each([&](int r, int c, float v) {
                if (r < t.rows && c < t.cols) dst[r * a.K + c] = v;
            });
        }
    };
    run_tiles<BM, BN, false, false>((lds_t*)lds, more, next, finish);
}

// Fold the partials of every expert cut into more than one chunk, in chunk
// order, in FP32, then round once; zero-fill experts without tokens.
// Grid: (ceil(N*K / 2048), E); 256 threads x 8 consecutive elements.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gg_wgrad_fold_kernel(GemmArgs a) {
    const int e = blockIdx.y;
    __shared__ int32_t s_info[3];   // T_e, chunks_e, slot base
    if (threadIdx.x == 0) {
        // clamp like build_schedule: offsets into [0, M], running max
        int64_t run = 0, sb = 0, Te = 0, ce = 0;
        int64_t prev = 0;
        for (int x = 0; x <= e + 1 && x <= a.E; ++x) {
            int64_t v = a.offs[x];
            v = v < 0 ? 0 : (v > a.M ? a.M : v);
            run = v > run ? v : run;
            if (x > 0) {
                const int64_t T = run - prev;
                const int32_t c = chunks_dev((int32_t)T, a.chunk_max);
                if (x - 1 < e && c > 1) sb += c;
                if (x - 1 == e) { Te = T; ce = c; }
            }
            prev = run;
        }
        s_info[0] = (int32_t)Te;
        s_info[1] = (int32_t)ce;
        s_info[2] = (int32_t)sb;
    }
    __syncthreads();
    const int32_t Te = s_info[0], ce = s_info[1], sb = s_info[2];
    if (Te > 0 && ce <= 1) return;   // written directly by the chunk kernel
    const int64_t nk = a.N * a.K;
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
    if (i0 >= nk) return;            // nk is a multiple of 8
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
        for (int c = 1; c < ce; ++c) {
            p += nk;
            x0 = *reinterpret_cast<const f32x4*>(p);
            x1 = *reinterpret_cast<const f32x4*>(p + 4);
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
// non-deterministic weight gradient: stream-K over 512-token units with an
// atomic FP32 tile sum and a last-arrival ticket for split tiles

template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gg_wgrad_streamk_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[TileMma<BM, BN, false, false>::kLdsBytes];
    __shared__ Sched sch;
    __shared__ int32_t s_last;
    const int32_t tn = (int32_t)((a.N + BM - 1) / BM), tk = (int32_t)((a.K + BN - 1) / BN);
    const int32_t P = tn * tk;
    build_schedule(sch, a.offs, a.E, a.M, [=](int, int32_t T) {
        return P * (int32_t)((T + kStreamKUnit - 1) / kStreamKUnit);
    });
    const int64_t U = uni(sch.prefix[a.E]);
    const int64_t b = blockIdx.x;
    // Workgroup b of G takes units [b*U/G, (b+1)*U/G).  With G <= U every
    // range is non-empty, so the workgroups touching a tile are exactly
    // owner(first unit) .. owner(last unit).
    const int64_t G = U < (int64_t)gridDim.x ? U : (int64_t)gridDim.x;
    const int64_t u_end = b < G ? (b + 1) * U / G : 0;
    int64_t u = b < G ? b * U / G : 0;
    // the workgroup whose unit range holds unit v
    auto owner = [&](int64_t v) { return ((v + 1) * G - 1) / U; };
    // segments: the part of one tile's unit range inside this workgroup's range
    auto more = [&]() { return u < u_end; };
    auto next = [&](TileInfo& t) {
        const int e = uni(find_expert(sch, a.E, (int32_t)u));
        const int32_t oe = uni(sch.offs[e]), oe1 = uni(sch.offs[e + 1]), pe = uni(sch.prefix[e]);
        const int32_t T = oe1 - oe;
        const int32_t Ue = (int32_t)((T + kStreamKUnit - 1) / kStreamKUnit);
        const int32_t local = (int32_t)(u - pe);
        const int32_t tile = local / Ue, unit = local % Ue;
        const int64_t tile_u0 = pe + (int64_t)tile * Ue;
        const int64_t seg_end = min(u_end, tile_u0 + Ue);
        const int32_t unit_hi = (int32_t)(seg_end - tile_u0);
        const int32_t ti = tile / tk, tj = tile % tk;
        const int64_t n0 = (int64_t)ti * BM, k0 = (int64_t)tj * BN;
        const int64_t tb = oe + (int64_t)unit * kStreamKUnit;
        const int64_t te = min<int64_t>(oe + (int64_t)unit_hi * kStreamKUnit, oe1);
        t.o0 = n0;
        t.o1 = k0;
        t.rows = (int32_t)min<int64_t>(BM, a.N - n0);
        t.cols = (int32_t)min<int64_t>(BN, a.K - k0);
        t.e = e;
        const bool whole = unit == 0 && unit_hi == Ue;
        t.aux = whole ? -1 : tile;
        t.aux2 = whole ? 1 : (int32_t)(owner(tile_u0 + Ue - 1) - owner(tile_u0) + 1);
        t.A = Operand{a.A + tb * a.N + n0, a.N, t.rows, (int32_t)(te - tb)};
        t.B = Operand{a.B + tb * a.K + k0, a.K, t.cols, (int32_t)(te - tb)};
        u = seg_end;
    };
    auto finish = [&](const TileInfo& t, const TileMma<BM, BN, false, false>& mma) {
        const int64_t base = (int64_t)t.e * a.N * a.K + t.o0 * a.K + t.o1;
        void* out = a.out;
        if (t.aux < 0) {   // the whole tile in this workgroup: store directly
            mma.for_each([&](int r, int c, float v) {
                if (r < t.rows && c < t.cols) store1<OUT_BF16>(out, base + r * a.K + c, v);
            });
            return;
        }
        const int64_t slot = (int64_t)t.e * P + t.aux;
        float* ts = a.tilesum + slot * (BM * BN);
        mma.for_each([&](int r, int c, float v) {
            if (r < t.rows && c < t.cols)
                __hip_atomic_fetch_add(ts + r * BN + c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        });
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t old = __hip_atomic_fetch_add(a.tickets + slot, 1u, __ATOMIC_ACQ_REL,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            s_last = (old + 1 == (uint32_t)t.aux2);
        }
        __syncthreads();
        if (s_last) {   // last arrival: read and clear the sum, write the tile
            __threadfence();
            for (int i = threadIdx.x * 4; i < BM * BN; i += kGemmThreads * 4) {
                const int r = i / BN, c = i % BN;
                if (r < t.rows && c < t.cols) {
                    f32x4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[q] = __hip_atomic_load(ts + i + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(ts + i + q, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    store4<OUT_BF16>(out, base + r * a.K + c, v);
                }
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(a.tickets + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    };
    run_tiles<BM, BN, false, false>((lds_t*)lds, more, next, finish);
    // experts without tokens: dW[e] = +0, shared out over the grid
    const int64_t nk = a.N * a.K;
    for (int e = 0; e < a.E; ++e) {
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
// "FP32 router GEMM (256 experts, BF16x3 emulation)").
//   out[m,n] = sum_k X[m,k] Wr[n,k];  v = hi + lo, hi = bf16(v), lo = bf16(v - hi)
//   per 16-step: acc += hi_x hi_w, then hi_x lo_w, then lo_x hi_w.

constexpr int kRouterBM = 128, kRouterBN = 128;

struct RouterArgs {
    const float* X;
    const float* Wr;
    float* out;
    int64_t M, N, K;
};

struct RouterLoader {
    // 128 rows x 64 floats = 1024 chunks of 8 floats; 4 chunks per thread
    f32x4 r[8];
    __device__ __forceinline__ void load(const float* base, int64_t ld, int32_t nvalid, int32_t klen,
                                         int kstep) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = j * kThreads + threadIdx.x;
            const int row = v >> 3, ch = v & 7;
            const int kk = kstep * kTileK + ch * 8;
            const bool ok = kk < klen;
            const int rr = row < nvalid ? row : nvalid - 1;
            const float* p = base + (int64_t)rr * ld + (ok ? kk : 0);
            f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
            f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
            r[2 * j] = ok ? x0 : f32x4{0.f, 0.f, 0.f, 0.f};
            r[2 * j + 1] = ok ? x1 : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ __forceinline__ void store(uint16_t* shi, uint16_t* slo) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = j * kThreads + threadIdx.x;
            u32x4 h, l;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = r[2 * j + (q >> 1)][(q & 1) * 2];
                const float x1 = r[2 * j + (q >> 1)][(q & 1) * 2 + 1];
                const uint16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
                const uint16_t l0 = f32_to_bf16(x0 - bf16_to_f32(h0));
                const uint16_t l1 = f32_to_bf16(x1 - bf16_to_f32(h1));
                h[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                l[q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            const int off = lds_off(v >> 3, v & 7);
            st_lds16(shi, off, h);
            st_lds16(slo, off, l);
        }
    }
};

__global__ __launch_bounds__(kThreads, 1) void router_bf16x3_kernel(RouterArgs a) {
    constexpr int BM = kRouterBM, BN = kRouterBN, TS = BM * kTileK;
    __shared__ __attribute__((aligned(16))) uint16_t sAh[2 * TS], sAl[2 * TS], sBh[2 * TS], sBl[2 * TS];
    const int64_t ntn = (a.N + BN - 1) / BN;
    const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t mt = w / ntn, nt = w % ntn;
    const int64_t m0 = mt * BM, n0 = nt * BN;
    const int32_t rows = (int32_t)min<int64_t>(BM, a.M - m0);
    const int32_t cols = (int32_t)min<int64_t>(BN, a.N - n0);
    const int32_t klen = (int32_t)a.K;
    const float* Xb = a.X + m0 * a.K;
    const float* Wb = a.Wr + n0 * a.K;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (klen + kTileK - 1) / kTileK;
    RouterLoader la, lb;
    la.load(Xb, a.K, rows, klen, 0);
    lb.load(Wb, a.K, cols, klen, 0);
    la.store(sAh, sAl);
    lb.store(sBh, sBl);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(Xb, a.K, rows, klen, kt + 1);
            lb.load(Wb, a.K, cols, klen, kt + 1);
        }
        const uint16_t *ah = sAh + cur * TS, *al = sAl + cur * TS;
        const uint16_t *bh = sBh + cur * TS, *bl = sBl + cur * TS;
#pragma unroll
        for (int ks = 0; ks < kTileK / kMfmaK; ++ks) {
            const int ch = ks * 2 + (lane >> 5);
            bf16x8 xh[2], xl[2], wh[2], wl[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = wm * 64 + i * 32 + (lane & 31);
                const int rb = wn * 64 + i * 32 + (lane & 31);
                xh[i] = ld_lds_frag(ah, lds_off(ra, ch));
                xl[i] = ld_lds_frag(al, lds_off(ra, ch));
                wh[i] = ld_lds_frag(bh, lds_off(rb, ch));
                wl[i] = ld_lds_frag(bl, lds_off(rb, ch));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh[i], wh[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh[i], wl[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl[i], wh[j], acc[i][j], 0, 0, 0);
                }
        }
        if (more) {
            la.store(sAh + (cur ^ 1) * TS, sAl + (cur ^ 1) * TS);
            lb.store(sBh + (cur ^ 1) * TS, sBl + (cur ^ 1) * TS);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = wn * 64 + j * 32 + (lane & 31);
                if (row < rows && col < cols) a.out[(m0 + row) * a.N + n0 + col] = acc[i][j][r];
            }
}

// ---------------------------------------------------------------------------
// host launchers (called from api.cpp)

template <int OP, int BM, int BN>
static hipError_t launch_fwd_dgrad_t(const GemmArgs& a, bool bf16, hipStream_t s) {
    dim3 grid((unsigned)a.items_max), block(kGemmThreads);
    timing_mark(OP == 0 ? "gg_fwd_kernel" : "gg_dgrad_kernel", s);
    if (bf16) hipLaunchKernelGGL((gg_fwd_dgrad_kernel<OP, BM, BN, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gg_fwd_dgrad_kernel<OP, BM, BN, false>), grid, block, 0, s, a);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_fwd_dgrad(int op, int tile, const GemmArgs& a, bool bf16, hipStream_t s) {
    switch (tile) {
        case kTile128x128:
            return op == 0 ? launch_fwd_dgrad_t<0, 128, 128>(a, bf16, s) : launch_fwd_dgrad_t<1, 128, 128>(a, bf16, s);
        case kTile256x128:
            return op == 0 ? launch_fwd_dgrad_t<0, 256, 128>(a, bf16, s) : launch_fwd_dgrad_t<1, 256, 128>(a, bf16, s);
        case kTile128x256:
            return op == 0 ? launch_fwd_dgrad_t<0, 128, 256>(a, bf16, s) : launch_fwd_dgrad_t<1, 128, 256>(a, bf16, s);
        default:
            return op == 0 ? launch_fwd_dgrad_t<0, 256, 256>(a, bf16, s) : launch_fwd_dgrad_t<1, 256, 256>(a, bf16, s);
    }
}

template <int BM, int BN>
static hipError_t launch_wgrad_det_t(const GemmArgs& a, bool bf16, hipStream_t s) {
    if (a.items_max > 0) {
        dim3 grid((unsigned)a.items_max), block(kGemmThreads);
        timing_mark("gg_wgrad_det_kernel", s);
        if (bf16) hipLaunchKernelGGL((gg_wgrad_det_kernel<BM, BN, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gg_wgrad_det_kernel<BM, BN, false>), grid, block, 0, s, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
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
static hipError_t launch_wgrad_streamk_t(const GemmArgs& a, int64_t grid_n, bool bf16, hipStream_t s) {
    dim3 grid((unsigned)grid_n), block(kGemmThreads);
    timing_mark("gg_wgrad_streamk_kernel", s);
    if (bf16) hipLaunchKernelGGL((gg_wgrad_streamk_kernel<BM, BN, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gg_wgrad_streamk_kernel<BM, BN, false>), grid, block, 0, s, a);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_wgrad_streamk(int tile, const GemmArgs& a, int64_t grid_n, bool bf16, hipStream_t s) {
    switch (tile) {
        case kTile128x128: return launch_wgrad_streamk_t<128, 128>(a, grid_n, bf16, s);
        case kTile256x128: return launch_wgrad_streamk_t<256, 128>(a, grid_n, bf16, s);
        case kTile128x256: return launch_wgrad_streamk_t<128, 256>(a, grid_n, bf16, s);
        case kTile64x256: return launch_wgrad_streamk_t<64, 256>(a, grid_n, bf16, s);
        default: return launch_wgrad_streamk_t<256, 256>(a, grid_n, bf16, s);
    }
}

hipError_t launch_router(const float* X, const float* Wr, float* out, int64_t M, int64_t N, int64_t K,
                         hipStream_t s) {
    RouterArgs a{X, Wr, out, M, N, K};
    const int64_t tiles = ((M + kRouterBM - 1) / kRouterBM) * ((N + kRouterBN - 1) / kRouterBN);
    timing_mark("router_bf16x3_kernel", s);
    hipLaunchKernelGGL(router_bf16x3_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    timing_end(s);
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

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    size_t blocks = (bytes + kThreads * 16 - 1) / (kThreads * 16);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, static_cast<uint8_t*>(p), bytes);
    return hipGetLastError();
}

}  // namespace drgg
