// plan.hpp -- host-side planning for the ragged grouped GEMM on gfx950.
//
// Pure functions of the problem (and, for the non-deterministic weight
// gradient only, of the CU count).  Shared by the C ABI (api.cpp) and the
// kernel launchers (kernels.hip); nothing here touches the GPU.
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

// Functions the kernels evaluate too are host-and-device when hipcc compiles
// this header, plain host functions otherwise.
#if defined(__HIPCC__)
#define DRGG_HD __host__ __device__
#else
#define DRGG_HD
#endif

namespace drgg {

// The MFMA shape every program uses: v_mfma_f32_32x32x16_bf16 (32x32 output
// block, 16 reduction values per instruction).  Each output element is
// accumulated by one chain of these instructions in reduction order, so its
// value does not depend on the tile shape or the pipeline depth.
constexpr int kMfmaM = 32, kMfmaN = 32, kMfmaK = 16;

// Grouped-GEMM main loop: LDS stages of kStageK reduction values, kStages
// buffers per operand.
constexpr int kStageK = 32;
constexpr int kStages = 4;

// Token alignment of the deterministic weight gradient's chunks (and the
// reduction step of the router kernel).
constexpr int kTileK = 64;

// Token unit of the non-deterministic (stream-K) weight gradient: the K range
// of a split tile is handed out in 512-token units (flashinfer PR #8258,
// Summary: the k512 path, whose 512-token pieces are summed in no fixed order).
constexpr int64_t kStreamKUnit = 512;

// The reference CU count the deterministic chunk rule is written against.  It
// is a constant of the rule, never the live device's count, so that the
// deterministic weight gradient is the same on any number of CUs.
constexpr int64_t kRuleCUs = 256;

constexpr int kMaxExperts = 1024;

enum TileId { kTileAuto = 0, kTile256x256 = 1, kTile128x128 = 2, kTile256x128 = 3,
              kTile128x256 = 4, kTile64x256 = 5 };

struct TileShape { int bm, bn; };

inline TileShape tile_shape(int id) {
    switch (id) {
        case kTile128x128: return {128, 128};
        case kTile256x128: return {256, 128};
        case kTile128x256: return {128, 256};
        case kTile64x256: return {64, 256};
        default: return {256, 256};
    }
}

DRGG_HD inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
DRGG_HD inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Chunk rule part 2 (host mirror of the device function): an expert with T
// tokens is cut into chunks of `len` tokens (the last one shorter), starting
// at its first token.  S = ceil(T / chunk_max), len = ceil(T / S) rounded up
// to a multiple of 64, chunks = ceil(T / len).
DRGG_HD inline void wgrad_chunking(int64_t T, int64_t chunk_max, int64_t* len, int64_t* chunks) {
    if (T <= 0) { *len = 0; *chunks = 0; return; }
    const int64_t s = ceil_div(T, chunk_max);
    const int64_t l = round_up(ceil_div(T, s), kTileK);
    *len = l;
    *chunks = ceil_div(T, l);
}

// What one work item costs beyond its reduction steps (pipeline fill and the
// store of a 256x256 FP32 tile), in tokens of reduction: about eight 32-token
// steps.
constexpr int64_t kItemOverheadTokens = 256;

// The data gradient transposes W into its workspace (W^T, so that both
// operands are reduction-contiguous) only when the experts average at least
// this many tokens.  The transposed program saves a fraction of the
// product's time, which grows with the tokens that meet each W element,
// while the transpose costs a read and a write of every W element and a
// launch; on MI355X it pays from about 4096 tokens per expert on and loses
// at 2048 and below.
constexpr int64_t kTransposeMinTokens = 3072;
DRGG_HD inline bool dgrad_transposes_w(int64_t E, int64_t M) { return M >= kTransposeMinTokens * E; }

// Deterministic weight gradient, chunk rule part 1 (host): the longest chunk
// an expert's token range is cut into.  A function of (E, M, N, K) only.
//   P0    = output tiles per expert at a 256x256 reference tile
//   floor = max(half a reference CU's share of the token-tile work, 512)
//   chunk_max(S) = max(ceil(M / (E*S)), floor) rounded up to a multiple of 64
//   S     = the chunk count per balanced expert (ceil(M/E) tokens) that
//           minimises the estimated time on kRuleCUs workgroups: the waves
//           of its P0*E*chunks items times (its chunk length + the item
//           overhead); the smallest S on ties (fewest partials).
//   share = one reference CU's share of the token-tile work,
//           ceil(M * P0 / kRuleCUs) rounded up to 64: when the balanced
//           expert stays whole (one chunk), only experts longer than the
//           balanced size are cut, and into chunks of at least one share
//           (fewer and longer items, fewer partials to fold; measured faster
//           on skewed routings).
// Long experts are cut into more chunks; short ones are never cut.
inline int64_t wgrad_chunk_max(int32_t E, int64_t M, int64_t N, int64_t K) {
    if (M <= 0) return 512;
    const int64_t p0 = ceil_div(N, 256) * ceil_div(K, 256);
    const int64_t tb = ceil_div(M, (int64_t)E);
    int64_t floor = ceil_div(ceil_div(M * p0, kRuleCUs), 2);
    if (floor < 512) floor = 512;
    int64_t best = 0, best_cost = 0;
    for (int64_t s = 1; s <= 64; ++s) {
        int64_t c = ceil_div(M, (int64_t)E * s);
        c = round_up(c > floor ? c : floor, kTileK);
        int64_t len, chunks;
        wgrad_chunking(tb, c, &len, &chunks);
        const int64_t cost = ceil_div(p0 * E * chunks, kRuleCUs) * (len + kItemOverheadTokens);
        if (best == 0 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    int64_t len, chunks;
    wgrad_chunking(tb, best, &len, &chunks);
    const int64_t share = round_up(ceil_div(M * p0, kRuleCUs), kTileK);
    return chunks <= 1 && share > best ? share : best;
}

// Deterministic weight gradient, chunk rule part 3: the tail-only plan.
// Whole output tiles in full waves, only the tail split (flashinfer PR
// #8258, Summary: the last output tiles, the "tail", are the ones whose K
// range is split).  An expert cut into S > 1 chunks (part 2) has P0 output
// tiles of 256 x 256 (the reference tile, as in part 1) and a share
// R_e = kRuleCUs * T / M of the kRuleCUs reference workgroups (its share of
// the work).  Its whole tiles fill the F = floor(P0 / R_e) full waves on
// that share, floor(F * R_e) tiles, rounded down to whole rows of reference
// tiles; every other tile is cut into the S chunks.  Returns the number of
// 256-row reference rows of the expert's output (dW rows n < 256 * result)
// that run as whole tiles: all of them (ceil(N / 256)) when S <= 1.  A pure
// function of the problem, never of the device; the result does not depend
// on the kernel's tile shape either (its tiles nest in the 256-row bands).
// (The split program uses the same rule on the live grid: `workers`.)
DRGG_HD inline int64_t wgrad_whole_rows(int64_t T, int64_t M, int64_t N, int64_t K, int64_t S,
                                        int64_t workers = kRuleCUs) {
    const int64_t tn0 = ceil_div(N, 256), tk0 = ceil_div(K, 256);
    if (S <= 1 || T <= 0 || M <= 0 || workers <= 0) return tn0;
    const int64_t F = (tn0 * tk0 * M) / (workers * T);
    const int64_t full = (F * workers * T) / M;
    const int64_t h = full / tk0;
    return h < tn0 ? h : tn0;
}

// The non-deterministic split program's whole bands: full waves on the
// expert's share of the live grid (`workers` persistent workgroups), as
// wgrad_whole_rows, and then the tail-split rule below (tailsplit_units) on
// that share: the tail tiles are cut into chunks only when twice their
// number fits in the share, R_e = workers * T / M (2 * tail <= R_e);
// otherwise every tile of the expert stays whole (returns all bands).
DRGG_HD inline int64_t split_whole_rows(int64_t T, int64_t M, int64_t N, int64_t K, int64_t S, int64_t workers) {
    const int64_t tn0 = ceil_div(N, 256), tk0 = ceil_div(K, 256);
    const int64_t h = wgrad_whole_rows(T, M, N, K, S, workers);
    if (h >= tn0) return tn0;
    const int64_t tail = (tn0 - h) * tk0;
    return 2 * tail * M <= workers * T ? h : tn0;
}

// The split program's token unit: its chunks are the deterministic chunk
// lengths rounded up to whole kStreamKUnit-token units.
DRGG_HD inline void split_chunking(int64_t T, int64_t chunk_max, int64_t* len, int64_t* chunks) {
    int64_t l, c;
    wgrad_chunking(T, chunk_max, &l, &c);
    l = round_up(l, kStreamKUnit);
    *len = T > 0 ? l : 0;
    *chunks = T > 0 ? ceil_div(T, l) : 0;
}

// Slack placement of the split program's tail needs every workgroup's load
// at kernel start; grids above this size skip it (the tail is split).
constexpr int64_t kSlackMaxGrid = 1024;

// Experts above this count always run the all-split plan: the tail-only
// plan's walk has two positions per expert (whole tiles first, then the
// chunks), and the kernels' schedule tables hold kMaxExperts + 1 entries.
constexpr int kTailPlanMaxExperts = kMaxExperts / 2;

// Estimated time of a walk (host mirror of the kernels' walk_makespan):
// position q holds work[q] items of len[q] tokens each, handed out in snake
// rounds over `workers` workgroups; every item costs len + kItemOverheadTokens.
inline uint64_t walk_makespan_host(const std::vector<int64_t>& work, const std::vector<int64_t>& len,
                                   int64_t workers) {
    std::vector<uint64_t> load(workers, 0);
    int64_t i = 0;
    for (size_t q = 0; q < work.size(); ++q)
        for (int64_t j = 0; j < work[q]; ++j, ++i) {
            const int64_t r = i / workers, b = i % workers;
            load[(r & 1) ? workers - 1 - b : b] += (uint64_t)(len[q] + kItemOverheadTokens);
        }
    return *std::max_element(load.begin(), load.end());
}

// Host mirror of the deterministic weight gradient's plan choice, which the
// chunk kernel makes on the device from the group offsets (same integer
// arithmetic): the estimated time of each plan's walk on kRuleCUs reference
// workgroups, in tokens (snake rounds over the walk positions, each item
// costing its token count plus kItemOverheadTokens), with 256x256 reference
// tiles; the tail-only plan when it differs and is not slower.  `offs` are
// valid host offsets [E + 1] (o[0] = 0, non-decreasing, o[E] = M).  Fills row0[e] (if
// given) with the first dW row of expert e that the fold writes (0 in the
// all-split plan, and for experts not cut into chunks).  For tests and
// inspection only.
inline bool wgrad_tail_plan(const int32_t* offs, int32_t E, int64_t N, int64_t K, int32_t* row0) {
    std::vector<int64_t> T(E > 0 ? E : 0);
    int64_t M = 0, prev = 0;
    const int64_t last = E > 0 ? std::max<int64_t>(offs[E], 0) : 0;
    for (int32_t e = 0; e < E; ++e) {   // clamp into [0, M], non-decreasing
        const int64_t lo = std::max(prev, std::min<int64_t>(std::max<int64_t>(offs[e], 0), last));
        const int64_t hi = std::max(lo, std::min<int64_t>(std::max<int64_t>(offs[e + 1], 0), last));
        T[e] = hi - lo;
        prev = hi;
    }
    M = last;
    for (int32_t e = 0; e < E && row0; ++e) row0[e] = 0;
    if (E > kTailPlanMaxExperts || M <= 0) return false;
    const int64_t cmax = wgrad_chunk_max(E, M, N, K);
    std::vector<int64_t> L(E), S(E), band(E);
    for (int32_t e = 0; e < E; ++e) {
        wgrad_chunking(T[e], cmax, &L[e], &S[e]);
        band[e] = wgrad_whole_rows(T[e], M, N, K, S[e]);
    }
    std::vector<int32_t> perm(E);
    for (int32_t e = 0; e < E; ++e) perm[e] = e;
    std::stable_sort(perm.begin(), perm.end(), [&](int32_t x, int32_t y) { return L[x] > L[y]; });
    const int64_t tk0 = ceil_div(K, 256), P0 = ceil_div(N, 256) * tk0;

    std::vector<int64_t> w1(E), l1(E), w2(2 * E), l2(2 * E);
    int64_t whole_tiles = 0;
    for (int32_t q = 0; q < E; ++q) {
        const int32_t e = perm[q];
        w1[q] = P0 * S[e];
        l1[q] = S[e] > 1 ? L[e] : T[e];
        const int64_t w0 = S[e] > 1 ? band[e] * tk0 : 0;
        whole_tiles += w0;
        w2[q] = w0;
        l2[q] = T[e];
        w2[E + q] = S[e] > 1 ? (P0 - w0) * S[e] : S[e] == 1 ? P0 : 0;   // no tokens: no items
        l2[E + q] = S[e] > 1 ? L[e] : T[e];
    }
    const bool tail = whole_tiles > 0 && walk_makespan_host(w2, l2, kRuleCUs) <= walk_makespan_host(w1, l1, kRuleCUs);
    for (int32_t e = 0; e < E && row0 && tail; ++e)
        row0[e] = S[e] > 1 ? (int32_t)std::min<int64_t>(N, band[e] * 256) : 0;
    return tail;
}

// Host mirror of the split program's choice for a grid of G workgroups and
// kernel tiles of bm x bn (the kernel makes it on the device; same
// arithmetic).  Experts in decreasing order of chunk length.  Banded walk:
// a first pass of every expert's whole tiles (split_whole_rows; all of an
// expert not cut into chunks) in snake rounds over the G workgroups, each
// item its token count plus kItemOverheadTokens, then the tail tiles.  Slack
// placement (flashinfer PR #8258, Summary): the workgroups are ranked by
// their first-pass load; if there are at most G tail tiles and the i-th tail
// tile (in walk order) fits whole on the i-th least-loaded workgroup without
// taking it beyond the largest load plus one tail share (one chunk of that
// expert), every tail tile runs whole there (no tile sum, no ticket);
// otherwise the tail runs as chunk items.  The banded walk runs if its
// estimated time is not above the all-split walk's (every tile of an expert
// cut into chunks as chunk items); without slack placement and with no
// expert cut into chunks keeping whole tiles both walks hold the same items
// and the all-split one runs.  Returns true for the slack placement;
// out[0] = tail tiles, out[1] = 1 if the banded walk runs.  For tests only.
inline bool wgrad_split_plan(const int32_t* offs, int32_t E, int64_t N, int64_t K, int bm, int bn, int64_t G,
                             int64_t* out) {
    out[0] = out[1] = 0;
    if (E < 1 || G < 1) return false;
    const int64_t M = offs[E];
    if (M <= 0) return false;
    const int64_t cmax = wgrad_chunk_max(E, M, N, K);
    const int64_t tn = ceil_div(N, bm), tk = ceil_div(K, bn), P = tn * tk;
    const bool banded = E <= kTailPlanMaxExperts;
    std::vector<int64_t> T(E), L(E), S(E), nw(E);
    for (int32_t e = 0; e < E; ++e) {
        T[e] = (int64_t)offs[e + 1] - offs[e];
        split_chunking(T[e], cmax, &L[e], &S[e]);
        if (S[e] == 0) nw[e] = 0;   // no tokens: no items
        else if (S[e] == 1) nw[e] = P;
        else if (!banded) nw[e] = 0;
        else nw[e] = std::min<int64_t>(tn, split_whole_rows(T[e], M, N, K, S[e], G) * (256 / bm)) * tk;
    }
    std::vector<int32_t> perm(E);
    for (int32_t e = 0; e < E; ++e) perm[e] = e;
    std::stable_sort(perm.begin(), perm.end(), [&](int32_t x, int32_t y) { return L[x] > L[y]; });
    if (!banded) return false;
    std::vector<int64_t> w1(E), l1(E), wb(2 * E), lb(2 * E), ws(E), ls(E), tail_T, tail_L;
    int64_t total1 = 0;
    for (int32_t q = 0; q < E; ++q) {
        const int32_t e = perm[q];
        w1[q] = T[e] > 0 ? nw[e] : 0;
        l1[q] = T[e];
        total1 += w1[q];
        wb[q] = w1[q];
        lb[q] = T[e];
        wb[E + q] = T[e] > 0 ? (P - nw[e]) * S[e] : 0;
        lb[E + q] = L[e];
        ws[q] = S[e] > 1 ? P * S[e] : S[e] == 1 ? P : 0;
        ls[q] = S[e] > 1 ? L[e] : T[e];
        for (int64_t j = nw[e]; j < P && T[e] > 0; ++j) {
            tail_T.push_back(T[e]);
            tail_L.push_back(L[e]);
        }
    }
    const int64_t ntail = (int64_t)tail_T.size();
    out[0] = ntail;
    if (total1 == 0) return false;   // the banded walk is the all-split walk
    std::vector<uint64_t> load(G, 0);
    for (int64_t i = 0, q = 0, j = 0; i < total1; ++i, ++j) {
        while (j >= w1[q]) { ++q; j = 0; }
        const int64_t r = i / G, b = i % G;
        load[(r & 1) ? G - 1 - b : b] += (uint64_t)(l1[q] + kItemOverheadTokens);
    }
    const uint64_t lmax = *std::max_element(load.begin(), load.end());
    const uint64_t lmin = *std::min_element(load.begin(), load.end());
    bool slack = false;
    uint64_t top = lmax;
    if (ntail > 0 && ntail <= G && G <= kSlackMaxGrid && lmin + (uint64_t)tail_T[0] <= lmax + (uint64_t)tail_L[0]) {
        std::vector<uint64_t> sorted = load;
        std::sort(sorted.begin(), sorted.end());
        slack = true;
        for (int64_t t = 0; t < ntail; ++t) {
            if (sorted[t] + (uint64_t)tail_T[t] > lmax + (uint64_t)tail_L[t]) slack = false;
            top = std::max<uint64_t>(top, sorted[t] + (uint64_t)tail_T[t] + kItemOverheadTokens);
        }
    }
    bool keeps = false;   // an expert cut into chunks keeps whole tiles
    for (int32_t e = 0; e < E; ++e) keeps = keeps || (S[e] > 1 && nw[e] > 0);
    if (!keeps && !slack) return false;   // both walks hold the same items: the all-split one runs
    const uint64_t mk_band = slack ? top : walk_makespan_host(wb, lb, G);
    const bool use_band = mk_band <= walk_makespan_host(ws, ls, G);
    out[1] = use_band;
    return slack && use_band;
}

// Partial slots the deterministic weight gradient may need: only experts cut
// into more than one chunk write partials.  Such an expert has
// T > chunk_max and at most T / chunk_max + 1 < 2 T / chunk_max chunks, so the
// total is below 2 M / chunk_max.  With M <= chunk_max no expert can be cut
// (T <= M): no slots, no fold, and no workspace at all.
inline int64_t wgrad_max_partials(int64_t M, int64_t chunk_max) {
    return M <= chunk_max ? 0 : (2 * M) / chunk_max + 1;
}

// The tail-split rule of a persistent schedule (flashinfer PR #7516, the
// #7632 commit body, its tail-split routing test): `tiles` equal output
// tiles run on `workers` persistent workers in full waves plus a partial
// last wave of tail = tiles mod workers tiles.  When 2 * tail <= workers the
// tail tiles are cut in two along the reduction, giving 2 * tail half units
// next to the `full` whole tiles; otherwise every tile stays whole.
// Returns (tiles, units, full, split): units = work units handed out,
// full = tiles that run whole, split = pieces per tail tile (1 or 2).
struct TailSplit {
    int64_t tiles, units, full, split;
};
inline TailSplit tailsplit_units(int64_t tiles, int64_t workers) {
    const int64_t tail = workers > 0 ? tiles % workers : 0;
    if (tail > 0 && 2 * tail <= workers) return {tiles, tiles - tail + 2 * tail, tiles - tail, 2};
    return {tiles, tiles, tiles, 1};
}

// Rows per round of the staged epilogue of the forward and data-gradient
// kernels (kernels.hip): its LDS scratch is that many 128-byte rows per
// wave.  Tiles below 256x128 share a CU and get the smaller scratch.
constexpr int ep_rows(int bm, int bn) { return bm * bn >= 256 * 128 ? 16 : 8; }
// Whether the deterministic weight gradient writes its tiles through a
// per-wave LDS scratch in whole 128-byte lines (as the forward does): every
// tile shape but 128x128, where the scratch would leave room for one
// workgroup per CU instead of two.
constexpr bool wgrad_det_staged(int bm, int bn) { return !(bm == 128 && bn == 128); }
// Workgroups of a persistent grouped-GEMM kernel that fit on one CU's 160 KB
// of LDS: kStages stages of (BM + BN) x kStageK BF16, the schedule tables
// (10 KB; the deterministic weight gradient adds 4 KB of partial-slot
// bases), the epilogue scratch (forward, data gradient, and the deterministic
// weight gradient where wgrad_det_staged), and 1 KB for alignment.
// Workgroups have 4 waves, except the 8 of the 256x256 forward,
// data-gradient and deterministic weight-gradient kernels.
inline int64_t wgs_per_cu(TileShape t, bool fwd_dgrad, bool det_wgrad) {
    const int64_t waves = (fwd_dgrad || det_wgrad) && t.bm == 256 && t.bn == 256 ? 8 : 4;
    const bool ep = fwd_dgrad || (det_wgrad && wgrad_det_staged(t.bm, t.bn));
    const int64_t lds = (int64_t)kStages * (t.bm + t.bn) * kStageK * 2 + 10248 + (det_wgrad ? 4100 : 0) +
                        (ep ? waves * ep_rows(t.bm, t.bn) * 128 : 0) + 1024;
    const int64_t n = (160 * 1024) / lds;
    return n < 1 ? 1 : n;
}

// FP32 router program choice and slices.  The single-pass program (128x128
// tiles) runs when its tiles alone fill kRuleCUs workgroups, or for K > 2^21
// (ks = 0, kq = K); otherwise the sliced program (router_ks_kernel): 256x256
// output tiles and ks slices of kq values (a multiple of 32: whole 128-byte
// rows) so that tiles * ks reaches kRuleCUs workgroups, at most 8 slices and
// none shorter than 256 values.  A function of (M, N, K) only: the slices are
// added in a fixed order.
struct RouterSplit {
    int64_t ks, kq;
};
inline RouterSplit router_split(int64_t M, int64_t N, int64_t K) {
    if (ceil_div(M, 128) * ceil_div(N, 128) >= kRuleCUs || K > (int64_t(1) << 21)) return {0, K};
    const int64_t tiles = ceil_div(M, 256) * ceil_div(N, 256);
    int64_t ks = tiles > 0 ? ceil_div(kRuleCUs, tiles) : 1;
    const int64_t cap = K / 256 > 1 ? K / 256 : 1;
    if (ks > cap) ks = cap;
    if (ks > 8) ks = 8;
    if (ks < 1) ks = 1;
    const int64_t kq = round_up(ceil_div(K, ks), 32);
    return {ceil_div(K, kq), kq};   // every slice non-empty
}

// Default output tile per program: 256x256, except the skinny weight
// gradient (N <= 64: 64x256) and outputs of at most 128 columns (Y has N,
// dX and dW have K), where a 256-wide tile would be at least half masked:
// 128x128 (measured on per-head projections with K = 128: data gradient
// -12 %, weight gradient -5 %).  The forward and data gradient then look at
// how many 256x256 tiles the call has: between lo = ceil(M/256) * ct (every
// group's rows packed, ct = ceil(cols/256)) and hi = floor((M + 255 E)/256)
// * ct (each group adds at most one partial row tile).
//  * lo <= kRuleCUs / 2: 128x128.  The persistent grid would run one
//    256x256 tile per busy workgroup while most CUs idle; four times the
//    tiles of a quarter the work finish sooner (kernel times, 4 groups of 128
//    tokens with K = 256, N = 512: forward 12.6 -> 10.0 us, data gradient
//    17.4 -> 12.5 us; one group of 2048 tokens at 4096 x 4096: 89 -> 71 us
//    and 93 -> 77 us; 128 groups of 64 tokens at 1024 x 1024: 60 -> 52 us
//    and 71 -> 62 us).  The same when the groups average fewer than 128
//    tokens (M < 128 E), whatever lo says: 256-row tiles would then be at
//    least half padding (64 groups of 86 tokens on average, N = 4096, K =
//    1024: forward 125.3 -> 111.5 us; 32 groups of 70 at 768 x 4096: data
//    gradient 50.7 -> 41.5 us; 128x128 was the fastest tile at all 18 such
//    points measured).
//  * kRuleCUs < lo and hi <= 3 kRuleCUs / 2 (between one and one and a half
//    waves), with both operands reduction-contiguous (the forward, and the
//    data gradient on W^T): 128x256.  A second round of 256x256 tiles would
//    run at most half full; 128x256 tiles (4 waves) fill their rounds better
//    (8 groups of 1536 tokens at gate_up's N = 1536, K = 2048: forward 105.5
//    -> 100.9 us, data gradient 90.8 -> 83.5 us; one group of 5120 / 6144
//    tokens at 4096 x 4096: forward 207.9 -> 186.7 / 211.6 -> 200.3 us, data
//    gradient 206.2 -> 186.0 / 210.7 -> 194.4 us).  At one wave and from
//    1.9 waves on 256x256 was as fast or faster at every measured point, and
//    the data gradient that reads W transposed lost 15 % on 128x256.
// The output bits do not depend on the tile (every element sums its
// reduction in the same order).  The deterministic weight gradient's work
// items are output tiles over token chunks; with few of them smaller tiles
// spread the work (the chunks do not depend on the tile, so neither do the
// bits).  Unchunked (M <= chunk_max: no expert can be cut, every item is a
// whole expert's tile, often of few tokens) the E * ceil(N/256) *
// ceil(K/256) items take 128x128 up to kRuleCUs / 8 and 128x256 up to
// kRuleCUs / 2 (kernel times, 256x256 -> chosen tile: 4 groups of 128 tokens
// at N = 512, K = 256: 17.0 -> 13.4 us; one group of 384 at 768 x 768: 21.0
// -> 15.6 us; one group of 512 at 2048 x 2048: 27.0 -> 24.6 us; 8 groups of
// 64 at 1024 x 1024: 20.8 -> 19.1 us; at 256 items 256x256 stays faster,
// 29.6 against 31.5 us).  Chunked, U = ceil(N/256) * ceil(K/256) * (E +
// M / chunk_max) bounds the items; U <= kRuleCUs / 2 takes 128x128, whose
// four times as many items still fit one round of two workgroups per CU
// (one group of 4096 tokens at N = 256, K = 1024, U = 36: 35.6 -> 28.5 us;
// 8192 tokens, U = 68: 39.8 -> 34.3 us; 4 groups, 8192 tokens at 512 x 512,
// U = 80: 39.9 -> 36.0 us; at U = 160, 144 items, 128x128 lost 23 %).  The
// split program (det false) keeps 256x256.
inline int default_tile(int op, int64_t E, int64_t M, int64_t N, int64_t K, bool kmajor, bool det) {
    if (op == 2 && N <= 64) return kTile64x256;
    const int64_t cols = op == 0 ? N : K;
    if (cols <= 128) return kTile128x128;
    if (op == 2) {
        if (!det || M <= 0) return kTile256x256;
        const int64_t cm = wgrad_chunk_max((int32_t)E, M, N, K);
        const int64_t p0 = ceil_div(N, 256) * ceil_div(K, 256);
        if (M <= cm) {
            const int64_t t = E * p0;
            if (t <= kRuleCUs / 8) return kTile128x128;
            if (t <= kRuleCUs / 2) return kTile128x256;
        } else if (p0 * (E + M / cm) <= kRuleCUs / 2) {
            return kTile128x128;
        }
        return kTile256x256;
    }
    const int64_t ct = ceil_div(cols, 256);
    const int64_t lo = ceil_div(M, 256) * ct;
    const int64_t hi = (M + 255 * E) / 256 * ct;
    if (lo <= kRuleCUs / 2 || M < 128 * E) return kTile128x128;
    if (kmajor && lo > kRuleCUs && hi <= kRuleCUs * 3 / 2) return kTile128x256;
    return kTile256x256;
}

}  // namespace drgg
