// gdn_step.hip - gdn_step and gdn_pair: the HBM-streaming one- and
// two-position kernels.

#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kXcds = 8;

// ------------------------------------------------------------- gdn_step
// HBM-bound: the state is streamed once in and once out, 4 KiB tiles (8 rows)
// at a time.  Two launch shapes:
//  - small launches (up to kOneShotTiles tiles): one one-wave workgroup per
//    tile, which spreads the few tiles over every CU (k_step_tile);
//  - large launches: two tiles per 8-wave workgroup, staged through LDS
//    (k_step_staged).
// Workgroup g runs on XCD g % 8; the small kernel remaps workgroups to tiles
// so that the 16 tiles of a head share one XCD and its k and q are fetched
// into one L2 only.

// Small launches.  q is fetched together with the state: with one tile per
// wave, fetching it after the key reduction measured 0.08 us slower at B = 1.
template <bool NT>
__global__ __launch_bounds__(64) void k_step_tile(StepArgs a) {
    const int lane = threadIdx.x;
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int t = (G % kXcds == 0) ? (g % kXcds) * (G / kXcds) + g / kXcds : g;
    const int head = t / kTilesPerHead;
    const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
    const int b = head / a.Hv;
    const int h = head - b * a.Hv;
    int kh = h;
    while (kh >= a.Hk) kh -= a.Hk;                            // key-head broadcast
    float *Mrow = a.state + static_cast<int64_t>(head) * (D * D) + row * D;
    const float gt = a.gate[head];
    const float bt = a.beta[head];
    const float vj = a.v[b * a.v_bstride + h * D + row];
    RowSlice r;
    load_row<NT>(r, Mrow, c);
    VecSlice kv, qv;
    load_vec(kv, a.k + b * a.qk_bstride + kh * D, c);
    load_vec(qv, a.q + b * a.qk_bstride + kh * D, c);
    const float e = expf(gt);
    const float sk = group_sum(head_part(r, kv, e));         // decay, key product
    update_part(r, (vj - sk) * bt, kv);                       // correction, rank-1
    store_row<NT>(Mrow, r, c);
    const float o = group_sum(dot_part(r, qv)) * kInvSqrtD;   // read-out
    if (c == 0) a.out[static_cast<int64_t>(head) * D + row] = o;
}

// Large launches: staged tiles.  A workgroup of 8 waves takes two
// consecutive tiles of one head.  Every thread streams one float4
// of the pair into LDS with a nontemporal load, so each load instruction of
// a wave covers 1 KiB of contiguous state (four waves per tile); after a
// barrier, waves 0 and 4 read their tile back from LDS in the row layout,
// run the step's row arithmetic on it (that of k_step_tile) and store the
// rows straight from registers.
// Same per-row arithmetic, so the same bits.  Measured on MI355X against
// the persistent walk (the same pattern with each wave loading its own tile
// row by row): 5.90-5.92 against 6.19-6.21 ms for the B = 256 x 36-layer
// step, 5.84-5.89 against 6.12 ms for those layers as one B = 9216 call,
// 3-4 % faster from B = 32 to 512.  An in-place probe shows why: one
// float4 per thread in 1 KiB-contiguous instructions reads and writes
// 6.56-6.66 TB/s where the walk's pattern reaches 6.29-6.37.  Measured and
// not taken: one tile per 256-thread workgroup (1.5 % slower on the 36
// layers), 4 or 8 tiles per workgroup, one or two waves per tile (slower),
// every wave computing a share of the rows (up to 50 % slower), the stores
// also staged through LDS behind a second barrier (6.6-6.7 ms) or by the
// computing wave alone (5.98 against 5.90 ms), workgroups
// remapped so that one XCD takes a contiguous share of the tiles (2 %
// slower), and a grid-stride loop over tile pairs inside the kernel (its
// live values took 68 VGPRs instead of 56: three workgroups per CU instead
// of four, 25 % slower).  A launch with more tile pairs than one dispatch
// holds (2^22 workgroups: states beyond 32 GiB) is split into several
// launches.
constexpr int kStagedThreads = 512;
constexpr int kStagedTiles = 2;
constexpr int kF4PerTile = kRowsPerTile * D / 4;   // 256
static_assert(kStagedThreads == kStagedTiles * kF4PerTile, "one float4 per thread");

template <bool NT>
__global__ __launch_bounds__(kStagedThreads) void k_step_staged(StepArgs a, int pair0) {
    constexpr int kWavesPerTile = kF4PerTile / 64;   // 4
    __shared__ f4 tile[kStagedTiles][kF4PerTile];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int mine = wave / kWavesPerTile;           // the tile of the pair this wave streams
    const int p = (wave % kWavesPerTile) * 64 + lane;   // this lane's float4 in it
    const bool computes = wave % kWavesPerTile == 0;    // waves 0 and 4 compute tile `mine`
    const int t = (pair0 + static_cast<int>(blockIdx.x)) * kStagedTiles + mine;
    const int head = t / kTilesPerHead;
    const int row0 = (t % kTilesPerHead) * kRowsPerTile;
    float *Mt = a.state + static_cast<int64_t>(head) * (D * D) + row0 * D;
    const f4 *src = reinterpret_cast<const f4 *>(Mt) + p;
    if constexpr (NT)
        tile[mine][p] = __builtin_nontemporal_load(src);
    else
        tile[mine][p] = *src;
    // The computing waves fetch their vectors only now: the barrier below
    // then waits for the tile alone, the six other waves leave as soon as it
    // is in LDS, and the vector loads complete while the next workgroup
    // starts (fetching them before the LDS write measured 4 % slower).
    VecSlice kv, qv;
    float gt = 0.0f, bt = 0.0f, vj = 0.0f;
    if (computes) {
        const int b = head / a.Hv;
        const int h = head - b * a.Hv;
        int kh = h;
        while (kh >= a.Hk) kh -= a.Hk;                      // key-head broadcast
        load_vec(kv, a.k + b * a.qk_bstride + kh * D, c);
        load_vec(qv, a.q + b * a.qk_bstride + kh * D, c);
        gt = a.gate[head];
        bt = a.beta[head];
        vj = a.v[b * a.v_bstride + h * D + row0 + grp];
    }
    __syncthreads();                 // every wave: its share of the tiles is in LDS
    if (!computes) return;
    RowSlice r;
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) r.m[i] = tile[mine][grp * (D / 4) + kLanesPerRow * i + c];
    const float e = expf(gt);
    const float sk = group_sum(head_part(r, kv, e));         // decay, key product
    update_part(r, (vj - sk) * bt, kv);                       // correction, rank-1
    store_row<NT>(Mt + grp * D, r, c);
    const float o = group_sum(dot_part(r, qv)) * kInvSqrtD;   // read-out
    if (c == 0) a.out[static_cast<int64_t>(head) * D + row0 + grp] = o;
}

// --------------------------------------------------- gdn_step, cached state
// gdn_step_ex with GDN_STATE_CACHED: the caller's states stay resident in
// the Infinity Cache across calls, so the state goes through the caches and
// the launch is laid out for latency rather than for a streaming window.
// Each wave takes TPW consecutive tiles of one head (every head's 16 tiles
// split over 16 / TPW waves), issues all their state loads at once, reads
// the head's k, q, beta and gate once, and then updates and stores its tiles
// one after the other.  Same per-row arithmetic as k_step_tile and
// k_step_staged, so the same bits.
// Measured on MI355X, 100 calls with fresh inputs per call: B = 64 (a
// 128 MiB state) 4.15 ms against 4.48 ms for the nontemporal walk and
// 4.95 ms for the walk with cached state access; B = 32 2.04 against
// 2.37 ms.  With 4 tiles per wave 0.5-2 % slower.  Beyond the Infinity
// Cache (one 512 MiB state) it is 20 % slower than the default.
template <int TPW, int W>
__global__ __launch_bounds__(W * 64) void k_step_cached(StepArgs a, int n_tiles) {
    static_assert(kTilesPerHead % TPW == 0, "a wave's tiles must share a head");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int t0 = (static_cast<int>(blockIdx.x) * W + wave) * TPW;
    if (t0 >= n_tiles) return;
    const int head = t0 / kTilesPerHead;
    const int b = head / a.Hv;
    const int h = head - b * a.Hv;
    const int kh = h % a.Hk;                                   // key-head broadcast
    float *Mh = a.state + static_cast<int64_t>(head) * (D * D);
    const int row0 = (t0 % kTilesPerHead) * kRowsPerTile + grp;
    RowSlice r[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) load_row<false>(r[j], Mh + (row0 + j * kRowsPerTile) * D, c);
    VecSlice kv, qv;
    load_vec(kv, a.k + b * a.qk_bstride + kh * D, c);
    load_vec(qv, a.q + b * a.qk_bstride + kh * D, c);
    const float bt = a.beta[head];
    const float e = expf(a.gate[head]);
    float vj[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) vj[j] = a.v[b * a.v_bstride + h * D + row0 + j * kRowsPerTile];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const float sk = group_sum(head_part(r[j], kv, e));   // decay, key product
        update_part(r[j], (vj[j] - sk) * bt, kv);              // correction, rank-1
        store_row<false>(Mh + (row0 + j * kRowsPerTile) * D, r[j], c);
        const float o = group_sum(dot_part(r[j], qv)) * kInvSqrtD;   // read-out
        if (c == 0) a.out[static_cast<int64_t>(head) * D + row0 + j * kRowsPerTile] = o;
    }
}

// ------------------------------------------------------------- gdn_pair
// Speculative two-position step (docs.rs "Module linear_core", gdn_pair):
// each row is read once, advanced by position 1 and written back to `state`
// (committed), then advanced by position 2 in registers and written to
// `state_next` (tentative).  Three state transfers instead of the four of
// two separate steps.  A persistent grid of W-wave workgroups (one per CU)
// walks the tiles in a grid-stride loop, one tile per wave per pass, so the
// addresses in flight form one contiguous window that sweeps the state; W =
// 1 with one workgroup per tile for small launches.  Workgroups are grouped
// in epochs of GE: epoch e walks tiles [e * span, (e + 1) * span), span =
// GE * W * iters, like one persistent launch of GE workgroups; the
// dispatcher starts epoch e + 1 as epoch e retires, which keeps the window
// contiguous (one long walk lets the waves drift apart).  The staged layout
// of k_step_staged measured slower here (265 against 257 us at B = 256,
// 1078 against 1013 us at B = 1024, equal at B = 64): with one read and two
// writes per row the writes dominate, and staging helps the reads.  Fetching
// q after the key reduction measured 7 % slower.
template <int W>
__global__ __launch_bounds__(W * 64) void k_pair(PairArgs a, int n_tiles, int GE, int iters) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;

    const int epoch = blockIdx.x / GE;
    const int g = blockIdx.x - epoch * GE;
    const int lg = (GE % kXcds == 0) ? (g % kXcds) * (GE / kXcds) + g / kXcds : g;
    const int stride = GE * W;
    const int span = stride * iters;
    const int base = epoch * span;
    const int end = n_tiles - base < span ? n_tiles : base + span;

    for (int u = base + lg * W + wave; u < end; u += stride) {
        const int head = u / kTilesPerHead;
        const int row = (u % kTilesPerHead) * kRowsPerTile + grp;
        const int b = head / a.Hv;
        const int h = head - b * a.Hv;
        const int kh = h % a.Hk;
        const int64_t roff = static_cast<int64_t>(head) * (D * D) + row * D;

        RowSlice r;
        load_row<true>(r, a.state + roff, c);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t bp = static_cast<int64_t>(b) * 2 + p;
            VecSlice kv, qv;
            load_vec(kv, a.k + (bp * a.Hk + kh) * D, c);
            load_vec(qv, a.q + (bp * a.Hk + kh) * D, c);
            const int64_t hp = bp * a.Hv + h;
            const float e = expf(a.gate[hp]);
            const float o = row_token(r, kv, qv, e, a.beta[hp], a.v[hp * D + row]);
            store_row<true>((p == 0 ? a.state : a.state_next) + roff, r, c);
            if (c == 0) a.out[hp * D + row] = o;
        }
    }
}

}  // namespace

// Launches of up to this many tiles (B * Hv <= 512) run one wave per tile
// (k_step_tile): measured per call over 36 layers, replayed from a graph,
// 2.73 against 2.94 us at B = 1, 3.18 against 3.35 at B = 2, 7.3 against
// 7.9 at B = 8 and equal at B = 16 for the staged kernel, which is ahead
// from B = 32.
constexpr int64_t kOneShotTiles = 8192;
// Staged launches are split so that each stays under 2^31 work-items (the
// dispatch's grid size is a 32-bit count): 2^22 workgroups, a 32 GiB share
// of the state.
constexpr int64_t kMaxStagedWgs = int64_t(1) << 22;

constexpr int kCachedTilesPerWave = 8;
constexpr int kCachedWaves = 4;

// gdn_pair's walk: 8-wave workgroups, one per CU.  Its 32-bit tile index may
// run one stride (grid x kPairWaves) past the last tile; the C ABI leaves
// 65536 of headroom below INT32_MAX, so the grid is capped at 8192
// workgroups.
constexpr int kPairWaves = 8;
constexpr int64_t kMaxGrid = 65536 / kPairWaves;
// Up to 2048 tiles (B * Hv <= 128) the pair runs one wave per tile: 21 %
// lower latency at B = 1 (3.4 vs 4.25 us), 14 % at B = 2; from B = 8 the
// walk is as fast or faster.
constexpr int64_t kPairOneShotTiles = 2048;
// Epochs of kEpochIters passes; each epoch workgroup reserves 96 KiB of
// (unused) LDS so that only one fits per CU, as in the persistent walk (more
// waves per CU measured slower).  Epoch launches are kept under 2^22
// workgroups (2^31 work-items); larger ones, states far beyond one GPU's
// memory, run as the plain persistent walk.
constexpr int kEpochIters = 4;
constexpr size_t kEpochLdsBytes = 96 * 1024;
constexpr int64_t kMaxEpochWgs = int64_t(1) << 22;

template <bool NT>
hipError_t launch_step_policy(const StepArgs &a, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>(a.B) * a.Hv * kTilesPerHead;
    const int nt = static_cast<int>(tiles);
    if (tiles <= kOneShotTiles) {
        k_step_tile<NT><<<dim3(static_cast<unsigned>(tiles)), dim3(64), 0, s>>>(a);
        return hipGetLastError();
    }
    // (a launch past 2^32 work-items, a state far beyond any GPU's memory,
    // falls back to the staged kernel with cached access)
    constexpr int64_t per_wg = kCachedTilesPerWave * kCachedWaves;
    if (!NT && (tiles + per_wg - 1) / per_wg * kCachedWaves * 64 <= INT64_C(0xffffffff)) {
        k_step_cached<kCachedTilesPerWave, kCachedWaves>
            <<<dim3(static_cast<unsigned>((tiles + per_wg - 1) / per_wg)), dim3(kCachedWaves * 64),
               0, s>>>(a, nt);
        return hipGetLastError();
    }
    // tiles = B * Hv * 16 is even; each launch stays under 2^31 work-items
    const int64_t pairs = tiles / kStagedTiles;
    for (int64_t p0 = 0; p0 < pairs; p0 += kMaxStagedWgs) {
        const int64_t wgs = pairs - p0 < kMaxStagedWgs ? pairs - p0 : kMaxStagedWgs;
        k_step_staged<NT><<<dim3(static_cast<unsigned>(wgs)), dim3(kStagedThreads), 0, s>>>(
            a, static_cast<int>(p0));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_step(const StepArgs &a, hipStream_t s, bool cached) {
    return cached ? launch_step_policy<false>(a, s) : launch_step_policy<true>(a, s);
}

// The pair kernel runs its persistent walk in epochs of kEpochIters passes
// at every size (one epoch, the plain walk, when it has at most that many
// passes): measured per 256 sequences, 257 against 265-271 us at B = 256,
// 255 against 285-295 us at B = 512..2048, and 6-7 % faster at B = 64, 128
// than one long persistent walk.
hipError_t launch_pair(const PairArgs &a, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>(a.B) * a.Hv * kTilesPerHead;
    const int nt = static_cast<int>(tiles);
    if (tiles <= kPairOneShotTiles) {
        k_pair<1><<<dim3(static_cast<unsigned>(tiles)), dim3(64), 0, s>>>(a, nt, nt, 1);
        return hipGetLastError();
    }
    int64_t full = static_cast<int64_t>(device_cus());
    if (full > kMaxGrid) full = kMaxGrid;
    const int64_t need = (tiles + kPairWaves - 1) / kPairWaves;
    const int grid = static_cast<int>(need < full ? need : full);
    const int64_t span = static_cast<int64_t>(grid) * kPairWaves * kEpochIters;
    const int64_t epochs = (tiles + span - 1) / span;
    if (epochs > 1 && grid * epochs <= kMaxEpochWgs) {
        k_pair<kPairWaves><<<dim3(static_cast<unsigned>(grid * epochs)), dim3(kPairWaves * 64),
                             kEpochLdsBytes, s>>>(a, nt, grid, kEpochIters);
    } else {
        const int64_t passes = (tiles + static_cast<int64_t>(grid) * kPairWaves - 1) /
                               (static_cast<int64_t>(grid) * kPairWaves);
        k_pair<kPairWaves><<<dim3(grid), dim3(kPairWaves * 64), 0, s>>>(
            a, nt, grid, static_cast<int>(passes));
    }
    return hipGetLastError();
}

}  // namespace gdn
