// gdn_step.hip - gdn_step and gdn_pair: the HBM-streaming one- and
// two-position kernels (persistent tile walk over the state).

#include "gdn_device.hpp"

namespace gdn {
namespace {

// ------------------------------------------------------------- gdn_step
// HBM-bound: the state is streamed once in and once out.  A persistent grid
// of one 8-wave workgroup per CU walks the tiles (8 rows = 4 KiB each) of all
// heads in a grid-stride loop, one tile per wave per iteration, so the
// addresses in flight at any moment form one contiguous window of ~8 MiB
// that advances through the state.  Measured on MI355X this beats one
// workgroup per head, more or fewer waves per CU, deeper per-wave queues and
// prefetching the next tile.  Workgroup g runs on XCD g % 8; the tile order
// is remapped so that the 16 tiles of a head go to workgroups of one XCD and
// its k and q are fetched into one L2 only.  Small launches (kOneShotTiles)
// instead give every tile a one-wave workgroup of its own.
constexpr int kStepWaves = 8;
constexpr int kXcds = 8;

// k_step's grid-stride walk over tiles u = (head = b * Hv + h, row block).
// With a stride of whole heads (an even grid) the row block never changes
// and (b, h) advance by constants, so the loop carries no integer division
// (measured ~2 % faster at B = 256 than dividing on every pass).
//
// Epochs: workgroups g = e * GE + l (l < GE) walk the tiles of epoch e,
// [e * E, (e + 1) * E) with E = GE * W * iters, together, like one
// persistent launch of GE workgroups.  Large launches use many short epochs:
// the dispatcher starts epoch e + 1's workgroups as epoch e's retire, which
// keeps the tiles in flight in one contiguous window (one long persistent
// walk lets the waves drift apart) and overlaps the end of one epoch with
// the start of the next.  A single epoch is the plain persistent walk.
struct TileWalk {
    int u, end, head, row, b, h;
    int stride, hstep, db, dh, Hv, grp;
    bool whole;

    // Positions this wave (of W per workgroup) on its first tile; false if
    // it has none.  GE: workgroups per epoch; iters: passes per epoch.
    template <int W>
    __device__ bool init(int n_tiles, int GE, int iters, int Hv_, int wave, int grp_) {
        const int epoch = blockIdx.x / GE;
        const int g = blockIdx.x - epoch * GE;
        const int lg = (GE % kXcds == 0) ? (g % kXcds) * (GE / kXcds) + g / kXcds : g;
        const int span = GE * W * iters;           // tiles per epoch
        const int base = epoch * span;
        end = n_tiles - base < span ? n_tiles : base + span;
        Hv = Hv_;
        grp = grp_;
        stride = GE * W;
        u = base + lg * W + wave;
        whole = (stride % kTilesPerHead) == 0;
        hstep = stride / kTilesPerHead;
        db = hstep / Hv;
        dh = hstep - db * Hv;
        if (u >= end) return false;
        place();
        return true;
    }

    // Advances to this wave's next tile; false when its epoch is done.
    __device__ bool next() {
        u += stride;
        if (u >= end) return false;
        if (whole) {
            head += hstep;
            h += dh;
            b += db;
            if (h >= Hv) {
                h -= Hv;
                ++b;
            }
        } else {
            place();
        }
        return true;
    }

    __device__ void place() {
        head = u / kTilesPerHead;
        row = (u % kTilesPerHead) * kRowsPerTile + grp;
        b = head / Hv;
        h = head - b * Hv;
    }
};

// kLateQ: fetch q only after the key reduction instead of together with the
// state.  When waves make several passes this measured ~3.5 % faster at
// B = 256 (the wave then pauses for q between its state stores and its next
// state loads; an explicit pause there gains about as much, so the spacing
// of each wave's reads and writes is the likely cause).  A single pass (small
// B) fetches q early, since there the extra L2 round trip is pure latency.
// W: waves per workgroup (kStepWaves for the persistent walk; 1 for small
// launches, where one wave per tile spreads the few tiles over every CU).
template <bool kLateQ, int W>
__global__ __launch_bounds__(W * 64) void k_step(StepArgs a, int n_tiles, int epoch_wgs,
                                                 int epoch_iters) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 7;

    TileWalk w;
    if (!w.template init<W>(n_tiles, epoch_wgs, epoch_iters, a.Hv, wave, lane >> 3)) return;
    do {
        int kh = w.h;
        while (kh >= a.Hk) kh -= a.Hk;                        // key-head broadcast
        float *Mrow = a.state + static_cast<int64_t>(w.head) * (D * D) + w.row * D;
        const float *kp = a.k + w.b * a.qk_bstride + kh * D;
        const float *qp = a.q + w.b * a.qk_bstride + kh * D;
        const float gt = a.gate[w.head];
        const float bt = a.beta[w.head];
        const float vj = a.v[w.b * a.v_bstride + w.h * D + w.row];
        RowSlice r;
        load_row<true>(r, Mrow, c);
        VecSlice kv, qv;
        load_vec(kv, kp, c);
        if constexpr (!kLateQ) load_vec(qv, qp, c);
        const float e = expf(gt);

        const float sk = group_sum(head_part(r, kv, e));     // steps 1-2
        if constexpr (kLateQ) {
            __builtin_amdgcn_sched_barrier(0);                // keep the q loads here
            load_vec(qv, qp, c);
            __builtin_amdgcn_sched_barrier(0);
        }
        update_part(r, (vj - sk) * bt, kv);                   // steps 3-4
        store_row<true>(Mrow, r, c);
        const float o = group_sum(dot_part(r, qv)) * kInvSqrtD;   // step 5
        if (c == 0) a.out[static_cast<int64_t>(w.head) * D + w.row] = o;
    } while (w.next());
}

// ------------------------------------------------------------- gdn_pair
// Speculative two-position step (docs.rs "Module linear_core", gdn_pair):
// the same persistent tile walk as k_step; each row is read once, advanced
// by position 1 and written back to `state` (committed), then advanced by
// position 2 in registers and written to `state_next` (tentative).  Three
// state transfers instead of the four of two separate steps.  Unlike k_step
// this kernel keeps q with the other loads and computes its tile indices
// afresh each pass: with one read and two writes per row, fetching q late
// measured 7 % slower and the incremental walk 1 % slower on MI355X.  W:
// waves per workgroup, as in k_step (1 for small launches).  Workgroups are
// grouped in epochs of GE as in k_step's walk: epoch e walks tiles
// [e * span, (e + 1) * span), span = GE * W * iters.
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

#ifndef GDN_STEP_WGS_PER_CU
#define GDN_STEP_WGS_PER_CU 1
#endif

// The walks' 32-bit tile index may run one stride (grid x kStepWaves) past
// the last tile; the C ABI leaves 65536 of headroom below INT32_MAX, so the
// grid is capped at 8192 workgroups.
constexpr int64_t kMaxGrid = 65536 / kStepWaves;

// Launches of up to this many tiles (B * Hv <= 512) run one wave per tile:
// measured 21 % lower latency at B = 1 (2.5 vs 3.2 us per call over 36
// layers), 14 % at B = 2 and 2-4 % at B = 8..16 than the persistent walk on
// 8-wave workgroups, which wins again from B = 64.
constexpr int64_t kOneShotTiles = 8192;
// The same for gdn_pair up to 2048 tiles (B * Hv <= 128): 21 % lower latency
// at B = 1 (3.4 vs 4.25 us), 14 % at B = 2; from B = 8 the walk is as fast
// or faster.
constexpr int64_t kPairOneShotTiles = 2048;

// Launches with more passes per wave than this run as epochs of
// kEpochIters passes (measured per 256 sequences: 172 vs 175 us at B = 512,
// 169 vs 195 us at B = 9216, where the 36 layers of the B = 256 decode in one
// call take 6.1 ms against 6.2 ms for 36 separate launches).  Each epoch
// workgroup reserves 96 KiB of (unused) LDS so that only one fits per CU,
// as in the persistent walk; more waves per CU measured slower.
// Epoch launches are kept under 2^22 workgroups (2^31 work-items: the
// dispatch's grid size is a 32-bit count of work-items); larger ones, states
// far beyond one GPU's memory, fall back to the persistent walk.
constexpr int kPersistentIters = 64;
constexpr int kEpochIters = 4;
constexpr size_t kEpochLdsBytes = 96 * 1024;
constexpr int64_t kMaxEpochWgs = int64_t(1) << 22;

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>(a.B) * a.Hv * kTilesPerHead;
    const int nt = static_cast<int>(tiles);
    if (tiles <= kOneShotTiles) {
        k_step<false, 1><<<dim3(static_cast<unsigned>(tiles)), dim3(64), 0, s>>>(a, nt, nt, 1);
        return hipGetLastError();
    }
    int64_t full = device_cus() * static_cast<int64_t>(GDN_STEP_WGS_PER_CU);
    if (full > kMaxGrid) full = kMaxGrid;
    const int64_t need = (tiles + kStepWaves - 1) / kStepWaves;
    const int grid = static_cast<int>(need < full ? need : full);
    const int64_t passes = (tiles + static_cast<int64_t>(grid) * kStepWaves - 1) /
                           (static_cast<int64_t>(grid) * kStepWaves);
    const int64_t span = static_cast<int64_t>(grid) * kStepWaves * kEpochIters;
    const int64_t epochs = (tiles + span - 1) / span;
    if (passes > kPersistentIters && grid * epochs <= kMaxEpochWgs) {
        k_step<true, kStepWaves><<<dim3(static_cast<unsigned>(grid * epochs)),
                                   dim3(kStepWaves * 64), kEpochLdsBytes, s>>>(a, nt, grid,
                                                                               kEpochIters);
    } else if (passes > 1) {
        k_step<true, kStepWaves><<<dim3(grid), dim3(kStepWaves * 64), 0, s>>>(
            a, nt, grid, static_cast<int>(passes));
    } else {
        k_step<false, kStepWaves><<<dim3(grid), dim3(kStepWaves * 64), 0, s>>>(a, nt, grid, 1);
    }
    return hipGetLastError();
}

// The pair kernel runs its persistent walk in epochs of kEpochIters passes
// at every size (one epoch, the plain walk, when it has at most that many
// passes): measured per 256 sequences, 257 against 265-271 us at B = 256,
// 255 against 285-295 us at B = 512..2048, and 6-7 % faster at B = 64, 128.
// Its read-once-write-twice traffic gains from the epochs' tighter window
// where the step's read-once-write-once traffic does not (at B <= 256).
hipError_t launch_pair(const PairArgs &a, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>(a.B) * a.Hv * kTilesPerHead;
    const int nt = static_cast<int>(tiles);
    if (tiles <= kPairOneShotTiles) {
        k_pair<1><<<dim3(static_cast<unsigned>(tiles)), dim3(64), 0, s>>>(a, nt, nt, 1);
        return hipGetLastError();
    }
    int64_t full = device_cus() * static_cast<int64_t>(GDN_STEP_WGS_PER_CU);
    if (full > kMaxGrid) full = kMaxGrid;
    const int64_t need = (tiles + kStepWaves - 1) / kStepWaves;
    const int grid = static_cast<int>(need < full ? need : full);
    const int64_t span = static_cast<int64_t>(grid) * kStepWaves * kEpochIters;
    const int64_t epochs = (tiles + span - 1) / span;
    if (epochs > 1 && grid * epochs <= kMaxEpochWgs) {
        k_pair<kStepWaves><<<dim3(static_cast<unsigned>(grid * epochs)), dim3(kStepWaves * 64),
                             kEpochLdsBytes, s>>>(a, nt, grid, kEpochIters);
    } else {
        const int64_t passes = (tiles + static_cast<int64_t>(grid) * kStepWaves - 1) /
                               (static_cast<int64_t>(grid) * kStepWaves);
        k_pair<kStepWaves><<<dim3(grid), dim3(kStepWaves * 64), 0, s>>>(
            a, nt, grid, static_cast<int>(passes));
    }
    return hipGetLastError();
}

}  // namespace gdn
