// launch.hpp -- the scan kernel template and its host-side launch logic,
// shared by the translation units that define the C ABI of include/lrs.h.
//
// One kernel template serves all seven estimators and the generic scan.  The [N, T] input is one
// flat stream of N*T elements; row ends are segment boundaries like episode
// ends, so rows never need separate handling.  A block owns a tile of
// E*64*W consecutive elements; each lane owns E of them:
//   1. vector-load the raw streams once, build (alpha, beta) in registers;
//   2. compose the lane's E maps serially, then a 6-step wave64 scan;
//   3. combine the W wave aggregates through LDS;
//   4. if rows straddle tiles, obtain the value entering the tile from the
//      neighbouring tiles' published aggregates (decoupled look-back over
//      aggregates only, in ticket order);
//   5. apply the carry, run each lane's recursion, store once.
// Nothing but the final outputs (and 16 bytes of aggregate per tile on the
// look-back path) is written to HBM: one read of each input, one write of
// each output, as the rl-triton paper's fused kernels do (gist.science
// technical summary, Methodology 2).
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/lrs.h"
#include "estimators.hpp"

namespace lrs {

struct Sched {
    uint64_t total;      // N*T
    uint8_t* ws;         // workspace (look-back only)
    uint32_t T;
    uint32_t num_tiles;
    // Look-back only.  When every row spans a whole number of tiles and
    // there are many rows, tiles_per_row > 1 and block b takes position
    // b / rows (counted from the end of the row for backward scans) of row
    // b % rows: all rows' outermost tiles first, so a tile's neighbour ran
    // `rows` blocks earlier and its aggregate is usually published before
    // this block needs it.  Otherwise tiles_per_row = 0 and tiles are taken
    // in flat order.
    uint32_t tiles_per_row;
    uint32_t rows;
    int lookback;
    int vec;
    // Division by T without a divide: shifts when T is a power of two
    // (log2T), else a multiply by magic = floor(2^64 / T) + 1.
    uint64_t magic;
    uint32_t log2T;
    int pow2;
    // T is a multiple of the elements per lane: a lane's elements never
    // cross a row end, so their row-start and row-end bits take two compares.
    int lane_in_row;
};

// Row and step of a flat index below 2^35.  The multiply-high estimate
// floor(n * magic / 2^64) exceeds n / T by less than n / 2^64, so it is the
// quotient or one above it; one correction makes it exact.
__device__ __forceinline__ void split_index(uint64_t n, const Sched& s, uint64_t& row, uint32_t& t)
{
    if (s.pow2) {
        row = n >> s.log2T;
        t = (uint32_t)n & (s.T - 1u);
        return;
    }
    uint64_t q = __umul64hi(n, s.magic);
    int64_t r = (int64_t)(n - q * s.T);
    if (r < 0) {
        --q;
        r += s.T;
    }
    row = q;
    t = (uint32_t)r;
}

// Same for a 32-bit index u: the overshoot u / 2^64 * (magic - 2^64 / T) is
// below 2^-32 < 1 / T, so the estimate is already the quotient.  Only the
// high 64 bits of the 96-bit product u * magic are formed.
__device__ __forceinline__ void split_index32(uint32_t u, const Sched& s, uint32_t& q, uint32_t& t)
{
    if (s.pow2) {
        q = u >> s.log2T;
        t = u & (s.T - 1u);
        return;
    }
    const uint32_t mlo = (uint32_t)s.magic, mhi = (uint32_t)(s.magic >> 32);
    q = (uint32_t)(((uint64_t)u * mhi + __umulhi(u, mlo)) >> 32);
    t = u - q * s.T;
}

// The tile block b works on.  Look-back launches take tiles so that every
// tile a block may wait for belongs to a block of lower index (workgroups of
// a dispatch start in index order, so that block is running or done):
// position-major order (all rows' outermost tiles first, counted from the
// row end for backward scans) when every row spans tiles_per_row > 1 whole
// tiles, else flat order from the end of the array (backward) or its start
// (forward).  Launches without carries take tiles in flat order.  Shared by
// the kernel and the host's schedule diagnostics (lrs_debug_schedule).
struct TilePlace {
    uint32_t tile;
    uint32_t row;  // position-major only: the tile's row and its place in it
    uint32_t pos;
};

__host__ __device__ inline TilePlace place_tile(uint32_t b, const Sched& s, bool backward)
{
    if (s.lookback && s.tiles_per_row > 1) {
        const uint32_t pos = b / s.rows, row = b % s.rows;
        const uint32_t p = backward ? s.tiles_per_row - 1u - pos : pos;
        return {row * s.tiles_per_row + p, row, p};
    }
    return {(s.lookback && backward) ? s.num_tiles - 1u - b : b, 0u, 0u};
}

template <class A, int W>
struct BlockShared {
    A a[W];
    A b[W];
    A carry;
    uint32_t open;
};

// Everything after the positions are known.  F: the tile lies wholly inside
// the array and the base pointers are vector aligned (straight-line vector
// loads and stores); otherwise every access is guarded by the lane's count.
template <class Op, int E, int W, class A, bool F, bool NT, bool S>
__device__ __forceinline__ void tile_body(const typename Op::Args& args, const Sched& s,
                                          uint32_t tile, const Pos<E, F, false, NT, S>& P, const Ctx& c,
                                          BlockShared<A, W>& sh)
{
    using T = typename Op::T;  // A: the composition type (fp32 or fp64 for fp32 maps)
    constexpr bool kB = Op::kBackward;
    const int tid = threadIdx.x;
    const int lane = c.lane;
    const int wave = tid / kWave;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(s.ws);
    uint64_t* rec = reinterpret_cast<uint64_t*>(s.ws + sizeof(WsHeader));

    // The block count (which returns the launch tag) and the neighbour's record
    // are issued first, in flight with the tile's loads.  (Publishing one
    // record per wave instead, so that a waiting neighbour needs only the
    // waves nearest to it, measured 15-90% slower on long rows: every wave
    // then needs the launch tag before the block's barrier, and the reads of
    // the one header word that carries it serialize.)
    const bool far_most = kB ? (tile == s.num_tiles - 1u) : (tile == 0u);
    Record early{{0, 0, 0, 0}};
    uint64_t entry = 0;
    uint32_t tag = 0, top_seen = ~0u;
    if (s.lookback && wave == 0) {
        if (lane == 0) entry = count_block(hdr, blockIdx.x);
        if (!far_most) early = read_adjacent<kB, A>(rec, tile);
    }

    T alpha[E], beta[E];
    typename Op::State st;
    Op::prepare(args, P, c, alpha, beta, st);

    // Lane aggregate, then the wave scan.  fp32 maps keep a in fp32 but form
    // the product of the lane's betas in fp64 and round it once: with a
    // constant beta every lane would otherwise hold the same rounded beta^E,
    // and the scan would multiply that one relative error once per lane of
    // distance.
    Aff<A> agg = identity<A>();
    if constexpr (std::is_same<A, float>::value) {
        float a = 0.0f;
        double b = 1.0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int j = kB ? E - 1 - k : k;
            a = fmaf(beta[j], a, alpha[j]);
            b *= (double)beta[j];
        }
        agg = {a, (float)b};
    } else if (kB) {
#pragma unroll
        for (int j = E - 1; j >= 0; --j) agg = combine(Aff<A>{A(alpha[j]), A(beta[j])}, agg);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) agg = combine(Aff<A>{A(alpha[j]), A(beta[j])}, agg);
    }
    const Aff<A> inc = lane_scan(agg);  // lane 63 holds the wave total
    const Aff<A> exc = lane_exclusive(inc);

    // The tile's far boundary element (backward: its last; forward: its
    // first) sits in lane 0 of wave W-1 (backward) or of wave 0 (forward).
    Aff<A> tile_agg = identity<A>(), beyond = identity<A>();
    A carry = A(0);
    if constexpr (W == 1) {
        // One wave per block: everything stays in registers, no barrier.
        tile_agg = readlane(inc, kWave - 1);
        if (s.lookback) {
            tag = launch_tag(entry);
            if (lane == 0) top_seen = count_group(hdr, entry, s.num_tiles, blockIdx.x);
            const uint32_t open = readlane(Op::far_open(st) ? 1u : 0u, 0);
            if (lane == 0) publish_aggregate<A>(rec, tile, tag, tile_agg);
            if (!far_most && open)
                carry = lookback_carry<kB, A>(rec, tile, s.num_tiles, tag, lane, &hdr->error, early);
        }
    } else {
        if (lane == kWave - 1) {
            sh.a[wave] = inc.a;
            sh.b[wave] = inc.b;
        }
        if (lane == 0 && wave == (kB ? W - 1 : 0)) sh.open = Op::far_open(st) ? 1u : 0u;
        __syncthreads();

        // Compose the wave totals: lane v holds wave v's; a row scan gives
        // the whole tile and, for each wave, the waves beyond it (backward:
        // the later waves; forward: the earlier ones).
        Aff<A> x = identity<A>();
        if (lane < W) x = {sh.a[lane], sh.b[lane]};
        x = row_scan<kB, W>(x);
        const int w = __builtin_amdgcn_readfirstlane(wave);
        tile_agg = readlane(x, kB ? 0 : W - 1);
        if (kB ? (w < W - 1) : (w > 0)) beyond = readlane(x, kB ? w + 1 : w - 1);

        if (s.lookback) {
            if (wave == 0) {
                tag = launch_tag(entry);
                if (lane == 0) top_seen = count_group(hdr, entry, s.num_tiles, blockIdx.x);
                if (lane == 0) publish_aggregate<A>(rec, tile, tag, tile_agg);
                A cin = A(0);
                if (!far_most && sh.open)
                    cin = lookback_carry<kB, A>(rec, tile, s.num_tiles, tag, lane, &hdr->error,
                                                early);
                if (lane == 0) sh.carry = cin;
            }
            __syncthreads();
            carry = sh.carry;
        }
    }

    const A wave_in = apply(beyond, carry);
    const T lane_in = T(apply(exc, wave_in));
    Op::finish(args, P, c, alpha, beta, st, lane_in);
    if (s.lookback && wave == 0 && lane == 0) close_launch(hdr, top_seen, s.num_tiles, tag);
}

template <class Op, int E, int W, class A, bool NT, bool S>
__device__ __forceinline__ void scan_body(const typename Op::Args& args, const Sched& s)
{
    warm_kernargs<kernarg_bytes<typename Op::Args, Sched>()>();
    constexpr bool kB = Op::kBackward;
    constexpr uint32_t kTile = (uint32_t)E * kWave * W;
    __shared__ BlockShared<A, W> sh;

    const int tid = threadIdx.x;
    // On the look-back path the tile a block depends on always belongs to a
    // block of lower index (place_tile).
    const TilePlace tp = place_tile(blockIdx.x, s, kB);
    const uint32_t tile = tp.tile;
    uint64_t tile_row;
    uint32_t tile_t;
    if (s.lookback && s.tiles_per_row > 1) {
        tile_row = tp.row;
        tile_t = tp.pos * kTile;
    } else {
        split_index((uint64_t)tile * kTile, s, tile_row, tile_t);
    }
    const uint64_t tile_start = (uint64_t)tile * kTile;

    // Where this lane's elements sit in their rows.
    // Backward estimators give lane L chunk 63-L of its wave (see scan_core.hpp).
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t chunk = (tid - lane) + (kB ? kWave - 1 - lane : lane);
    const uint32_t off = chunk * E;
    const uint64_t i0 = tile_start + off;
    const int count = i0 >= s.total ? 0 : (int)((s.total - i0) < (uint64_t)E ? (s.total - i0) : E);
    uint32_t q, t;
    split_index32(tile_t + off, s, q, t);  // tile_t + off < 2^31 + 2^14
    const uint64_t n0 = tile_row + q;
    uint32_t last = 0, first = 0;
    if (s.lane_in_row) {
        if (t + (uint32_t)E == s.T) last = 1u << (E - 1);
        if (t == 0) first = 1u;
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (t == s.T - 1) last |= 1u << j;
            if (t == 0) first |= 1u << j;
            t = (t == s.T - 1) ? 0u : t + 1u;
        }
    }
    const Ctx c{s.total, s.T, tid & (kWave - 1), s.vec != 0};

    if (s.vec && tile_start + kTile <= s.total && s.T >= (uint32_t)E) {
        const Pos<E, true, false, NT, S> P{i0, n0, E, last, first, 0, n0};
        tile_body<Op, E, W, A, true, NT, S>(args, s, tile, P, c, sh);
    } else {
        const uint32_t valid = (count >= 32) ? ~0u : ((1u << count) - 1u);
        const Pos<E, false, false, NT, S> P{i0, n0, count, last & valid, first & valid, 0, n0};
        tile_body<Op, E, W, A, false, NT, S>(args, s, tile, P, c, sh);
    }
}

template <class Op, int E, int W, class A, bool NT, bool S>
__global__ __launch_bounds__(W * kWave) void scan_kernel(const typename Op::Args args, const Sched s)
{
    scan_body<Op, E, W, A, NT, S>(args, s);
}

// The same kernel with its scalar registers capped at 72: a gfx950 SIMD held
// eight waves of a kernel only while it needed at most about that many
// (measured from per-block timestamps: kernels of 68-72 SGPRs ran eight waves
// per SIMD, one of 87 six, ones of 77 and 88 could not fit a second 16-wave
// block per CU), although the compiler estimates full occupancy up to about
// 100.  The excess spills to vector lanes.
template <class Op, int E, int W, class A, bool NT, bool S>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_num_sgpr(72))) void scan_kernel_lean(
    const typename Op::Args args, const Sched s)
{
    scan_body<Op, E, W, A, NT, S>(args, s);
}

// Look-back launches with four or more waves per block take the capped
// kernel for maps composed in fp64, for strided arrays (each array's row gap
// adds scalar registers: GAE+trunc 72 -> 84, Retrace+trunc 77 -> 93; capped,
// strided Retrace+trunc at 64 x 131072 went 48.1 -> 37.7 us, GAE+trunc
// 27.0 -> 25.0, level with contiguous arrays) and for ops that ask for it
// (kLeanSgprs): there a block waiting for its carry holds its slot, and more
// resident blocks keep loads in flight.  Launches without carries keep the
// uncapped kernel (the capped one measured 1-3% slower there: the spills cost
// and the loads already saturate).
template <class Op, int W, class A, bool S>
constexpr bool lean_sgprs()
{
    return W >= 4 && (std::is_same<A, double>::value || Op::kLeanSgprs || S);
}

// ------------------------------------------------------------ host side


struct Cfg {
    int E, W;
    uint32_t tile() const { return (uint32_t)(E * kWave * W); }
};
constexpr int kNumCfg = 7;  // ordered by tile size
constexpr Cfg kCfgs[kNumCfg] = {{4, 1}, {4, 4}, {8, 4}, {4, 8}, {16, 4}, {4, 16}, {8, 16}};
constexpr uint32_t kMinTile = 256;  // smallest tile the look-back path may use
constexpr int kAlignedCfgs[5] = {0, 1, 3, 5, 6};  // 4x1, 4x4, 4x8, 4x16, 8x16
constexpr uint32_t kNarrowMaxTile = 2048;  // ops without kWideTiles stop at 4x8
constexpr uint64_t kWideMinTiles = 1024;   // whole-row tiles above 2048 need this many
constexpr int kLookbackCfg = 3;            // 4x8: 2048-element tiles
constexpr int kLookbackCfgWide4 = 5;       // 4x16: prefix sums, maps composed in fp64
constexpr uint64_t kFewWide4Tiles = 128;   // fewer 4x16 look-back tiles than this: 4x8
constexpr int kLookbackCfgLight = 2;       // 8x4: kLbLight ops, below kWideMinTiles
// 16-bit data: eight elements per lane make each data load 16 bytes
constexpr int kLookbackCfgHalfWide = 6;    // 8x16: 8192-element tiles (ops with kWideTiles)
constexpr int kLookbackCfgHalf = 2;        // 8x4: 2048-element tiles
constexpr int64_t kPositionMajorRows = 1024;
// Largest beta for which fp32 maps compose in fp32 (see run()).
constexpr float kFp32BetaMax = 0.99f;

// Defined in abi.hip.
extern std::atomic<int> g_force_lookback;
extern std::atomic<int> g_forced_cfg;
extern std::atomic<int> g_forced_tm_waves;  // 0: automatic
extern thread_local char g_err[512];

inline lrs_status fail(lrs_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

inline bool valid_sizes(int64_t N, int64_t T)
{
    if (N < 1 || T < 1 || T >= (int64_t(1) << 31)) return false;
    if (N > (int64_t(1) << 34) / T) return false;
    return N * T < (int64_t(1) << 34);
}

inline size_t workspace_bytes_for(uint64_t total)
{
    return sizeof(WsHeader) + 8 * kRecordWords * ((total + kMinTile - 1) / kMinTile);
}

// Pick the tile.  Measured on MI355X: four elements per lane stream best
// for tiles up to 2048 elements, and a tile that holds whole rows needs no
// look-back, so: the smallest tile that holds whole rows, among 256, 1024
// and 2048 elements (4 per lane) and, for ops whose registers allow it and
// when at least kWideMinTiles such tiles fill the chip, 4096 (4 per lane,
// 16 waves) and 8192 (8 per lane, 16 waves).  Otherwise the look-back path:
// fp32 data on 2048-element tiles of eight waves; 16-bit data on eight
// elements per lane (16-byte loads), in 8192-element tiles for ops with
// kWideTiles when at least kWideMinTiles of them fill the chip, else in
// 2048-element tiles of four waves.  16-bit rows that divide 2048 also take
// those 2048-element tiles when at least kWideMinTiles of them fill the chip.
// Long fp32 rows (measured at 64 x 131072 and 1024 x 16384 on inputs
// cycled over >= 1 GiB) follow the op's LookbackTile: kLbLight ops take
// eight elements per lane, in 8192-element tiles when kWideMinTiles of them
// fill the chip, else in 2048-element ones (also when composed in fp64);
// kLbWide4 ops, and kLbNarrow ops composed in fp64, 4096-element tiles of
// four per lane (kLbWide4 ops on fewer than kFewWide4Tiles of them: 2048);
// kLbNarrow ops 2048-element tiles of four per lane.
inline int choose_cfg(uint64_t total, uint64_t T, bool wide_ok, LookbackTile lb, bool fp64, int elem_bytes,
                      bool* lookback)
{
    const int forced = g_forced_cfg.load();
    const bool force_lb = g_force_lookback.load() != 0;
    if (forced >= 0 || force_lb) {
        const int c = forced >= 0 ? forced : 0;
        const uint64_t tiles = (total + kCfgs[c].tile() - 1) / kCfgs[c].tile();
        *lookback = force_lb || (tiles > 1 && kCfgs[c].tile() % T != 0);
        return c;
    }
    if (elem_bytes == 2) {
        // 16-bit rows that fit 2048-element tiles: eight elements per lane
        // (16-byte loads) when enough such tiles fill the chip
        const Cfg& h = kCfgs[kLookbackCfgHalf];
        if (h.tile() % T == 0 && (total + h.tile() - 1) / h.tile() >= kWideMinTiles) {
            *lookback = false;
            return kLookbackCfgHalf;
        }
    }
    for (int c : kAlignedCfgs) {
        const uint64_t tiles = (total + kCfgs[c].tile() - 1) / kCfgs[c].tile();
        if (kCfgs[c].tile() > kNarrowMaxTile && (!wide_ok || tiles < kWideMinTiles)) break;
        if (kCfgs[c].tile() % T == 0 || tiles == 1) {
            *lookback = false;
            return c;
        }
    }
    *lookback = true;
    const uint64_t wide_tiles = (total + kCfgs[kLookbackCfgHalfWide].tile() - 1) /
                                kCfgs[kLookbackCfgHalfWide].tile();
    if (elem_bytes == 2)
        return wide_ok && wide_tiles >= kWideMinTiles ? kLookbackCfgHalfWide : kLookbackCfgHalf;
    if (lb == kLbWide4 || (fp64 && lb == kLbNarrow)) {
        // Retrace and the affine scan on fewer 4096-element tiles than half
        // the device's CUs: 2048-element tiles, twice the blocks (4096 x 100,
        // 100 tiles: Retrace 12-14% and the affine scan 11% faster; at 150-250
        // tiles Retrace measured up to 5% slower, the affine scan 4-6% faster)
        const uint64_t wide4_tiles = (total + kCfgs[kLookbackCfgWide4].tile() - 1) /
                                     kCfgs[kLookbackCfgWide4].tile();
        if (lb == kLbWide4 && wide4_tiles < kFewWide4Tiles) return kLookbackCfg;
        return kLookbackCfgWide4;
    }
    if (lb == kLbLight) return wide_tiles >= kWideMinTiles ? kLookbackCfgHalfWide : kLookbackCfgLight;
    return kLookbackCfg;
}

// Work items of a launch over `total` elements on tiles of configuration c.
inline uint64_t launch_items(uint64_t total, const Cfg& c)
{
    return (total + c.tile() - 1) / c.tile() * (uint64_t)(c.W * kWave);
}
constexpr uint64_t kMaxLaunchItems = 0xffffffffull;  // a dispatch's grid size is 32-bit
constexpr int kWideCfg = 6;                          // 8x16: 8192-element tiles

inline bool aligned(const void* p, uintptr_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; }

// Compute units of the device that `stream` belongs to, queried once per
// device (256 on MI355X; also the answer if the query fails).
inline uint32_t device_cus(hipStream_t stream)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<uint32_t> cache[kMaxDevices];
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    uint32_t n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        n = (uint32_t)v;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <class Op, int E, int W, class A, bool S, bool NT = false>
hipError_t launch_cfg(const typename Op::Args& a, const Sched& s, hipStream_t stream)
{
    void* kargs[] = {(void*)&a, (void*)&s};
    const void* k = (const void*)&scan_kernel<Op, E, W, A, NT, S>;
    if constexpr (lean_sgprs<Op, W, A, S>())
        if (s.lookback) k = (const void*)&scan_kernel_lean<Op, E, W, A, NT, S>;
    return hipLaunchKernel(k, dim3(s.num_tiles), dim3(W * kWave), kargs, 0, stream);
}

// S: some array of the call has a row stride other than its row length.
template <template <int> class Op, class A, bool S>
hipError_t launch_any(int cfg, const typename Op<4>::Args& a, const Sched& s, hipStream_t stream)
{
    constexpr bool kNT = Op<4>::kStreamLoads;
    switch (cfg) {
        case 0: return launch_cfg<Op<4>, 4, 1, A, S>(a, s, stream);
        case 1: return launch_cfg<Op<4>, 4, 4, A, S>(a, s, stream);
        // Non-temporal input loads on long rows: the look-back tiles (4x8,
        // and 8x4 for 16-bit data) and the 8192-element tiles.
        case 2:
            return s.lookback ? launch_cfg<Op<8>, 8, 4, A, S, kNT>(a, s, stream)
                              : launch_cfg<Op<8>, 8, 4, A, S>(a, s, stream);
        case 3:
            return s.lookback ? launch_cfg<Op<4>, 4, 8, A, S, kNT>(a, s, stream)
                              : launch_cfg<Op<4>, 4, 8, A, S>(a, s, stream);
        case 4: return launch_cfg<Op<16>, 16, 4, A, S>(a, s, stream);
        case 5: return launch_cfg<Op<4>, 4, 16, A, S>(a, s, stream);
        default: return launch_cfg<Op<8>, 8, 16, A, S, kNT>(a, s, stream);
    }
}

template <template <int> class Op, class A>
hipError_t launch_any(bool strided, int cfg, const typename Op<4>::Args& a, const Sched& s,
                      hipStream_t stream)
{
    return strided ? launch_any<Op, A, true>(cfg, a, s, stream)
                   : launch_any<Op, A, false>(cfg, a, s, stream);
}

// The schedule of a row-major call: tile shape (an index into kCfgs), the
// Sched fields that do not depend on pointers, and the composition type.
struct Plan {
    int cfg;
    bool fp64;
    Sched s;
};

// fp32 maps compose in fp64 when the call's betas may come close to 1:
// long near-undamped chains (sums) accumulate fp32 rounding beyond the
// parity bound, while damped chains forget it within ~1/(1 - beta) steps.
template <template <int> class Op>
Plan plan_row_major(int64_t N, int64_t T, float beta_max)
{
    const uint64_t total = (uint64_t)N * (uint64_t)T;
    bool lookback = false;
    using Val = typename Op<4>::T;
    const bool fp64 = std::is_same<Val, float>::value && beta_max > kFp32BetaMax;
    int cfg = choose_cfg(total, (uint64_t)T, Op<4>::kWideTiles, Op<4>::kLookbackTile, fp64,
                         Op<4>::kElemBytes, &lookback);
    // A dispatch holds at most 2^32 - 1 work items.  Four elements per lane
    // exceed that only within one tile of 2^34 elements; eight elements per
    // lane in 8192-element tiles stay below 2^31 for every accepted size.
    if (launch_items(total, kCfgs[cfg]) > kMaxLaunchItems) {
        cfg = kWideCfg;
        const uint64_t tiles = (total + kCfgs[cfg].tile() - 1) / kCfgs[cfg].tile();
        lookback = lookback || (tiles > 1 && kCfgs[cfg].tile() % (uint64_t)T != 0);
    }
    const Cfg& k = kCfgs[cfg];
    Sched s{};
    s.total = total;
    s.T = (uint32_t)T;
    s.num_tiles = (uint32_t)((total + k.tile() - 1) / k.tile());
    s.lookback = lookback ? 1 : 0;
    // Position-major order pays when rows outnumber the blocks resident at
    // once (about 1000 here), so that a tile's neighbour has finished; with
    // fewer rows, flat order keeps concurrent blocks on contiguous memory.
    if ((uint64_t)T % k.tile() == 0 && N >= kPositionMajorRows) {
        s.tiles_per_row = (uint32_t)((uint64_t)T / k.tile());
        s.rows = (uint32_t)N;
    } else {
        s.tiles_per_row = 0;
        s.rows = 0;
    }
    s.pow2 = (T & (T - 1)) == 0 ? 1 : 0;
    s.log2T = 0;
    while ((1ull << s.log2T) < (uint64_t)T) ++s.log2T;
    s.magic = s.pow2 ? 0 : ~0ull / (uint64_t)T + 1ull;  // T >= 3 here: no overflow
    s.lane_in_row = (uint64_t)T % (uint64_t)k.E == 0 ? 1 : 0;
    s.ws = nullptr;
    s.vec = 0;
    return Plan{cfg, fp64, s};
}

// An [N, T] array argument as the vector-access decision sees it.
struct ArrayRef {
    const void* p;
    uint64_t gap;    // row stride - seq_len, in elements
    int elem_bytes;  // 1 (masks), 2 or 4
};

// Shared checks and launch.  arrays: every [N, T] array the kernel may
// vector-load or -store, for the alignment decision.
template <template <int> class Op>
lrs_status run(const char* name, int64_t N, int64_t T, float beta_max, const typename Op<4>::Args& a,
               const ArrayRef* arrays, int narrays, void* ws, size_t ws_bytes, hipStream_t stream)
{
    using Val = typename Op<4>::T;
    Plan plan = plan_row_major<Op>(N, T, beta_max);
    const int cfg = plan.cfg;
    const bool fp64 = plan.fp64;
    const Cfg& k = kCfgs[cfg];
    Sched s = plan.s;
    s.ws = static_cast<uint8_t*>(ws);
    if (s.lookback) {
        const size_t need = sizeof(WsHeader) + 8 * kRecordWords * (size_t)s.num_tiles;
        if (ws == nullptr || ws_bytes < need)
            return fail(LRS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name,
                        need, ws == nullptr ? (size_t)0 : ws_bytes);
        if (!aligned(ws, 16)) return fail(LRS_ERR_WORKSPACE, "%s: workspace not 16-byte aligned", name);
    }
    // One vector access per lane covers its E elements, at most 16 bytes: every
    // array's base must be aligned to it, and a strided array's rows too, with
    // no lane straddling a row end (seq_len a multiple of E), so that a lane's
    // elements stay contiguous.
    bool vec = true, strided = false;
    for (int i = 0; i < narrays; ++i) {
        const ArrayRef& r = arrays[i];
        if (r.p == nullptr) continue;
        strided = strided || r.gap != 0;
        const uint64_t align = (uint64_t)k.E * r.elem_bytes < 16 ? (uint64_t)k.E * r.elem_bytes : 16;
        vec = vec && aligned(r.p, (uintptr_t)align);
        if (r.gap != 0) vec = vec && s.lane_in_row && (r.gap * (uint64_t)r.elem_bytes) % align == 0;
    }
    s.vec = vec ? 1 : 0;
    hipError_t e;
    if constexpr (std::is_same<Val, float>::value)
        e = fp64 ? launch_any<Op, double>(strided, cfg, a, s, stream)
                 : launch_any<Op, float>(strided, cfg, a, s, stream);
    else
        e = launch_any<Op, Val>(strided, cfg, a, s, stream);
    if (e != hipSuccess)
        return fail(LRS_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    g_err[0] = '\0';
    return LRS_OK;
}

inline bool unit_interval(float x) { return x >= 0.0f && x <= 1.0f; }  // false for NaN
inline bool positive(float x) { return x > 0.0f; }                       // +inf allowed, NaN not

inline lrs_status check_common(const char* name, int64_t N, int64_t T)
{
    if (!valid_sizes(N, T))
        return fail(LRS_ERR_INVALID_ARG,
                    "%s: need num_envs >= 1, 1 <= seq_len < 2^31, num_envs*seq_len < 2^34 "
                    "(got %lld x %lld)",
                    name, (long long)N, (long long)T);
    return LRS_OK;
}

inline lrs_status check_boundary(const char* name, const uint8_t* term, const uint8_t* trunc,
                                 const void* tv)
{
    if (term == nullptr) return fail(LRS_ERR_INVALID_ARG, "%s: terminateds is required", name);
    if (trunc != nullptr && tv == nullptr)
        return fail(LRS_ERR_INVALID_ARG, "%s: truncateds given without trunc_values", name);
    return LRS_OK;
}

// Memory an array argument covers (a null pointer covers nothing).
struct Span {
    const void* p;
    uint64_t bytes;
};

inline bool spans_overlap(const Span& x, const Span& y)
{
    if (x.p == nullptr || y.p == nullptr || x.bytes == 0 || y.bytes == 0) return false;
    const uintptr_t a = (uintptr_t)x.p, b = (uintptr_t)y.p;
    return a < b + y.bytes && b < a + x.bytes;
}

// Every array a call writes (its outputs and the workspace) must be disjoint
// from every array it reads and from every other one it writes: a tile reads
// its neighbours' inputs (successor values, the predecessor's done flag)
// while other tiles store, so overlapping memory would race.
inline lrs_status check_disjoint(const char* name, const Span* outs, int nouts, const Span* ins,
                                 int nins)
{
    for (int i = 0; i < nouts; ++i) {
        for (int j = 0; j < nins; ++j)
            if (spans_overlap(outs[i], ins[j]))
                return fail(LRS_ERR_INVALID_ARG,
                            "%s: output array %d overlaps input array %d (outputs and the "
                            "workspace must not share memory with any input)",
                            name, i, j);
        for (int k = i + 1; k < nouts; ++k)
            if (spans_overlap(outs[i], outs[k]))
                return fail(LRS_ERR_INVALID_ARG,
                            "%s: output arrays %d and %d overlap (outputs and the workspace must "
                            "not share memory)",
                            name, i, k);
    }
    return LRS_OK;
}

#define LRS_REQUIRE(cond, ...)                                   \
    do {                                                         \
        if (!(cond)) return fail(LRS_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

#define LRS_TRY(expr)                      \
    do {                                   \
        const lrs_status st_ = (expr);     \
        if (st_ != LRS_OK) return st_;     \
    } while (0)

}  // namespace lrs
