// timemajor.hpp -- the same recurrences on time-major rollouts: arrays of
// shape [T, N] (row = time step, column = environment), element (n, t) at
// t * N + n, the layout of rollout buffers written one step at a time.
//
// A lane owns one environment, so each load instruction of a wave reads 64
// consecutive columns of one time row (coalesced).  A wave holds E
// consecutive steps of its 64 environments; a block holds G groups of 64
// environments (1, or 2 on long rows with many environments) and stacks
// W / G waves along time per group, so a tile is 64 G environments x E W / G
// steps.  The estimator functors are the row-major ones, fed a time-major Pos
// (strided, guarded accesses; all of a lane's steps belong to one
// environment).
//
// Carries between tiles run along time, per environment: each tile publishes
// its aggregate as soon as its own maps are composed, and its inclusive value
// (the value at its near edge) once it has its carry.  A tile looks back over
// up to kWindowTM<W> earlier-in-scan tiles, to the first published inclusive
// value or cut, and applies the aggregates in between from the far one to the
// near one.  That is exactly the arithmetic by which those tiles form their
// own inclusive values, so the result is the same bits however far a tile
// had to look: deterministic.  Blocks take tiles time-tile-major from the
// scan's far end, so every tile a block reads belongs to a block of lower
// index, which is running or done.  Every wait is bounded (kMaxPolls); a
// wait that gives up flags the header and makes the tile's outputs NaN.
#pragma once

#include "launch.hpp"

namespace lrs {

struct SchedTM {
    uint8_t* ws;          // header + per-(tile, environment) records
    uint32_t N, T;
    uint32_t groups;      // ceil(N / 64): environment groups
    uint32_t time_tiles;  // ceil(T / (E * W))
    uint32_t num_blocks;  // groups * time_tiles
};

// Records: three planes of time_tiles * N tagged 64-bit words (tag << 32 |
// 32 payload bits): the tile's aggregate a and b per environment, and its
// inclusive value y (the value at its near edge, which the next tile in
// scan order needs).  Planar, so a wave's 64 environments read 512
// contiguous bytes.  The payload is fp32 for fp32 maps whatever their
// composition type (uint32 for the integer prefix sum): a tile defines y as
// apply(published aggregate, carry) in that type, so any reader that
// rebuilds y from published aggregates gets the same bits.
constexpr uint32_t kPlanesTM = 3;
// Aggregates a waiting tile may compose: inclusive values then propagate up
// to that many tiles per hop.  32 for the 16-wave blocks that carry long rows
// (64 environments x 131072 steps: 20% faster than 16); 16 for smaller
// blocks, which carry only under a forced wave count and would otherwise
// give up occupancy to the window's LDS.
template <int W>
constexpr int kWindowTM = W >= 16 ? 32 : 16;

// Record payload type of a composition type: uint32 stays, fp32/fp64 -> fp32.
template <class A>
using RecOf = typename std::conditional<std::is_same<A, uint32_t>::value, uint32_t, float>::type;

template <class R>
__device__ __forceinline__ uint64_t tagged(uint32_t tag, R v)
{
    return ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, v);
}
template <class R>
__device__ __forceinline__ bool untag(uint64_t w, uint32_t tag, R& v)
{
    if ((uint32_t)(w >> 32) != tag) return false;
    v = __builtin_bit_cast(R, (uint32_t)w);
    return true;
}

// The tile (time tile k, environment group g) block b works on: tiles are
// taken time-tile-major from the scan's far end, so the tile one step
// farther in scan order, the only kind a tile waits for, belongs to block
// b - groups.  Shared by the kernel and lrs_debug_schedule.
struct TilePlaceTM {
    uint32_t k, g;
};

__host__ __device__ inline TilePlaceTM place_tile_tm(uint32_t b, const SchedTM& s, bool backward)
{
    const uint32_t pos = b / s.groups, g = b % s.groups;
    return {backward ? s.time_tiles - 1u - pos : pos, g};
}

// G groups of 64 environments per block; per group W / G waves along time.
// Environment (group q, lane l) at column q * 64 + l.
template <class A, int W, int G>
struct BlockSharedTM {
    A a[W / G][kWave * G];
    A b[W / G][kWave * G];
    RecOf<A> win_a[kWindowTM<W>][kWave * G];  // aggregates gathered by the look-back
    RecOf<A> win_b[kWindowTM<W>][kWave * G];
    RecOf<A> carry[kWave * G];
};

// One tile: 64 G environments x E W / G steps.  Wave w works on environment
// group w % G and on the E steps w / G of the tile, so the G waves of a time
// step read G adjacent 256-byte runs of each time row together (4096 x 2048:
// a load/store kernel on 128 x 128-step tiles of two groups took 14.3 us,
// on 64 x 256-step tiles of one group 15.9).  F: every environment of the
// block and every step of the tile exist (unconditional accesses); otherwise
// accesses are guarded.
template <class Op, int E, int W, int G, class A, bool F, bool S>
__device__ __forceinline__ void tile_body_tm(const typename Op::Args& args, const SchedTM& s,
                                             uint32_t k, uint32_t g, BlockSharedTM<A, W, G>& sh)
{
    using T = typename Op::T;
    using R = RecOf<A>;
    constexpr bool kB = Op::kBackward;
    constexpr int kWavesT = W / G;  // waves along time
    constexpr uint32_t kSteps = (uint32_t)E * kWavesT;
    constexpr int kNear = kB ? 0 : kWavesT - 1;  // the time wave holding the tile's near edge

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // The wave index is uniform across the wave; saying so lets the compiler
    // keep time-row bases in scalar registers (4096 x 2048: 4-12 fewer VGPRs
    // per kernel, discounted returns with truncations 23% faster, the other
    // calls 0-3%; the same change in the row-major kernel made it slower).
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int grp = wave % G;
    const int tw = wave / G;
    const int col_l = grp * kWave + lane;  // the environment's column in the shared arrays
    const uint32_t n = (g * G + (uint32_t)grp) * kWave + lane;
    const bool active = n < s.N;
    const uint32_t t0 = k * kSteps + (uint32_t)tw * E;

    int count = 0;
    uint32_t last = 0, first = 0;
    if (active && t0 < s.T) {
        count = (int)(s.T - t0 < (uint32_t)E ? s.T - t0 : E);
        if (s.T - 1u - t0 < (uint32_t)count) last = 1u << (s.T - 1u - t0);
        if (t0 == 0) first = 1u;
    }
    const uint32_t col = active ? n : 0u;  // inactive lanes touch nothing (count = 0)
    // Wide tiles read non-temporally: 0-4% faster than plain loads with one
    // group of 64 (64 x 131072 to 4096 x 256), more with two.
    const Pos<E, F, true, true, S> P{(uint64_t)t0 * s.N + col, col, count, last, first, s.N, t0};
    const Ctx c{(uint64_t)s.N * s.T, s.T, lane, false};

    // The launch tag is read first, in flight with the tile's loads.  These
    // blocks count themselves in at their end instead, after their stores
    // are issued (measured faster here than counting in at the start, as the
    // row-major kernel does; both keep the same header state between
    // launches).
    WsHeader* hdr = reinterpret_cast<WsHeader*>(s.ws);
    const bool carries = tw == kNear && s.time_tiles > 1;
    uint32_t tag = 0;
    if (carries)
        tag = __builtin_amdgcn_readfirstlane(
                  __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) + 1u;

    T alpha[E], beta[E];
    typename Op::State st;
    Op::prepare(args, P, c, alpha, beta, st);

    // The lane's own map over its E steps (as in the row-major kernel: fp32
    // maps keep a in fp32 and form the product of betas in fp64).
    Aff<A> x = identity<A>();
    if constexpr (std::is_same<A, float>::value) {
        float a = 0.0f;
        double b = 1.0;
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const int j = kB ? E - 1 - q : q;
            a = fmaf(beta[j], a, alpha[j]);
            b *= (double)beta[j];
        }
        x = {a, (float)b};
    } else if (kB) {
#pragma unroll
        for (int j = E - 1; j >= 0; --j) x = combine(Aff<A>{A(alpha[j]), A(beta[j])}, x);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) x = combine(Aff<A>{A(alpha[j]), A(beta[j])}, x);
    }
    if constexpr (W > 1) {
        sh.a[tw][col_l] = x.a;
        sh.b[tw][col_l] = x.b;
        __syncthreads();
    }

    // The group's waves between this one and the tile's far edge, nearest
    // first.
    Aff<A> beyond = identity<A>();
#pragma unroll
    for (int d = 1; d < kWavesT; ++d) {
        const int w = kB ? tw + d : tw - d;
        if (w >= 0 && w < kWavesT) beyond = combine(beyond, Aff<A>{sh.a[w][col_l], sh.b[w][col_l]});
    }

    R carry = R(0);
    if (carries) {
        uint64_t* rec = reinterpret_cast<uint64_t*>(s.ws + sizeof(WsHeader));
        const uint64_t plane = (uint64_t)s.time_tiles * s.N;
        uint64_t* rec_a = rec;
        uint64_t* rec_b = rec + plane;
        uint64_t* rec_y = rec + 2 * plane;
        const Aff<A> tile_map = combine(x, beyond);
        const Aff<R> tile = {(R)tile_map.a, (R)tile_map.b};  // as published
        const bool far_most = kB ? (k == s.time_tiles - 1u) : (k == 0u);
        const bool near_most = kB ? (k == 0u) : (k == s.time_tiles - 1u);
        const uint64_t own = (uint64_t)k * s.N + n;
        if (active && !near_most) {
            // the aggregate first, so that later tiles can look past this one
            st_agent(rec_a + own, tagged(tag, tile.a));
            st_agent(rec_b + own, tagged(tag, tile.b));
            if (far_most || tile.b == R(0)) st_agent(rec_y + own, tagged(tag, tile.a));
        }
        if (!far_most) {
            // Look back along time, per environment, up to the first tile
            // whose inclusive value is published or whose aggregate has a cut
            // (b = 0: its value is its a), keeping the open aggregates in
            // between; then apply them from the far one to the near one.
            const int step = kB ? 1 : -1;
            const int64_t last_tile = kB ? (int64_t)s.time_tiles - 1 : 0;  // the far-most one
            int64_t j = (int64_t)k + step;
            int depth = 0;
            bool done = !active;
            R base = R(0);
            uint32_t polls = 0;
            bool gave_up = false;
            while (__ballot(!done) != 0) {
                bool moved = false;
                if (!done) {
                    // the tile's three words are read together: one round
                    // trip per step of the walk
                    const uint64_t slot = (uint64_t)j * s.N + n;
                    R y, a, b;
                    const uint64_t wy = ld_agent(rec_y + slot);
                    const uint64_t wa = ld_agent(rec_a + slot);
                    const uint64_t wb = ld_agent(rec_b + slot);
                    if (untag(wy, tag, y)) {
                        base = y;
                        done = true;
                    } else if (j != last_tile && depth < kWindowTM<W> &&
                               untag(wa, tag, a) && untag(wb, tag, b)) {
                        moved = true;
                        // (at the far-most tile only its y is awaited, so j
                        // never leaves the array)
                        if (b == R(0)) {
                            base = a;
                            done = true;
                        } else {
                            sh.win_a[depth][col_l] = a;
                            sh.win_b[depth][col_l] = b;
                            ++depth;
                            j += step;
                        }
                    }
                }
                if (++polls > kMaxPolls) {
                    if (lane == 0)
                        __hip_atomic_fetch_or(&hdr->error, kErrTimeout, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    gave_up = true;
                    break;
                }
                // pause only when no lane moved on
                if (__ballot(!done && !moved) != 0) __builtin_amdgcn_s_sleep(1);
            }
            carry = base;
            for (int d = depth - 1; d >= 0; --d)
                carry = apply(Aff<R>{sh.win_a[d][col_l], sh.win_b[d][col_l]}, carry);
            // a wait that gave up leaves every lane of the tile without its
            // carry: NaN for fp32 maps (0 for the integer prefix sum)
            if (gave_up) carry = give_up_carry<R>();
            if (active && !near_most && tile.b != R(0))
                st_agent(rec_y + own, tagged(tag, apply(tile, carry)));
        }
    }
    if constexpr (W > 1) {
        if (tw == kNear) sh.carry[col_l] = carry;
        __syncthreads();
        carry = sh.carry[col_l];
    }

    const T lane_in = T(apply(beyond, A(carry)));
    Op::finish(args, P, c, alpha, beta, st, lane_in);
    // One wave counts the block, after the barrier above: each group's near
    // wave, the only ones that read the launch tag, has it by then.
    if (carries && grp == 0 && lane == 0) {
        const uint64_t entry = count_block(hdr, blockIdx.x);
        close_launch(hdr, count_group(hdr, entry, s.num_blocks, blockIdx.x), s.num_blocks, tag);
    }
}

template <class Op, int E, int W, int G, class A, bool S>
__device__ __forceinline__ void scan_body_tm(const typename Op::Args& args, const SchedTM& s)
{
    warm_kernargs<kernarg_bytes<typename Op::Args, SchedTM>()>();
    constexpr uint32_t kSteps = (uint32_t)E * (W / G);
    __shared__ BlockSharedTM<A, W, G> sh;
    const TilePlaceTM tp = place_tile_tm(blockIdx.x, s, Op::kBackward);
    const uint32_t k = tp.k, g = tp.g;
    const bool full = (uint64_t)(k + 1u) * kSteps <= s.T && (uint64_t)(g + 1u) * kWave * G <= s.N;
    if (full)
        tile_body_tm<Op, E, W, G, A, true, S>(args, s, k, g, sh);
    else
        tile_body_tm<Op, E, W, G, A, false, S>(args, s, k, g, sh);
}

// Rows that fit one tile, on few environments: V environments per block
// instead of 64, so that a 4096-environment batch spreads over 4096 / V
// blocks rather than 64.  A wave holds C = 64 / V chunks of E steps of
// its V environments (lane l: environment l mod V, chunk l / V), so each load
// instruction reads C time rows of V consecutive environments; a block of W
// waves covers E * W * C steps, the whole row, and needs no carry.  The chunk
// maps combine through LDS as the wave maps of the wide kernel do.
template <class A, int Q, int V>
struct BlockSharedTMRows {
    A a[Q][V];
    A b[Q][V];
};

template <class Op, int E, int W, int V, class A, bool F, bool S>
__device__ __forceinline__ void rows_body_tm(const typename Op::Args& args, const SchedTM& s,
                                             uint32_t g, BlockSharedTMRows<A, W * (kWave / V), V>& sh)
{
    using T = typename Op::T;
    constexpr bool kB = Op::kBackward;
    constexpr int C = kWave / V;
    constexpr int Q = W * C;  // chunks along time

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int v = lane % V;
    const int q = __builtin_amdgcn_readfirstlane(tid / kWave) * C + lane / V;
    const uint32_t n = g * V + (uint32_t)v;
    const bool active = n < s.N;
    const uint32_t t0 = (uint32_t)q * E;

    int count = 0;
    uint32_t last = 0, first = 0;
    if (active && t0 < s.T) {
        count = (int)(s.T - t0 < (uint32_t)E ? s.T - t0 : E);
        if (s.T - 1u - t0 < (uint32_t)count) last = 1u << (s.T - 1u - t0);
        if (t0 == 0) first = 1u;
    }
    const uint32_t col = active ? n : 0u;  // inactive lanes touch nothing (count = 0)
    // Plain loads: non-temporal ones measured up to 13% slower on these short
    // rows (4096 x 32, 4096 x 100, 4096 x 128).
    const Pos<E, F, true, false, S> P{(uint64_t)t0 * s.N + col, col, count, last, first, s.N, t0};
    const Ctx c{(uint64_t)s.N * s.T, s.T, lane, false};

    T alpha[E], beta[E];
    typename Op::State st;
    Op::prepare(args, P, c, alpha, beta, st);

    Aff<A> x = identity<A>();
    if constexpr (std::is_same<A, float>::value) {
        float a = 0.0f;
        double b = 1.0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int j = kB ? E - 1 - k : k;
            a = fmaf(beta[j], a, alpha[j]);
            b *= (double)beta[j];
        }
        x = {a, (float)b};
    } else if (kB) {
#pragma unroll
        for (int j = E - 1; j >= 0; --j) x = combine(Aff<A>{A(alpha[j]), A(beta[j])}, x);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) x = combine(Aff<A>{A(alpha[j]), A(beta[j])}, x);
    }
    sh.a[q][v] = x.a;
    sh.b[q][v] = x.b;
    __syncthreads();

    // Chunks between this one and the row's far end, nearest first.
    Aff<A> beyond = identity<A>();
#pragma unroll
    for (int d = 1; d < Q; ++d) {
        const int w = kB ? q + d : q - d;
        if (w >= 0 && w < Q) beyond = combine(beyond, Aff<A>{sh.a[w][v], sh.b[w][v]});
    }
    const T lane_in = T(apply(beyond, A(0)));
    Op::finish(args, P, c, alpha, beta, st, lane_in);
}

template <class Op, int E, int W, int G, class A, bool S>
__global__ __launch_bounds__(W * kWave) void scan_kernel_tm(const typename Op::Args args,
                                                            const SchedTM s)
{
    scan_body_tm<Op, E, W, G, A, S>(args, s);
}

// The same kernel capped for eight waves per SIMD (64 VGPRs, 72 SGPRs): two
// 16-wave blocks per CU instead of one.  The uncapped 16-step kernels hold
// 64-74 VGPRs and 95-106 SGPRs; calls that fit the caps without spilling
// take this twin on grids larger than the CU count (kLeanTm).
template <class Op, int E, int W, int G, class A, bool S>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_num_sgpr(72), amdgpu_waves_per_eu(8, 8))) void scan_kernel_tm_lean(
    const typename Op::Args args, const SchedTM s)
{
    scan_body_tm<Op, E, W, G, A, S>(args, s);
}


template <class Op, int E, int W, int V, class A, bool S>
__global__ __launch_bounds__(W * kWave) void scan_kernel_tm_rows(const typename Op::Args args,
                                                                 const SchedTM s)
{
    warm_kernargs<kernarg_bytes<typename Op::Args, SchedTM>()>();
    constexpr uint32_t kSteps = (uint32_t)E * W * (kWave / V);
    __shared__ BlockSharedTMRows<A, W * (kWave / V), V> sh;
    const uint32_t g = blockIdx.x;
    const bool full = kSteps == s.T && (uint64_t)(g + 1u) * V <= s.N;
    if (full)
        rows_body_tm<Op, E, W, V, A, true, S>(args, s, g, sh);
    else
        rows_body_tm<Op, E, W, V, A, false, S>(args, s, g, sh);
}

// ------------------------------------------------------------- host side
constexpr int kTmE = 8;        // steps per lane
// Rows longer than 128 steps take 16 steps per lane in 16-wave blocks:
// 256-step tiles, so the carries run along time in half as many tiles as
// with 128-step ones (64 environments x 131072 steps: GAE 89 -> 58 us;
// 256 x 32768: 13-21% faster; 4096 x 2048: 0-6%).  V-trace then spills a few
// bytes per lane and is still faster (95 -> 70 us at 64 x 131072).
constexpr int kTmELong = 16;
constexpr uint64_t kTmLongRow = 128;
constexpr int kTmWSmall = 8;   // waves per block: 64-step tiles
// Long rows on many environments take two groups of 64 per block (128
// environments x 128 steps: twice the time tiles of one group's 256-step
// tiles, and adjacent 256-byte runs per row read together).  Measured against
// one group: 1-13% faster at 4096 x 1024, 4096 x 2048, 8192 x 1024,
// 8192 x 2048 and 16384 x 512; at 4096 x 8192 5-11% faster for the calls of
// three or more streams, the others within 1%; slower with fewer
// environments (2048 x 2048: +2-11%, 256 x 32768: +11-23%) and on rows of
// 256 steps (4096 x 256: +7-22%), which one group holds in a single tile.
inline bool tm_two_groups(uint64_t N, uint64_t T)
{
    return (N >= 4096 && T >= 1024) || (N >= 8192 && T >= 512);
}
constexpr int kTmWLarge = 16;  // 128-step tiles

inline uint64_t tm_tiles(uint64_t T, int W) { return (T + (uint64_t)kTmE * W - 1) / ((uint64_t)kTmE * W); }

inline bool tm_waves_supported(int W) { return W == 2 || W == 4 || W == 8 || W == 16; }

// Narrow blocks for rows that fit one tile (measured at 4096 x {32, 128}):
// when the wide kernel would have fewer than kTmRowsMaxGroups blocks of 64
// environments, rows of at most 128 steps take blocks of kTmRowsV = 32
// environments (twice the blocks; each load instruction reads two time rows
// of 128 bytes for fp32): 17-21% faster at 4096 x 128, 11% at 4096 x 32; 16
// environments per block measured slower than 32 at 128 steps.  Returns the
// waves per narrow block (1, 2, 4 or 8: 16 to 128 steps), or 0 for the wide
// kernel, which a forced wave count also selects.
constexpr int kTmRowsV = 32;
constexpr uint64_t kTmRowsMaxGroups = 256;
inline int tm_rows_waves(uint64_t N, uint64_t T)
{
    if (g_forced_tm_waves.load() != 0) return 0;
    if ((N + kWave - 1) / kWave >= kTmRowsMaxGroups) return 0;
    for (int W = 1; W <= 8; W *= 2)
        if ((uint64_t)kTmE * W * (kWave / kTmRowsV) >= T) return W;
    return 0;
}

// Waves per block (measured at 4096 x {32 .. 8192} and at 64 to 1024
// environments with 2^23 elements): rows of at most 64 steps take the
// smallest block that holds them whole (16-, 32- or 64-step tiles: no
// carries, no idle waves); longer rows take 128-step tiles, whose carries
// run along time in half as many steps as 64-step tiles' (3-44% faster than
// those, most with few environments: 64 x 131072 GAE 160 -> 89 us).  Smaller
// tiles with carries measured slower everywhere (at 4096 x 128: 4.7 us on
// one 128-step tile, 6.1-8.1 us on 2-8 tiles).
inline int tm_waves(uint64_t T)
{
    const int forced = g_forced_tm_waves.load();
    if (forced > 0) return forced;
    if (T <= 2u * kTmE) return 2;
    if (T <= 4u * kTmE) return 4;
    if (T <= (uint64_t)kTmWSmall * kTmE) return kTmWSmall;
    return kTmWLarge;
}

// Workspace of a time-major call: the header and three words per
// (64-step tile, environment).  Only a forced smaller block (a diagnostic
// setting) needs more, and then this reports that.
inline size_t workspace_bytes_tm(uint64_t N, uint64_t T)
{
    const int forced = g_forced_tm_waves.load();
    const int w = forced > 0 && forced < kTmWSmall ? forced : kTmWSmall;
    return sizeof(WsHeader) + 8 * kPlanesTM * N * tm_tiles(T, w);
}

template <template <int> class Op, int E, int W, int G, class A>
hipError_t launch_tm(bool strided, const typename Op<kTmE>::Args& a, const SchedTM& s,
                     hipStream_t stream)
{
    void* params[] = {(void*)&a, (void*)&s};
    const void* k = strided ? (const void*)&scan_kernel_tm<Op<E>, E, W, G, A, true>
                            : (const void*)&scan_kernel_tm<Op<E>, E, W, G, A, false>;
    constexpr LeanTm kLean = Op<E>::kLeanTm;
    constexpr bool kLeanOk = kLean == kLeanTmAny ||
                             (kLean == kLeanTmFp32 && !std::is_same<A, double>::value);
    if constexpr (kLeanOk && E == kTmELong && W == 16) {
        if (!strided && s.num_blocks > device_cus(stream))
            k = (const void*)&scan_kernel_tm_lean<Op<E>, E, W, G, A, false>;
    }
    return hipLaunchKernel(k, dim3(s.num_blocks), dim3(W * kWave), params, 0, stream);
}

template <template <int> class Op, int W, int V, class A>
hipError_t launch_tm_rows(bool strided, const typename Op<kTmE>::Args& a, const SchedTM& s,
                          hipStream_t stream)
{
    void* params[] = {(void*)&a, (void*)&s};
    const void* k = strided ? (const void*)&scan_kernel_tm_rows<Op<kTmE>, kTmE, W, V, A, true>
                            : (const void*)&scan_kernel_tm_rows<Op<kTmE>, kTmE, W, V, A, false>;
    return hipLaunchKernel(k, dim3(s.num_blocks), dim3(W * kWave), params, 0, stream);
}

template <template <int> class Op, int W, int V>
hipError_t launch_tm_rows_acc(float beta_max, bool strided, const typename Op<kTmE>::Args& a,
                              const SchedTM& s, hipStream_t stream)
{
    using Val = typename Op<kTmE>::T;
    if constexpr (std::is_same<Val, float>::value)
        return beta_max > kFp32BetaMax ? launch_tm_rows<Op, W, V, double>(strided, a, s, stream)
                                       : launch_tm_rows<Op, W, V, float>(strided, a, s, stream);
    else
        return launch_tm_rows<Op, W, V, Val>(strided, a, s, stream);
}

template <template <int> class Op, int W, int E = kTmE, int G = 1>
hipError_t launch_tm_acc(float beta_max, bool strided, const typename Op<kTmE>::Args& a,
                         const SchedTM& s, hipStream_t stream)
{
    using Val = typename Op<kTmE>::T;
    if constexpr (std::is_same<Val, float>::value)
        return beta_max > kFp32BetaMax ? launch_tm<Op, E, W, G, double>(strided, a, s, stream)
                                       : launch_tm<Op, E, W, G, float>(strided, a, s, stream);
    else
        return launch_tm<Op, E, W, G, Val>(strided, a, s, stream);
}

// The schedule of a time-major call: narrow whole-row blocks (rows_waves > 0
// waves of kTmRowsV environments) or the wide kernel (waves W, 16 steps per
// lane when long_rows), and its SchedTM without the workspace.  The launch
// checks that the grid fits a dispatch.
struct PlanTM {
    int rows_waves;
    int W;
    bool long_rows;
    int G;  // environment groups of 64 per block of the wide kernel
    uint64_t tile_steps;
    SchedTM s;
};

// Calls whose kernels fit the capped twin (kLeanTm, with maps composed in
// fp32 where that matters).  The others hold 69-128 VGPRs: one block per CU.
template <template <int> class Op>
inline bool tm_lean_capable(float beta_max)
{
    constexpr LeanTm kLean = Op<kTmE>::kLeanTm;
    using Val = typename Op<kTmE>::T;
    const bool fp64 = std::is_same<Val, float>::value && beta_max > kFp32BetaMax;
    return kLean == kLeanTmAny || (kLean == kLeanTmFp32 && !fp64);
}

// Long rows whose 256-step tiles would make fewer blocks than the device's
// 256 CUs.  The calls that run one block per CU then take 128-step tiles
// (8 steps per lane): twice the blocks (V-trace, Retrace and GAE with
// truncations 5-23% faster at 4096 x 256, 4096 x 512, 2048 x 512 and
// 1024 x 1024; GAE and TD(lambda) within 2% or faster).  The others keep
// 256-step tiles (up to 19% faster than 128-step ones there).
constexpr uint64_t kTmFewBlocks = 256;
inline bool tm_few_blocks(uint64_t N, uint64_t T)
{
    const uint64_t tiles = (T + (uint64_t)kTmELong * kTmWLarge - 1) / ((uint64_t)kTmELong * kTmWLarge);
    return (N + kWave - 1) / kWave * tiles < kTmFewBlocks;
}

inline PlanTM plan_time_major(int64_t N, int64_t T, bool lean_capable)
{
    PlanTM p{};
    p.s.N = (uint32_t)N;
    p.s.T = (uint32_t)T;
    p.s.ws = nullptr;
    p.rows_waves = tm_rows_waves((uint64_t)N, (uint64_t)T);
    p.G = 1;
    if (p.rows_waves) {
        p.W = p.rows_waves;
        p.tile_steps = (uint64_t)T;
        p.s.groups = (uint32_t)((N + kTmRowsV - 1) / kTmRowsV);
        p.s.time_tiles = 1;
        p.s.num_blocks = p.s.groups;
        return p;
    }
    p.W = tm_waves((uint64_t)T);
    p.long_rows = g_forced_tm_waves.load() == 0 && (uint64_t)T > kTmLongRow;
    if (p.long_rows && tm_two_groups((uint64_t)N, (uint64_t)T))
        p.G = 2;
    else if (p.long_rows && !lean_capable && tm_few_blocks((uint64_t)N, (uint64_t)T))
        p.long_rows = false;
    p.s.groups = (uint32_t)((N + (int64_t)kWave * p.G - 1) / ((int64_t)kWave * p.G));
    p.tile_steps = (uint64_t)(p.long_rows ? kTmELong : kTmE) * (uint64_t)(p.W / p.G);
    p.s.time_tiles = (uint32_t)(((uint64_t)T + p.tile_steps - 1) / p.tile_steps);
    p.s.num_blocks = p.s.groups * p.s.time_tiles;
    return p;
}

template <template <int> class Op>
lrs_status run_tm(const char* name, int64_t N, int64_t T, float beta_max,
                  const typename Op<kTmE>::Args& a, bool strided, void* ws, size_t ws_bytes,
                  hipStream_t stream)
{
    if (N >= (int64_t(1) << 32))
        return fail(LRS_ERR_INVALID_ARG, "%s: time-major calls need num_envs < 2^32", name);
    const PlanTM plan = plan_time_major(N, T, tm_lean_capable<Op>(beta_max));
    if (const int Wr = plan.rows_waves) {
        SchedTM s = plan.s;
        s.ws = static_cast<uint8_t*>(ws);
        hipError_t e;
        switch (Wr) {
            case 1: e = launch_tm_rows_acc<Op, 1, kTmRowsV>(beta_max, strided, a, s, stream); break;
            case 2: e = launch_tm_rows_acc<Op, 2, kTmRowsV>(beta_max, strided, a, s, stream); break;
            case 4: e = launch_tm_rows_acc<Op, 4, kTmRowsV>(beta_max, strided, a, s, stream); break;
            default: e = launch_tm_rows_acc<Op, 8, kTmRowsV>(beta_max, strided, a, s, stream); break;
        }
        if (e != hipSuccess)
            return fail(LRS_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
        g_err[0] = '\0';
        return LRS_OK;
    }
    const int W = plan.W;
    const bool long_rows = plan.long_rows;
    const uint64_t tile_steps = plan.tile_steps;
    SchedTM s = plan.s;
    // One lane per environment, padded to whole groups of 64: with few
    // environments and very long rows the launch could exceed the 2^32 - 1
    // work items a dispatch holds.
    if ((uint64_t)s.num_blocks * (uint64_t)(W * kWave) > 0xffffffffull)
        return fail(LRS_ERR_INVALID_ARG,
                    "%s: time-major launch of %llu work items (ceil(num_envs/64)*64 lanes x "
                    "%llu steps / %d) exceeds 2^32 - 1; use the row-major call for so few, so "
                    "long rows",
                    name, (unsigned long long)s.num_blocks * (unsigned long long)(W * kWave),
                    (unsigned long long)(s.time_tiles * tile_steps), (int)(tile_steps / W));
    s.ws = static_cast<uint8_t*>(ws);
    if (s.time_tiles > 1) {
        const size_t need = sizeof(WsHeader) + 8 * kPlanesTM * (size_t)N * s.time_tiles;
        if (ws == nullptr || ws_bytes < need)
            return fail(LRS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name,
                        need, ws == nullptr ? (size_t)0 : ws_bytes);
        if (!aligned(ws, 16)) return fail(LRS_ERR_WORKSPACE, "%s: workspace not 16-byte aligned", name);
    }
    hipError_t e;
    if (long_rows && plan.G == 2) {
        e = launch_tm_acc<Op, kTmWLarge, kTmELong, 2>(beta_max, strided, a, s, stream);
    } else if (long_rows) {
        e = launch_tm_acc<Op, kTmWLarge, kTmELong>(beta_max, strided, a, s, stream);
    } else switch (W) {
        case 2: e = launch_tm_acc<Op, 2>(beta_max, strided, a, s, stream); break;
        case 4: e = launch_tm_acc<Op, 4>(beta_max, strided, a, s, stream); break;
        case 8: e = launch_tm_acc<Op, 8>(beta_max, strided, a, s, stream); break;
        default: e = launch_tm_acc<Op, 16>(beta_max, strided, a, s, stream); break;
    }
    if (e != hipSuccess)
        return fail(LRS_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    g_err[0] = '\0';
    return LRS_OK;
}

}  // namespace lrs
