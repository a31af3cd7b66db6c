// timemajor.hpp -- the same recurrences on time-major rollouts: arrays of
// shape [T, N] (row = time step, column = environment), element (n, t) at
// t * N + n, the layout of rollout buffers written one step at a time.
//
// A lane owns one environment, so each load instruction of a wave reads 64
// consecutive columns of one time row (coalesced).  A wave holds E
// consecutive steps of its 64 environments; a block stacks W waves along
// time, so a tile is 64 environments x E*W steps.  The estimator functors are
// the row-major ones, fed a time-major Pos (strided, guarded accesses; all
// of a lane's steps belong to one environment).
//
// Carries between tiles run along time, per environment: tile k publishes,
// for each of its environments, the value at its near edge (the inclusive
// result that the next tile in scan order needs), tagged with the launch
// epoch, and the next tile waits for exactly that value: a chained scan,
// deterministic, with no look-back.  Blocks take tiles time-tile-major from
// the scan's far end, so a tile's predecessor belongs to the block
// `groups` lower, which is running or done.  A lane whose tile holds a cut
// publishes before it waits.  Every wait is bounded (kMaxPolls).
#pragma once

#include "launch.hpp"

namespace lrs {

struct SchedTM {
    uint8_t* ws;          // header + per-(tile, environment) values
    uint32_t N, T;
    uint32_t groups;      // ceil(N / 64): environment groups
    uint32_t time_tiles;  // ceil(T / (E * W))
    uint32_t num_blocks;  // groups * time_tiles
};

// Words per published value: one 64-bit word (tag << 32 | bits) for 32-bit
// values, two (low and high halves, each tagged) for fp64.
template <class A>
constexpr uint32_t kWordsTM = sizeof(A) == 8 ? 2u : 1u;

template <class A>
__device__ __forceinline__ void publish_tm(uint64_t* rec, uint64_t slot, uint32_t tag, A v)
{
    const uint64_t t = (uint64_t)tag << 32;
    const uint64_t bits = payload_bits(v);
    if constexpr (kWordsTM<A> == 2) {
        st_agent(rec + 2 * slot, t | (bits & 0xffffffffu));
        st_agent(rec + 2 * slot + 1, t | (bits >> 32));
    } else {
        st_agent(rec + slot, t | bits);
    }
}

// true and the value once both halves carry `tag`
template <class A>
__device__ __forceinline__ bool read_tm(const uint64_t* rec, uint64_t slot, uint32_t tag, A& v)
{
    if constexpr (kWordsTM<A> == 2) {
        const uint64_t lo = ld_agent(rec + 2 * slot), hi = ld_agent(rec + 2 * slot + 1);
        if ((uint32_t)(lo >> 32) != tag || (uint32_t)(hi >> 32) != tag) return false;
        v = from_payload<A>((uint32_t)lo, (uint32_t)hi);
    } else {
        const uint64_t w = ld_agent(rec + slot);
        if ((uint32_t)(w >> 32) != tag) return false;
        v = from_payload<A>((uint32_t)w, 0u);
    }
    return true;
}

template <class A, int W>
struct BlockSharedTM {
    A a[W][kWave];
    A b[W][kWave];
    A carry[kWave];
};

template <class Op, int E, int W, class A>
__global__ __launch_bounds__(W * kWave) void scan_kernel_tm(const typename Op::Args args,
                                                            const SchedTM s)
{
    using T = typename Op::T;
    constexpr bool kB = Op::kBackward;
    constexpr uint32_t kSteps = (uint32_t)E * W;
    constexpr int kNear = kB ? 0 : W - 1;  // the wave holding the tile's near edge
    __shared__ BlockSharedTM<A, W> sh;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t pos = blockIdx.x / s.groups, g = blockIdx.x % s.groups;
    const uint32_t k = kB ? s.time_tiles - 1u - pos : pos;  // time tile
    const uint32_t n = g * kWave + lane;
    const bool active = n < s.N;
    const uint32_t t0 = k * kSteps + (uint32_t)wave * E;

    int count = 0;
    uint32_t last = 0, first = 0;
    if (active && t0 < s.T) {
        count = (int)(s.T - t0 < (uint32_t)E ? s.T - t0 : E);
        if (s.T - 1u - t0 < (uint32_t)count) last = 1u << (s.T - 1u - t0);
        if (t0 == 0) first = 1u;
    }
    const uint32_t col = active ? n : 0u;  // inactive lanes touch nothing (count = 0)
    const Pos<E, false, true> P{(uint64_t)t0 * s.N + col, col, count, last, first, s.N};
    const Ctx c{(uint64_t)s.N * s.T, s.T, lane, false};

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
    sh.a[wave][lane] = x.a;
    sh.b[wave][lane] = x.b;
    __syncthreads();

    // Waves between this one and the tile's far edge, nearest first.
    Aff<A> beyond = identity<A>();
#pragma unroll
    for (int d = 1; d < W; ++d) {
        const int w = kB ? wave + d : wave - d;
        if (w >= 0 && w < W) beyond = combine(beyond, Aff<A>{sh.a[w][lane], sh.b[w][lane]});
    }

    if (wave == kNear) {
        WsHeader* hdr = reinterpret_cast<WsHeader*>(s.ws);
        uint64_t* rec = reinterpret_cast<uint64_t*>(s.ws + sizeof(WsHeader));
        A carry = A(0);
        if (s.time_tiles > 1) {
            const uint32_t tag = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                                     &hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) + 1u;
            const Aff<A> tile = combine(x, beyond);
            const bool far_most = kB ? (k == s.time_tiles - 1u) : (k == 0u);
            const bool near_most = kB ? (k == 0u) : (k == s.time_tiles - 1u);
            const uint64_t own = (uint64_t)k * s.N + n;
            // a cut inside the tile (or nothing beyond it): publish now
            bool published = !active || near_most;
            if (!published && (far_most || tile.b == A(0))) {
                publish_tm<A>(rec, own, tag, tile.a);
                published = true;
            }
            if (active && !far_most) {
                const uint64_t pred = (uint64_t)(kB ? k + 1u : k - 1u) * s.N + n;
                uint32_t polls = 0;
                bool have = false;
                for (;;) {
                    if (!have) have = read_tm<A>(rec, pred, tag, carry);
                    if (__ballot(!have) == 0) break;  // the active lanes poll together
                    if (++polls > kMaxPolls) {
                        if (lane == 0)
                            __hip_atomic_fetch_or(&hdr->error, kErrTimeout, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                        if (!have) carry = A(0);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (!published) publish_tm<A>(rec, own, tag, apply(tile, carry));
            if (lane == 0) finish_launch(hdr, s.num_blocks, blockIdx.x, tag);
        }
        sh.carry[lane] = carry;
    }
    __syncthreads();

    const T lane_in = T(apply(beyond, sh.carry[lane]));
    Op::finish(args, P, c, alpha, beta, st, lane_in);
}

// ------------------------------------------------------------- host side
constexpr int kTmE = 8;   // steps per lane
constexpr int kTmW = 16;  // waves per block: 128-step tiles

inline uint64_t tm_time_tiles(uint64_t T) { return (T + kTmE * kTmW - 1) / (kTmE * kTmW); }

// Workspace of a time-major call: the header and up to two words per
// (tile, environment).  At most the row-major need (32 bytes per 256
// elements) plus 16 bytes per environment.
inline size_t workspace_bytes_tm(uint64_t N, uint64_t T)
{
    return sizeof(WsHeader) + 16 * N * tm_time_tiles(T);
}

template <template <int> class Op, class A>
hipError_t launch_tm(const typename Op<kTmE>::Args& a, const SchedTM& s, hipStream_t stream)
{
    void* params[] = {(void*)&a, (void*)&s};
    return hipLaunchKernel((const void*)&scan_kernel_tm<Op<kTmE>, kTmE, kTmW, A>,
                           dim3(s.num_blocks), dim3(kTmW * kWave), params, 0, stream);
}

template <template <int> class Op>
lrs_status run_tm(const char* name, int64_t N, int64_t T, float beta_max,
                  const typename Op<kTmE>::Args& a, void* ws, size_t ws_bytes, hipStream_t stream)
{
    SchedTM s{};
    s.N = (uint32_t)N;
    s.T = (uint32_t)T;
    s.groups = (uint32_t)((N + kWave - 1) / kWave);
    s.time_tiles = (uint32_t)tm_time_tiles((uint64_t)T);
    s.num_blocks = s.groups * s.time_tiles;
    s.ws = static_cast<uint8_t*>(ws);
    if (N >= (int64_t(1) << 32))
        return fail(LRS_ERR_INVALID_ARG, "%s: time-major calls need num_envs < 2^32", name);
    if (s.time_tiles > 1) {
        const size_t need = workspace_bytes_tm((uint64_t)N, (uint64_t)T);
        if (ws == nullptr || ws_bytes < need)
            return fail(LRS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name,
                        need, ws == nullptr ? (size_t)0 : ws_bytes);
        if (!aligned(ws, 16)) return fail(LRS_ERR_WORKSPACE, "%s: workspace not 16-byte aligned", name);
    }
    using Val = typename Op<kTmE>::T;
    hipError_t e;
    if constexpr (std::is_same<Val, float>::value)
        e = beta_max > kFp32BetaMax ? launch_tm<Op, double>(a, s, stream)
                                    : launch_tm<Op, float>(a, s, stream);
    else
        e = launch_tm<Op, Val>(a, s, stream);
    if (e != hipSuccess)
        return fail(LRS_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    g_err[0] = '\0';
    return LRS_OK;
}

}  // namespace lrs
