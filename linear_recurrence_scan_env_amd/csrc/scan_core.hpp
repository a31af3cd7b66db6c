// scan_core.hpp -- device building blocks of the segmented affine scan on
// gfx950 (wave64).
//
// An element of the recurrence is the affine map x -> a + b*x.  Scanning
// composes maps: the element nearer the output end ("near") is applied last,
// (a_n, b_n) (+) (a_f, b_f) = (a_n + b_n*a_f, b_n*b_f), which is the operator
// of the rl-triton paper (gist.science technical summary, Methodology 1).
// For a backward scan "far" is the later time step; for a forward scan it is
// the earlier one.  A segment boundary is b = 0, which makes everything
// beyond it irrelevant (exactly, for finite values).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrs {

constexpr int kWave = 64;

template <class T>
struct Aff {
    T a, b;
};

__device__ __forceinline__ Aff<float> combine(Aff<float> near, Aff<float> far)
{
    return {fmaf(near.b, far.a, near.a), near.b * far.b};
}

// Integer maps only ever have b in {0, 1}; arithmetic is modulo 2^32.
__device__ __forceinline__ Aff<uint32_t> combine(Aff<uint32_t> near, Aff<uint32_t> far)
{
    return {near.b ? near.a + far.a : near.a, near.b & far.b};
}

__device__ __forceinline__ float apply(Aff<float> f, float x) { return fmaf(f.b, x, f.a); }
__device__ __forceinline__ uint32_t apply(Aff<uint32_t> f, uint32_t x) { return f.b ? f.a + x : f.a; }

template <class T>
__device__ __forceinline__ Aff<T> identity() { return {T(0), T(1)}; }

__device__ __forceinline__ float shfl_down(float v, int d) { return __shfl_down(v, d, kWave); }
__device__ __forceinline__ uint32_t shfl_down(uint32_t v, int d)
{
    return (uint32_t)__shfl_down((int)v, d, kWave);
}
__device__ __forceinline__ float shfl_up(float v, int d) { return __shfl_up(v, d, kWave); }
__device__ __forceinline__ uint32_t shfl_up(uint32_t v, int d)
{
    return (uint32_t)__shfl_up((int)v, d, kWave);
}
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, kWave); }
__device__ __forceinline__ uint32_t shfl(uint32_t v, int src)
{
    return (uint32_t)__shfl((int)v, src, kWave);
}

// Inclusive scan over the 64 lanes of a wave.  Backward: lane L ends up with
// the composition of lanes L..63 (far = higher lanes).  Forward: lanes 0..L.
template <bool kBackward, class T>
__device__ __forceinline__ Aff<T> wave_scan(Aff<T> x, int lane)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        Aff<T> f;
        if (kBackward) {
            f.a = shfl_down(x.a, d);
            f.b = shfl_down(x.b, d);
            if (lane + d < kWave) x = combine(x, f);
        } else {
            f.a = shfl_up(x.a, d);
            f.b = shfl_up(x.b, d);
            if (lane >= d) x = combine(x, f);
        }
    }
    return x;
}

// Exclusive value of a lane: the inclusive scan of its far neighbour.
template <bool kBackward, class T>
__device__ __forceinline__ Aff<T> wave_exclusive(Aff<T> inc, int lane)
{
    Aff<T> e;
    if (kBackward) {
        e.a = shfl_down(inc.a, 1);
        e.b = shfl_down(inc.b, 1);
        if (lane == kWave - 1) e = identity<T>();
    } else {
        e.a = shfl_up(inc.a, 1);
        e.b = shfl_up(inc.b, 1);
        if (lane == 0) e = identity<T>();
    }
    return e;
}

// ----------------------------------------------------------------- loads
// E consecutive elements starting at flat index i0 (a multiple of E).  The
// vector form needs `vec` (base pointer alignment checked on the host) and a
// full chunk; the ragged tail and misaligned bases take scalar loads.

template <int E>
__device__ __forceinline__ void load_f32(float (&v)[E], const float* __restrict__ p, uint64_t i0,
                                         int count, bool vec)
{
    if (vec && count == E) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            float4 q = *reinterpret_cast<const float4*>(p + i0 + 4 * k);
            v[4 * k + 0] = q.x;
            v[4 * k + 1] = q.y;
            v[4 * k + 2] = q.z;
            v[4 * k + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = (j < count) ? p[i0 + j] : 0.0f;
    }
}

template <int E>
__device__ __forceinline__ void load_u32(uint32_t (&v)[E], const int32_t* __restrict__ p,
                                         uint64_t i0, int count, bool vec)
{
    if (vec && count == E) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            int4 q = *reinterpret_cast<const int4*>(p + i0 + 4 * k);
            v[4 * k + 0] = (uint32_t)q.x;
            v[4 * k + 1] = (uint32_t)q.y;
            v[4 * k + 2] = (uint32_t)q.z;
            v[4 * k + 3] = (uint32_t)q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = (j < count) ? (uint32_t)p[i0 + j] : 0u;
    }
}

// Bit j of the result is (mask[i0 + j] != 0).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w)
{
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) bits |= (((w >> (8 * k)) & 0xffu) != 0u ? 1u : 0u) << k;
    return bits;
}

template <int E>
__device__ __forceinline__ uint32_t load_mask(const uint8_t* __restrict__ p, uint64_t i0,
                                              int count, bool vec)
{
    static_assert(E == 4 || E == 8, "mask loads are 4 or 8 bytes");
    if (p == nullptr) return 0u;
    if (vec && count == E) {
        if (E == 4) return nonzero_bytes(*reinterpret_cast<const uint32_t*>(p + i0));
        uint2 w = *reinterpret_cast<const uint2*>(p + i0);
        return nonzero_bytes(w.x) | (nonzero_bytes(w.y) << 4);
    }
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < E; ++j)
        if (j < count && p[i0 + j] != 0) bits |= 1u << j;
    return bits;
}

template <int E>
__device__ __forceinline__ void store_f32(float* __restrict__ p, const float (&v)[E], uint64_t i0,
                                          int count, bool vec)
{
    if (vec && count == E) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
            *reinterpret_cast<float4*>(p + i0 + 4 * k) =
                make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (j < count) p[i0 + j] = v[j];
    }
}

template <int E>
__device__ __forceinline__ void store_u32(int32_t* __restrict__ p, const uint32_t (&v)[E],
                                          uint64_t i0, int count, bool vec)
{
    if (vec && count == E) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
            *reinterpret_cast<int4*>(p + i0 + 4 * k) =
                make_int4((int)v[4 * k], (int)v[4 * k + 1], (int)v[4 * k + 2], (int)v[4 * k + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (j < count) p[i0 + j] = (int32_t)v[j];
    }
}

// ------------------------------------------------ cross-tile carry protocol
//
// Workspace: a header followed by one 16-byte record per tile: two 64-bit
// words, each (tag << 32 | payload), the payloads being the bit patterns of
// the tile aggregate's a and b.  Every word is written and read with
// single-copy-atomic 64-bit accesses at agent scope, and each word carries
// its own tag, so a reader that sees both tags equal to this launch's tag
// holds a consistent aggregate without any fence.
//
// Header: the launch epoch, an error word, and block-completion counters
// spread over kGroups cache lines (block b counts itself in group b % kGroups;
// the block completing a group counts the group in `top`).  tag = epoch + 1.
// Every block reads the epoch before counting itself out; the block that
// completes the last group zeroes the counters and advances the epoch, so
// the next launch on the same stream starts clean and stale records (older
// tags, or the zero fill) are never mistaken for fresh ones.  Spreading the
// counters keeps same-address atomics, which serialize, to a few per line.
//
// Tiles are taken in dispatch order (backward scans from the end of the
// array), so a tile only waits for tiles of lower block index.  Workgroups
// of a dispatch are started in index order, so those blocks are running or
// finished and every wait ends; each wait is also bounded (kMaxPolls), so a
// violated assumption or a corrupted workspace yields a flagged error in the
// header instead of a hang.

constexpr uint32_t kGroups = 32;
constexpr uint32_t kLine = 128;  // bytes between counters

struct WsHeader {
    uint32_t epoch;
    uint32_t error;  // nonzero: a wait gave up (kErrTimeout)
    uint32_t top;    // number of completed groups
    uint32_t pad0[kLine / 4 - 3];
    struct {
        uint32_t count;
        uint32_t pad[kLine / 4 - 1];
    } group[kGroups];
};
static_assert(sizeof(WsHeader) == kLine * (kGroups + 1), "header layout");

// Upper bound on the polls of one look-back wait (about a second).
constexpr uint32_t kMaxPolls = 1u << 20;
constexpr uint32_t kErrTimeout = 2u;

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t bits_of(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t bits_of(uint32_t x) { return x; }
template <class T>
__device__ __forceinline__ T from_bits(uint32_t x);
template <>
__device__ __forceinline__ float from_bits<float>(uint32_t x) { return __uint_as_float(x); }
template <>
__device__ __forceinline__ uint32_t from_bits<uint32_t>(uint32_t x) { return x; }

template <class T>
__device__ __forceinline__ void publish_aggregate(uint64_t* rec, uint32_t tile, uint32_t tag,
                                                  Aff<T> agg)
{
    const uint64_t hi = (uint64_t)tag << 32;
    st_agent(rec + 2 * (uint64_t)tile, hi | bits_of(agg.a));
    st_agent(rec + 2 * (uint64_t)tile + 1, hi | bits_of(agg.b));
}

// Executed by one full wave.  Returns the value entering `tile` from its far
// side (backward: the scan value at the first element of tile+1; forward:
// the value at the last element of tile-1).  Composes the aggregates of the
// neighbouring tiles, nearest first, up to and including the first one whose
// b is zero (a segment boundary) or the end of the array.  Only aggregates
// are used, combined in a fixed order, so the result does not depend on
// timing (deterministic run to run).
template <bool kBackward, class T>
__device__ T lookback_carry(const uint64_t* rec, uint32_t tile, uint32_t num_tiles, uint32_t tag,
                            int lane, uint32_t* error)
{
    Aff<T> acc = identity<T>();
    uint32_t polls = 0;
    for (uint32_t base = 0;; base += kWave) {
        const int64_t j = kBackward ? (int64_t)tile + 1 + base + lane
                                    : (int64_t)tile - 1 - (int64_t)base - lane;
        const bool exists = j >= 0 && j < (int64_t)num_tiles;
        Aff<T> v = {T(0), T(0)};  // beyond the array: nothing flows in
        bool have = !exists;
        for (;;) {
            if (!have) {
                const uint64_t wa = ld_agent(rec + 2 * (uint64_t)j);
                const uint64_t wb = ld_agent(rec + 2 * (uint64_t)j + 1);
                if ((uint32_t)(wa >> 32) == tag && (uint32_t)(wb >> 32) == tag) {
                    have = true;
                    v.a = from_bits<T>((uint32_t)wa);
                    v.b = from_bits<T>((uint32_t)wb);
                }
            }
            const uint64_t zero_b = __ballot(have && v.b == T(0));
            const uint64_t missing = __ballot(!have);
            const int k = zero_b ? __ffsll((unsigned long long)zero_b) - 1 : kWave - 1;
            const uint64_t needed = (k == kWave - 1) ? ~0ull : ((2ull << k) - 1ull);
            if ((missing & needed) == 0) {
                if (lane > k) v = identity<T>();
                Aff<T> tot = wave_scan<true>(v, lane);  // lane 0 = composition of 0..k
                tot.a = shfl(tot.a, 0);
                tot.b = shfl(tot.b, 0);
                acc = combine(acc, tot);
                if (zero_b) return acc.a;
                break;  // all 64 neighbours continue the segment: next window
            }
            if (++polls > kMaxPolls) {
                if (lane == 0)
                    __hip_atomic_fetch_or(error, kErrTimeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                return T(0);
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
}

}  // namespace lrs
