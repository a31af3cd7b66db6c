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

// ------------------------------------------------------- lane exchange
// DPP row shifts move data between lanes of a 16-lane row inside one VALU
// instruction (row_shl:n -- lane i reads lane i+n; row_shr:n -- lane i reads
// lane i-n; a lane whose source is outside its row keeps `old`).  The three
// row boundaries of a wave64 are bridged with v_readlane.
constexpr int kDppRowShl = 0x100;
constexpr int kDppRowShr = 0x110;

template <int kCtrl>
__device__ __forceinline__ float dpp(float old, float src)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                      kCtrl, 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t src)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, kCtrl, 0xf, 0xf, false);
}

__device__ __forceinline__ float readlane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Value held by lane+1 (lane 63 gets `edge`).
template <class T>
__device__ __forceinline__ T lane_next(T v, int lane, T edge)
{
    T r = dpp<kDppRowShl + 1>(edge, v);
    const T r16 = readlane(v, 16), r32 = readlane(v, 32), r48 = readlane(v, 48);
    if (lane == 15) r = r16;
    if (lane == 31) r = r32;
    if (lane == 47) r = r48;
    return r;
}

// Value held by lane-1 (lane 0 gets `edge`).
template <class T>
__device__ __forceinline__ T lane_prev(T v, int lane, T edge)
{
    T r = dpp<kDppRowShr + 1>(edge, v);
    const T r15 = readlane(v, 15), r31 = readlane(v, 31), r47 = readlane(v, 47);
    if (lane == 16) r = r15;
    if (lane == 32) r = r31;
    if (lane == 48) r = r47;
    return r;
}

// Inclusive scan over the 64 lanes of a wave.  Backward: lane L ends up with
// the composition of lanes L..63 (far = higher lanes).  Forward: lanes 0..L.
// Four DPP steps scan each 16-lane row; the row totals are then combined
// through v_readlane and folded into each row.
template <bool kBackward, class T>
__device__ __forceinline__ Aff<T> wave_scan(Aff<T> x, int lane)
{
    const Aff<T> id = identity<T>();
#define LRS_ROW_STEP(n)                                                          \
    {                                                                            \
        Aff<T> f;                                                                \
        if (kBackward) {                                                         \
            f.a = dpp<kDppRowShl + (n)>(id.a, x.a);                              \
            f.b = dpp<kDppRowShl + (n)>(id.b, x.b);                              \
        } else {                                                                 \
            f.a = dpp<kDppRowShr + (n)>(id.a, x.a);                              \
            f.b = dpp<kDppRowShr + (n)>(id.b, x.b);                              \
        }                                                                        \
        x = combine(x, f);                                                       \
    }
    LRS_ROW_STEP(1)
    LRS_ROW_STEP(2)
    LRS_ROW_STEP(4)
    LRS_ROW_STEP(8)
#undef LRS_ROW_STEP
    const int row = lane >> 4;
    if (kBackward) {
        // row totals sit in lanes 16r; suffix over rows 3..1
        const Aff<T> s3{readlane(x.a, 48), readlane(x.b, 48)};
        const Aff<T> s2 = combine(Aff<T>{readlane(x.a, 32), readlane(x.b, 32)}, s3);
        const Aff<T> s1 = combine(Aff<T>{readlane(x.a, 16), readlane(x.b, 16)}, s2);
        const Aff<T> far = row == 0 ? s1 : (row == 1 ? s2 : (row == 2 ? s3 : id));
        x = combine(x, far);
    } else {
        // row totals sit in lanes 16r+15; prefix over rows 0..2
        const Aff<T> p0{readlane(x.a, 15), readlane(x.b, 15)};
        const Aff<T> p1 = combine(Aff<T>{readlane(x.a, 31), readlane(x.b, 31)}, p0);
        const Aff<T> p2 = combine(Aff<T>{readlane(x.a, 47), readlane(x.b, 47)}, p1);
        const Aff<T> far = row == 3 ? p2 : (row == 2 ? p1 : (row == 1 ? p0 : id));
        x = combine(x, far);
    }
    return x;
}

// Exclusive value of a lane: the inclusive scan of its far neighbour.
template <bool kBackward, class T>
__device__ __forceinline__ Aff<T> wave_exclusive(Aff<T> inc, int lane)
{
    const Aff<T> id = identity<T>();
    if (kBackward) return {lane_next(inc.a, lane, id.a), lane_next(inc.b, lane, id.b)};
    return {lane_prev(inc.a, lane, id.a), lane_prev(inc.b, lane, id.b)};
}

// ----------------------------------------------------------------- loads
// A lane owns E consecutive elements starting at flat index i0 (a multiple
// of E).  Pos<E, kFull> says where they are; kFull marks a tile that lies
// wholly inside the array with vector-aligned base pointers, in which case
// every access below is an unconditional vector load or store.  Otherwise
// (the last tile, misaligned views) each access checks the lane's count.

template <int E, bool kFull>
struct Pos {
    uint64_t i0;     // flat index of element 0
    uint64_t n0;     // row of element 0
    int count;       // valid elements (E except at the end of the array)
    uint32_t last;   // bit j: element j is the last step of its row
    uint32_t first;  // bit j: element j is the first step of its row
};

template <int E, bool kFull>
__device__ __forceinline__ bool vector_ok(const Pos<E, kFull>& P, bool vec)
{
    return kFull || (vec && P.count == E);
}

template <int E, bool kFull>
__device__ __forceinline__ void load_f32(float (&v)[E], const float* __restrict__ p,
                                         const Pos<E, kFull>& P, bool vec)
{
    if (vector_ok(P, vec)) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            const float4 q = *reinterpret_cast<const float4*>(p + P.i0 + 4 * k);
            v[4 * k + 0] = q.x;
            v[4 * k + 1] = q.y;
            v[4 * k + 2] = q.z;
            v[4 * k + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = (j < P.count) ? p[P.i0 + j] : 0.0f;
    }
}

template <int E, bool kFull>
__device__ __forceinline__ void load_u32(uint32_t (&v)[E], const int32_t* __restrict__ p,
                                         const Pos<E, kFull>& P, bool vec)
{
    if (vector_ok(P, vec)) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            const int4 q = *reinterpret_cast<const int4*>(p + P.i0 + 4 * k);
            v[4 * k + 0] = (uint32_t)q.x;
            v[4 * k + 1] = (uint32_t)q.y;
            v[4 * k + 2] = (uint32_t)q.z;
            v[4 * k + 3] = (uint32_t)q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = (j < P.count) ? (uint32_t)p[P.i0 + j] : 0u;
    }
}

// Bit k of the result is (byte k of w != 0).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w)
{
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) bits |= (((w >> (8 * k)) & 0xffu) != 0u ? 1u : 0u) << k;
    return bits;
}

// Bit j of the result is (mask[i0 + j] != 0); a null mask reads as all zero.
template <int E, bool kFull>
__device__ __forceinline__ uint32_t load_mask(const uint8_t* __restrict__ p, const Pos<E, kFull>& P,
                                              bool vec)
{
    static_assert(E == 4 || E == 8 || E == 16, "mask loads are 4, 8 or 16 bytes");
    if (vector_ok(P, vec)) {
        if (E == 4) return nonzero_bytes(*reinterpret_cast<const uint32_t*>(p + P.i0));
        if (E == 8) {
            const uint2 w = *reinterpret_cast<const uint2*>(p + P.i0);
            return nonzero_bytes(w.x) | (nonzero_bytes(w.y) << 4);
        }
        const uint4 w = *reinterpret_cast<const uint4*>(p + P.i0);
        return nonzero_bytes(w.x) | (nonzero_bytes(w.y) << 4) | (nonzero_bytes(w.z) << 8) |
               (nonzero_bytes(w.w) << 12);
    }
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < E; ++j)
        if (j < P.count && p[P.i0 + j] != 0) bits |= 1u << j;
    return bits;
}

// Outputs are written once and not read again by this launch: full-tile
// stores are non-temporal (streamed past the caches).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int E, bool kFull>
__device__ __forceinline__ void store_f32(float* __restrict__ p, const float (&v)[E],
                                          const Pos<E, kFull>& P, bool vec)
{
    if (vector_ok(P, vec)) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
            __builtin_nontemporal_store(f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]},
                                        reinterpret_cast<f32x4*>(p + P.i0 + 4 * k));
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (j < P.count) p[P.i0 + j] = v[j];
    }
}

template <int E, bool kFull>
__device__ __forceinline__ void store_u32(int32_t* __restrict__ p, const uint32_t (&v)[E],
                                          const Pos<E, kFull>& P, bool vec)
{
    if (vector_ok(P, vec)) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
            __builtin_nontemporal_store(u32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]},
                                        reinterpret_cast<u32x4*>(p + P.i0 + 4 * k));
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (j < P.count) p[P.i0 + j] = (int32_t)v[j];
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
    uint32_t polls = 0;
    // Common case first: the adjacent tile's aggregate alone settles the
    // carry when its b is zero (a cut inside it, or gamma*lambda products
    // that underflow across a tile).  Poll just that record, one load pair.
    {
        const uint64_t j = kBackward ? (uint64_t)tile + 1 : (uint64_t)tile - 1;
        for (;;) {
            const uint64_t wa = ld_agent(rec + 2 * j);
            const uint64_t wb = ld_agent(rec + 2 * j + 1);
            if ((uint32_t)(wa >> 32) == tag && (uint32_t)(wb >> 32) == tag) {
                if (from_bits<T>((uint32_t)wb) == T(0)) return from_bits<T>((uint32_t)wa);
                break;  // the segment continues past it: full look-back below
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
    Aff<T> acc = identity<T>();
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
                tot.a = readlane(tot.a, 0);
                tot.b = readlane(tot.b, 0);
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
