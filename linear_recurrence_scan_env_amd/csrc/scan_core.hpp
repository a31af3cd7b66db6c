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

#include <type_traits>

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

__device__ __forceinline__ Aff<double> combine(Aff<double> near, Aff<double> far)
{
    return {fma(near.b, far.a, near.a), near.b * far.b};
}

__device__ __forceinline__ float apply(Aff<float> f, float x) { return fmaf(f.b, x, f.a); }
__device__ __forceinline__ double apply(Aff<double> f, double x) { return fma(f.b, x, f.a); }
__device__ __forceinline__ uint32_t apply(Aff<uint32_t> f, uint32_t x) { return f.b ? f.a + x : f.a; }

template <class T>
__device__ __forceinline__ Aff<T> identity() { return {T(0), T(1)}; }

// Maps are composed in AccOf<T>: fp32 maps in fp32 and integer maps exactly
// in uint32.  The one fp32 composition that needs more precision is a lane's
// own product of betas (see lane_aggregate in the kernel): a constant beta
// makes that product, and its rounding, the same in every lane, and the
// scan would multiply the same relative error once per lane of distance.
template <class T>
struct AccOf {
    using type = T;
};

// ------------------------------------------------------- lane exchange
//
// Lane order.  Every scan runs forward in lane order: lane L's inclusive
// value composes lanes 0..L with lane L nearest the output.  Forward
// estimators give lane L the L-th chunk of the wave; backward estimators
// give it chunk 63-L, so that "nearer the output" (earlier in time) is again
// the higher lane.  Either way the wave total sits in lane 63 and a lane's
// exclusive value comes from lane L-1.
//
// DPP (GFX9 encodings): row_shr:n -- lane i reads lane i-n of its 16-lane
// row; row_shl:n -- lane i+n; row_bcast:15 / row_bcast:31 -- lane 15 of a
// row / lane 31 feed the following row(s) selected by the row mask;
// wave_shr:1 -- lane i reads lane i-1 across the wave.  A lane whose source
// is invalid or whose row is masked off keeps `old`.
constexpr int kDppRowShl = 0x100;
constexpr int kDppRowShr = 0x110;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp(float old, float src)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                      kCtrl, kRowMask, 0xf, false));
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t src)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, kCtrl, kRowMask, 0xf, false);
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp(double old, double src)
{
    const int2 o = __builtin_bit_cast(int2, old), x = __builtin_bit_cast(int2, src);
    const int2 r = make_int2(__builtin_amdgcn_update_dpp(o.x, x.x, kCtrl, kRowMask, 0xf, false),
                             __builtin_amdgcn_update_dpp(o.y, x.y, kCtrl, kRowMask, 0xf, false));
    return __builtin_bit_cast(double, r);
}

template <int kCtrl, int kRowMask = 0xf, class T>
__device__ __forceinline__ Aff<T> dpp(Aff<T> old, Aff<T> src)
{
    return {dpp<kCtrl, kRowMask>(old.a, src.a), dpp<kCtrl, kRowMask>(old.b, src.b)};
}

__device__ __forceinline__ float readlane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ double readlane(double v, int l)
{
    const int2 x = __builtin_bit_cast(int2, v);
    return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(x.x, l),
                                                __builtin_amdgcn_readlane(x.y, l)));
}
template <class T>
__device__ __forceinline__ Aff<T> readlane(Aff<T> v, int l)
{
    return {readlane(v.a, l), readlane(v.b, l)};
}

// Value held by lane-1 (lane 0 gets `edge`).
template <class T>
__device__ __forceinline__ T lane_prev(T v, T edge)
{
    return dpp<kDppWaveShr1>(edge, v);
}

// Inclusive forward scan over the 64 lanes: four row_shr steps inside each
// 16-lane row, then row_bcast:15 and row_bcast:31 carry row totals into the
// rows above.
template <class T>
__device__ __forceinline__ Aff<T> lane_scan(Aff<T> x)
{
    const Aff<T> id = identity<T>();
    x = combine(x, dpp<kDppRowShr + 1>(id, x));
    x = combine(x, dpp<kDppRowShr + 2>(id, x));
    x = combine(x, dpp<kDppRowShr + 4>(id, x));
    x = combine(x, dpp<kDppRowShr + 8>(id, x));
    x = combine(x, dpp<kDppRowBcast15, 0xa>(id, x));
    x = combine(x, dpp<kDppRowBcast31, 0xc>(id, x));
    return x;
}

// Exclusive value of a lane: the inclusive value of lane-1.
template <class T>
__device__ __forceinline__ Aff<T> lane_exclusive(Aff<T> inc)
{
    return dpp<kDppWaveShr1>(identity<T>(), inc);
}

// Inclusive scan of lanes 0..W-1 (W <= 16, all in row 0).  kSuffix: lane v
// composes lanes v..W-1 (far = higher lanes); otherwise lanes 0..v.
template <bool kSuffix, int W, class T>
__device__ __forceinline__ Aff<T> row_scan(Aff<T> x)
{
    static_assert(W >= 1 && W <= 16, "one 16-lane row");
    const Aff<T> id = identity<T>();
    if (W > 1) x = combine(x, kSuffix ? dpp<kDppRowShl + 1>(id, x) : dpp<kDppRowShr + 1>(id, x));
    if (W > 2) x = combine(x, kSuffix ? dpp<kDppRowShl + 2>(id, x) : dpp<kDppRowShr + 2>(id, x));
    if (W > 4) x = combine(x, kSuffix ? dpp<kDppRowShl + 4>(id, x) : dpp<kDppRowShr + 4>(id, x));
    if (W > 8) x = combine(x, kSuffix ? dpp<kDppRowShl + 8>(id, x) : dpp<kDppRowShr + 8>(id, x));
    return x;
}

// ------------------------------------------------------- kernel arguments
// A kernel's arguments are read through the scalar cache, which starts each
// dispatch cold.  Left alone, the compiler loads each argument where it is
// first used: the schedule fields that pick the branch first, then the
// array pointers inside it, so a wave waits for several dependent cache
// misses before its first data load (at 4096 x 128 about 1 us of a 3-5 us
// call).  Reading one word of every 64-byte line of the argument block at
// entry, and consuming their xor in an empty asm statement, issues all those
// misses together; the later loads of the same lines then hit.
template <int kBytes>
__device__ __forceinline__ void warm_kernargs()
{
    typedef __attribute__((address_space(4))) const uint32_t kword;
    const kword* k = (const kword*)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t x = 0u;
#pragma unroll
    for (int off = 0; off < kBytes; off += 64) x ^= k[off / 4];
    asm volatile("" ::"s"(x));
}

// Bytes of the explicit arguments (args, sched) of a scan kernel.
template <class Args, class Sch>
constexpr int kernarg_bytes()
{
    return (int)((sizeof(Args) + alignof(Sch) - 1) / alignof(Sch) * alignof(Sch) + sizeof(Sch));
}

// ----------------------------------------------------------------- loads
// A lane owns E consecutive elements starting at flat index i0 (a multiple
// of E).  Pos<E, kFull> says where they are; kFull marks a tile that lies
// wholly inside the array with vector-aligned base pointers, in which case
// every access below is an unconditional vector load or store.  Otherwise
// (the last tile, misaligned views) each access checks the lane's count.

template <int E, bool kFull, bool kTM = false, bool kNT = false, bool kStrided = false>
struct Pos {
    uint64_t i0;     // flat index of element 0
    uint64_t n0;     // row (environment) of element 0
    int count;       // valid elements (E except at the end of the array)
    uint32_t last;   // bit j: element j is the last step of its row
    uint32_t first;  // bit j: element j is the first step of its row
    // Time-major ([T, N]) lanes: element j sits at flat index i0 + j * stride
    // (stride = N) and all E elements are steps of row n0; every access is a
    // scalar access, coalesced across the lanes of a wave, and unconditional
    // when kFull (the lane's E steps all exist).
    uint64_t stride;
    // Outer index of element 0: its row (row-major) or its time step
    // (time-major).  A strided array places the element at flat index i and
    // outer index o at p[i + o * gap] (see Strided).
    uint64_t o0;
};

// An [N, T] array (or [T, N] for time-major calls) whose rows (time steps)
// start ld elements apart, ld >= T (>= N): element (n, t) at n * ld + t, so at
// flat index i = n * T + t plus n * gap, gap = ld - T.  gap = 0 for a
// contiguous array.
template <class D>
struct Strided {
    D* p;
    uint64_t gap;
};

template <class D>
__device__ __forceinline__ Strided<const D> as_const(Strided<D> s)
{
    return {s.p, s.gap};
}

template <int E, bool kFull, bool TM, bool NT, bool S>
__device__ __forceinline__ bool vector_ok(const Pos<E, kFull, TM, NT, S>& P, bool vec)
{
    return !TM && (kFull || (vec && P.count == E));
}

// Offset of a lane's element j (0 <= j <= E) in an array with the given gap.
// Row-major: element j lies in row o0 plus the number of row ends among the
// lane's elements before it.  Time-major: element j is time step o0 + j.
// Launches whose arrays are all contiguous (S = false) ignore the gaps, which
// are then 0, and keep their address arithmetic to the flat index.
template <int E, bool kFull, bool TM, bool NT, bool S>
__device__ __forceinline__ uint64_t elem_offset(const Pos<E, kFull, TM, NT, S>& P, int j, uint64_t gap)
{
    const uint64_t flat = TM ? P.i0 + (uint64_t)j * P.stride : P.i0 + (uint64_t)j;
    if constexpr (!S) return flat;
    if constexpr (TM) return flat + (P.o0 + (uint64_t)j) * gap;
    const uint32_t before = P.last & ((1u << j) - 1u);
    return flat + (P.o0 + (uint64_t)__builtin_popcount(before)) * gap;
}

// Offset of element 0, where a lane's vector accesses start: the host allows
// vector access to a strided array only when no lane straddles a row end.
template <int E, bool kFull, bool TM, bool NT, bool S>
__device__ __forceinline__ uint64_t base_offset(const Pos<E, kFull, TM, NT, S>& P, uint64_t gap)
{
    if constexpr (!S) return P.i0;
    return P.i0 + P.o0 * gap;
}

// ------------------------------------------------------- element storage
// Data streams are fp32, or 16-bit (bfloat16 or IEEE half) with fp32
// arithmetic: loads widen exactly, stores round to nearest even (gfx950
// converts a pair of floats in one instruction).  The 16-bit types are bit
// containers; their values only ever exist as floats in registers.
struct bf16_t {
    uint16_t bits;
};
struct f16_t {
    uint16_t bits;
};
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <class D>
constexpr bool kHalfWidth = sizeof(D) == 2;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)__builtin_bit_cast(_Float16, x.bits); }

template <class D>
__device__ __forceinline__ D from_f32(float x)
{
    if constexpr (std::is_same<D, float>::value) return x;
    else if constexpr (std::is_same<D, bf16_t>::value) return D{__builtin_bit_cast(uint16_t, (__bf16)x)};
    else return D{__builtin_bit_cast(uint16_t, (_Float16)x)};
}

// Two 16-bit values packed in a word (element 2k in the low half).
template <class D>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi)
{
    if constexpr (std::is_same<D, bf16_t>::value) {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xffff0000u);
    } else {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        lo = (float)h.x;
        hi = (float)h.y;
    }
}

template <class D>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (std::is_same<D, bf16_t>::value)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Input vectors are read once per launch.  With NT set (long rows: look-back
// launches and 8192-element tiles, where it measures faster) they are loaded
// non-temporally, like the output stores; elsewhere plain loads measure
// faster.  Both go component by component through HIP's vector structs, so
// that the compiler can drop components a lane never reads (a lane that only
// needs elements 1..3 issues one 12-byte load).
template <class V, bool NT, class S>
__device__ __forceinline__ V ld_vec(const S* p)
{
    if constexpr (!NT) {
        return *reinterpret_cast<const V*>(p);
    } else if constexpr (std::is_arithmetic<V>::value) {
        return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
    } else {
        using C = typename V::value_type;
        constexpr int n = sizeof(V) / sizeof(C);
        static_assert(n == 2 || n == 4, "two- or four-component vectors");
        const C* q = reinterpret_cast<const C*>(p);
        V r;
        r.x = __builtin_nontemporal_load(q);
        r.y = __builtin_nontemporal_load(q + 1);
        if constexpr (n == 4) {
            r.z = __builtin_nontemporal_load(q + 2);
            r.w = __builtin_nontemporal_load(q + 3);
        }
        return r;
    }
}

// One element; non-temporal for time-major tiles with NT set.
template <bool NTL, class D>
__device__ __forceinline__ D get(const D* p)
{
    if constexpr (!NTL) {
        return *p;
    } else if constexpr (std::is_arithmetic<D>::value) {
        return __builtin_nontemporal_load(p);
    } else {
        static_assert(sizeof(D) == 2, "16-bit storage types");
        return D{__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p))};
    }
}

template <int E, bool kFull, bool TM, bool NT, bool S, class D>
__device__ __forceinline__ void load_f32(float (&v)[E], Strided<const D> a,
                                         const Pos<E, kFull, TM, NT, S>& P, bool vec)
{
    const D* __restrict__ p = a.p;
    if (vector_ok(P, vec)) {
        const uint64_t b = base_offset(P, a.gap);
        if constexpr (std::is_same<D, float>::value) {
#pragma unroll
            for (int k = 0; k < E / 4; ++k) {
                const float4 q = ld_vec<float4, NT>(p + b + 4 * k);
                v[4 * k + 0] = q.x;
                v[4 * k + 1] = q.y;
                v[4 * k + 2] = q.z;
                v[4 * k + 3] = q.w;
            }
        } else if constexpr (E == 4) {
            const uint2 q = ld_vec<uint2, NT>(p + b);
            unpack2<D>(q.x, v[0], v[1]);
            unpack2<D>(q.y, v[2], v[3]);
        } else {
#pragma unroll
            for (int k = 0; k < E / 8; ++k) {
                const uint4 q = ld_vec<uint4, NT>(p + b + 8 * k);
                unpack2<D>(q.x, v[8 * k + 0], v[8 * k + 1]);
                unpack2<D>(q.y, v[8 * k + 2], v[8 * k + 3]);
                unpack2<D>(q.z, v[8 * k + 4], v[8 * k + 5]);
                unpack2<D>(q.w, v[8 * k + 6], v[8 * k + 7]);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool in = kFull || j < P.count;
            if constexpr (TM) {
                // as in load_mask: every element loaded (element 0 of the array
                // for those past the count), then masked
                const float x = to_f32(get<NT>(p + (in ? elem_offset(P, j, a.gap) : 0)));
                v[j] = in ? x : 0.0f;
            } else {
                v[j] = in ? to_f32(p[elem_offset(P, j, a.gap)]) : 0.0f;
            }
        }
    }
}

template <int E, bool kFull, bool TM, bool NT, bool S>
__device__ __forceinline__ void load_u32(uint32_t (&v)[E], Strided<const int32_t> a,
                                         const Pos<E, kFull, TM, NT, S>& P, bool vec)
{
    const int32_t* __restrict__ p = a.p;
    if (vector_ok(P, vec)) {
        const uint64_t b = base_offset(P, a.gap);
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            const uint4 q = ld_vec<uint4, NT>(p + b + 4 * k);
            v[4 * k + 0] = q.x;
            v[4 * k + 1] = q.y;
            v[4 * k + 2] = q.z;
            v[4 * k + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool in = kFull || j < P.count;
            if constexpr (TM) {
                const uint32_t x = (uint32_t)get<NT>(p + (in ? elem_offset(P, j, a.gap) : 0));
                v[j] = in ? x : 0u;
            } else {
                v[j] = in ? (uint32_t)p[elem_offset(P, j, a.gap)] : 0u;
            }
        }
    }
}

// Bit k of the result is (byte k of w != 0).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w)
{
    // Bit 7 of each byte of h is set iff that byte of w is nonzero (the low
    // seven bits plus 0x7f carry into bit 7 without leaving the byte).
    const uint32_t h = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
    // Multiplying by 2^21 + 2^14 + 2^7 + 1 moves bits 7, 15, 23, 31 to bits
    // 28..31; no two partial products share a bit, so nothing carries.
    return (h * 0x00204081u) >> 28;
}

// Bit j of the result is (mask[i0 + j] != 0); a null mask reads as all zero.
template <int E, bool kFull, bool TM, bool NT, bool S>
__device__ __forceinline__ uint32_t load_mask(Strided<const uint8_t> a, const Pos<E, kFull, TM, NT, S>& P,
                                              bool vec)
{
    static_assert(E == 4 || E == 8 || E == 16, "mask loads are 4, 8 or 16 bytes");
    const uint8_t* __restrict__ p = a.p;
    if (vector_ok(P, vec)) {
        const uint64_t b = base_offset(P, a.gap);
        if (E == 4) return nonzero_bytes(ld_vec<uint32_t, NT>(p + b));
        if (E == 8) {
            const uint2 w = ld_vec<uint2, NT>(p + b);
            return nonzero_bytes(w.x) | (nonzero_bytes(w.y) << 4);
        }
        const uint4 w = ld_vec<uint4, NT>(p + b);
        return nonzero_bytes(w.x) | (nonzero_bytes(w.y) << 4) | (nonzero_bytes(w.z) << 8) |
               (nonzero_bytes(w.w) << 12);
    }
    uint32_t bits = 0;
    if constexpr (TM) {
        // Time-major lanes take this path for every partial tile.  Every
        // element is loaded, those past the lane's count from element 0 of the
        // array (which exists), and masked after: no load sits under a branch
        // or is overwritten while in flight, so the lane's loads are all
        // issued before the first wait instead of one round trip each
        // (4096 x 100: 37-58% faster; row-major tiles, which come here only
        // for a tail lane, measured 0-7% slower with it).
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool in = kFull || j < P.count;
            const uint8_t m = get<NT>(p + (in ? elem_offset(P, j, a.gap) : 0));
            bits |= (uint32_t)(in && m != 0) << j;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if ((kFull || j < P.count) && p[elem_offset(P, j, a.gap)] != 0) bits |= 1u << j;
    }
    return bits;
}

// Outputs are written once and not read again by this launch: full-tile
// stores are non-temporal (streamed past the caches), and so are the
// element-wise stores of time-major tiles, whose wave stores cover 64
// consecutive environments of one time step (4096 environments x 2048 steps:
// a plain load/store kernel of that tiling took 17.4 us with plain stores,
// 15.8 with non-temporal ones).
template <bool NTS, class D>
__device__ __forceinline__ void put(D* p, D v)
{
    if constexpr (!NTS) {
        *p = v;
    } else if constexpr (std::is_arithmetic<D>::value) {
        __builtin_nontemporal_store(v, p);
    } else {
        static_assert(sizeof(D) == 2, "16-bit storage types");
        __builtin_nontemporal_store(v.bits, reinterpret_cast<uint16_t*>(p));
    }
}

template <int E, bool kFull, bool TM, bool NT, bool S, class D>
__device__ __forceinline__ void store_f32(Strided<D> a, const float (&v)[E],
                                          const Pos<E, kFull, TM, NT, S>& P, bool vec)
{
    D* __restrict__ p = a.p;
    if (vector_ok(P, vec)) {
        const uint64_t b = base_offset(P, a.gap);
        if constexpr (std::is_same<D, float>::value) {
#pragma unroll
            for (int k = 0; k < E / 4; ++k)
                __builtin_nontemporal_store(f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]},
                                            reinterpret_cast<f32x4*>(p + b + 4 * k));
        } else if constexpr (E == 4) {
            __builtin_nontemporal_store(u32x2{pack2<D>(v[0], v[1]), pack2<D>(v[2], v[3])},
                                        reinterpret_cast<u32x2*>(p + b));
        } else {
#pragma unroll
            for (int k = 0; k < E / 8; ++k)
                __builtin_nontemporal_store(
                    u32x4{pack2<D>(v[8 * k + 0], v[8 * k + 1]), pack2<D>(v[8 * k + 2], v[8 * k + 3]),
                          pack2<D>(v[8 * k + 4], v[8 * k + 5]), pack2<D>(v[8 * k + 6], v[8 * k + 7])},
                    reinterpret_cast<u32x4*>(p + b + 8 * k));
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (kFull || j < P.count) put<TM>(p + elem_offset(P, j, a.gap), from_f32<D>(v[j]));
    }
}

template <int E, bool kFull, bool TM, bool NT, bool S>
__device__ __forceinline__ void store_u32(Strided<int32_t> a, const uint32_t (&v)[E],
                                          const Pos<E, kFull, TM, NT, S>& P, bool vec)
{
    int32_t* __restrict__ p = a.p;
    if (vector_ok(P, vec)) {
        const uint64_t b = base_offset(P, a.gap);
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
            __builtin_nontemporal_store(u32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]},
                                        reinterpret_cast<u32x4*>(p + b + 4 * k));
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (kFull || j < P.count) put<TM>(p + elem_offset(P, j, a.gap), (int32_t)v[j]);
    }
}

// ------------------------------------------------ cross-tile carry protocol
//
// Workspace: a header followed by one 32-byte record per tile: four 64-bit
// words, each (tag << 32 | payload), the payloads being the low and high
// halves of the tile aggregate's a and b (64-bit composition values; the
// integer prefix sum leaves the high halves zero).  Every word is written
// and read with single-copy-atomic 64-bit accesses at agent scope, and each
// word carries its own tag, so a reader that sees all four tags equal to this
// launch's tag holds a consistent aggregate without any fence.
//
// Header: the launch epoch, an error word, a group counter `top`, and
// kGroups count words on separate cache lines, each (epoch << 32 | blocks
// of the current launch counted so far).  Block b counts itself with one
// atomic add on word b % kGroups.  The row-major kernel does this at the
// block's start, in flight with the tile's loads, and takes its tag from the
// word's old value, so the tag read and the count are one access that no
// wave waits for until the tag is needed.  The time-major kernel reads the
// epoch at the start and counts at the block's end.  Either way a block has
// its tag before it is counted.  The block that counted last in its group
// counts the group in `top`; the one that completes `top` has seen every
// block of the launch take its tag, so it rewrites every count word as
// (epoch + 1) << 32, zeroes `top` and advances `epoch`.  The next launch on
// the same stream thus starts clean, and stale records (older tags, or the
// zero fill) are never mistaken for fresh ones.  Spreading the counts keeps
// same-address atomics, which serialize, to a few per line.
//
// A tile only ever waits for tiles of lower block index (the host maps
// blocks to tiles so).  Workgroups of a dispatch are started in index order,
// so those blocks are running or finished and every wait ends; each wait is
// also bounded (kMaxPolls), so a violated assumption or a corrupted
// workspace yields a flagged error in the header and NaN outputs (see
// give_up_carry) instead of a hang.

constexpr uint32_t kGroups = 32;
constexpr uint32_t kLine = 128;  // bytes between counters

struct WsHeader {
    uint32_t epoch;
    uint32_t error;  // nonzero: a wait gave up (kErrTimeout)
    uint32_t top;    // number of groups whose blocks have all counted in
    uint32_t pad0[kLine / 4 - 3];
    struct {
        uint64_t word;  // epoch << 32 | blocks counted in (low half first in memory)
        uint32_t pad[kLine / 4 - 2];
    } group[kGroups];
};
static_assert(sizeof(WsHeader) == kLine * (kGroups + 1), "header layout");

__device__ __forceinline__ void st_agent_hdr(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One lane per block: count the block; the returned word holds the launch's
// epoch.  Only launches with carries between tiles call these.
__device__ __forceinline__ uint64_t count_block(WsHeader* hdr, uint32_t block)
{
    return __hip_atomic_fetch_add(&hdr->group[block % kGroups].word, 1ull, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// The launch tag from a count word held by lane 0 of the calling wave
// (wave-uniform result).
__device__ __forceinline__ uint32_t launch_tag(uint64_t entry)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(entry >> 32), 0) + 1u;
}

// Lane 0, once its count word is in: if the block was its group's last to
// be counted, count the group in `top` and return top's old value (the
// launch is complete when it is groups - 1); otherwise ~0u.
__device__ __forceinline__ uint32_t count_group(WsHeader* hdr, uint64_t entry, uint32_t num_blocks,
                                                uint32_t block)
{
    const uint32_t g = block % kGroups;
    const uint32_t members = (num_blocks - g + kGroups - 1) / kGroups;  // blocks in group g
    if ((uint32_t)entry != members - 1u) return ~0u;
    return __hip_atomic_fetch_add(&hdr->top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0, at the block's end, with count_group's result: the block that
// completed `top` resets the counters and advances the epoch.  Every block
// holds its tag by then, and none touches the header again in this launch.
__device__ __forceinline__ void close_launch(WsHeader* hdr, uint32_t top_seen, uint32_t num_blocks,
                                             uint32_t tag)
{
    const uint32_t groups = num_blocks < kGroups ? num_blocks : kGroups;
    if (top_seen != groups - 1u) return;
    uint32_t next = tag;                 // = epoch + 1
    if (next == 0xffffffffu) next = 0u;  // keep tags (epoch + 1) nonzero
    for (uint32_t i = 0; i < kGroups; ++i) st_agent_hdr(&hdr->group[i].word, (uint64_t)next << 32);
    __hip_atomic_store(&hdr->top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&hdr->epoch, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Upper bound on the polls of one look-back wait (about a second).
constexpr uint32_t kMaxPolls = 1u << 20;
constexpr uint32_t kErrTimeout = 2u;

// The carry a tile takes when its wait gave up: a quiet NaN for floating-point
// maps, so that every output that depends on the missing carry is NaN rather
// than a plausible wrong value; 0 for the integer prefix sum (its outputs in
// that tile are then wrong, and the header's error word says so).
template <class A>
__device__ __forceinline__ A give_up_carry()
{
    if constexpr (std::is_floating_point<A>::value)
        return __builtin_nan("");
    else
        return A(0);
}

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr uint32_t kRecordWords = 4;

// 32-bit aggregates fill two words of a record, 64-bit ones all four.
template <class A>
constexpr uint32_t kWordsOf = sizeof(A) == 8 ? 4u : 2u;

__device__ __forceinline__ uint64_t payload_bits(double x) { return __builtin_bit_cast(uint64_t, x); }
__device__ __forceinline__ uint64_t payload_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint64_t payload_bits(uint32_t x) { return x; }
template <class A>
__device__ __forceinline__ A from_payload(uint32_t lo, uint32_t hi);
template <>
__device__ __forceinline__ double from_payload<double>(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <>
__device__ __forceinline__ float from_payload<float>(uint32_t lo, uint32_t)
{
    return __builtin_bit_cast(float, lo);
}
template <>
__device__ __forceinline__ uint32_t from_payload<uint32_t>(uint32_t lo, uint32_t)
{
    return lo;
}

template <class A>
__device__ __forceinline__ void publish_aggregate(uint64_t* rec, uint32_t tile, uint32_t tag,
                                                  Aff<A> agg)
{
    const uint64_t t = (uint64_t)tag << 32;
    const uint64_t a = payload_bits(agg.a), b = payload_bits(agg.b);
    uint64_t* r = rec + kRecordWords * (uint64_t)tile;
    if constexpr (kWordsOf<A> == 4) {
        st_agent(r + 0, t | (a & 0xffffffffu));
        st_agent(r + 1, t | (a >> 32));
        st_agent(r + 2, t | (b & 0xffffffffu));
        st_agent(r + 3, t | (b >> 32));
    } else {
        st_agent(r + 0, t | a);
        st_agent(r + 1, t | b);
    }
}

// One tile's record as read (possibly stale).
struct Record {
    uint64_t w[kRecordWords];
};

template <class A>
__device__ __forceinline__ Record read_record(const uint64_t* rec, uint64_t tile)
{
    const uint64_t* r = rec + kRecordWords * tile;
    if constexpr (kWordsOf<A> == 4)
        return {{ld_agent(r + 0), ld_agent(r + 1), ld_agent(r + 2), ld_agent(r + 3)}};
    else
        return {{ld_agent(r + 0), ld_agent(r + 1), 0, 0}};
}

template <class A>
__device__ __forceinline__ bool record_current(const Record& x, uint32_t tag)
{
    bool ok = (uint32_t)(x.w[0] >> 32) == tag && (uint32_t)(x.w[1] >> 32) == tag;
    if constexpr (kWordsOf<A> == 4)
        ok = ok && (uint32_t)(x.w[2] >> 32) == tag && (uint32_t)(x.w[3] >> 32) == tag;
    return ok;
}

template <class A>
__device__ __forceinline__ Aff<A> record_value(const Record& x)
{
    if constexpr (kWordsOf<A> == 4)
        return {from_payload<A>((uint32_t)x.w[0], (uint32_t)x.w[1]),
                from_payload<A>((uint32_t)x.w[2], (uint32_t)x.w[3])};
    else
        return {from_payload<A>((uint32_t)x.w[0], 0u), from_payload<A>((uint32_t)x.w[1], 0u)};
}

// The adjacent tile's record, read as early as possible (issued with the
// tile's own loads); lookback_carry() re-polls it only if this copy is stale.
template <bool kBackward, class A>
__device__ __forceinline__ Record read_adjacent(const uint64_t* rec, uint32_t tile)
{
    return read_record<A>(rec, kBackward ? (uint64_t)tile + 1 : (uint64_t)tile - 1);
}

// Executed by one full wave.  Returns the value entering `tile` from its far
// side (backward: the scan value at the first element of tile+1; forward:
// the value at the last element of tile-1).  Composes the aggregates of the
// neighbouring tiles, nearest first, up to and including the first one whose
// b is zero (a segment boundary) or the end of the array.  Only aggregates
// are used, combined in a fixed order, so the result does not depend on
// timing (deterministic run to run).
template <bool kBackward, class A>
__device__ A lookback_carry(const uint64_t* rec, uint32_t tile, uint32_t num_tiles, uint32_t tag,
                            int lane, uint32_t* error, const Record& early)
{
    uint32_t polls = 0;
    // Common case first: the adjacent tile's aggregate alone settles the
    // carry when its b is zero (a cut inside it, or gamma*lambda products
    // that underflow across a tile).  Check the early copy, then poll just
    // that record.
    {
        const uint64_t j = kBackward ? (uint64_t)tile + 1 : (uint64_t)tile - 1;
        for (bool first = true;; first = false) {
            const Record x = first ? early : read_record<A>(rec, j);
            if (record_current<A>(x, tag)) {
                const Aff<A> v = record_value<A>(x);
                if (v.b == A(0)) return v.a;
                break;  // the segment continues past it: full look-back below
            }
            if (++polls > kMaxPolls) {
                if (lane == 0)
                    __hip_atomic_fetch_or(error, kErrTimeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                return give_up_carry<A>();
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    // Window of 64 neighbours: lane l holds the one at distance 63 - l (lane
    // 63 the adjacent tile), so that the forward lane scan composes them
    // nearest-first and lane 63 ends with the whole composition.
    Aff<A> acc = identity<A>();
    for (uint32_t base = 0;; base += kWave) {
        const int64_t d = (int64_t)base + (kWave - 1 - lane);
        const int64_t j = kBackward ? (int64_t)tile + 1 + d : (int64_t)tile - 1 - d;
        const bool exists = j >= 0 && j < (int64_t)num_tiles;
        Aff<A> v = {A(0), A(0)};  // beyond the array: nothing flows in
        bool have = !exists;
        for (;;) {
            if (!have) {
                const Record x = read_record<A>(rec, (uint64_t)j);
                if (record_current<A>(x, tag)) {
                    have = true;
                    v = record_value<A>(x);
                }
            }
            const uint64_t zero_b = __ballot(have && v.b == A(0));
            const uint64_t missing = __ballot(!have);
            // nearest neighbour with b == 0 = the highest such lane
            const int l0 = zero_b ? 63 - __clzll((long long)zero_b) : 0;
            const uint64_t needed = ~0ull << l0;  // lanes l0..63
            if ((missing & needed) == 0) {
                if (lane < l0) v = identity<A>();
                const Aff<A> tot = readlane(lane_scan(v), kWave - 1);
                acc = combine(acc, tot);
                if (zero_b) return acc.a;
                break;  // all 64 neighbours continue the segment: next window
            }
            if (++polls > kMaxPolls) {
                if (lane == 0)
                    __hip_atomic_fetch_or(error, kErrTimeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                return give_up_carry<A>();
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
}

}  // namespace lrs
