// estimators.hpp -- per-estimator coefficient construction and epilogues.
//
// Each functor Op<E> handles the E consecutive elements a lane owns:
//   prepare(): load the raw streams once (vector loads), build alpha_j and
//              beta_j in registers, keep what the epilogue needs;
//   far_open(): whether the lane's far boundary element takes a value from
//              beyond the lane (backward: not an episode end; forward: not a
//              reset), used to skip the cross-tile carry when a tile ends on
//              a boundary;
//   finish():  given the value entering from the far side, run the lane's
//              serial recursion, apply the epilogue, store once.
// The [N, T] arrays are treated as one flat stream of N*T elements in which
// row ends are ordinary segment boundaries; Pos gives each element's place
// in its row.  Every load depends on positions only, never on another loaded
// value, so all of a lane's loads are in flight together.
//
// Definitions follow the rl-triton README Kernels table (one row per
// estimator) and the boundary rules of the gist.science technical summary,
// Methodology 3 (terminated: successor value 0; truncated: supplied value;
// rollout-window end: bootstrap value in the local term only).
#pragma once

#include "scan_core.hpp"

namespace lrs {

struct Ctx {
    uint64_t total;  // N*T
    uint32_t T;      // seq_len
    int lane;
    bool vec;        // base pointers allow vector access
};

// e^x on the hardware base-2 exponential (v_exp_f32, correct to about one
// unit in the last place): e^x = 2^(x * log2(e)).  Rounding x * log2(e) to
// fp32 adds a relative error of about |x| * 2^-24 to the result, so for
// log-ratios of moderate size the result stays within a few units in the last
// place, far inside the parity bound of the estimators that take it.
__device__ __forceinline__ float exp_e(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// Tile shape of an op's look-back launches on fp32 data (measured on long
// rows): four elements per lane in 2048-element tiles for GAE and V-trace;
// four per lane in 4096-element tiles for Retrace (its four input streams
// and shifted traces; 1-2% faster than 2048 at 64 x 131072, 12% with
// truncations at 1024 x 16384) and the affine scan; eight per lane for the
// ops with few streams, the prefix sums included (int32: 12-21% faster
// than four per lane in 4096-element tiles).
enum LookbackTile { kLbNarrow, kLbLight, kLbWide4 };

// kLeanSgprs: the op's look-back launches (four or more waves per block) use
// a kernel built with a cap on scalar registers.  A block of W waves needs W / 4 wave
// slots on each SIMD, and on gfx950 a kernel measured to need at most about 72
// SGPRs for eight waves per SIMD (more cost it blocks per CU, whatever the
// compiler's occupancy estimate says).  V-trace's kernels hold 83-100; capped,
// they spill a few to vector lanes and run 2-3% faster on long rows.  Maps
// composed in fp64 are capped for every op (the fp32 prefix sum at 64 x 131072:
// one block per CU instead of two, 22.9 -> 19.0 us).
// kLeanTm: the op's time-major kernels with 16 steps per lane take a twin
// capped for eight waves per SIMD (64 VGPRs and 72 SGPRs) on grids larger
// than the CU count, for contiguous arrays.  Only where they fit without
// spills: discounted returns and traces with maps composed in fp32
// (kLeanTmFp32), the prefix sums with either composition (kLeanTmAny).  At
// 4096 x 2048: discounted 21.5 -> 19.0 us, traces 21.5 -> 19.5, fp32 prefix
// sum 22.1 -> 19.3.  GAE, TD(lambda), V-trace and Retrace spill under the
// caps and ran 7% to 2.3x slower.
enum LeanTm { kLeanTmNo, kLeanTmFp32, kLeanTmAny };

// Value of stream p at flat index i0+E (element 0 of the next chunk).  Full
// tiles load it in every lane (same cache line as the neighbouring chunk's
// vector load), unconditionally, so it is in flight with the lane's other
// loads; it is discarded where unused.  (Taking it from the neighbouring lane
// instead, with a DPP shift after the vector load, measured 3-12% slower at
// 4096 x 128: the wave then waits for that load before issuing the rest.)
// The guarded path takes it from the lane holding the next chunk (backward
// estimators hold chunks in reversed lane order: lane L-1) and reads memory
// only in lane 0, which holds the wave's last chunk.  `used` (the lane's last
// element is not a row end) guarantees i0+E < N*T.
template <int E, bool F, bool TM, bool NT, bool S, class D>
__device__ __forceinline__ float next_elem(float my0, Strided<const D> a,
                                           const Pos<E, F, TM, NT, S>& P, const Ctx& c, bool used)
{
    const D* __restrict__ p = a.p;
    if constexpr (TM) {
        // time-major: the successor is the same row's next step, E rows on
        // (it exists whenever `used`); full lanes load unconditionally (their
        // own first element when unused)
        if constexpr (F) {
            const float v = to_f32(p[used ? elem_offset(P, E, a.gap) : elem_offset(P, 0, a.gap)]);
            return used ? v : 0.0f;
        }
        // partial tiles: element 0 of the array when unused (as the guarded
        // loads do), so no wait follows the load
        const float v = to_f32(p[used ? elem_offset(P, E, a.gap) : 0]);
        return used ? v : 0.0f;
    } else if constexpr (F) {
        // unused: re-read the lane's own first element (a line already
        // fetched) rather than touch the next tile.  Full tiles of a strided
        // array never straddle a row end, so element E is in row o0.
        const uint64_t b = base_offset(P, a.gap);
        const float v = to_f32(p[used ? b + E : b]);
        return used ? v : 0.0f;
    } else {
        float v = lane_prev(my0, 0.0f);
        if (c.lane == 0) v = used ? to_f32(p[elem_offset(P, E, a.gap)]) : 0.0f;
        return v;
    }
}

// The successor of the lane's last element is read only when that element
// is not the last of its row.
template <int E, bool F, bool TM, bool NT, bool S>
__device__ __forceinline__ bool successor_used(const Pos<E, F, TM, NT, S>& P)
{
    return P.count == E && !((P.last >> (E - 1)) & 1u);
}

// ------------------------------------------------ backward episode ends
// end_j  = terminated_j | truncated_j | last-in-row_j
// vend_j = successor value at an end: 0 if terminated, else trunc_values if
//          truncated, else the row's bootstrap value (0 if none).
template <int E>
struct Ends {
    uint32_t end;
    float vend[E];
};

template <class D>
struct BoundaryArgs {
    Strided<const uint8_t> term;
    Strided<const uint8_t> trunc;  // used iff the kernel is the truncating variant
    Strided<const D> tv;           // idem
    const D* boot;                 // [N]; never null: without bootstrap values the
    int has_boot;                  // host passes another input array and has_boot = 0
};

// trunc_values only matter where truncated: on row-major arrays a lane
// reads them only when it holds a truncation (with vector access, all E at
// once; otherwise element by element), and the others read as 0.  The
// stream then costs HBM traffic around truncations only.  The load depends
// on the truncation mask, so callers issue it after every other load of the
// tile.  Time-major lanes (one scalar load per step) measure faster loading
// them unconditionally with the other streams.  On row-major calls of
// 4096 x 128, where most waves hold a truncation and so wait for the mask, a
// dense load issued with the others measured no faster (-1.5% to +1.3%).
template <int E, bool F, bool TM, bool NT, bool S, class D>
__device__ __forceinline__ void load_trunc_values(float (&tv)[E], Strided<const D> p, uint32_t kap,
                                                  const Pos<E, F, TM, NT, S>& P, bool vec)
{
    if constexpr (TM) {
        load_f32<E>(tv, p, P, vec);
    } else if (vector_ok(P, vec)) {
        if (kap != 0u) {
            load_f32<E>(tv, p, P, vec);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) tv[j] = 0.0f;
        }
    } else {
        // kap has bits only for the lane's valid elements
#pragma unroll
        for (int j = 0; j < E; ++j)
            tv[j] = ((kap >> j) & 1u) ? to_f32(p.p[elem_offset(P, j, p.gap)]) : 0.0f;
    }
}

// The truncation mask of the lane's elements (0 for the non-truncating
// variants).  Estimators read it before their other streams: the
// trunc_values read waits for it, and so leaves while those are in flight.
template <int E, bool F, bool TM, bool NT, bool S, bool kTrunc, class D>
__device__ __forceinline__ uint32_t trunc_mask(const BoundaryArgs<D>& b, const Pos<E, F, TM, NT, S>& P,
                                               const Ctx& c)
{
    return kTrunc ? load_mask<E>(b.trunc, P, c.vec) : 0u;
}

// kap: trunc_mask's result.
template <int E, bool F, bool TM, bool NT, bool S, bool kTrunc, class D>
__device__ __forceinline__ Ends<E> load_ends(const BoundaryArgs<D>& b, const Pos<E, F, TM, NT, S>& P,
                                             const Ctx& c, uint32_t kap)
{
    const uint32_t tau = load_mask<E>(b.term, P, c.vec);
    // Bootstrap of each row end in the lane.  Full tiles have seq_len >= E,
    // so a lane holds at most one row end, which belongs to its first row:
    // one unconditional load.  The guarded path loads per row end.
    float bv[E];
    if constexpr (F) {
        const float b0 = to_f32(b.boot[b.has_boot ? P.n0 : 0]);
#pragma unroll
        for (int j = 0; j < E; ++j) bv[j] = b.has_boot ? b0 : 0.0f;
    } else {
        uint64_t n = P.n0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool last = (P.last >> j) & 1u;
            bv[j] = (last && b.has_boot) ? to_f32(b.boot[n]) : 0.0f;
            if (last) ++n;
        }
    }
    float tv[E];
    if constexpr (kTrunc) {
        load_trunc_values<E>(tv, b.tv, kap, P, c.vec);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) tv[j] = 0.0f;
    }
    Ends<E> r;
    r.end = tau | kap | P.last;
#pragma unroll
    for (int j = 0; j < E; ++j)
        r.vend[j] = ((tau >> j) & 1u) ? 0.0f : (((kap >> j) & 1u) ? tv[j] : bv[j]);
    return r;
}

// Elements past the end of the array are identities.
template <int E, bool F, bool TM, bool NT, bool S, class T>
__device__ __forceinline__ void clear_tail(T (&alpha)[E], T (&beta)[E], const Pos<E, F, TM, NT, S>& P)
{
    if (F) return;
#pragma unroll
    for (int j = 0; j < E; ++j)
        if (j >= P.count) {
            alpha[j] = T(0);
            beta[j] = T(1);
        }
}

template <int E>
__device__ __forceinline__ void backward_pass(float (&out)[E], const float (&alpha)[E],
                                              const float (&beta)[E], float carry)
{
    float a = carry;
#pragma unroll
    for (int j = E - 1; j >= 0; --j) {
        a = fmaf(beta[j], a, alpha[j]);
        out[j] = a;
    }
}

// --------------------------------------------------------------- GAE
// README Kernels table (compute_gae): delta_t = r_t + gamma*Vnext_t - V_t,
// A_t = delta_t + gamma*lambda*A_{t+1} inside an episode.
template <class D>
struct GaeArgs {
    BoundaryArgs<D> b;
    Strided<const D> rewards;
    Strided<const D> values;
    float gamma, gl;  // gl = fp32(gamma*lambda)
    Strided<D> adv;
};

template <int E, bool kTrunc, class D = float>
struct GaeOp {
    using T = float;
    using Args = GaeArgs<D>;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = true;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbNarrow;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmNo;
    struct State {
        uint32_t end;
    };

    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        const uint32_t kap = trunc_mask<E, F, TM, NT, S, kTrunc>(a.b, P, c);  // first: see trunc_mask
        float r[E], v[E];
        load_f32<E>(r, a.rewards, P, c.vec);
        load_f32<E>(v, a.values, P, c.vec);
        const float vnx = next_elem<E>(v[0], a.values, P, c, successor_used(P));
        const Ends<E> e = load_ends<E, F, TM, NT, S, kTrunc>(a.b, P, c, kap);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool end = (e.end >> j) & 1u;
            const float v1 = (j + 1 < E) ? v[(j + 1) % E] : vnx;
            const float vn = end ? e.vend[j] : v1;
            alpha[j] = fmaf(a.gamma, vn, r[j]) - v[j];
            beta[j] = end ? 0.0f : a.gl;
        }
        clear_tail(alpha, beta, P);
        s.end = e.end;
    }
    __device__ static bool far_open(const State& s) { return !((s.end >> (E - 1)) & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State&,
                                  float carry)
    {
        float out[E];
        backward_pass<E>(out, alpha, beta, carry);
        store_f32<E>(a.adv, out, P, c.vec);
    }
};

// -------------------------------------------------------- TD(lambda) returns
// README Kernels table (compute_lambda_returns):
// G_t = r_t + gamma*((1-lambda)*V_{t+1} + lambda*G_{t+1}) inside an episode,
// G_t = r_t + gamma*Vnext_t at its end.
template <class D>
struct LambdaArgs {
    BoundaryArgs<D> b;
    Strided<const D> rewards;
    Strided<const D> values;
    float gamma, gl, g1l;  // gl = fp32(gamma*lambda), g1l = fp32(gamma*(1-lambda))
    Strided<D> out;
};

template <int E, bool kTrunc, class D = float>
struct LambdaOp {
    using T = float;
    using Args = LambdaArgs<D>;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = true;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbLight;
    // non-temporal input loads measure slower for this op on long rows
    static constexpr bool kStreamLoads = false;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmNo;
    struct State {
        uint32_t end;
    };

    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        const uint32_t kap = trunc_mask<E, F, TM, NT, S, kTrunc>(a.b, P, c);  // first: see trunc_mask
        float r[E], v[E];
        load_f32<E>(r, a.rewards, P, c.vec);
        load_f32<E>(v, a.values, P, c.vec);
        const float vnx = next_elem<E>(v[0], a.values, P, c, successor_used(P));
        const Ends<E> e = load_ends<E, F, TM, NT, S, kTrunc>(a.b, P, c, kap);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool end = (e.end >> j) & 1u;
            const float v1 = (j + 1 < E) ? v[(j + 1) % E] : vnx;
            alpha[j] = end ? fmaf(a.gamma, e.vend[j], r[j]) : fmaf(a.g1l, v1, r[j]);
            beta[j] = end ? 0.0f : a.gl;
        }
        clear_tail(alpha, beta, P);
        s.end = e.end;
    }
    __device__ static bool far_open(const State& s) { return !((s.end >> (E - 1)) & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State&,
                                  float carry)
    {
        float out[E];
        backward_pass<E>(out, alpha, beta, carry);
        store_f32<E>(a.out, out, P, c.vec);
    }
};

// --------------------------------------------------------- discounted returns
// README Kernels table (compute_discounted_returns): G_t = r_t + gamma*G_{t+1}
// inside an episode, r_t + gamma*Vnext_t at its end (values never read).
template <class D>
struct DiscArgs {
    BoundaryArgs<D> b;
    Strided<const D> rewards;
    float gamma;
    Strided<D> out;
};

template <int E, bool kTrunc, class D = float>
struct DiscOp {
    using T = float;
    using Args = DiscArgs<D>;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = true;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbLight;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmFp32;
    struct State {
        uint32_t end;
    };

    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        const uint32_t kap = trunc_mask<E, F, TM, NT, S, kTrunc>(a.b, P, c);  // first: see trunc_mask
        float r[E];
        load_f32<E>(r, a.rewards, P, c.vec);
        const Ends<E> e = load_ends<E, F, TM, NT, S, kTrunc>(a.b, P, c, kap);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool end = (e.end >> j) & 1u;
            alpha[j] = end ? fmaf(a.gamma, e.vend[j], r[j]) : r[j];
            beta[j] = end ? 0.0f : a.gamma;
        }
        clear_tail(alpha, beta, P);
        s.end = e.end;
    }
    __device__ static bool far_open(const State& s) { return !((s.end >> (E - 1)) & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State&,
                                  float carry)
    {
        float out[E];
        backward_pass<E>(out, alpha, beta, carry);
        store_f32<E>(a.out, out, P, c.vec);
    }
};

// ------------------------------------------------------------------ V-trace
// README Kernels table (compute_vtrace: importance-weighted targets and
// advantages); Espeholt et al. 2018 eq. 1 with c_t = lambda*min(c_bar, w_t):
// A_t = rho_t*(r_t + gamma*Vnext_t - V_t) + gamma*c_t*A_{t+1}, vs_t = V_t + A_t,
// pg_t = min(pg_rho_bar, w_t)*(r_t + gamma*(end_t ? Vnext_t : vs_{t+1}) - V_t).
template <class D>
struct VtraceArgs {
    BoundaryArgs<D> b;
    Strided<const D> log_rhos;
    Strided<const D> rewards;
    Strided<const D> values;
    float gamma, lambda, rho_bar, c_bar, pg_rho_bar;
    Strided<D> vs;
    Strided<D> pg;
};

template <int E, bool kTrunc, class D = float>
struct VtraceOp {
    using T = float;
    using Args = VtraceArgs<D>;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = true;
    // Whole rows of 4096 or 8192 in one block (E = 8 or 16 waves) cost
    // this op occupancy: its per-element state needs more registers.
    static constexpr bool kWideTiles = false;
    static constexpr LookbackTile kLookbackTile = kLbNarrow;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = true;
    static constexpr LeanTm kLeanTm = kLeanTmNo;
    struct State {
        uint32_t end;
        float r[E], v[E], tgt[E], rho_pg[E];  // tgt: Vnext at ends, V_{t+1} elsewhere
    };

    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        const uint32_t kap = trunc_mask<E, F, TM, NT, S, kTrunc>(a.b, P, c);  // first: see trunc_mask
        float lr[E];
        load_f32<E>(lr, a.log_rhos, P, c.vec);
        load_f32<E>(s.r, a.rewards, P, c.vec);
        load_f32<E>(s.v, a.values, P, c.vec);
        const float vnx = next_elem<E>(s.v[0], a.values, P, c, successor_used(P));
        const Ends<E> e = load_ends<E, F, TM, NT, S, kTrunc>(a.b, P, c, kap);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool end = (e.end >> j) & 1u;
            const float w = exp_e(lr[j]);
            const float rho = fminf(a.rho_bar, w);
            const float cc = a.lambda * fminf(a.c_bar, w);
            const float v1 = (j + 1 < E) ? s.v[(j + 1) % E] : vnx;
            const float vn = end ? e.vend[j] : v1;
            s.tgt[j] = vn;
            s.rho_pg[j] = fminf(a.pg_rho_bar, w);
            alpha[j] = rho * (fmaf(a.gamma, vn, s.r[j]) - s.v[j]);
            beta[j] = end ? 0.0f : a.gamma * cc;
        }
        clear_tail(alpha, beta, P);
        s.end = e.end;
    }
    __device__ static bool far_open(const State& s) { return !((s.end >> (E - 1)) & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State& s,
                                  float carry)
    {
        float vs[E], pg[E];
        float a_next = carry;  // A at the element after j
#pragma unroll
        for (int j = E - 1; j >= 0; --j) {
            const float A = fmaf(beta[j], a_next, alpha[j]);
            const bool end = (s.end >> j) & 1u;
            const float target = end ? s.tgt[j] : s.tgt[j] + a_next;  // Vnext or vs_{t+1}
            vs[j] = s.v[j] + A;
            pg[j] = s.rho_pg[j] * (fmaf(a.gamma, target, s.r[j]) - s.v[j]);
            a_next = A;
        }
        store_f32<E>(a.vs, vs, P, c.vec);
        store_f32<E>(a.pg, pg, P, c.vec);
    }
};

// ------------------------------------------------------------------ Retrace
// README Kernels table (compute_retrace: off-policy return with truncated
// importance ratios); Munos et al. 2016 with c_{t+1} = lambda*min(c_bar, w_{t+1}):
// G_t = r_t + gamma*(V_{t+1} - c_{t+1}*Q_{t+1}) + gamma*c_{t+1}*G_{t+1} inside
// an episode, r_t + gamma*Vnext_t at its end.
template <class D>
struct RetraceArgs {
    BoundaryArgs<D> b;
    Strided<const D> log_rhos;
    Strided<const D> rewards;
    Strided<const D> q_values;
    Strided<const D> values;
    float gamma, lambda, c_bar;
    Strided<D> out;
};

template <int E, bool kTrunc, class D = float>
struct RetraceOp {
    using T = float;
    using Args = RetraceArgs<D>;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = true;
    // Whole rows of 4096 or 8192 in one block (E = 8 or 16 waves) cost
    // this op occupancy: its per-element state needs more registers.
    static constexpr bool kWideTiles = false;
    static constexpr LookbackTile kLookbackTile = kLbWide4;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmNo;
    struct State {
        uint32_t end;
    };

    __device__ static float trace(const Args& a, float lr)
    {
        return a.lambda * fminf(a.c_bar, exp_e(lr));
    }

    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        const uint32_t kap = trunc_mask<E, F, TM, NT, S, kTrunc>(a.b, P, c);  // first: see trunc_mask
        float lr[E], r[E], q[E], v[E], cc[E];
        load_f32<E>(lr, a.log_rhos, P, c.vec);
        load_f32<E>(r, a.rewards, P, c.vec);
        load_f32<E>(q, a.q_values, P, c.vec);
        load_f32<E>(v, a.values, P, c.vec);
        const bool used = successor_used(P);
        // successor (t+1) quantities of the lane's last element
        const float lrnx = next_elem<E>(lr[0], a.log_rhos, P, c, used);
        const float qnx = next_elem<E>(q[0], a.q_values, P, c, used);
        const float vnx = next_elem<E>(v[0], a.values, P, c, used);
        const Ends<E> e = load_ends<E, F, TM, NT, S, kTrunc>(a.b, P, c, kap);
#pragma unroll
        for (int j = 0; j < E; ++j) cc[j] = trace(a, lr[j]);
        const float cnx = trace(a, lrnx);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool end = (e.end >> j) & 1u;
            const float c1 = (j + 1 < E) ? cc[(j + 1) % E] : cnx;
            const float q1 = (j + 1 < E) ? q[(j + 1) % E] : qnx;
            const float v1 = (j + 1 < E) ? v[(j + 1) % E] : vnx;
            alpha[j] = end ? fmaf(a.gamma, e.vend[j], r[j]) : fmaf(a.gamma, fmaf(-c1, q1, v1), r[j]);
            beta[j] = end ? 0.0f : a.gamma * c1;
        }
        clear_tail(alpha, beta, P);
        s.end = e.end;
    }
    __device__ static bool far_open(const State& s) { return !((s.end >> (E - 1)) & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State&,
                                  float carry)
    {
        float out[E];
        backward_pass<E>(out, alpha, beta, carry);
        store_f32<E>(a.out, out, P, c.vec);
    }
};

// --------------------------------------------------- forward estimators
// reset_j = first-in-row_j | dones_{j-1}.  dones of the element before the
// lane comes from the neighbouring lane (lane 0 of a wave reads it, except
// at a row start where it is not needed).
template <int E, bool F, bool TM, bool NT, bool S>
__device__ __forceinline__ uint32_t load_resets(Strided<const uint8_t> dn,
                                                const Pos<E, F, TM, NT, S>& P, const Ctx& c)
{
    const uint8_t* __restrict__ dones = dn.p;
    const uint32_t d = load_mask<E>(dn, P, c.vec);
    // The predecessor of element 0 is in the same row whenever it is used
    // (element 0 is not a row start): base offset - 1 (row-major) or one
    // time step back (time-major).
    uint32_t dprev;
    if constexpr (TM) {
        // time-major: the predecessor is the same row's previous step
        const bool used = P.count > 0 && !(P.first & 1u);
        const uint64_t own = elem_offset(P, 0, dn.gap);
        if constexpr (F) {
            const uint32_t w = dones[used ? own - P.stride - dn.gap : own] != 0 ? 1u : 0u;
            dprev = used ? w : 0u;
        } else {
            dprev = used ? (dones[own - P.stride - dn.gap] != 0 ? 1u : 0u) : 0u;
        }
    } else if constexpr (F) {
        // every lane loads its predecessor's flag unconditionally, in flight
        // with the other loads (its own first flag where none is needed)
        const bool used = P.i0 > 0 && !(P.first & 1u);
        const uint64_t b = base_offset(P, dn.gap);
        const uint32_t w = dones[used ? b - 1 : b] != 0 ? 1u : 0u;
        dprev = used ? w : 0u;
    } else {
        dprev = lane_prev((d >> (E - 1)) & 1u, 0u);
        if (c.lane == 0 && !(P.first & 1u) && P.count > 0 && P.i0 > 0)
            dprev = dones[base_offset(P, dn.gap) - 1] != 0 ? 1u : 0u;
    }
    return P.first | (d << 1) | dprev;  // bit j: reset at element j
}

struct ForwardArgs {
    Strided<const void> x;  // D (the storage type) or int32 elements
    Strided<const uint8_t> dones;
    float gl;  // eligibility traces: fp32(gamma*lambda)
    Strided<void> out;
};

template <class D>
__device__ __forceinline__ Strided<const D> typed(Strided<const void> a)
{
    return {static_cast<const D*>(a.p), a.gap};
}
template <class D>
__device__ __forceinline__ Strided<D> typed(Strided<void> a)
{
    return {static_cast<D*>(a.p), a.gap};
}

// README Kernels table (compute_eligibility_traces):
// e_t = x_t + gamma*lambda*(1 - d_{t-1})*e_{t-1}.
template <int E, class D = float>
struct EligOp {
    using T = float;
    using Args = ForwardArgs;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = false;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbLight;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmFp32;
    struct State {
        uint32_t reset;
    };
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        load_f32<E>(alpha, typed<D>(a.x), P, c.vec);
        s.reset = load_resets<E>(a.dones, P, c);
#pragma unroll
        for (int j = 0; j < E; ++j) beta[j] = ((s.reset >> j) & 1u) ? 0.0f : a.gl;
        clear_tail(alpha, beta, P);
    }
    __device__ static bool far_open(const State& s) { return !(s.reset & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State&,
                                  float carry)
    {
        float out[E];
        float e = carry;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            e = fmaf(beta[j], e, alpha[j]);
            out[j] = e;
        }
        store_f32<E>(typed<D>(a.out), out, P, c.vec);
    }
};

// README Kernels table (compute_episodic_prefix_sum): S_t = x_t + (1 - d_{t-1})*S_{t-1}.
template <int E, class D = float>
struct PrefixF32Op {
    using T = float;
    using Args = ForwardArgs;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = false;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbLight;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmAny;
    struct State {
        uint32_t reset;
    };
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        load_f32<E>(alpha, typed<D>(a.x), P, c.vec);
        s.reset = load_resets<E>(a.dones, P, c);
#pragma unroll
        for (int j = 0; j < E; ++j) beta[j] = ((s.reset >> j) & 1u) ? 0.0f : 1.0f;
        clear_tail(alpha, beta, P);
    }
    __device__ static bool far_open(const State& s) { return !(s.reset & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State& s,
                                  float carry)
    {
        float out[E];
        float e = carry;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            e = ((s.reset >> j) & 1u) ? alpha[j] : e + alpha[j];
            out[j] = e;
        }
        (void)beta;
        store_f32<E>(typed<D>(a.out), out, P, c.vec);
    }
};

template <int E>
struct PrefixI32Op {
    using T = uint32_t;
    using Args = ForwardArgs;
    static constexpr int kElemBytes = 4;
    static constexpr bool kBackward = false;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbLight;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmAny;
    struct State {
        uint32_t reset;
    };
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   uint32_t (&alpha)[E], uint32_t (&beta)[E], State& s)
    {
        load_u32<E>(alpha, typed<int32_t>(a.x), P, c.vec);
        s.reset = load_resets<E>(a.dones, P, c);
#pragma unroll
        for (int j = 0; j < E; ++j) beta[j] = ((s.reset >> j) & 1u) ? 0u : 1u;
        clear_tail(alpha, beta, P);
    }
    __device__ static bool far_open(const State& s) { return !(s.reset & 1u); }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const uint32_t (&alpha)[E], const uint32_t (&beta)[E],
                                  const State& s, uint32_t carry)
    {
        uint32_t out[E];
        uint32_t e = carry;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            e = ((s.reset >> j) & 1u) ? alpha[j] : e + alpha[j];
            out[j] = e;
        }
        (void)beta;
        store_u32<E>(typed<int32_t>(a.out), out, P, c.vec);
    }
};

// ---------------------------------------------- generic segmented affine scan
// Summary page, Methodology 1 (Unified Algebraic Framework): every estimator
// above is the recurrence y_t = alpha_t + beta_t * y_prev over per-step pairs;
// here the pairs come from memory.  y_prev is y_{t+1} when kRev (scan from
// the row end), else y_{t-1}.  Before the row's first step in scan order it
// is carry[n] (0 without carries).  A set reset[t] drops beta_t * y_prev.
template <class D>
struct AffineArgs {
    Strided<const D> alpha;
    Strided<const D> beta;
    Strided<const uint8_t> reset;  // used iff the kernel is the resetting variant
    const D* carry;                // [N]; never null: without carries the host
    int has_carry;                 // passes another input array and has_carry = 0
    Strided<D> out;
};

template <int E, bool kRev, bool kReset, class D = float>
struct AffineOp {
    using T = float;
    using Args = AffineArgs<D>;
    static constexpr int kElemBytes = sizeof(D);
    static constexpr bool kBackward = kRev;
    static constexpr bool kWideTiles = true;
    static constexpr LookbackTile kLookbackTile = kLbWide4;
    static constexpr bool kStreamLoads = true;
    static constexpr bool kLeanSgprs = false;
    static constexpr LeanTm kLeanTm = kLeanTmNo;
    struct State {
        uint32_t cut;
    };

    template <bool F, bool TM, bool NT, bool S>
    __device__ static void prepare(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                   float (&alpha)[E], float (&beta)[E], State& s)
    {
        load_f32<E>(alpha, a.alpha, P, c.vec);
        load_f32<E>(beta, a.beta, P, c.vec);
        uint32_t reset = 0u;
        if constexpr (kReset) reset = load_mask<E>(a.reset, P, c.vec);
        // Steps whose predecessor in scan order lies outside the row.
        const uint32_t edge = kRev ? P.last : P.first;
        float cv[E];
        if constexpr (F) {
            // seq_len >= E: at most one such step per lane.  Reverse, it ends
            // the lane's first row.  Forward, it starts the lane's first row
            // if it is the lane's first element, else the next row.
            const bool next_row = !kRev && edge != 0u && !(edge & 1u);
            const float c0 = to_f32(a.carry[a.has_carry ? P.n0 + (next_row ? 1 : 0) : 0]);
#pragma unroll
            for (int j = 0; j < E; ++j) cv[j] = a.has_carry ? c0 : 0.0f;
        } else {
            uint64_t n = P.n0;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const bool e = (edge >> j) & 1u;
                if (!kRev && e && j > 0) ++n;
                cv[j] = (e && a.has_carry) ? to_f32(a.carry[n]) : 0.0f;
                if (kRev && e) ++n;
            }
        }
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool r = (reset >> j) & 1u, e = (edge >> j) & 1u;
            if (e && !r) alpha[j] = fmaf(beta[j], cv[j], alpha[j]);
            if (r || e) beta[j] = 0.0f;
        }
        clear_tail(alpha, beta, P);
        s.cut = reset | edge;
    }
    __device__ static bool far_open(const State& s)
    {
        return kRev ? !((s.cut >> (E - 1)) & 1u) : !(s.cut & 1u);
    }
    template <bool F, bool TM, bool NT, bool S>
    __device__ static void finish(const Args& a, const Pos<E, F, TM, NT, S>& P, const Ctx& c,
                                  const float (&alpha)[E], const float (&beta)[E], const State&,
                                  float carry)
    {
        float out[E];
        if constexpr (kRev) {
            backward_pass<E>(out, alpha, beta, carry);
        } else {
            float y = carry;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                y = fmaf(beta[j], y, alpha[j]);
                out[j] = y;
            }
        }
        store_f32<E>(a.out, out, P, c.vec);
    }
};

}  // namespace lrs
