// entries.hpp -- argument checks and launch of every estimator and of the
// generic affine scan, for any element type D of the data streams (float,
// bf16_t, f16_t).  Each call also states the largest beta its maps can hold
// (gamma*lambda, gamma, gamma*lambda*c_bar, 1 for sums, unbounded for caller
// coefficients), which sets the composition precision, and the layout of its
// arrays (row-major [N, T] or time-major [T, N], each with its own row
// stride).  The extern "C" functions of include/lrs.h are thin wrappers over
// these templates, one translation unit per group and storage type.
#pragma once

#include "launch.hpp"
#include "timemajor.hpp"

namespace lrs {

// Row-major [N, T] (one flat segmented scan) or time-major [T, N] (chained
// per-environment carries along time) launch of one functor.
template <template <int> class Op>
lrs_status run_layout(bool tm, const char* nm, int64_t N, int64_t T, float beta_max,
                      const typename Op<4>::Args& a, const ArrayRef* arrays, int narrays, void* ws,
                      size_t ws_bytes, hipStream_t stream)
{
    if (tm) {
        bool strided = false;
        for (int i = 0; i < narrays; ++i) strided = strided || (arrays[i].p && arrays[i].gap != 0);
        return run_tm<Op>(nm, N, T, beta_max, a, strided, ws, ws_bytes, stream);
    }
    return run<Op>(nm, N, T, beta_max, a, arrays, narrays, ws, ws_bytes, stream);
}

template <class D> struct GaeSel {
    template <int E> using T = GaeOp<E, true, D>;
    template <int E> using N = GaeOp<E, false, D>;
};
template <class D> struct LambdaSel {
    template <int E> using T = LambdaOp<E, true, D>;
    template <int E> using N = LambdaOp<E, false, D>;
};
template <class D> struct DiscSel {
    template <int E> using T = DiscOp<E, true, D>;
    template <int E> using N = DiscOp<E, false, D>;
};
template <class D> struct VtraceSel {
    template <int E> using T = VtraceOp<E, true, D>;
    template <int E> using N = VtraceOp<E, false, D>;
};
template <class D> struct RetraceSel {
    template <int E> using T = RetraceOp<E, true, D>;
    template <int E> using N = RetraceOp<E, false, D>;
};
template <class D> struct ForwardSel {
    template <int E> using Elig = EligOp<E, D>;
    template <int E> using Prefix = PrefixF32Op<E, D>;
};
template <class D> struct AffineSel {
    template <int E> using FwdR = AffineOp<E, false, true, D>;
    template <int E> using FwdN = AffineOp<E, false, false, D>;
    template <int E> using RevR = AffineOp<E, true, true, D>;
    template <int E> using RevN = AffineOp<E, true, false, D>;
};

// ------------------------------------------------------------ array layout

// The per-step arrays of one call: [N, T] row-major or [T, N] time-major,
// with one row stride per array argument (elements between consecutive rows,
// or between consecutive time steps for time-major calls), 0 meaning
// contiguous.
struct Layout {
    bool tm;
    int64_t N, T;
    const int64_t* strides;  // host array in signature order, or null
    int64_t inner() const { return tm ? N : T; }
    int64_t outer() const { return tm ? T : N; }
};

// A per-step array argument: its pointer, element size and whether the call
// writes it.
struct Arg {
    const void* p;
    int elem_bytes;
    bool out;
};

// Largest extent of a strided array, in elements (keeps every offset the
// kernels form far below 2^64).
constexpr int64_t kMaxExtent = int64_t(1) << 60;

// Checks the strides of the call's per-step arrays (args, in signature
// order), fills their gaps (row stride - contiguous row stride), and checks
// that no written array (the outputs and the workspace) shares memory with
// any other array (per-step ones by their extents, and the per-env arrays
// in `envs`).
template <int K>
lrs_status check_arrays(const char* nm, const Layout& L, const Arg (&args)[K], const Span* envs,
                        int nenvs, const void* ws, size_t ws_bytes, uint64_t (&gaps)[K])
{
    Span ins[K + 2], outs[K + 1];
    int ni = 0, no = 0;
    for (int i = 0; i < K; ++i) {
        gaps[i] = 0;
        const int64_t ld = L.strides != nullptr && args[i].p != nullptr ? L.strides[i] : 0;
        if (ld != 0) {
            if (ld < L.inner())
                return fail(LRS_ERR_INVALID_ARG,
                            "%s: row stride %lld of array argument %d is below %s = %lld (0 means "
                            "contiguous)",
                            nm, (long long)ld, i, L.tm ? "num_envs" : "seq_len",
                            (long long)L.inner());
            if (L.outer() > 1 && ld > (kMaxExtent - L.inner()) / (L.outer() - 1))
                return fail(LRS_ERR_INVALID_ARG, "%s: row stride %lld of array argument %d is too large",
                            nm, (long long)ld, i);
            gaps[i] = (uint64_t)(ld - L.inner());
        }
        const uint64_t rows = (uint64_t)L.outer(), inner = (uint64_t)L.inner();
        const uint64_t extent = ((rows - 1) * (inner + gaps[i]) + inner) * (uint64_t)args[i].elem_bytes;
        (args[i].out ? outs[no++] : ins[ni++]) = Span{args[i].p, extent};
    }
    for (int i = 0; i < nenvs && ni < K + 2; ++i) ins[ni++] = envs[i];
    outs[no++] = Span{ws, ws_bytes};
    return check_disjoint(nm, outs, no, ins, ni);
}

template <class D>
Strided<const D> in_arr(const D* p, uint64_t gap)
{
    return {p, gap};
}
template <class D>
Strided<D> out_arr(D* p, uint64_t gap)
{
    return {p, gap};
}

template <int K>
void array_refs(const Arg (&args)[K], const uint64_t (&gaps)[K], ArrayRef (&refs)[K])
{
    for (int i = 0; i < K; ++i) refs[i] = ArrayRef{args[i].p, gaps[i], args[i].elem_bytes};
}

// -------------------------------------------------------------- estimators

// Argument checks of a GAE call; fills the gaps of its six per-step arrays.
template <class D>
lrs_status gae_check(const char* nm, const Layout& L, const D* rewards, const D* values,
                     const uint8_t* term, const uint8_t* trunc, const D* tv, const D* boot,
                     float gamma, float lambda, D* adv, void* ws, size_t ws_bytes, uint64_t (&g)[6])
{
    LRS_TRY(check_common(nm, L.N, L.T));
    LRS_REQUIRE(rewards && values && adv, "%s: rewards, values and advantages are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    constexpr int s = sizeof(D);
    const Arg args[6] = {{rewards, s, false}, {values, s, false}, {term, 1, false},
                         {trunc, 1, false},   {tv, s, false},     {adv, s, true}};
    const Span envs[] = {{boot, (uint64_t)L.N * s}};
    return check_arrays(nm, L, args, envs, 1, ws, ws_bytes, g);
}

template <class D>
lrs_status gae_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* rewards,
                     const D* values, const uint8_t* term, const uint8_t* trunc, const D* tv,
                     const D* boot, float gamma, float lambda, D* adv, const int64_t* strides,
                     void* ws, size_t ws_bytes, hipStream_t stream)
{
    const Layout L{tm, N, T, strides};
    uint64_t g[6];
    LRS_TRY(gae_check<D>(nm, L, rewards, values, term, trunc, tv, boot, gamma, lambda, adv, ws,
                         ws_bytes, g));
    GaeArgs<D> a{{in_arr(term, g[2]), in_arr(trunc, g[3]), in_arr(tv, g[4]), boot ? boot : rewards,
                  boot != nullptr},
                 in_arr(rewards, g[0]), in_arr(values, g[1]), gamma,
                 (float)((double)gamma * (double)lambda), out_arr(adv, g[5])};
    constexpr int s = sizeof(D);
    const Arg args[6] = {{rewards, s, false}, {values, s, false}, {term, 1, false},
                         {trunc, 1, false},   {tv, s, false},     {adv, s, true}};
    ArrayRef r[6];
    array_refs(args, g, r);
    using S = GaeSel<D>;
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, a.gl, a, r, 6, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, a.gl, a, r, 6, ws, ws_bytes, stream);
}

template <class D>
lrs_status vtrace_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* log_rhos,
                        const D* rewards, const D* values, const uint8_t* term,
                        const uint8_t* trunc, const D* tv, const D* boot, float gamma, float lambda,
                        float rho_bar, float c_bar, float pg_rho_bar, D* vs, D* pg_adv,
                        const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(log_rhos && rewards && values && vs && pg_adv,
                "%s: log_rhos, rewards, values, vs and pg_advantages are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    LRS_REQUIRE(positive(rho_bar) && positive(c_bar) && positive(pg_rho_bar),
                "%s: rho_bar, c_bar and pg_rho_bar must be > 0", nm);
    const Layout L{tm, N, T, strides};
    constexpr int s = sizeof(D);
    const Arg args[8] = {{log_rhos, s, false}, {rewards, s, false}, {values, s, false},
                         {term, 1, false},     {trunc, 1, false},   {tv, s, false},
                         {vs, s, true},        {pg_adv, s, true}};
    const Span envs[] = {{boot, (uint64_t)N * s}};
    uint64_t g[8];
    LRS_TRY(check_arrays(nm, L, args, envs, 1, ws, ws_bytes, g));
    VtraceArgs<D> a{{in_arr(term, g[3]), in_arr(trunc, g[4]), in_arr(tv, g[5]),
                     boot ? boot : rewards, boot != nullptr},
                    in_arr(log_rhos, g[0]), in_arr(rewards, g[1]), in_arr(values, g[2]), gamma,
                    lambda, rho_bar, c_bar, pg_rho_bar, out_arr(vs, g[6]), out_arr(pg_adv, g[7])};
    ArrayRef r[8];
    array_refs(args, g, r);
    using S = VtraceSel<D>;
    const float beta_max = gamma * lambda * c_bar;  // beta_t = gamma * c_t <= this
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, beta_max, a, r, 8, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, beta_max, a, r, 8, ws, ws_bytes, stream);
}

template <class D>
lrs_status retrace_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* log_rhos,
                         const D* rewards, const D* q_values, const D* values, const uint8_t* term,
                         const uint8_t* trunc, const D* tv, const D* boot, float gamma,
                         float lambda, float c_bar, D* q_ret, const int64_t* strides, void* ws,
                         size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(log_rhos && rewards && q_values && values && q_ret,
                "%s: log_rhos, rewards, q_values, values and q_ret are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    LRS_REQUIRE(positive(c_bar), "%s: c_bar must be > 0", nm);
    const Layout L{tm, N, T, strides};
    constexpr int s = sizeof(D);
    const Arg args[8] = {{log_rhos, s, false}, {rewards, s, false}, {q_values, s, false},
                         {values, s, false},   {term, 1, false},    {trunc, 1, false},
                         {tv, s, false},       {q_ret, s, true}};
    const Span envs[] = {{boot, (uint64_t)N * s}};
    uint64_t g[8];
    LRS_TRY(check_arrays(nm, L, args, envs, 1, ws, ws_bytes, g));
    RetraceArgs<D> a{{in_arr(term, g[4]), in_arr(trunc, g[5]), in_arr(tv, g[6]),
                      boot ? boot : rewards, boot != nullptr},
                     in_arr(log_rhos, g[0]), in_arr(rewards, g[1]), in_arr(q_values, g[2]),
                     in_arr(values, g[3]), gamma, lambda, c_bar, out_arr(q_ret, g[7])};
    ArrayRef r[8];
    array_refs(args, g, r);
    using S = RetraceSel<D>;
    const float beta_max = gamma * lambda * c_bar;  // beta_t = gamma * c_t <= this
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, beta_max, a, r, 8, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, beta_max, a, r, 8, ws, ws_bytes, stream);
}

template <class D>
lrs_status lambda_returns_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* rewards,
                                const D* values, const uint8_t* term, const uint8_t* trunc,
                                const D* tv, const D* boot, float gamma, float lambda, D* out,
                                const int64_t* strides, void* ws, size_t ws_bytes,
                                hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && values && out, "%s: rewards, values and returns are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    const Layout L{tm, N, T, strides};
    constexpr int s = sizeof(D);
    const Arg args[6] = {{rewards, s, false}, {values, s, false}, {term, 1, false},
                         {trunc, 1, false},   {tv, s, false},     {out, s, true}};
    const Span envs[] = {{boot, (uint64_t)N * s}};
    uint64_t g[6];
    LRS_TRY(check_arrays(nm, L, args, envs, 1, ws, ws_bytes, g));
    LambdaArgs<D> a{{in_arr(term, g[2]), in_arr(trunc, g[3]), in_arr(tv, g[4]),
                     boot ? boot : rewards, boot != nullptr},
                    in_arr(rewards, g[0]), in_arr(values, g[1]), gamma,
                    (float)((double)gamma * (double)lambda),
                    (float)((double)gamma * (1.0 - (double)lambda)), out_arr(out, g[5])};
    ArrayRef r[6];
    array_refs(args, g, r);
    using S = LambdaSel<D>;
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, a.gl, a, r, 6, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, a.gl, a, r, 6, ws, ws_bytes, stream);
}

template <class D>
lrs_status discounted_returns_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* rewards,
                                    const uint8_t* term, const uint8_t* trunc, const D* tv,
                                    const D* boot, float gamma, D* out, const int64_t* strides,
                                    void* ws, size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && out, "%s: rewards and returns are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma), "%s: gamma must be in [0, 1]", nm);
    const Layout L{tm, N, T, strides};
    constexpr int s = sizeof(D);
    const Arg args[5] = {{rewards, s, false}, {term, 1, false}, {trunc, 1, false}, {tv, s, false},
                         {out, s, true}};
    const Span envs[] = {{boot, (uint64_t)N * s}};
    uint64_t g[5];
    LRS_TRY(check_arrays(nm, L, args, envs, 1, ws, ws_bytes, g));
    DiscArgs<D> a{{in_arr(term, g[1]), in_arr(trunc, g[2]), in_arr(tv, g[3]), boot ? boot : rewards,
                   boot != nullptr},
                  in_arr(rewards, g[0]), gamma, out_arr(out, g[4])};
    ArrayRef r[5];
    array_refs(args, g, r);
    using S = DiscSel<D>;
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, gamma, a, r, 5, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, gamma, a, r, 5, ws, ws_bytes, stream);
}

// The forward estimators' three per-step arrays: x, dones, out.
template <class X>
lrs_status forward_arrays(const char* nm, const Layout& L, const X* x, const uint8_t* dones,
                          X* out, void* ws, size_t ws_bytes, ForwardArgs* a, ArrayRef (&r)[3])
{
    constexpr int s = sizeof(X);
    const Arg args[3] = {{x, s, false}, {dones, 1, false}, {out, s, true}};
    uint64_t g[3];
    LRS_TRY(check_arrays(nm, L, args, nullptr, 0, ws, ws_bytes, g));
    a->x = Strided<const void>{x, g[0]};
    a->dones = Strided<const uint8_t>{dones, g[1]};
    a->out = Strided<void>{out, g[2]};
    array_refs(args, g, r);
    return LRS_OK;
}

template <class D>
lrs_status eligibility_traces_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* x,
                                    const uint8_t* dones, float gamma, float lambda, D* out,
                                    const int64_t* strides, void* ws, size_t ws_bytes,
                                    hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and traces are required", nm);
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    ForwardArgs a{};
    a.gl = (float)((double)gamma * (double)lambda);
    ArrayRef r[3];
    LRS_TRY(forward_arrays(nm, Layout{tm, N, T, strides}, x, dones, out, ws, ws_bytes, &a, r));
    return run_layout<ForwardSel<D>::template Elig>(tm, nm, N, T, a.gl, a, r, 3, ws, ws_bytes,
                                                    stream);
}

template <class D>
lrs_status prefix_sum_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* x,
                            const uint8_t* dones, D* out, const int64_t* strides, void* ws,
                            size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and sums are required", nm);
    ForwardArgs a{};
    a.gl = 1.0f;
    ArrayRef r[3];
    LRS_TRY(forward_arrays(nm, Layout{tm, N, T, strides}, x, dones, out, ws, ws_bytes, &a, r));
    return run_layout<ForwardSel<D>::template Prefix>(tm, nm, N, T, 1.0f, a, r, 3, ws, ws_bytes,
                                                      stream);
}

// A template only so that the kernels it launches are compiled in the one
// translation unit that calls it (I = int32_t).
template <class I>
lrs_status prefix_sum_int_entry(const char* nm, bool tm, int64_t N, int64_t T, const I* x,
                                const uint8_t* dones, I* out, const int64_t* strides, void* ws,
                                size_t ws_bytes, hipStream_t stream)
{
    static_assert(std::is_same<I, int32_t>::value, "int32 sums only");
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and sums are required", nm);
    ForwardArgs a{};
    a.gl = 1.0f;
    ArrayRef r[3];
    LRS_TRY(forward_arrays(nm, Layout{tm, N, T, strides}, x, dones, out, ws, ws_bytes, &a, r));
    return run_layout<PrefixI32Op>(tm, nm, N, T, 1.0f, a, r, 3, ws, ws_bytes, stream);
}

template <class D>
lrs_status affine_scan_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* alpha,
                             const D* beta, const uint8_t* reset, const D* carry_in, int reverse,
                             D* out, const int64_t* strides, void* ws, size_t ws_bytes,
                             hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(alpha && beta && out, "%s: alpha, beta and out are required", nm);
    LRS_REQUIRE(reverse == 0 || reverse == 1, "%s: reverse must be 0 or 1", nm);
    const Layout L{tm, N, T, strides};
    constexpr int s = sizeof(D);
    const Arg args[4] = {{alpha, s, false}, {beta, s, false}, {reset, 1, false}, {out, s, true}};
    const Span envs[] = {{carry_in, (uint64_t)N * s}};
    uint64_t g[4];
    LRS_TRY(check_arrays(nm, L, args, envs, 1, ws, ws_bytes, g));
    AffineArgs<D> a{in_arr(alpha, g[0]), in_arr(beta, g[1]),          in_arr(reset, g[2]),
                    carry_in ? carry_in : alpha, carry_in != nullptr, out_arr(out, g[3])};
    ArrayRef r[4];
    array_refs(args, g, r);
    using S = AffineSel<D>;
    const float bm = INFINITY;  // caller coefficients: no bound on beta is known
    if (reverse)
        return reset ? run_layout<S::template RevR>(tm, nm, N, T, bm, a, r, 4, ws, ws_bytes, stream)
                     : run_layout<S::template RevN>(tm, nm, N, T, bm, a, r, 4, ws, ws_bytes, stream);
    return reset ? run_layout<S::template FwdR>(tm, nm, N, T, bm, a, r, 4, ws, ws_bytes, stream)
                 : run_layout<S::template FwdN>(tm, nm, N, T, bm, a, r, 4, ws, ws_bytes, stream);
}

}  // namespace lrs
