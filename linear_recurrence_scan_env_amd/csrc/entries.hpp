// entries.hpp -- argument checks and launch of every estimator and of the
// generic affine scan, for any element type D of the data streams (float,
// bf16_t, f16_t).  Each call also states the largest beta its maps can hold
// (gamma*lambda, gamma, gamma*lambda*c_bar, 1 for sums, unbounded for caller
// coefficients), which sets the composition precision, and the layout of its
// arrays (row-major [N, T] or time-major [T, N]).  The extern "C" functions
// of include/lrs.h are thin wrappers over these templates, one translation
// unit per group and storage type.
#pragma once

#include "launch.hpp"
#include "timemajor.hpp"

namespace lrs {

// Row-major [N, T] (one flat segmented scan) or time-major [T, N] (chained
// per-environment carries along time) launch of one functor.
template <template <int> class Op>
lrs_status run_layout(bool tm, const char* nm, int64_t N, int64_t T, float beta_max,
                      const typename Op<4>::Args& a, const void* const* floats, int nfloats,
                      const void* const* masks, int nmasks, void* ws, size_t ws_bytes,
                      hipStream_t stream)
{
    if (tm) return run_tm<Op>(nm, N, T, beta_max, a, ws, ws_bytes, stream);
    return run<Op>(nm, N, T, beta_max, a, floats, nfloats, masks, nmasks, ws, ws_bytes, stream);
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

// Argument checks of a GAE call (everything but the workspace's size).
template <class D>
lrs_status gae_check(const char* nm, int64_t N, int64_t T, const D* rewards, const D* values,
                     const uint8_t* term, const uint8_t* trunc, const D* tv, const D* boot,
                     float gamma, float lambda, D* adv, void* ws, size_t ws_bytes)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && values && adv, "%s: rewards, values and advantages are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D), eb = (uint64_t)N * sizeof(D);
    const Span outs[] = {{adv, nb}, {ws, ws_bytes}};
    const Span ins[] = {{rewards, nb}, {values, nb}, {term, nt}, {trunc, nt}, {tv, nb}, {boot, eb}};
    return check_disjoint(nm, outs, 2, ins, 6);
}

template <class D>
lrs_status gae_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* rewards,
                     const D* values, const uint8_t* term, const uint8_t* trunc, const D* tv,
                     const D* boot, float gamma, float lambda, D* adv, void* ws, size_t ws_bytes,
                     hipStream_t stream)
{
    LRS_TRY(gae_check<D>(nm, N, T, rewards, values, term, trunc, tv, boot, gamma, lambda, adv, ws,
                         ws_bytes));
    GaeArgs<D> a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, rewards, values, gamma,
                 (float)((double)gamma * (double)lambda), adv};
    const void* f[] = {rewards, values, adv, tv};
    const void* m[] = {term, trunc};
    using S = GaeSel<D>;
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, a.gl, a, f, 4, m, 2, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, a.gl, a, f, 4, m, 2, ws, ws_bytes, stream);
}

template <class D>
lrs_status vtrace_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* log_rhos,
                        const D* rewards, const D* values, const uint8_t* term,
                        const uint8_t* trunc, const D* tv, const D* boot, float gamma, float lambda,
                        float rho_bar, float c_bar, float pg_rho_bar, D* vs, D* pg_adv, void* ws,
                        size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(log_rhos && rewards && values && vs && pg_adv,
                "%s: log_rhos, rewards, values, vs and pg_advantages are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    LRS_REQUIRE(positive(rho_bar) && positive(c_bar) && positive(pg_rho_bar),
                "%s: rho_bar, c_bar and pg_rho_bar must be > 0", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D), eb = (uint64_t)N * sizeof(D);
    const Span outs[] = {{vs, nb}, {pg_adv, nb}, {ws, ws_bytes}};
    const Span ins[] = {{log_rhos, nb}, {rewards, nb}, {values, nb}, {term, nt},
                        {trunc, nt},    {tv, nb},      {boot, eb}};
    LRS_TRY(check_disjoint(nm, outs, 3, ins, 7));
    VtraceArgs<D> a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, log_rhos, rewards,
                    values, gamma, lambda, rho_bar, c_bar, pg_rho_bar, vs, pg_adv};
    const void* f[] = {log_rhos, rewards, values, vs, pg_adv, tv};
    const void* m[] = {term, trunc};
    using S = VtraceSel<D>;
    const float beta_max = gamma * lambda * c_bar;  // beta_t = gamma * c_t <= this
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, beta_max, a, f, 6, m, 2, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, beta_max, a, f, 6, m, 2, ws, ws_bytes, stream);
}

template <class D>
lrs_status retrace_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* log_rhos,
                         const D* rewards, const D* q_values, const D* values, const uint8_t* term,
                         const uint8_t* trunc, const D* tv, const D* boot, float gamma,
                         float lambda, float c_bar, D* q_ret, void* ws, size_t ws_bytes,
                         hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(log_rhos && rewards && q_values && values && q_ret,
                "%s: log_rhos, rewards, q_values, values and q_ret are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    LRS_REQUIRE(positive(c_bar), "%s: c_bar must be > 0", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D), eb = (uint64_t)N * sizeof(D);
    const Span outs[] = {{q_ret, nb}, {ws, ws_bytes}};
    const Span ins[] = {{log_rhos, nb}, {rewards, nb}, {q_values, nb}, {values, nb},
                        {term, nt},     {trunc, nt},   {tv, nb},       {boot, eb}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 8));
    RetraceArgs<D> a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, log_rhos, rewards,
                     q_values, values, gamma, lambda, c_bar, q_ret};
    const void* f[] = {log_rhos, rewards, q_values, values, q_ret, tv};
    const void* m[] = {term, trunc};
    using S = RetraceSel<D>;
    const float beta_max = gamma * lambda * c_bar;  // beta_t = gamma * c_t <= this
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, beta_max, a, f, 6, m, 2, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, beta_max, a, f, 6, m, 2, ws, ws_bytes, stream);
}

template <class D>
lrs_status lambda_returns_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* rewards,
                                const D* values, const uint8_t* term, const uint8_t* trunc,
                                const D* tv, const D* boot, float gamma, float lambda, D* out,
                                void* ws, size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && values && out, "%s: rewards, values and returns are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D), eb = (uint64_t)N * sizeof(D);
    const Span outs[] = {{out, nb}, {ws, ws_bytes}};
    const Span ins[] = {{rewards, nb}, {values, nb}, {term, nt}, {trunc, nt}, {tv, nb}, {boot, eb}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 6));
    LambdaArgs<D> a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, rewards, values,
                    gamma,
                    (float)((double)gamma * (double)lambda),
                    (float)((double)gamma * (1.0 - (double)lambda)), out};
    const void* f[] = {rewards, values, out, tv};
    const void* m[] = {term, trunc};
    using S = LambdaSel<D>;
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, a.gl, a, f, 4, m, 2, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, a.gl, a, f, 4, m, 2, ws, ws_bytes, stream);
}

template <class D>
lrs_status discounted_returns_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* rewards,
                                    const uint8_t* term, const uint8_t* trunc, const D* tv,
                                    const D* boot, float gamma, D* out, void* ws, size_t ws_bytes,
                                    hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && out, "%s: rewards and returns are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma), "%s: gamma must be in [0, 1]", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D), eb = (uint64_t)N * sizeof(D);
    const Span outs[] = {{out, nb}, {ws, ws_bytes}};
    const Span ins[] = {{rewards, nb}, {term, nt}, {trunc, nt}, {tv, nb}, {boot, eb}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 5));
    DiscArgs<D> a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, rewards, gamma, out};
    const void* f[] = {rewards, out, tv};
    const void* m[] = {term, trunc};
    using S = DiscSel<D>;
    return trunc
        ? run_layout<S::template T>(tm, nm, N, T, gamma, a, f, 3, m, 2, ws, ws_bytes, stream)
        : run_layout<S::template N>(tm, nm, N, T, gamma, a, f, 3, m, 2, ws, ws_bytes, stream);
}

template <class D>
lrs_status eligibility_traces_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* x,
                                    const uint8_t* dones, float gamma, float lambda, D* out,
                                    void* ws, size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and traces are required", nm);
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda),
                "%s: gamma and lambda must be in [0, 1]", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D);
    const Span outs[] = {{out, nb}, {ws, ws_bytes}};
    const Span ins[] = {{x, nb}, {dones, nt}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 2));
    ForwardArgs a{x, dones, (float)((double)gamma * (double)lambda), out};
    const void* f[] = {x, out};
    const void* m[] = {dones};
    return run_layout<ForwardSel<D>::template Elig>(tm, nm, N, T, a.gl, a, f, 2, m, 1, ws, ws_bytes,
                                                    stream);
}

template <class D>
lrs_status prefix_sum_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* x,
                            const uint8_t* dones, D* out, void* ws, size_t ws_bytes,
                            hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and sums are required", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D);
    const Span outs[] = {{out, nb}, {ws, ws_bytes}};
    const Span ins[] = {{x, nb}, {dones, nt}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 2));
    ForwardArgs a{x, dones, 1.0f, out};
    const void* f[] = {x, out};
    const void* m[] = {dones};
    return run_layout<ForwardSel<D>::template Prefix>(tm, nm, N, T, 1.0f, a, f, 2, m, 1, ws,
                                                      ws_bytes, stream);
}

inline lrs_status prefix_sum_i32_entry(const char* nm, bool tm, int64_t N, int64_t T,
                                       const int32_t* x, const uint8_t* dones, int32_t* out,
                                       void* ws, size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and sums are required", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(int32_t);
    const Span outs[] = {{out, nb}, {ws, ws_bytes}};
    const Span ins[] = {{x, nb}, {dones, nt}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 2));
    ForwardArgs a{x, dones, 1.0f, out};
    const void* f[] = {x, out};
    const void* m[] = {dones};
    return run_layout<PrefixI32Op>(tm, nm, N, T, 1.0f, a, f, 2, m, 1, ws, ws_bytes, stream);
}

template <class D>
lrs_status affine_scan_entry(const char* nm, bool tm, int64_t N, int64_t T, const D* alpha,
                             const D* beta, const uint8_t* reset, const D* carry_in, int reverse,
                             D* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(alpha && beta && out, "%s: alpha, beta and out are required", nm);
    LRS_REQUIRE(reverse == 0 || reverse == 1, "%s: reverse must be 0 or 1", nm);
    const uint64_t nt = (uint64_t)N * (uint64_t)T, nb = nt * sizeof(D), eb = (uint64_t)N * sizeof(D);
    const Span outs[] = {{out, nb}, {ws, ws_bytes}};
    const Span ins[] = {{alpha, nb}, {beta, nb}, {reset, nt}, {carry_in, eb}};
    LRS_TRY(check_disjoint(nm, outs, 2, ins, 4));
    AffineArgs<D> a{alpha, beta, reset, carry_in ? carry_in : alpha, carry_in != nullptr, out};
    const void* f[] = {alpha, beta, out};
    const void* m[] = {reset};
    using S = AffineSel<D>;
    const float bm = INFINITY;  // caller coefficients: no bound on beta is known
    if (reverse)
        return reset ? run_layout<S::template RevR>(tm, nm, N, T, bm, a, f, 3, m, 1, ws, ws_bytes,
                                                    stream)
                     : run_layout<S::template RevN>(tm, nm, N, T, bm, a, f, 3, m, 1, ws, ws_bytes,
                                                    stream);
    return reset
        ? run_layout<S::template FwdR>(tm, nm, N, T, bm, a, f, 3, m, 1, ws, ws_bytes, stream)
        : run_layout<S::template FwdN>(tm, nm, N, T, bm, a, f, 3, m, 1, ws, ws_bytes, stream);
}

}  // namespace lrs
