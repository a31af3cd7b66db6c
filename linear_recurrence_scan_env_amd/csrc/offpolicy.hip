// offpolicy.hip -- entry points of the two importance-weighted backward estimators:
// V-trace and Retrace(lambda).
#include "launch.hpp"

namespace lrs {
template <int E> using VtraceT = VtraceOp<E, true>;
template <int E> using VtraceN = VtraceOp<E, false>;
template <int E> using RetraceT = RetraceOp<E, true>;
template <int E> using RetraceN = RetraceOp<E, false>;
}  // namespace lrs

using namespace lrs;

extern "C" {

lrs_status lrs_vtrace_f32(int64_t N, int64_t T, const float* log_rhos, const float* rewards,
                          const float* values, const uint8_t* term, const uint8_t* trunc,
                          const float* tv, const float* boot, float gamma, float lambda,
                          float rho_bar, float c_bar, float pg_rho_bar, float* vs,
                          float* pg_adv, void* ws, size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_vtrace_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(log_rhos && rewards && values && vs && pg_adv,
                "%s: log_rhos, rewards, values, vs and pg_advantages are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda), "%s: gamma and lambda must be in [0, 1]", nm);
    LRS_REQUIRE(positive(rho_bar) && positive(c_bar) && positive(pg_rho_bar),
                "%s: rho_bar, c_bar and pg_rho_bar must be > 0", nm);
    VtraceArgs a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, log_rhos, rewards, values, gamma, lambda,
                 rho_bar, c_bar, pg_rho_bar, vs, pg_adv};
    const void* f[] = {log_rhos, rewards, values, vs, pg_adv, tv};
    const void* m[] = {term, trunc};
    return trunc ? run<VtraceT>(nm, N, T, a, f, 6, m, 2, ws, ws_bytes, stream) : run<VtraceN>(nm, N, T, a, f, 6, m, 2, ws, ws_bytes, stream);
}

lrs_status lrs_retrace_f32(int64_t N, int64_t T, const float* log_rhos, const float* rewards,
                           const float* q_values, const float* values, const uint8_t* term,
                           const uint8_t* trunc, const float* tv, const float* boot, float gamma,
                           float lambda, float c_bar, float* q_ret, void* ws, size_t ws_bytes,
                           hipStream_t stream)
{
    const char* nm = "lrs_retrace_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(log_rhos && rewards && q_values && values && q_ret,
                "%s: log_rhos, rewards, q_values, values and q_ret are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda), "%s: gamma and lambda must be in [0, 1]", nm);
    LRS_REQUIRE(positive(c_bar), "%s: c_bar must be > 0", nm);
    RetraceArgs a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, log_rhos, rewards, q_values, values,
                  gamma, lambda, c_bar, q_ret};
    const void* f[] = {log_rhos, rewards, q_values, values, q_ret, tv};
    const void* m[] = {term, trunc};
    return trunc ? run<RetraceT>(nm, N, T, a, f, 6, m, 2, ws, ws_bytes, stream) : run<RetraceN>(nm, N, T, a, f, 6, m, 2, ws, ws_bytes, stream);
}

}  // extern "C"
