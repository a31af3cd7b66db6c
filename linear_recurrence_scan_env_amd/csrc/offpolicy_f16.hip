// offpolicy_f16.hip -- IEEE half (binary16) entry points of V-trace and
// Retrace(lambda).
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_vtrace_f16(int64_t N, int64_t T, const lrs_f16* log_rhos, const lrs_f16* rewards,
                          const lrs_f16* values, const uint8_t* term, const uint8_t* trunc,
                          const lrs_f16* tv, const lrs_f16* boot, float gamma, float lambda,
                          float rho_bar, float c_bar, float pg_rho_bar, lrs_f16* vs,
                          lrs_f16* pg_adv, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return vtrace_entry<f16_t>("lrs_vtrace_f16", false, N, T,
        reinterpret_cast<const f16_t*>(log_rhos), reinterpret_cast<const f16_t*>(rewards),
        reinterpret_cast<const f16_t*>(values), term, trunc, reinterpret_cast<const f16_t*>(tv),
        reinterpret_cast<const f16_t*>(boot), gamma, lambda, rho_bar, c_bar, pg_rho_bar,
        reinterpret_cast<f16_t*>(vs), reinterpret_cast<f16_t*>(pg_adv), strides, ws, ws_bytes, stream);
}

lrs_status lrs_vtrace_tm_f16(int64_t N, int64_t T, const lrs_f16* log_rhos, const lrs_f16* rewards,
                             const lrs_f16* values, const uint8_t* term, const uint8_t* trunc,
                             const lrs_f16* tv, const lrs_f16* boot, float gamma, float lambda,
                             float rho_bar, float c_bar, float pg_rho_bar, lrs_f16* vs,
                             lrs_f16* pg_adv, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return vtrace_entry<f16_t>("lrs_vtrace_tm_f16", true, N, T,
        reinterpret_cast<const f16_t*>(log_rhos), reinterpret_cast<const f16_t*>(rewards),
        reinterpret_cast<const f16_t*>(values), term, trunc, reinterpret_cast<const f16_t*>(tv),
        reinterpret_cast<const f16_t*>(boot), gamma, lambda, rho_bar, c_bar, pg_rho_bar,
        reinterpret_cast<f16_t*>(vs), reinterpret_cast<f16_t*>(pg_adv), strides, ws, ws_bytes, stream);
}

lrs_status lrs_retrace_f16(int64_t N, int64_t T, const lrs_f16* log_rhos, const lrs_f16* rewards,
                           const lrs_f16* q_values, const lrs_f16* values, const uint8_t* term,
                           const uint8_t* trunc, const lrs_f16* tv, const lrs_f16* boot,
                           float gamma, float lambda, float c_bar, lrs_f16* q_ret, const int64_t* strides, void* ws,
                           size_t ws_bytes, hipStream_t stream)
{
    return retrace_entry<f16_t>("lrs_retrace_f16", false, N, T,
        reinterpret_cast<const f16_t*>(log_rhos), reinterpret_cast<const f16_t*>(rewards),
        reinterpret_cast<const f16_t*>(q_values), reinterpret_cast<const f16_t*>(values), term,
        trunc, reinterpret_cast<const f16_t*>(tv), reinterpret_cast<const f16_t*>(boot), gamma,
        lambda, c_bar, reinterpret_cast<f16_t*>(q_ret), strides, ws, ws_bytes, stream);
}

lrs_status lrs_retrace_tm_f16(int64_t N, int64_t T, const lrs_f16* log_rhos,
                              const lrs_f16* rewards, const lrs_f16* q_values,
                              const lrs_f16* values, const uint8_t* term, const uint8_t* trunc,
                              const lrs_f16* tv, const lrs_f16* boot, float gamma, float lambda,
                              float c_bar, lrs_f16* q_ret, const int64_t* strides, void* ws, size_t ws_bytes,
                              hipStream_t stream)
{
    return retrace_entry<f16_t>("lrs_retrace_tm_f16", true, N, T,
        reinterpret_cast<const f16_t*>(log_rhos), reinterpret_cast<const f16_t*>(rewards),
        reinterpret_cast<const f16_t*>(q_values), reinterpret_cast<const f16_t*>(values), term,
        trunc, reinterpret_cast<const f16_t*>(tv), reinterpret_cast<const f16_t*>(boot), gamma,
        lambda, c_bar, reinterpret_cast<f16_t*>(q_ret), strides, ws, ws_bytes, stream);
}

}  // extern "C"
