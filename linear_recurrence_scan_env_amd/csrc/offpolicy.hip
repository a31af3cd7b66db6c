// offpolicy.hip -- fp32 entry points of V-trace and Retrace(lambda).
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_vtrace_f32(int64_t N, int64_t T, const float* log_rhos, const float* rewards,
                          const float* values, const uint8_t* term, const uint8_t* trunc,
                          const float* tv, const float* boot, float gamma, float lambda,
                          float rho_bar, float c_bar, float pg_rho_bar, float* vs, float* pg_adv,
                          const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return vtrace_entry<float>("lrs_vtrace_f32", false, N, T, log_rhos, rewards, values, term,
        trunc, tv, boot, gamma, lambda, rho_bar, c_bar, pg_rho_bar, vs, pg_adv, strides, ws, ws_bytes,
        stream);
}

lrs_status lrs_vtrace_tm_f32(int64_t N, int64_t T, const float* log_rhos, const float* rewards,
                             const float* values, const uint8_t* term, const uint8_t* trunc,
                             const float* tv, const float* boot, float gamma, float lambda,
                             float rho_bar, float c_bar, float pg_rho_bar, float* vs,
                             float* pg_adv, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return vtrace_entry<float>("lrs_vtrace_tm_f32", true, N, T, log_rhos, rewards, values, term,
        trunc, tv, boot, gamma, lambda, rho_bar, c_bar, pg_rho_bar, vs, pg_adv, strides, ws, ws_bytes,
        stream);
}

lrs_status lrs_retrace_f32(int64_t N, int64_t T, const float* log_rhos, const float* rewards,
                           const float* q_values, const float* values, const uint8_t* term,
                           const uint8_t* trunc, const float* tv, const float* boot, float gamma,
                           float lambda, float c_bar, float* q_ret, const int64_t* strides, void* ws, size_t ws_bytes,
                           hipStream_t stream)
{
    return retrace_entry<float>("lrs_retrace_f32", false, N, T, log_rhos, rewards, q_values,
        values, term, trunc, tv, boot, gamma, lambda, c_bar, q_ret, strides, ws, ws_bytes, stream);
}

lrs_status lrs_retrace_tm_f32(int64_t N, int64_t T, const float* log_rhos, const float* rewards,
                              const float* q_values, const float* values, const uint8_t* term,
                              const uint8_t* trunc, const float* tv, const float* boot,
                              float gamma, float lambda, float c_bar, float* q_ret, const int64_t* strides, void* ws,
                              size_t ws_bytes, hipStream_t stream)
{
    return retrace_entry<float>("lrs_retrace_tm_f32", true, N, T, log_rhos, rewards, q_values,
        values, term, trunc, tv, boot, gamma, lambda, c_bar, q_ret, strides, ws, ws_bytes, stream);
}

}  // extern "C"
