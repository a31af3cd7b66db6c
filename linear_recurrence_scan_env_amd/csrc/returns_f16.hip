// returns_f16.hip -- IEEE half (binary16) entry points of GAE, TD(lambda)
// returns and discounted returns.
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_gae_f16(int64_t N, int64_t T, const lrs_f16* rewards, const lrs_f16* values,
                       const uint8_t* term, const uint8_t* trunc, const lrs_f16* tv,
                       const lrs_f16* boot, float gamma, float lambda, lrs_f16* adv, const int64_t* strides, void* ws,
                       size_t ws_bytes, hipStream_t stream)
{
    return gae_entry<f16_t>("lrs_gae_f16", false, N, T, reinterpret_cast<const f16_t*>(rewards),
        reinterpret_cast<const f16_t*>(values), term, trunc, reinterpret_cast<const f16_t*>(tv),
        reinterpret_cast<const f16_t*>(boot), gamma, lambda, reinterpret_cast<f16_t*>(adv), strides, ws,
        ws_bytes, stream);
}

lrs_status lrs_gae_tm_f16(int64_t N, int64_t T, const lrs_f16* rewards, const lrs_f16* values,
                          const uint8_t* term, const uint8_t* trunc, const lrs_f16* tv,
                          const lrs_f16* boot, float gamma, float lambda, lrs_f16* adv, const int64_t* strides, void* ws,
                          size_t ws_bytes, hipStream_t stream)
{
    return gae_entry<f16_t>("lrs_gae_tm_f16", true, N, T, reinterpret_cast<const f16_t*>(rewards),
        reinterpret_cast<const f16_t*>(values), term, trunc, reinterpret_cast<const f16_t*>(tv),
        reinterpret_cast<const f16_t*>(boot), gamma, lambda, reinterpret_cast<f16_t*>(adv), strides, ws,
        ws_bytes, stream);
}

lrs_status lrs_lambda_returns_f16(int64_t N, int64_t T, const lrs_f16* rewards,
                                  const lrs_f16* values, const uint8_t* term, const uint8_t* trunc,
                                  const lrs_f16* tv, const lrs_f16* boot, float gamma,
                                  float lambda, lrs_f16* out, const int64_t* strides, void* ws, size_t ws_bytes,
                                  hipStream_t stream)
{
    return lambda_returns_entry<f16_t>("lrs_lambda_returns_f16", false, N, T,
        reinterpret_cast<const f16_t*>(rewards), reinterpret_cast<const f16_t*>(values), term,
        trunc, reinterpret_cast<const f16_t*>(tv), reinterpret_cast<const f16_t*>(boot), gamma,
        lambda, reinterpret_cast<f16_t*>(out), strides, ws, ws_bytes, stream);
}

lrs_status lrs_lambda_returns_tm_f16(int64_t N, int64_t T, const lrs_f16* rewards,
                                     const lrs_f16* values, const uint8_t* term,
                                     const uint8_t* trunc, const lrs_f16* tv, const lrs_f16* boot,
                                     float gamma, float lambda, lrs_f16* out, const int64_t* strides, void* ws,
                                     size_t ws_bytes, hipStream_t stream)
{
    return lambda_returns_entry<f16_t>("lrs_lambda_returns_tm_f16", true, N, T,
        reinterpret_cast<const f16_t*>(rewards), reinterpret_cast<const f16_t*>(values), term,
        trunc, reinterpret_cast<const f16_t*>(tv), reinterpret_cast<const f16_t*>(boot), gamma,
        lambda, reinterpret_cast<f16_t*>(out), strides, ws, ws_bytes, stream);
}

lrs_status lrs_discounted_returns_f16(int64_t N, int64_t T, const lrs_f16* rewards,
                                      const uint8_t* term, const uint8_t* trunc, const lrs_f16* tv,
                                      const lrs_f16* boot, float gamma, lrs_f16* out, const int64_t* strides, void* ws,
                                      size_t ws_bytes, hipStream_t stream)
{
    return discounted_returns_entry<f16_t>("lrs_discounted_returns_f16", false, N, T,
        reinterpret_cast<const f16_t*>(rewards), term, trunc, reinterpret_cast<const f16_t*>(tv),
        reinterpret_cast<const f16_t*>(boot), gamma, reinterpret_cast<f16_t*>(out), strides, ws, ws_bytes,
        stream);
}

lrs_status lrs_discounted_returns_tm_f16(int64_t N, int64_t T, const lrs_f16* rewards,
                                         const uint8_t* term, const uint8_t* trunc,
                                         const lrs_f16* tv, const lrs_f16* boot, float gamma,
                                         lrs_f16* out, const int64_t* strides, void* ws, size_t ws_bytes,
                                         hipStream_t stream)
{
    return discounted_returns_entry<f16_t>("lrs_discounted_returns_tm_f16", true, N, T,
        reinterpret_cast<const f16_t*>(rewards), term, trunc, reinterpret_cast<const f16_t*>(tv),
        reinterpret_cast<const f16_t*>(boot), gamma, reinterpret_cast<f16_t*>(out), strides, ws, ws_bytes,
        stream);
}

}  // extern "C"
