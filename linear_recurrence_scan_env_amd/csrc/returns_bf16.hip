// returns_bf16.hip -- bfloat16 entry points of GAE, TD(lambda) returns and
// discounted returns.
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_gae_bf16(int64_t N, int64_t T, const lrs_bf16* rewards, const lrs_bf16* values,
                        const uint8_t* term, const uint8_t* trunc, const lrs_bf16* tv,
                        const lrs_bf16* boot, float gamma, float lambda, lrs_bf16* adv, const int64_t* strides, void* ws,
                        size_t ws_bytes, hipStream_t stream)
{
    return gae_entry<bf16_t>("lrs_gae_bf16", false, N, T, reinterpret_cast<const bf16_t*>(rewards),
        reinterpret_cast<const bf16_t*>(values), term, trunc, reinterpret_cast<const bf16_t*>(tv),
        reinterpret_cast<const bf16_t*>(boot), gamma, lambda, reinterpret_cast<bf16_t*>(adv), strides, ws,
        ws_bytes, stream);
}

lrs_status lrs_gae_tm_bf16(int64_t N, int64_t T, const lrs_bf16* rewards, const lrs_bf16* values,
                           const uint8_t* term, const uint8_t* trunc, const lrs_bf16* tv,
                           const lrs_bf16* boot, float gamma, float lambda, lrs_bf16* adv,
                           const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return gae_entry<bf16_t>("lrs_gae_tm_bf16", true, N, T,
        reinterpret_cast<const bf16_t*>(rewards), reinterpret_cast<const bf16_t*>(values), term,
        trunc, reinterpret_cast<const bf16_t*>(tv), reinterpret_cast<const bf16_t*>(boot), gamma,
        lambda, reinterpret_cast<bf16_t*>(adv), strides, ws, ws_bytes, stream);
}

lrs_status lrs_lambda_returns_bf16(int64_t N, int64_t T, const lrs_bf16* rewards,
                                   const lrs_bf16* values, const uint8_t* term,
                                   const uint8_t* trunc, const lrs_bf16* tv, const lrs_bf16* boot,
                                   float gamma, float lambda, lrs_bf16* out, const int64_t* strides, void* ws,
                                   size_t ws_bytes, hipStream_t stream)
{
    return lambda_returns_entry<bf16_t>("lrs_lambda_returns_bf16", false, N, T,
        reinterpret_cast<const bf16_t*>(rewards), reinterpret_cast<const bf16_t*>(values), term,
        trunc, reinterpret_cast<const bf16_t*>(tv), reinterpret_cast<const bf16_t*>(boot), gamma,
        lambda, reinterpret_cast<bf16_t*>(out), strides, ws, ws_bytes, stream);
}

lrs_status lrs_lambda_returns_tm_bf16(int64_t N, int64_t T, const lrs_bf16* rewards,
                                      const lrs_bf16* values, const uint8_t* term,
                                      const uint8_t* trunc, const lrs_bf16* tv,
                                      const lrs_bf16* boot, float gamma, float lambda,
                                      lrs_bf16* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return lambda_returns_entry<bf16_t>("lrs_lambda_returns_tm_bf16", true, N, T,
        reinterpret_cast<const bf16_t*>(rewards), reinterpret_cast<const bf16_t*>(values), term,
        trunc, reinterpret_cast<const bf16_t*>(tv), reinterpret_cast<const bf16_t*>(boot), gamma,
        lambda, reinterpret_cast<bf16_t*>(out), strides, ws, ws_bytes, stream);
}

lrs_status lrs_discounted_returns_bf16(int64_t N, int64_t T, const lrs_bf16* rewards,
                                       const uint8_t* term, const uint8_t* trunc,
                                       const lrs_bf16* tv, const lrs_bf16* boot, float gamma,
                                       lrs_bf16* out, const int64_t* strides, void* ws, size_t ws_bytes,
                                       hipStream_t stream)
{
    return discounted_returns_entry<bf16_t>("lrs_discounted_returns_bf16", false, N, T,
        reinterpret_cast<const bf16_t*>(rewards), term, trunc, reinterpret_cast<const bf16_t*>(tv),
        reinterpret_cast<const bf16_t*>(boot), gamma, reinterpret_cast<bf16_t*>(out), strides, ws, ws_bytes,
        stream);
}

lrs_status lrs_discounted_returns_tm_bf16(int64_t N, int64_t T, const lrs_bf16* rewards,
                                          const uint8_t* term, const uint8_t* trunc,
                                          const lrs_bf16* tv, const lrs_bf16* boot, float gamma,
                                          lrs_bf16* out, const int64_t* strides, void* ws, size_t ws_bytes,
                                          hipStream_t stream)
{
    return discounted_returns_entry<bf16_t>("lrs_discounted_returns_tm_bf16", true, N, T,
        reinterpret_cast<const bf16_t*>(rewards), term, trunc, reinterpret_cast<const bf16_t*>(tv),
        reinterpret_cast<const bf16_t*>(boot), gamma, reinterpret_cast<bf16_t*>(out), strides, ws, ws_bytes,
        stream);
}

}  // extern "C"
