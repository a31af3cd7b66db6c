// returns.hip -- fp32 entry points of GAE, TD(lambda) returns and discounted
// returns.
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_gae_f32(int64_t N, int64_t T, const float* rewards, const float* values,
                       const uint8_t* term, const uint8_t* trunc, const float* tv,
                       const float* boot, float gamma, float lambda, float* adv, const int64_t* strides, void* ws,
                       size_t ws_bytes, hipStream_t stream)
{
    return gae_entry<float>("lrs_gae_f32", false, N, T, rewards, values, term, trunc, tv, boot,
        gamma, lambda, adv, strides, ws, ws_bytes, stream);
}

lrs_status lrs_gae_tm_f32(int64_t N, int64_t T, const float* rewards, const float* values,
                          const uint8_t* term, const uint8_t* trunc, const float* tv,
                          const float* boot, float gamma, float lambda, float* adv, const int64_t* strides, void* ws,
                          size_t ws_bytes, hipStream_t stream)
{
    return gae_entry<float>("lrs_gae_tm_f32", true, N, T, rewards, values, term, trunc, tv, boot,
        gamma, lambda, adv, strides, ws, ws_bytes, stream);
}

lrs_status lrs_lambda_returns_f32(int64_t N, int64_t T, const float* rewards, const float* values,
                                  const uint8_t* term, const uint8_t* trunc, const float* tv,
                                  const float* boot, float gamma, float lambda, float* out,
                                  const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return lambda_returns_entry<float>("lrs_lambda_returns_f32", false, N, T, rewards, values,
        term, trunc, tv, boot, gamma, lambda, out, strides, ws, ws_bytes, stream);
}

lrs_status lrs_lambda_returns_tm_f32(int64_t N, int64_t T, const float* rewards,
                                     const float* values, const uint8_t* term,
                                     const uint8_t* trunc, const float* tv, const float* boot,
                                     float gamma, float lambda, float* out, const int64_t* strides, void* ws,
                                     size_t ws_bytes, hipStream_t stream)
{
    return lambda_returns_entry<float>("lrs_lambda_returns_tm_f32", true, N, T, rewards, values,
        term, trunc, tv, boot, gamma, lambda, out, strides, ws, ws_bytes, stream);
}

lrs_status lrs_discounted_returns_f32(int64_t N, int64_t T, const float* rewards,
                                      const uint8_t* term, const uint8_t* trunc, const float* tv,
                                      const float* boot, float gamma, float* out, const int64_t* strides, void* ws,
                                      size_t ws_bytes, hipStream_t stream)
{
    return discounted_returns_entry<float>("lrs_discounted_returns_f32", false, N, T, rewards,
        term, trunc, tv, boot, gamma, out, strides, ws, ws_bytes, stream);
}

lrs_status lrs_discounted_returns_tm_f32(int64_t N, int64_t T, const float* rewards,
                                         const uint8_t* term, const uint8_t* trunc,
                                         const float* tv, const float* boot, float gamma,
                                         float* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return discounted_returns_entry<float>("lrs_discounted_returns_tm_f32", true, N, T, rewards,
        term, trunc, tv, boot, gamma, out, strides, ws, ws_bytes, stream);
}

}  // extern "C"
