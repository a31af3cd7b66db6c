// returns.hip -- entry points of the three value-based backward estimators: GAE,
// TD(lambda) returns and discounted returns.
#include "launch.hpp"

namespace lrs {
template <int E> using GaeT = GaeOp<E, true>;
template <int E> using GaeN = GaeOp<E, false>;
template <int E> using LambdaT = LambdaOp<E, true>;
template <int E> using LambdaN = LambdaOp<E, false>;
template <int E> using DiscT = DiscOp<E, true>;
template <int E> using DiscN = DiscOp<E, false>;
}  // namespace lrs

using namespace lrs;

extern "C" {

lrs_status lrs_gae_f32(int64_t N, int64_t T, const float* rewards, const float* values,
                       const uint8_t* term, const uint8_t* trunc, const float* tv,
                       const float* boot, float gamma, float lambda, float* adv, void* ws,
                       size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_gae_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && values && adv, "%s: rewards, values and advantages are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda), "%s: gamma and lambda must be in [0, 1]", nm);
    GaeArgs a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, rewards, values, gamma,
              (float)((double)gamma * (double)lambda), adv};
    const void* f[] = {rewards, values, adv, tv};
    const void* m[] = {term, trunc};
    return trunc ? run<GaeT>(nm, N, T, a, f, 4, m, 2, ws, ws_bytes, stream) : run<GaeN>(nm, N, T, a, f, 4, m, 2, ws, ws_bytes, stream);
}

lrs_status lrs_lambda_returns_f32(int64_t N, int64_t T, const float* rewards, const float* values,
                                  const uint8_t* term, const uint8_t* trunc, const float* tv,
                                  const float* boot, float gamma, float lambda, float* out,
                                  void* ws, size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_lambda_returns_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && values && out, "%s: rewards, values and returns are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda), "%s: gamma and lambda must be in [0, 1]", nm);
    LambdaArgs a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, rewards, values, gamma,
                 (float)((double)gamma * (double)lambda),
                 (float)((double)gamma * (1.0 - (double)lambda)), out};
    const void* f[] = {rewards, values, out, tv};
    const void* m[] = {term, trunc};
    return trunc ? run<LambdaT>(nm, N, T, a, f, 4, m, 2, ws, ws_bytes, stream) : run<LambdaN>(nm, N, T, a, f, 4, m, 2, ws, ws_bytes, stream);
}

lrs_status lrs_discounted_returns_f32(int64_t N, int64_t T, const float* rewards,
                                      const uint8_t* term, const uint8_t* trunc, const float* tv,
                                      const float* boot, float gamma, float* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_discounted_returns_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(rewards && out, "%s: rewards and returns are required", nm);
    LRS_TRY(check_boundary(nm, term, trunc, tv));
    LRS_REQUIRE(unit_interval(gamma), "%s: gamma must be in [0, 1]", nm);
    DiscArgs a{{term, trunc, tv, boot ? boot : rewards, boot != nullptr}, rewards, gamma, out};
    const void* f[] = {rewards, out, tv};
    const void* m[] = {term, trunc};
    return trunc ? run<DiscT>(nm, N, T, a, f, 3, m, 2, ws, ws_bytes, stream) : run<DiscN>(nm, N, T, a, f, 3, m, 2, ws, ws_bytes, stream);
}

}  // extern "C"
