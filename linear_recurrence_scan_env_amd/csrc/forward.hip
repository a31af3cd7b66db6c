// forward.hip -- entry points of the forward estimators: eligibility traces and the
// episodic prefix sums.
#include "launch.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_eligibility_traces_f32(int64_t N, int64_t T, const float* x, const uint8_t* dones,
                                      float gamma, float lambda, float* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_eligibility_traces_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and traces are required", nm);
    LRS_REQUIRE(unit_interval(gamma) && unit_interval(lambda), "%s: gamma and lambda must be in [0, 1]", nm);
    ForwardArgs a{x, dones, (float)((double)gamma * (double)lambda), out};
    const void* f[] = {x, out};
    const void* m[] = {dones};
    return run<EligOp>(nm, N, T, a, f, 2, m, 1, ws, ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_i32(int64_t N, int64_t T, const int32_t* x,
                                       const uint8_t* dones, int32_t* out, void* ws,
                                       size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_episodic_prefix_sum_i32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and sums are required", nm);
    ForwardArgs a{x, dones, 1.0f, out};
    const void* f[] = {x, out};
    const void* m[] = {dones};
    return run<PrefixI32Op>(nm, N, T, a, f, 2, m, 1, ws, ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_f32(int64_t N, int64_t T, const float* x, const uint8_t* dones,
                                       float* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_episodic_prefix_sum_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(x && dones && out, "%s: x, dones and sums are required", nm);
    ForwardArgs a{x, dones, 1.0f, out};
    const void* f[] = {x, out};
    const void* m[] = {dones};
    return run<PrefixF32Op>(nm, N, T, a, f, 2, m, 1, ws, ws_bytes, stream);
}

}  // extern "C"
