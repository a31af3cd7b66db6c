// forward.hip -- fp32 entry points of the forward estimators (eligibility
// traces, episodic prefix sum).
// Also the int32 prefix sum.
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_eligibility_traces_f32(int64_t N, int64_t T, const float* x, const uint8_t* dones,
                                      float gamma, float lambda, float* out, const int64_t* strides, void* ws,
                                      size_t ws_bytes, hipStream_t stream)
{
    return eligibility_traces_entry<float>("lrs_eligibility_traces_f32", false, N, T, x, dones,
        gamma, lambda, out, strides, ws, ws_bytes, stream);
}

lrs_status lrs_eligibility_traces_tm_f32(int64_t N, int64_t T, const float* x,
                                         const uint8_t* dones, float gamma, float lambda,
                                         float* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return eligibility_traces_entry<float>("lrs_eligibility_traces_tm_f32", true, N, T, x, dones,
        gamma, lambda, out, strides, ws, ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_f32(int64_t N, int64_t T, const float* x, const uint8_t* dones,
                                       float* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return prefix_sum_entry<float>("lrs_episodic_prefix_sum_f32", false, N, T, x, dones, out, strides, ws,
        ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_tm_f32(int64_t N, int64_t T, const float* x,
                                          const uint8_t* dones, float* out, const int64_t* strides, void* ws,
                                          size_t ws_bytes, hipStream_t stream)
{
    return prefix_sum_entry<float>("lrs_episodic_prefix_sum_tm_f32", true, N, T, x, dones, out, strides, ws,
        ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_i32(int64_t N, int64_t T, const int32_t* x,
                                       const uint8_t* dones, int32_t* out, const int64_t* strides, void* ws,
                                       size_t ws_bytes, hipStream_t stream)
{
    return prefix_sum_int_entry<int32_t>("lrs_episodic_prefix_sum_i32", false, N, T, x, dones, out, strides, ws,
                                ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_tm_i32(int64_t N, int64_t T, const int32_t* x,
                                          const uint8_t* dones, int32_t* out, const int64_t* strides, void* ws,
                                          size_t ws_bytes, hipStream_t stream)
{
    return prefix_sum_int_entry<int32_t>("lrs_episodic_prefix_sum_tm_i32", true, N, T, x, dones, out, strides, ws,
                                ws_bytes, stream);
}

}  // extern "C"
