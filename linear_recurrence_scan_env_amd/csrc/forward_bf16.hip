// forward_bf16.hip -- bfloat16 entry points of the forward estimators
// (eligibility traces, episodic prefix sum).
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_eligibility_traces_bf16(int64_t N, int64_t T, const lrs_bf16* x,
                                       const uint8_t* dones, float gamma, float lambda,
                                       lrs_bf16* out, const int64_t* strides, void* ws, size_t ws_bytes,
                                       hipStream_t stream)
{
    return eligibility_traces_entry<bf16_t>("lrs_eligibility_traces_bf16", false, N, T,
        reinterpret_cast<const bf16_t*>(x), dones, gamma, lambda, reinterpret_cast<bf16_t*>(out),
        strides, ws, ws_bytes, stream);
}

lrs_status lrs_eligibility_traces_tm_bf16(int64_t N, int64_t T, const lrs_bf16* x,
                                          const uint8_t* dones, float gamma, float lambda,
                                          lrs_bf16* out, const int64_t* strides, void* ws, size_t ws_bytes,
                                          hipStream_t stream)
{
    return eligibility_traces_entry<bf16_t>("lrs_eligibility_traces_tm_bf16", true, N, T,
        reinterpret_cast<const bf16_t*>(x), dones, gamma, lambda, reinterpret_cast<bf16_t*>(out),
        strides, ws, ws_bytes, stream);
}

lrs_status lrs_episodic_prefix_sum_bf16(int64_t N, int64_t T, const lrs_bf16* x,
                                        const uint8_t* dones, lrs_bf16* out, const int64_t* strides, void* ws,
                                        size_t ws_bytes, hipStream_t stream)
{
    return prefix_sum_entry<bf16_t>("lrs_episodic_prefix_sum_bf16", false, N, T,
        reinterpret_cast<const bf16_t*>(x), dones, reinterpret_cast<bf16_t*>(out), strides, ws, ws_bytes,
        stream);
}

lrs_status lrs_episodic_prefix_sum_tm_bf16(int64_t N, int64_t T, const lrs_bf16* x,
                                           const uint8_t* dones, lrs_bf16* out, const int64_t* strides, void* ws,
                                           size_t ws_bytes, hipStream_t stream)
{
    return prefix_sum_entry<bf16_t>("lrs_episodic_prefix_sum_tm_bf16", true, N, T,
        reinterpret_cast<const bf16_t*>(x), dones, reinterpret_cast<bf16_t*>(out), strides, ws, ws_bytes,
        stream);
}

}  // extern "C"
