// affine.hip -- fp32 entry points of the generic segmented affine scan.
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_affine_scan_f32(int64_t N, int64_t T, const float* alpha, const float* beta,
                               const uint8_t* reset, const float* carry_in, int reverse,
                               float* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return affine_scan_entry<float>("lrs_affine_scan_f32", false, N, T, alpha, beta, reset,
        carry_in, reverse, out, strides, ws, ws_bytes, stream);
}

lrs_status lrs_affine_scan_tm_f32(int64_t N, int64_t T, const float* alpha, const float* beta,
                                  const uint8_t* reset, const float* carry_in, int reverse,
                                  float* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return affine_scan_entry<float>("lrs_affine_scan_tm_f32", true, N, T, alpha, beta, reset,
        carry_in, reverse, out, strides, ws, ws_bytes, stream);
}

}  // extern "C"
