// affine_bf16.hip -- bfloat16 entry points of the generic segmented affine scan.
#include "entries.hpp"

using namespace lrs;

extern "C" {

lrs_status lrs_affine_scan_bf16(int64_t N, int64_t T, const lrs_bf16* alpha, const lrs_bf16* beta,
                                const uint8_t* reset, const lrs_bf16* carry_in, int reverse,
                                lrs_bf16* out, const int64_t* strides, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return affine_scan_entry<bf16_t>("lrs_affine_scan_bf16", false, N, T,
        reinterpret_cast<const bf16_t*>(alpha), reinterpret_cast<const bf16_t*>(beta), reset,
        reinterpret_cast<const bf16_t*>(carry_in), reverse, reinterpret_cast<bf16_t*>(out), strides, ws,
        ws_bytes, stream);
}

lrs_status lrs_affine_scan_tm_bf16(int64_t N, int64_t T, const lrs_bf16* alpha,
                                   const lrs_bf16* beta, const uint8_t* reset,
                                   const lrs_bf16* carry_in, int reverse, lrs_bf16* out, const int64_t* strides, void* ws,
                                   size_t ws_bytes, hipStream_t stream)
{
    return affine_scan_entry<bf16_t>("lrs_affine_scan_tm_bf16", true, N, T,
        reinterpret_cast<const bf16_t*>(alpha), reinterpret_cast<const bf16_t*>(beta), reset,
        reinterpret_cast<const bf16_t*>(carry_in), reverse, reinterpret_cast<bf16_t*>(out), strides, ws,
        ws_bytes, stream);
}

}  // extern "C"
