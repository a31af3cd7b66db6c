// affine.hip -- entry point of the generic segmented affine scan over
// caller-supplied (alpha, beta) pairs.
#include "launch.hpp"

namespace lrs {
template <int E> using AffineFwdR = AffineOp<E, false, true>;
template <int E> using AffineFwdN = AffineOp<E, false, false>;
template <int E> using AffineRevR = AffineOp<E, true, true>;
template <int E> using AffineRevN = AffineOp<E, true, false>;
}  // namespace lrs

using namespace lrs;

extern "C" {

lrs_status lrs_affine_scan_f32(int64_t N, int64_t T, const float* alpha, const float* beta,
                               const uint8_t* reset, const float* carry_in, int reverse,
                               float* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    const char* nm = "lrs_affine_scan_f32";
    LRS_TRY(check_common(nm, N, T));
    LRS_REQUIRE(alpha && beta && out, "%s: alpha, beta and out are required", nm);
    LRS_REQUIRE(reverse == 0 || reverse == 1, "%s: reverse must be 0 or 1", nm);
    AffineArgs a{alpha, beta, reset, carry_in ? carry_in : alpha, carry_in != nullptr, out};
    const void* f[] = {alpha, beta, out};
    const void* m[] = {reset};
    if (reverse)
        return reset ? run<AffineRevR>(nm, N, T, a, f, 3, m, 1, ws, ws_bytes, stream)
                     : run<AffineRevN>(nm, N, T, a, f, 3, m, 1, ws, ws_bytes, stream);
    return reset ? run<AffineFwdR>(nm, N, T, a, f, 3, m, 1, ws, ws_bytes, stream)
                 : run<AffineFwdN>(nm, N, T, a, f, 3, m, 1, ws, ws_bytes, stream);
}

}  // extern "C"
