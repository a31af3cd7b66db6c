// floor.hip -- reference kernels for measurement: what a launch of a given
// grid costs with no work (an empty kernel), and with nothing but the bytes a
// call moves (a streaming kernel that reads and writes the same byte counts
// on the same grid, with no recurrence).  Timed beside a call, they split its
// duration into the launch floor, the memory traffic and the rest.  Not part
// of any estimator.
#include <array>
#include <utility>

#include "launch.hpp"

namespace lrs {
namespace {

__global__ void floor_empty() {}

// Lane g of L reads 16-byte vectors g, g + L, g + 2L, ... (coalesced across
// lanes; NLD of them at most, all issued before the first use), folds them
// into one value, and then writes vectors g, g + L, ... of dst with it, so
// that every store waits for every load, as a call's stores wait for its scan.
template <int NLD>
__global__ void floor_stream(const u32x4* __restrict__ src, uint64_t n_in, u32x4* __restrict__ dst,
                             uint64_t n_out)
{
    const uint64_t lanes = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 v[NLD];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
        const uint64_t i = (uint64_t)k * lanes + g;
        v[k] = i < n_in ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < NLD; ++k) acc ^= v[k];
    for (uint64_t i = g; i < n_out; i += lanes) {
        u32x4 w = acc;
        w.x ^= (uint32_t)i;
        __builtin_nontemporal_store(w, dst + i);
    }
}

template <int NLD>
hipError_t launch_stream(uint32_t blocks, uint32_t threads, const u32x4* src, uint64_t n_in,
                         u32x4* dst, uint64_t n_out, hipStream_t stream)
{
    void* args[] = {(void*)&src, (void*)&n_in, (void*)&dst, (void*)&n_out};
    return hipLaunchKernel((const void*)&floor_stream<NLD>, dim3(blocks), dim3(threads), args, 0,
                           stream);
}

// Up to 16 vectors per lane (the time-major grids are small: 64 blocks for
// 4096 environments of 128 steps).
constexpr int kMaxVectorsPerLane = 16;
using StreamLauncher = hipError_t (*)(uint32_t, uint32_t, const u32x4*, uint64_t, u32x4*, uint64_t,
                                      hipStream_t);
template <int... I>
constexpr auto stream_launchers(std::integer_sequence<int, I...>)
{
    return std::array<StreamLauncher, sizeof...(I)>{&launch_stream<I + 1>...};
}
constexpr auto kStreamLaunchers =
    stream_launchers(std::make_integer_sequence<int, kMaxVectorsPerLane>{});

}  // namespace
}  // namespace lrs

using namespace lrs;

extern "C" lrs_status lrs_debug_floor(int kind, int64_t blocks, int threads, const void* src,
                                      int64_t read_bytes, void* dst, int64_t write_bytes,
                                      hipStream_t stream)
{
    const char* nm = "lrs_debug_floor";
    if (blocks < 1 || blocks > 0x7fffffff || threads < 64 || threads > 1024 || threads % 64 != 0)
        return fail(LRS_ERR_INVALID_ARG, "%s: need 1 <= blocks < 2^31 and threads in 64..1024, a "
                    "multiple of 64", nm);
    hipError_t e = hipSuccess;
    if (kind == 0) {
        void* args[] = {nullptr};
        e = hipLaunchKernel((const void*)&floor_empty, dim3((uint32_t)blocks), dim3(threads), args,
                            0, stream);
    } else if (kind == 1) {
        if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 || write_bytes % 16 ||
            (read_bytes && (src == nullptr || !aligned(src, 16))) ||
            (write_bytes && (dst == nullptr || !aligned(dst, 16))))
            return fail(LRS_ERR_INVALID_ARG, "%s: byte counts must be multiples of 16 and the "
                        "arrays 16-byte aligned", nm);
        const uint64_t lanes = (uint64_t)blocks * (uint64_t)threads;
        const uint64_t n_in = (uint64_t)read_bytes / 16, n_out = (uint64_t)write_bytes / 16;
        const uint64_t per_lane = (n_in + lanes - 1) / lanes;
        const u32x4* s = static_cast<const u32x4*>(src);
        u32x4* d = static_cast<u32x4*>(dst);
        const uint32_t b = (uint32_t)blocks, t = (uint32_t)threads;
        if (per_lane > (uint64_t)kMaxVectorsPerLane)
            return fail(LRS_ERR_INVALID_ARG, "%s: at most %d vectors of 16 bytes read per lane "
                        "(%llu asked)", nm, kMaxVectorsPerLane, (unsigned long long)per_lane);
        e = kStreamLaunchers[per_lane == 0 ? 0 : per_lane - 1](b, t, s, n_in, d, n_out, stream);
    } else {
        return fail(LRS_ERR_INVALID_ARG, "%s: kind must be 0 (empty) or 1 (stream)", nm);
    }
    if (e != hipSuccess) return fail(LRS_ERR_HIP, "%s: launch failed: %s", nm, hipGetErrorString(e));
    g_err[0] = '\0';
    return LRS_OK;
}
