// noalloc.hip -- lrs_gae_noalloc_f32: lrs_gae_f32 without a caller workspace,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The look-back path's workspace (the header and the per-tile aggregate
// records) lives in a file-scope device array instead.  Each GPU holds its
// own copy of the array at its own address until the process ends; host code
// never uses the array's name as an address: on a call's first use of a
// device, with that device current, hipGetSymbolAddress yields the address,
// which is kept per device and passed to the kernels like a workspace
// pointer.  That first use also clears the array on the caller's stream with
// a fill kernel (the carry protocol needs the header zeroed once; every call
// leaves it consistent for the next), so the first call on a device must not
// be captured into a graph.  All calls on one GPU share the array,
// so calls that overlap in time on one GPU race, like calls sharing a
// workspace.
#include <mutex>

#include "entries.hpp"

namespace lrs {

constexpr size_t kScratchBytes = size_t(8) << 20;  // per GPU

// The area itself.  In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns is used.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void clear_scratch(uint4* p, uint64_t n)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's copy of the array (null on failure, with g_err set).
void* device_scratch(const char* name, hipStream_t stream, lrs_status* st)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *st = fail(LRS_ERR_HIP, "%s: hipGetDevice failed: %s", name, hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *st = fail(LRS_ERR_INVALID_ARG, "%s: device %d is beyond the %d supported", name, dev,
                   kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] != nullptr) return g_scratch_ptr[dev];
    // First use on this device: it must not be captured, since the clear
    // below runs once, not on every replay.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess || cap != hipStreamCaptureStatusNone) {
        *st = fail(LRS_ERR_INVALID_ARG,
                   "%s: the first call on a device clears its scratch area and must not be "
                   "captured into a graph: call it once before capturing",
                   name);
        return nullptr;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
        *st = fail(LRS_ERR_HIP, "%s: hipGetSymbolAddress failed: %s", name, hipGetErrorString(e));
        return nullptr;
    }
    const uint64_t n16 = kScratchBytes / 16;
    void* args[] = {&ptr, (void*)&n16};
    e = hipLaunchKernel((const void*)&clear_scratch, dim3((unsigned)((n16 + 255) / 256)), dim3(256),
                        args, 0, stream);
    if (e != hipSuccess) {
        *st = fail(LRS_ERR_HIP, "%s: clearing the scratch area failed: %s", name,
                   hipGetErrorString(e));
        return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

}  // namespace
}  // namespace lrs

using namespace lrs;

extern "C" lrs_status lrs_gae_noalloc_f32(int64_t N, int64_t T, const float* rewards,
                                          const float* values, const uint8_t* term,
                                          const uint8_t* trunc, const float* tv, const float* boot,
                                          float gamma, float lambda, float* adv,
                                          const int64_t* strides, hipStream_t stream)
{
    const char* nm = "lrs_gae_noalloc_f32";
    // every argument is checked before anything (the first use's clear
    // included) is enqueued
    uint64_t gaps[6];
    LRS_TRY(gae_check<float>(nm, Layout{false, N, T, strides}, rewards, values, term, trunc, tv,
                             boot, gamma, lambda, adv, nullptr, 0, gaps));
    const size_t need = workspace_bytes_for((uint64_t)N * (uint64_t)T);
    if (need > kScratchBytes)
        return fail(LRS_ERR_INVALID_ARG,
                    "%s: %lld x %lld needs %zu bytes of scratch; the static area holds %zu "
                    "(num_envs * seq_len <= %llu)",
                    nm, (long long)N, (long long)T, need, kScratchBytes,
                    (unsigned long long)((kScratchBytes - sizeof(WsHeader)) / (8 * kRecordWords) *
                                         kMinTile));
    lrs_status st = LRS_OK;
    void* ws = device_scratch(nm, stream, &st);
    if (ws == nullptr) return st;
    return gae_entry<float>(nm, false, N, T, rewards, values, term, trunc, tv, boot, gamma, lambda,
                            adv, strides, ws, kScratchBytes, stream);
}
