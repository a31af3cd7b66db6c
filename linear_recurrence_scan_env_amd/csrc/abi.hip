// abi.hip -- library-wide entry points of include/lrs.h (no kernels): version,
// status strings, the last-error buffer, workspace sizing and the debug
// schedule override.
#include "timemajor.hpp"

namespace lrs {

std::atomic<int> g_force_lookback{0};
std::atomic<int> g_forced_cfg{-1};
std::atomic<int> g_forced_tm_waves{0};
thread_local char g_err[512];

}  // namespace lrs

using namespace lrs;

extern "C" {

int lrs_version(void) { return 100; }

const char* lrs_status_string(lrs_status s)
{
    switch (s) {
        case LRS_OK: return "success";
        case LRS_ERR_INVALID_ARG: return "invalid argument";
        case LRS_ERR_WORKSPACE: return "workspace missing or too small";
        case LRS_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* lrs_last_error(void) { return g_err; }

size_t lrs_workspace_bytes(lrs_estimator est, int64_t num_envs, int64_t seq_len)
{
    if ((int)est < 0 || (int)est > (int)LRS_AFFINE_SCAN) return 0;
    if (!valid_sizes(num_envs, seq_len)) return 0;
    const size_t row_major = workspace_bytes_for((uint64_t)num_envs * (uint64_t)seq_len);
    const size_t time_major = workspace_bytes_tm((uint64_t)num_envs, (uint64_t)seq_len);
    return row_major > time_major ? row_major : time_major;
}

lrs_status lrs_debug_set_schedule(int force_lookback, int elems_per_lane, int waves_per_block)
{
    int cfg = -1;
    if (elems_per_lane != 0 || waves_per_block != 0) {
        for (int i = 0; i < kNumCfg; ++i)
            if (kCfgs[i].E == elems_per_lane && kCfgs[i].W == waves_per_block) cfg = i;
        if (cfg < 0)
            return fail(LRS_ERR_INVALID_ARG, "lrs_debug_set_schedule: unsupported tile %d x %d",
                        elems_per_lane, waves_per_block);
    }
    g_force_lookback.store(force_lookback != 0);
    g_forced_cfg.store(cfg);
    return LRS_OK;
}

lrs_status lrs_debug_set_time_major_waves(int waves_per_block)
{
    if (waves_per_block != 0 && !tm_waves_supported(waves_per_block))
        return fail(LRS_ERR_INVALID_ARG, "lrs_debug_set_time_major_waves: %d is not 0, 2, 4, 8 or 16",
                    waves_per_block);
    g_forced_tm_waves.store(waves_per_block);
    return LRS_OK;
}

}  // extern "C"
