// abi.hip -- library-wide entry points of include/lrs.h (no kernels): version,
// status strings, the last-error buffer, workspace sizing, the debug
// schedule override and the schedule diagnostics.
#include "entries.hpp"

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

namespace lrs {
namespace {

// The plan of one functor, as run() / run_tm() would make it.
template <template <int> class Op>
lrs_status describe(bool tm, int64_t N, int64_t T, float beta_max, lrs_schedule_info* info,
                    uint32_t* map, int64_t cap)
{
    constexpr bool kB = Op<4>::kBackward;
    *info = lrs_schedule_info{};
    info->time_major = tm ? 1 : 0;
    info->backward = kB ? 1 : 0;
    if (!tm) {
        const Plan p = plan_row_major<Op>(N, T, beta_max);
        const Cfg& k = kCfgs[p.cfg];
        info->num_blocks = p.s.num_tiles;
        info->num_tiles = p.s.num_tiles;
        info->tile_elems = k.tile();
        info->carries = p.s.lookback;
        info->tiles_per_row = (int32_t)p.s.tiles_per_row;
        info->elems_per_lane = k.E;
        info->waves_per_block = k.W;
        info->composition_fp64 = p.fp64 ? 1 : 0;
        if (map != nullptr && cap >= info->num_blocks)
            for (uint32_t b = 0; b < p.s.num_tiles; ++b) map[b] = place_tile(b, p.s, kB).tile;
        return LRS_OK;
    }
    if (N >= (int64_t(1) << 32))
        return fail(LRS_ERR_INVALID_ARG, "lrs_debug_schedule: time-major calls need num_envs < 2^32");
    const PlanTM p = plan_time_major(N, T, tm_lean_capable<Op>(beta_max));
    using Val = typename Op<4>::T;
    info->num_blocks = p.s.num_blocks;
    info->num_tiles = (int64_t)p.s.time_tiles * p.s.groups;
    info->tile_steps = (int64_t)p.tile_steps;
    info->groups = p.s.groups;
    info->envs_per_group = p.rows_waves ? kTmRowsV : kWave * p.G;
    info->carries = p.s.time_tiles > 1 ? 1 : 0;
    info->elems_per_lane = p.rows_waves ? kTmE : (p.long_rows ? kTmELong : kTmE);
    info->waves_per_block = p.W;
    info->composition_fp64 = std::is_same<Val, float>::value && beta_max > kFp32BetaMax ? 1 : 0;
    if (map != nullptr && cap >= info->num_blocks)
        for (uint32_t b = 0; b < p.s.num_blocks; ++b) {
            const TilePlaceTM t = place_tile_tm(b, p.s, kB);
            map[b] = t.k * p.s.groups + t.g;
        }
    return LRS_OK;
}

template <class D>
lrs_status describe_call(lrs_estimator est, int flags, int64_t N, int64_t T, float bm,
                         lrs_schedule_info* info, uint32_t* map, int64_t cap)
{
    const bool tr = flags & LRS_SCHED_TRUNCATED, tm = flags & LRS_SCHED_TIME_MAJOR;
    switch (est) {
        case LRS_GAE:
            return tr ? describe<GaeSel<D>::template T>(tm, N, T, bm, info, map, cap)
                      : describe<GaeSel<D>::template N>(tm, N, T, bm, info, map, cap);
        case LRS_VTRACE:
            return tr ? describe<VtraceSel<D>::template T>(tm, N, T, bm, info, map, cap)
                      : describe<VtraceSel<D>::template N>(tm, N, T, bm, info, map, cap);
        case LRS_RETRACE:
            return tr ? describe<RetraceSel<D>::template T>(tm, N, T, bm, info, map, cap)
                      : describe<RetraceSel<D>::template N>(tm, N, T, bm, info, map, cap);
        case LRS_LAMBDA_RETURNS:
            return tr ? describe<LambdaSel<D>::template T>(tm, N, T, bm, info, map, cap)
                      : describe<LambdaSel<D>::template N>(tm, N, T, bm, info, map, cap);
        case LRS_DISCOUNTED_RETURNS:
            return tr ? describe<DiscSel<D>::template T>(tm, N, T, bm, info, map, cap)
                      : describe<DiscSel<D>::template N>(tm, N, T, bm, info, map, cap);
        case LRS_ELIGIBILITY_TRACES:
            return describe<ForwardSel<D>::template Elig>(tm, N, T, bm, info, map, cap);
        case LRS_PREFIX_SUM_F32:
            return describe<ForwardSel<D>::template Prefix>(tm, N, T, bm, info, map, cap);
        case LRS_PREFIX_SUM_I32:
            return describe<PrefixI32Op>(tm, N, T, bm, info, map, cap);
        case LRS_AFFINE_SCAN:
            if (flags & LRS_SCHED_REVERSE)
                return tr ? describe<AffineSel<D>::template RevR>(tm, N, T, bm, info, map, cap)
                          : describe<AffineSel<D>::template RevN>(tm, N, T, bm, info, map, cap);
            return tr ? describe<AffineSel<D>::template FwdR>(tm, N, T, bm, info, map, cap)
                      : describe<AffineSel<D>::template FwdN>(tm, N, T, bm, info, map, cap);
    }
    return fail(LRS_ERR_INVALID_ARG, "lrs_debug_schedule: unknown estimator %d", (int)est);
}

}  // namespace
}  // namespace lrs

extern "C" lrs_status lrs_debug_schedule(lrs_estimator est, int flags, int64_t num_envs,
                                         int64_t seq_len, float beta_max, lrs_schedule_info* info,
                                         uint32_t* tile_of_block, int64_t capacity)
{
    if (info == nullptr) return fail(LRS_ERR_INVALID_ARG, "lrs_debug_schedule: info is required");
    if (!valid_sizes(num_envs, seq_len))
        return fail(LRS_ERR_INVALID_ARG, "lrs_debug_schedule: invalid sizes %lld x %lld",
                    (long long)num_envs, (long long)seq_len);
    if ((flags & ~0xf) != 0 || ((flags & LRS_SCHED_16BIT) && est == LRS_PREFIX_SUM_I32) ||
        ((flags & LRS_SCHED_REVERSE) && est != LRS_AFFINE_SCAN))
        return fail(LRS_ERR_INVALID_ARG, "lrs_debug_schedule: unsupported flags %d", flags);
    if (flags & LRS_SCHED_16BIT)
        return describe_call<bf16_t>(est, flags, num_envs, seq_len, beta_max, info, tile_of_block,
                                     capacity);
    return describe_call<float>(est, flags, num_envs, seq_len, beta_max, info, tile_of_block,
                                capacity);
}
