// Decoupled look-back over row groups taken in ticket order: each group learns the
// offset of its kept blocks in col_idx from the totals of the groups before it.
#pragma once

#include "common.h"
#include "kernels.h"

namespace sattn {

// Offset of group g in col_idx: decoupled look-back over the groups' look-back words,
// run by one wave.  The group's total is published first; then the words of the 64
// groups before the current position are read at once and summed up to the nearest
// one that carries a prefix; while one of those has published nothing yet the wave
// polls again.  Every group before g holds an earlier ticket, so it is running or
// done and publishes its total without waiting on anyone; the polls end.  After
// spin_cap polls the wave gives up: it counts the missing totals as 0 (so that the
// offsets of later groups can only come out low, never past the end of col_idx) and
// reports that it gave up through `gave_up`.
__device__ __forceinline__ int64_t group_lookback(uint64_t *status, int64_t g, int64_t total, int lane,
                                                  uint32_t spin_cap, bool &gave_up) {
    if (lane == 0)
        __hip_atomic_store(status + g, (g == 0 ? kStatPre : kStatAgg) | (uint64_t)total, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    int64_t base = 0, p = g - 1;
    uint32_t polls = 0;
    gave_up = false;
    while (p >= 0) {
        const int64_t idx = p - lane;
        const uint64_t w = idx >= 0 ? __hip_atomic_load(status + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                    : kStatPre;
        const uint64_t f = w & kStatFlags;
        const uint64_t pre = __ballot(f == kStatPre);
        const int first = pre ? __builtin_ctzll(pre) : 64;       // nearest group carrying a prefix
        const uint64_t upto = first >= 63 ? ~0ull : ((2ull << first) - 1);
        const bool missing = (__ballot(f == 0) & upto) != 0;
        if (missing && ++polls < spin_cap) {
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        gave_up = gave_up || missing;
        const int v = lane <= first && f != 0 ? (int)(w & ~kStatFlags) : 0;
        base += wave_sum_i(v);
        if (first < 64) break;
        p -= 64;
    }
    if (lane == 0)
        __hip_atomic_store(status + g, kStatPre | (uint64_t)(base + total), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return base;
}

}  // namespace sattn
