// Splitting a one-dimensional grid into dispatches the hardware accepts.
//
// An AQL kernel-dispatch packet gives the grid size in work-items as a 32-bit
// field per dimension, so one dispatch holds at most 2^32 - 1 work-items.  A
// grid of more workgroups than that is launched as consecutive slices; each
// slice is told the logical index of its first workgroup, and a kernel's
// logical workgroup is that offset plus its (remapped) index in the slice.
//
// Plain host C++ (no HIP): the plan is unit-tested on the CPU.
#pragma once

#include <stdint.h>

namespace pc {

constexpr uint64_t kDispatchItemLimit = 0xFFFFFFFFull;  // work-items per dispatch, per dimension

// Workgroups of `threads` lanes per slice under a cap of `items` work-items
// per dispatch (at least one workgroup).
inline int64_t slice_blocks(uint64_t items, int threads) {
    const uint64_t per = items / static_cast<uint64_t>(threads);
    return per > 0 ? static_cast<int64_t>(per) : 1;
}

// Calls launch(first, count) for consecutive slices [first, first + count)
// that cover [0, n_blocks) in order, each with count <= slice_blocks(items,
// threads); stops at, and returns, the first non-zero result.  n_blocks <= 0
// launches nothing.
template <class Status, class F>
Status for_each_slice(int64_t n_blocks, int threads, uint64_t items, Status ok, F &&launch) {
    const int64_t per = slice_blocks(items, threads);
    for (int64_t first = 0; first < n_blocks; first += per) {
        const int64_t left = n_blocks - first;
        const Status st = launch(first, static_cast<uint32_t>(left < per ? left : per));
        if (st != ok) return st;
    }
    return ok;
}

}  // namespace pc
