// Host-side launchers of the kernels, one per translation unit; called by the
// C ABI layer (api.hip) after it has validated every argument.
#pragma once

#include "common.hpp"
#include "dispatch.hpp"

namespace pc {

// Work-items per dispatch in force: the hardware's 2^32 - 1, or the lower cap
// set by the diagnostic pc_set_max_dispatch_items (api.hip).
uint64_t dispatch_items();

// Launches a grid of n_blocks workgroups of `threads` lanes as consecutive
// slices within the dispatch cap; launch(first, count) enqueues one slice
// whose kernel adds `first` to its workgroup index.
template <class F>
hipError_t launch_slices(int64_t n_blocks, int threads, F &&launch) {
    return for_each_slice(n_blocks, threads, dispatch_items(), hipSuccess, [&](int64_t first, uint32_t count) {
        launch(first, count);
        return hipGetLastError();
    });
}

hipError_t launch_fill(void *out, int64_t n_maps, uint32_t k0, uint32_t k1, uint32_t slot, bool raw,
                       hipStream_t stream);

// eps_c == nullptr: point-mass stand-in on the references x0c / x0u;
// otherwise eps_c / eps_u hold the network's noise predictions per map.
hipError_t launch_step_indep(float *state, const float *x0c, const float *x0u, const float *eps_c, const float *eps_u,
                             StepArgs a, bool noise, hipStream_t stream);

// init: draw x_T in the step (only with project, no pre_disc and references).
hipError_t launch_step_chain(float *state, const float *x0c, const float *x0u, const float *eps_c, const float *eps_u,
                             StepArgs a, ChainArgs ch, bool project, float *pre_disc, bool noise, bool init,
                             hipStream_t stream);

hipError_t launch_seam_project(float *state, int32_t n_chains, int32_t n_cols, ChainArgs ch, hipStream_t stream);

hipError_t launch_seam_discrepancy(const float *state, int32_t n_chains, int32_t n_cols, ChainArgs ch, float *rms,
                                   float *summary, hipStream_t stream);

hipError_t launch_seam_mean_abs(const float *state, int32_t n_chains, int32_t G, int32_t S, ChainArgs ch, float *out,
                                hipStream_t stream);

// proper: rotations only (det +1); otherwise any orthogonal map.
hipError_t launch_stitch(const float *coords, int32_t n_chains, int32_t G, int32_t S, ChainArgs ch, float *chain,
                         float *resid, bool proper, hipStream_t stream);

hipError_t launch_mds(const float *maps, int64_t n_maps, float *coords, float *eigvals, int32_t max_iters,
                      hipStream_t stream);

}  // namespace pc
