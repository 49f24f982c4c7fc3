/*
 * pc.h — C ABI of the MI355X (gfx950) hot path of tiled, ensemble 3D-genome
 * diffusion inference: guided DDIM reverse steps over batched 64-bead
 * distance maps, overlap-consistency projection of adjacent tiles, and
 * classical-MDS recovery of a point cloud per map.
 *
 * Method: "ParaChromo: a parallel inference framework for conditioned, tiled
 * 3D genome diffusion" (Electronics 15(13):2750), over the ChromoGen sampler
 * it wraps (section 3.1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Map:    64 beads; the 2016 distances of bead pairs i < j, float32, strict
 *         upper triangle row by row: idx(i, j) = i(127 - i)/2 + (j - i - 1).
 * State:  float32 [R][G][S][2016], row-major, for R regions (or tiles), G
 *         guidance weights and S trajectories per (region, weight).  Map
 *         (r, g, s) has trajectory id t = (r G + g) S + s.
 * Chains: with chain_len > 1, regions c*chain_len .. c*chain_len+chain_len-1
 *         are the consecutive tiles of chain c; adjacent tiles share
 *         `overlap` beads (the last `overlap` beads of tile k are the first of
 *         tile k+1).  The same (g, s) across a chain is one joint sample.
 * Noise:  Philox4x32-10 (Salmon et al., SC'11), key = (seed low word, seed
 *         high word), counter = (q, t, slot, 0) for the quad q = e / 4 of
 *         packed element e; word e % 4 belongs to element e.  Slot 0 draws
 *         x_T, slot i+1 the noise of DDIM step i.  Words (0,1) and (2,3) of a
 *         block become two normals each by Box-Muller on the 24-bit uniforms
 *         u1 = ((r >> 8) + 1) 2^-24 in (0, 1] and u2 = (r >> 8) 2^-24 in [0, 1):
 *         sqrt(-2 ln u1) cos(2 pi u2), then sqrt(-2 ln u1) sin(2 pi u2).
 * Memory: every array argument marked "device" is device memory owned by the
 *         caller and must be 16-byte aligned; "host" arrays are host memory.
 *         The library allocates no device memory and keeps no state between
 *         calls (pc_ddim_sample holds its schedule in a host buffer for the
 *         length of the call; the one setting, pc_set_max_dispatch_items, is
 *         a diagnostic); it is safe to call from several threads.
 * Sizes:  any layout with R G S <= 2^31 - 1 maps is accepted.  One dispatch
 *         holds at most 2^32 - 1 work-items, so a kernel whose grid needs
 *         more (e.g. the independent-map step beyond 16,777,214 maps, two
 *         maps per 512-lane workgroup) is launched as consecutive slices of
 *         the same grid on the same stream, with identical results.
 * Stream: `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *         enqueued asynchronously on it; nothing synchronises.
 * Errors: argument errors are detected before any launch and return a
 *         negative status with nothing enqueued; a failed launch returns
 *         PC_ERR_HIP.  pc_last_error() describes the last failure on the
 *         calling thread.  Nothing aborts and no exception crosses the ABI.
 */
#ifndef PC_H
#define PC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define PC_API __attribute__((visibility("default")))
#else
#define PC_API
#endif

typedef int32_t pc_status;
#define PC_OK 0
#define PC_ERR_NULL (-1)   /* a required pointer is NULL                      */
#define PC_ERR_SHAPE (-2)  /* sizes non-positive, inconsistent or overflowing */
#define PC_ERR_ALIGN (-3)  /* a device array is not 16-byte aligned           */
#define PC_ERR_PARAM (-4)  /* a scalar parameter is out of its range          */
#define PC_ERR_HIP (-5)    /* the HIP runtime reported an error at launch     */

#define PC_BEADS 64
#define PC_PACKED 2016
#define PC_MAX_GUIDANCE 16

typedef struct pc_layout {
    int32_t n_regions;  /* R >= 1: independent regions, or tiles of all chains      */
    int32_t n_guidance; /* G in 1..PC_MAX_GUIDANCE                                  */
    int32_t n_traj;     /* S >= 1 trajectories per (region, guidance weight)        */
    int32_t chain_len;  /* tiles per chain, >= 1, dividing R; 1 = no chains         */
    int32_t overlap;    /* beads shared by adjacent tiles, 2..32 (chain_len > 1)    */
} pc_layout;

/* Version string of the library. */
PC_API const char *pc_version(void);

/* Static text for a status code. */
PC_API const char *pc_status_string(pc_status status);

/* Message describing the last failing call on this thread ("" if none). */
PC_API const char *pc_last_error(void);

/*
 * Noise schedule and DDIM grid (host).  Linear beta schedule of the DDPM
 * sampler (Ho et al., ref. [19] of the paper): beta_s = beta_start +
 * (beta_end - beta_start) s / (T - 1), abar_t = prod_{s <= t} (1 - beta_s).
 * DDIM (Song et al., ref. [7]) with n_steps reverse steps of stride T/n_steps
 * visits tau_i = T - (T/n_steps)(i + 1); step i goes from abar[tau_i] to
 * abar[tau_{i+1}], and to 1 after the last step.  The paper reduces the
 * sampler to 50..1000 DDIM steps (Abstract; section 5.4.3).
 *   abar_t[i], abar_next[i]  host double [n_steps], written.
 * Errors: NULL outputs; T < 2; n_steps < 1 or not dividing T; betas not in
 * (0, 1).
 */
PC_API pc_status pc_ddim_schedule(int32_t n_steps, int32_t T, double beta_start, double beta_end,
                           double *abar_t, double *abar_next);

/*
 * Cosine noise schedule (host), the schedule of ChromoGen's sampler
 * (section 4.3.2), in the form of Nichol & Dhariwal (ICML 2021): with
 * f(u) = cos^2(pi/2 (u + s)/(1 + s)), beta_t = min(1 - f((t+1)/T) / f(t/T),
 * beta_max) and abar_t = prod_{u <= t} (1 - beta_u); the DDIM grid and
 * outputs are those of pc_ddim_schedule (s = 0.008, beta_max = 0.999 are the
 * published values).
 * Errors: NULL outputs; T < 2; n_steps < 1 or not dividing T; s outside
 * [0, 1) or beta_max outside (0, 1).
 */
PC_API pc_status pc_ddim_schedule_cosine(int32_t n_steps, int32_t T, double s, double beta_max, double *abar_t,
                                         double *abar_next);

/*
 * Initial state x_T: an independent N(0, 1) draw per packed entry of every
 * map, Philox slot 0 (each region starts from independent Gaussian noise,
 * section 4.3.1).
 *   state  device float [R][G][S][2016], written.
 */
PC_API pc_status pc_init_state(float *state, const pc_layout *layout, uint64_t seed, void *stream);

/*
 * One fused guided DDIM reverse step over every map, in place (sections 3.1
 * and 4.1; DDIM of ref. [7]; classifier-free guidance of ref. [15]).
 * Denoiser stand-in: the exact noise prediction for a point-mass prior at
 * the region's reference map, eps(x; x0) = (x - sqrt(a) x0) / sqrt(1 - a).
 * With a = abar_t, a' = abar_next, sigma = eta sqrt((1-a')/(1-a)) sqrt(1-a/a'):
 *   eps    = eps_u + w_g (eps_c - eps_u)
 *   x0_hat = (x - sqrt(1-a) eps) / sqrt(a)
 *   x      = sqrt(a') x0_hat + sqrt(max(0, 1-a'-sigma^2)) eps + sigma z,
 * z the normals of Philox slot `slot`.
 * If project_seams != 0 (chains only), every shared pair of adjacent tiles
 * is then replaced by the float32 mean (left + right) * 0.5 of its two
 * stepped copies, written identically to both tiles (overlap-consistency
 * projection, section 4.3.2 and Algorithm 1).
 *   state      device float [R][G][S][2016], read and written.
 *   x0_cond,
 *   x0_uncond  device float [R][2016]: conditional / unconditional reference.
 *   w          host float [G]: guidance weight per g (0 unconditional, 1 conditional).
 *   pre_disc   device float [n_chains*(chain_len-1)][G][S] or NULL (chains
 *              only): per seam and joint sample, the RMS over the shared
 *              pairs of (left copy - right copy) after the step and before
 *              any projection.
 * Errors: NULL state/x0/w/layout; bad layout; abar_t outside (0, 1) or
 * abar_next outside (0, 1]; abar_t > abar_next; eta < 0 or not finite; 1 - a' - sigma^2 < -1e-12
 * (eta too large); pre_disc or project_seams given without chains.
 */
PC_API pc_status pc_ddim_cfg_step(float *state, const float *x0_cond, const float *x0_uncond, const float *w,
                           const pc_layout *layout, double abar_t, double abar_next, double eta,
                           uint64_t seed, uint32_t slot, int32_t project_seams, float *pre_disc,
                           void *stream);

/*
 * The same guided DDIM step, projection and discrepancy as
 * pc_ddim_cfg_step, for a real denoiser: the conditional and unconditional
 * noise predictions of every map come from buffers (what the conditional
 * U-Net returns for the current state, section 3.1) instead of the
 * point-mass stand-in.  eps = eps_u + w_g (eps_c - eps_u), then the DDIM
 * update as above.  Algorithmic traffic: 16 B per element (state read and
 * written, both predictions read).  With eta = 1 on a stride-1 grid this is
 * the DDPM ancestral p-sample of the pages' spatial runs (section 5.1).
 *   eps_cond,
 *   eps_uncond  device float [R][G][S][2016], read.
 * Other arguments and errors as pc_ddim_cfg_step (references are not used).
 */
PC_API pc_status pc_ddim_cfg_step_eps(float *state, const float *eps_cond, const float *eps_uncond, const float *w,
                                      const pc_layout *layout, double abar_t, double abar_next, double eta,
                                      uint64_t seed, uint32_t slot, int32_t project_seams, float *pre_disc,
                                      void *stream);

/*
 * The whole reverse chain on the stream: optionally x_T (pc_init_state), then
 * the n_steps guided DDIM steps of pc_ddim_schedule(n_steps, T, beta_start,
 * beta_end), step i drawing Philox slot i + 1.  With chains and
 * project_every = K > 0, the seams are projected in the step kernel after
 * every K-th step (section 4.3.2: a synchronisation interval K); K = 0 never
 * projects.  Arguments as for pc_init_state and pc_ddim_cfg_step.
 *   init      1: start from x_T = the normals pc_init_state would write; the
 *             first step draws them in registers, so the state is not read
 *             before it (its prior contents are ignored).  0: start from the
 *             state as given.  The result is bitwise the same as
 *             pc_init_state followed by the steps.
 * Errors: those of pc_ddim_schedule and pc_ddim_cfg_step; project_every < 0;
 * project_every > 0 without chains.  On an error no step has been enqueued
 * unless it is PC_ERR_HIP.
 */
PC_API pc_status pc_ddim_sample(float *state, const float *x0_cond, const float *x0_uncond, const float *w,
                                const pc_layout *layout, int32_t n_steps, int32_t T, double beta_start,
                                double beta_end, double eta, uint64_t seed, int32_t project_every, int32_t init,
                                void *stream);

/*
 * Overlap-consistency projection alone (section 4.3.2, Algorithm 1): for
 * every chain, adjacent tile pair and (g, s), both copies of each shared pair
 * become their float32 mean (left + right) * 0.5.  Entries outside the seams
 * are not touched.
 *   state  device float [R][G][S][2016], read and written.
 * Errors: NULL pointers; bad layout; chain_len < 2.
 */
PC_API pc_status pc_seam_project(float *state, const pc_layout *layout, void *stream);

/*
 * Seam discrepancy (section 5.5, Eq. (6), read per joint sample): RMS over
 * the shared pairs of (left copy - right copy), per seam and (g, s).
 *   rms      device float [n_chains*(chain_len-1)][G][S], written.
 *   summary  device float [2] or NULL: mean and max of rms.
 * Errors: NULL pointers; bad layout; chain_len < 2.
 */
PC_API pc_status pc_seam_discrepancy(const float *state, const pc_layout *layout, float *rms, float *summary,
                              void *stream);

/*
 * Seam discrepancy in the paper's form (section 5.5, Eq. (6); the equation
 * itself was lost, read from its description): per seam and guidance weight,
 * the mean over the shared pairs of |mean_s left copy - mean_s right copy|,
 * the sample means taken over the S trajectories.  Sums run in float64 in a
 * fixed order, so the result is deterministic.
 *   out  device float [n_chains*(chain_len-1)][G], written.
 * Errors: NULL pointers; bad layout; chain_len < 2.
 */
PC_API pc_status pc_seam_mean_abs(const float *state, const pc_layout *layout, float *out, void *stream);

/*
 * Classical (Torgerson) MDS per map, the distance-geometry initialiser that
 * turns a final map into a 64-bead point cloud (sections 3.1 and 5.5):
 * B = -1/2 J (D o D) J, its three largest eigenpairs by block subspace
 * iteration (block 4, Rayleigh-Ritz), negative eigenvalues clamped to zero,
 * X = V_3 diag(sqrt(lambda)).  Each column of X is signed so that its
 * largest-magnitude entry is positive.  The iteration ranks by magnitude; when
 * large negative eigenvalues (a map far from Euclidean) could hide one of the
 * three wanted ones, their directions are projected out and the iteration
 * restarts, up to four passes.
 *   maps      device float [n_maps][2016].
 *   coords    device float [n_maps][64][3], written.
 *   eigvals   device float [n_maps][3] or NULL: the three eigenvalues, descending.
 *   max_iters cap on the Rayleigh-Ritz steps of a map over all passes, 1..256
 *             (0 selects 128).  Maps that are Euclidean up to rounding take 1-4;
 *             the cap is reached only by maps far from any point cloud.
 * Errors: NULL maps/coords (when n_maps > 0); n_maps < 0 or overflowing;
 * max_iters out of range.  n_maps = 0 is a no-op and accepts NULL pointers.
 */
PC_API pc_status pc_mds_recover(const float *maps, int64_t n_maps, float *coords, float *eigvals,
                         int32_t max_iters, void *stream);

/*
 * Chain stitching (section 5.5 and Figure 4: each tile's point cloud, rigidly
 * aligned on the shared beads, gives a chromosome-scale chain; the residual
 * after alignment is the coordinate-level seam diagnostic).  For every chain
 * and (g, s), tile 0 keeps its frame and tile k+1 is moved onto the aligned
 * tile k by the orthogonal map and translation that best superpose its first
 * `overlap` beads on tile k's last `overlap` beads (orthogonal Procrustes;
 * reflections allowed, since a distance map fixes a point cloud only up to
 * O(3)).  A shared bead takes the mean of its two aligned positions.
 *   coords    device float [R][G][S][64][3] (pc_mds_recover's output).
 *   chain     device float [n_chains][G][S][(chain_len-1)(64-overlap)+64][3], written.
 *   residual  device float [n_chains*(chain_len-1)][G][S], written: RMS
 *             distance over the shared beads after aligning seam k.
 * Shared beads must not be coplanar (the alignment is then not unique).
 * The seams are fitted independently in their tiles' own frames and the fits
 * composed along the chain, which equals fitting each tile onto the already
 * aligned one (a rigid motion of the target moves the best fit with it).
 * Errors: NULL pointers; bad layout; chain_len outside 2..1024; overlap below
 * 4 (three or fewer shared beads are always coplanar).
 */
PC_API pc_status pc_kabsch_stitch(const float *coords, const pc_layout *layout, float *chain, float *residual,
                                  void *stream);

/*
 * The same stitching with every fit restricted to rotations (det +1): Kabsch's
 * fit with the determinant correction, the other reading of the Kabsch
 * alignment of section 5.5 and Figure 4.  Where the best orthogonal map of a
 * seam is a reflection (adjacent tiles recovered as mirror images), the best
 * rotation is taken instead and the seam keeps a residual of the order of the
 * shared block's size: mirrored tiles are not superposed.  Arguments, layout
 * and errors as pc_kabsch_stitch.
 */
PC_API pc_status pc_kabsch_stitch_proper(const float *coords, const pc_layout *layout, float *chain, float *residual,
                                         void *stream);

/* Diagnostics ----------------------------------------------------------- */

/*
 * Lowers the number of work-items any one kernel dispatch may hold (process
 * wide; 0 restores the hardware's 2^32 - 1), so that tests can drive the
 * sliced launches of large grids (see "Sizes" above) with small inputs.
 * Results do not depend on it.  Not meant to change while other threads
 * enqueue work.
 * Errors: items outside 1024..2^32-1 (other than 0).
 */
PC_API pc_status pc_set_max_dispatch_items(uint64_t items);

/* One Philox4x32-10 block on the host: out = Philox(ctr, key(seed)). */
PC_API pc_status pc_philox_block(uint32_t out[4], const uint32_t ctr[4], uint64_t seed);

/*
 * The raw Philox words the sampler draws for slot `slot`:
 *   out  device uint32 [R][G][S][2016], word of every packed element.
 */
PC_API pc_status pc_philox_fill(uint32_t *out, const pc_layout *layout, uint64_t seed, uint32_t slot,
                         void *stream);

/*
 * The standard normals the sampler draws for slot `slot` (slot 0 equals
 * pc_init_state):
 *   out  device float [R][G][S][2016], written.
 */
PC_API pc_status pc_normal_fill(float *out, const pc_layout *layout, uint64_t seed, uint32_t slot, void *stream);

/*
 * Seam index map (host): for the overlap O, the O(O-1)/2 shared pairs
 * (p, q), p < q, in row-major order; out[2k] is the packed index of pair k in
 * the left tile (beads 64-O+p, 64-O+q) and out[2k+1] in the right tile
 * (beads p, q).  Section 4.3.2: the lower-right block of the left tile and
 * the upper-left block of the right tile.
 *   out  host int32 [O(O-1)/2][2], written.
 * Errors: NULL out; O outside 2..32.
 */
PC_API pc_status pc_seam_index_map(int32_t *out, int32_t overlap);

#ifdef __cplusplus
}
#endif

#endif /* PC_H */
