// C ABI of the library (include/pc.h): argument validation, the float64
// schedule and step coefficients, and kernel launches on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <new>

#include "pc.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[256] = "";

pc_status fail(pc_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
pc_status fail(pc_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

pc_status ok() {
    g_err[0] = '\0';
    return PC_OK;
}

pc_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(PC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a layout; on success stores the map count.
pc_status check_layout(const pc_layout *L, int64_t *n_maps) {
    if (!L) return fail(PC_ERR_NULL, "layout is NULL");
    if (L->n_regions < 1 || L->n_guidance < 1 || L->n_traj < 1)
        return fail(PC_ERR_SHAPE, "R, G, S must be >= 1 (got %d, %d, %d)", L->n_regions, L->n_guidance, L->n_traj);
    if (L->n_guidance > PC_MAX_GUIDANCE) return fail(PC_ERR_SHAPE, "G = %d exceeds %d", L->n_guidance, PC_MAX_GUIDANCE);
    if (L->chain_len < 1 || L->n_regions % L->chain_len != 0)
        return fail(PC_ERR_SHAPE, "chain_len %d must be >= 1 and divide R = %d", L->chain_len, L->n_regions);
    if (L->chain_len > 1 && (L->overlap < 2 || L->overlap > pc::kMaxOverlap))
        return fail(PC_ERR_SHAPE, "overlap %d outside 2..%d", L->overlap, pc::kMaxOverlap);
    const int64_t n = static_cast<int64_t>(L->n_regions) * L->n_guidance * L->n_traj;
    // trajectory ids are Philox counter words, kept below 2^31 for signed index
    // arithmetic; grids beyond one dispatch's 2^32 - 1 work-items are launched in slices
    if (n > 0x7FFFFFFFLL) return fail(PC_ERR_SHAPE, "R*G*S = %lld exceeds 2^31 - 1", static_cast<long long>(n));
    if (L->chain_len > 1 && static_cast<int64_t>(L->n_guidance) * L->n_traj > 0x7FFFFFFFLL / L->chain_len)
        return fail(PC_ERR_SHAPE, "chain layout too large");
    *n_maps = n;
    return PC_OK;
}

pc::ChainArgs chain_args(const pc_layout *L) {
    pc::ChainArgs ch;
    ch.chain_len = L->chain_len;
    ch.overlap = L->overlap;
    ch.n_pairs = L->overlap * (L->overlap - 1) / 2;
    return ch;
}

// Work-items per dispatch; lowered only by the diagnostic pc_set_max_dispatch_items.
std::atomic<uint64_t> g_dispatch_items{pc::kDispatchItemLimit};

}  // namespace

uint64_t pc::dispatch_items() { return g_dispatch_items.load(std::memory_order_relaxed); }

extern "C" {

const char *pc_version(void) { return "pc 0.1 (gfx950)"; }

const char *pc_status_string(pc_status s) {
    switch (s) {
        case PC_OK: return "ok";
        case PC_ERR_NULL: return "null pointer";
        case PC_ERR_SHAPE: return "bad shape";
        case PC_ERR_ALIGN: return "misaligned device pointer";
        case PC_ERR_PARAM: return "parameter out of range";
        case PC_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *pc_last_error(void) { return g_err; }

pc_status pc_set_max_dispatch_items(uint64_t items) {
    if (items == 0) items = pc::kDispatchItemLimit;
    if (items < 1024 || items > pc::kDispatchItemLimit)
        return fail(PC_ERR_PARAM, "dispatch cap %llu outside 1024..2^32-1", static_cast<unsigned long long>(items));
    g_dispatch_items.store(items, std::memory_order_relaxed);
    return ok();
}

pc_status pc_ddim_schedule(int32_t n_steps, int32_t T, double beta_start, double beta_end, double *abar_t,
                           double *abar_next) {
    if (!abar_t || !abar_next) return fail(PC_ERR_NULL, "output is NULL");
    if (T < 2) return fail(PC_ERR_PARAM, "T = %d must be >= 2", T);
    if (n_steps < 1 || T % n_steps != 0) return fail(PC_ERR_PARAM, "n_steps = %d must divide T = %d", n_steps, T);
    if (!(beta_start > 0.0 && beta_start < 1.0 && beta_end > 0.0 && beta_end < 1.0))
        return fail(PC_ERR_PARAM, "betas must lie in (0, 1)");
    // abar_t = prod_{s <= t} (1 - beta_s), accumulated in index order.
    const int stride = T / n_steps;
    double acc = 1.0;
    int next_i = n_steps - 1;  // tau_i = T - stride (i + 1); tau_{n-1} = 0 comes first
    for (int t = 0; t < T && next_i >= 0; ++t) {
        acc *= 1.0 - (beta_start + (beta_end - beta_start) * static_cast<double>(t) / static_cast<double>(T - 1));
        if (t == T - stride * (next_i + 1)) {
            abar_t[next_i] = acc;
            --next_i;
        }
    }
    for (int i = 0; i < n_steps; ++i) abar_next[i] = i + 1 < n_steps ? abar_t[i + 1] : 1.0;
    return ok();
}

pc_status pc_ddim_schedule_cosine(int32_t n_steps, int32_t T, double s, double beta_max, double *abar_t,
                                  double *abar_next) {
    if (!abar_t || !abar_next) return fail(PC_ERR_NULL, "output is NULL");
    if (T < 2) return fail(PC_ERR_PARAM, "T = %d must be >= 2", T);
    if (n_steps < 1 || T % n_steps != 0) return fail(PC_ERR_PARAM, "n_steps = %d must divide T = %d", n_steps, T);
    if (!(s >= 0.0 && s < 1.0) || !(beta_max > 0.0 && beta_max < 1.0))
        return fail(PC_ERR_PARAM, "need 0 <= s < 1 and 0 < beta_max < 1");
    // f(u) = cos^2(pi/2 (u + s)/(1 + s)); beta_t = min(1 - f((t+1)/T) / f(t/T), beta_max)
    const double pi = 3.141592653589793;
    const int stride = T / n_steps;
    double acc = 1.0;
    int next_i = n_steps - 1;
    for (int t = 0; t < T && next_i >= 0; ++t) {
        const double c0 = cos((static_cast<double>(t) / T + s) / (1.0 + s) * pi / 2.0);
        const double c1 = cos((static_cast<double>(t + 1) / T + s) / (1.0 + s) * pi / 2.0);
        double beta = 1.0 - (c1 * c1) / (c0 * c0);
        if (beta > beta_max) beta = beta_max;
        acc *= 1.0 - beta;
        if (t == T - stride * (next_i + 1)) {
            abar_t[next_i] = acc;
            --next_i;
        }
    }
    for (int i = 0; i < n_steps; ++i) abar_next[i] = i + 1 < n_steps ? abar_t[i + 1] : 1.0;
    return ok();
}

pc_status pc_init_state(float *state, const pc_layout *layout, uint64_t seed, void *stream) {
    return pc_normal_fill(state, layout, seed, 0u, stream);
}

pc_status pc_normal_fill(float *out, const pc_layout *layout, uint64_t seed, uint32_t slot, void *stream) {
    if (!out) return fail(PC_ERR_NULL, "output is NULL");
    int64_t n = 0;
    const pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (!aligned16(out)) return fail(PC_ERR_ALIGN, "output not 16-byte aligned");
    return hip_status(pc::launch_fill(out, n, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), slot,
                                      false, static_cast<hipStream_t>(stream)),
                      "normal fill launch");
}

pc_status pc_philox_fill(uint32_t *out, const pc_layout *layout, uint64_t seed, uint32_t slot, void *stream) {
    if (!out) return fail(PC_ERR_NULL, "output is NULL");
    int64_t n = 0;
    const pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (!aligned16(out)) return fail(PC_ERR_ALIGN, "output not 16-byte aligned");
    return hip_status(pc::launch_fill(out, n, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), slot,
                                      true, static_cast<hipStream_t>(stream)),
                      "philox fill launch");
}

}  // extern "C"

namespace {

// Shared by both step entry points: eps_c == nullptr selects the point-mass
// stand-in on the references, otherwise the per-map noise predictions.
pc_status ddim_step(const char *name, float *state, const float *x0_cond, const float *x0_uncond, const float *eps_c,
                    const float *eps_u, const float *w, const pc_layout *layout, double abar_t, double abar_next,
                    double eta, uint64_t seed, uint32_t slot, int32_t project_seams, float *pre_disc, void *stream,
                    bool init = false) {
    int64_t n = 0;
    pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    const bool eps = eps_c != nullptr;
    if (eps ? (!aligned16(eps_c) || !aligned16(eps_u)) : (!aligned16(x0_cond) || !aligned16(x0_uncond)))
        return fail(PC_ERR_ALIGN, "%s: device arrays must be 16-byte aligned", name);
    if (!aligned16(state) || (pre_disc && !aligned16(pre_disc)))
        return fail(PC_ERR_ALIGN, "%s: device arrays must be 16-byte aligned", name);
    if (!(abar_t > 0.0 && abar_t < 1.0)) return fail(PC_ERR_PARAM, "abar_t = %g outside (0, 1)", abar_t);
    if (!(abar_next > 0.0 && abar_next <= 1.0)) return fail(PC_ERR_PARAM, "abar_next = %g outside (0, 1]", abar_next);
    if (abar_t > abar_next) return fail(PC_ERR_PARAM, "abar_t %g > abar_next %g", abar_t, abar_next);
    if (!(eta >= 0.0) || !isfinite(eta)) return fail(PC_ERR_PARAM, "eta = %g must be finite and >= 0", eta);
    const bool chains = layout->chain_len > 1;
    if ((project_seams || pre_disc) && !chains)
        return fail(PC_ERR_PARAM, "seam projection / discrepancy need chain_len > 1");

    const double a = abar_t, an = abar_next;
    const double sigma = eta * sqrt((1.0 - an) / (1.0 - a)) * sqrt(1.0 - a / an);
    double dir2 = 1.0 - an - sigma * sigma;
    if (dir2 < -1e-12) return fail(PC_ERR_PARAM, "eta = %g too large: 1 - abar_next - sigma^2 = %g", eta, dir2);
    if (dir2 < 0.0) dir2 = 0.0;

    pc::StepArgs args;
    memset(&args, 0, sizeof args);
    args.c.sa = static_cast<float>(sqrt(a));
    args.c.inv_s1a = static_cast<float>(1.0 / sqrt(1.0 - a));
    args.c.s1a = static_cast<float>(sqrt(1.0 - a));
    args.c.inv_sa = static_cast<float>(1.0 / sqrt(a));
    args.c.sap = static_cast<float>(sqrt(an));
    args.c.cdir = static_cast<float>(sqrt(dir2));
    args.c.sigma = static_cast<float>(sigma);
    for (int g = 0; g < layout->n_guidance; ++g) {
        if (!isfinite(w[g])) return fail(PC_ERR_PARAM, "w[%d] is not finite", g);
        args.w[g] = w[g];
    }
    args.R = layout->n_regions;
    args.G = layout->n_guidance;
    args.S = layout->n_traj;
    args.k0 = static_cast<uint32_t>(seed);
    args.k1 = static_cast<uint32_t>(seed >> 32);
    args.slot = slot;
    args.init = init ? 1u : 0u;
    const bool noise = args.c.sigma != 0.0f;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (chains && (project_seams || pre_disc)) {
        // x_T in the seam-owning kernel: drawn in registers where it has that
        // form (projecting, no discrepancy output, references), else filled first
        const bool draw = init && project_seams && !pre_disc && !eps;
        if (init && !draw) {
            const hipError_t e = pc::launch_fill(state, n, args.k0, args.k1, 0u, false, s);
            if (e != hipSuccess) return hip_status(e, "x_T fill launch");
        }
        return hip_status(pc::launch_step_chain(state, x0_cond, x0_uncond, eps_c, eps_u, args, chain_args(layout),
                                                project_seams != 0, pre_disc, noise, draw, s),
                          "chain step launch");
    }
    return hip_status(pc::launch_step_indep(state, x0_cond, x0_uncond, eps_c, eps_u, args, noise, s), "step launch");
}

}  // namespace

extern "C" {

pc_status pc_ddim_cfg_step(float *state, const float *x0_cond, const float *x0_uncond, const float *w,
                           const pc_layout *layout, double abar_t, double abar_next, double eta, uint64_t seed,
                           uint32_t slot, int32_t project_seams, float *pre_disc, void *stream) {
    if (!state || !x0_cond || !x0_uncond || !w) return fail(PC_ERR_NULL, "state, references and w are required");
    return ddim_step("pc_ddim_cfg_step", state, x0_cond, x0_uncond, nullptr, nullptr, w, layout, abar_t, abar_next,
                     eta, seed, slot, project_seams, pre_disc, stream);
}

pc_status pc_ddim_cfg_step_eps(float *state, const float *eps_cond, const float *eps_uncond, const float *w,
                               const pc_layout *layout, double abar_t, double abar_next, double eta, uint64_t seed,
                               uint32_t slot, int32_t project_seams, float *pre_disc, void *stream) {
    if (!state || !eps_cond || !eps_uncond || !w)
        return fail(PC_ERR_NULL, "state, noise predictions and w are required");
    return ddim_step("pc_ddim_cfg_step_eps", state, nullptr, nullptr, eps_cond, eps_uncond, w, layout, abar_t,
                     abar_next, eta, seed, slot, project_seams, pre_disc, stream);
}

pc_status pc_ddim_sample(float *state, const float *x0_cond, const float *x0_uncond, const float *w,
                         const pc_layout *layout, int32_t n_steps, int32_t T, double beta_start, double beta_end,
                         double eta, uint64_t seed, int32_t project_every, int32_t init, void *stream) {
    if (!state || !x0_cond || !x0_uncond || !w) return fail(PC_ERR_NULL, "state, references and w are required");
    int64_t n = 0;
    pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (project_every < 0) return fail(PC_ERR_PARAM, "project_every = %d must be >= 0", project_every);
    if (project_every > 0 && layout->chain_len < 2)
        return fail(PC_ERR_PARAM, "seam projection needs chain_len > 1");
    if (n_steps < 1 || n_steps > 100000) return fail(PC_ERR_PARAM, "n_steps = %d outside 1..100000", n_steps);
    double *sched = new (std::nothrow) double[2 * static_cast<size_t>(n_steps)];
    if (!sched) return fail(PC_ERR_PARAM, "cannot hold the schedule");
    st = pc_ddim_schedule(n_steps, T, beta_start, beta_end, sched, sched + n_steps);
    // Validate every step's parameters before enqueuing anything.
    for (int i = 0; st == PC_OK && i < n_steps; ++i) {
        const double a = sched[i], an = sched[n_steps + i];
        if (!(a > 0.0 && a < 1.0 && an > 0.0 && an <= 1.0 && a <= an))
            st = fail(PC_ERR_PARAM, "schedule step %d out of range", i);
        else if (!(eta >= 0.0) || !isfinite(eta))
            st = fail(PC_ERR_PARAM, "eta = %g must be finite and >= 0", eta);
        else {
            const double sg = eta * sqrt((1.0 - an) / (1.0 - a)) * sqrt(1.0 - a / an);
            if (1.0 - an - sg * sg < -1e-12) st = fail(PC_ERR_PARAM, "eta = %g too large at step %d", eta, i);
        }
    }
    // With init, the first step draws x_T in registers (the same Philox slot 0
    // normals pc_init_state writes) instead of reading a filled state.
    for (int i = 0; st == PC_OK && i < n_steps; ++i) {
        const int proj = project_every > 0 && (i + 1) % project_every == 0;
        st = ddim_step("pc_ddim_sample", state, x0_cond, x0_uncond, nullptr, nullptr, w, layout, sched[i],
                       sched[n_steps + i], eta, seed, static_cast<uint32_t>(i + 1), proj, nullptr, stream,
                       init && i == 0);
    }
    delete[] sched;
    return st;
}

pc_status pc_seam_project(float *state, const pc_layout *layout, void *stream) {
    if (!state) return fail(PC_ERR_NULL, "state is NULL");
    int64_t n = 0;
    const pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (layout->chain_len < 2) return fail(PC_ERR_SHAPE, "seam projection needs chain_len >= 2");
    if (!aligned16(state)) return fail(PC_ERR_ALIGN, "state not 16-byte aligned");
    return hip_status(pc::launch_seam_project(state, layout->n_regions / layout->chain_len,
                                              layout->n_guidance * layout->n_traj, chain_args(layout),
                                              static_cast<hipStream_t>(stream)),
                      "seam projection launch");
}

pc_status pc_seam_discrepancy(const float *state, const pc_layout *layout, float *rms, float *summary, void *stream) {
    if (!state || !rms) return fail(PC_ERR_NULL, "state and rms are required");
    int64_t n = 0;
    const pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (layout->chain_len < 2) return fail(PC_ERR_SHAPE, "seam discrepancy needs chain_len >= 2");
    if (!aligned16(state) || !aligned16(rms) || (summary && !aligned16(summary)))
        return fail(PC_ERR_ALIGN, "device arrays must be 16-byte aligned");
    return hip_status(pc::launch_seam_discrepancy(state, layout->n_regions / layout->chain_len,
                                                  layout->n_guidance * layout->n_traj, chain_args(layout), rms,
                                                  summary, static_cast<hipStream_t>(stream)),
                      "seam discrepancy launch");
}

pc_status pc_seam_mean_abs(const float *state, const pc_layout *layout, float *out, void *stream) {
    if (!state || !out) return fail(PC_ERR_NULL, "state and out are required");
    int64_t n = 0;
    const pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (layout->chain_len < 2) return fail(PC_ERR_SHAPE, "seam discrepancy needs chain_len >= 2");
    if (!aligned16(state)) return fail(PC_ERR_ALIGN, "state not 16-byte aligned");
    return hip_status(pc::launch_seam_mean_abs(state, layout->n_regions / layout->chain_len, layout->n_guidance,
                                               layout->n_traj, chain_args(layout), out,
                                               static_cast<hipStream_t>(stream)),
                      "seam mean-abs launch");
}

pc_status pc_mds_recover(const float *maps, int64_t n_maps, float *coords, float *eigvals, int32_t max_iters,
                         void *stream) {
    if (n_maps < 0 || n_maps > 0x7FFFFFFFLL) return fail(PC_ERR_SHAPE, "n_maps = %lld outside 0..2^31-1",
                                                         static_cast<long long>(n_maps));
    if (max_iters == 0) max_iters = 128;
    if (max_iters < 1 || max_iters > 256) return fail(PC_ERR_PARAM, "max_iters = %d outside 1..256", max_iters);
    if (n_maps == 0) return ok();  // nothing to read or write; the pointers may be NULL
    if (!maps || !coords) return fail(PC_ERR_NULL, "maps and coords are required");
    if (!aligned16(maps) || !aligned16(coords) || (eigvals && !aligned16(eigvals)))
        return fail(PC_ERR_ALIGN, "device arrays must be 16-byte aligned");
    return hip_status(pc::launch_mds(maps, n_maps, coords, eigvals, max_iters, static_cast<hipStream_t>(stream)),
                      "mds launch");
}

}  // extern "C"

namespace {

// Shared by both stitching entry points: proper restricts the fits to rotations.
pc_status stitch(const float *coords, const pc_layout *layout, float *chain, float *residual, bool proper,
                 void *stream) {
    if (!coords || !chain || !residual) return fail(PC_ERR_NULL, "coords, chain and residual are required");
    int64_t n = 0;
    const pc_status st = check_layout(layout, &n);
    if (st != PC_OK) return st;
    if (layout->chain_len < 2 || layout->chain_len > 1024)
        return fail(PC_ERR_SHAPE, "stitching needs 2 <= chain_len <= 1024 (got %d)", layout->chain_len);
    if (layout->overlap < 4)  // three or fewer points are always coplanar: the fit is not unique
        return fail(PC_ERR_SHAPE, "stitching needs overlap >= 4 (got %d)", layout->overlap);
    if (!aligned16(coords) || !aligned16(chain) || !aligned16(residual))
        return fail(PC_ERR_ALIGN, "device arrays must be 16-byte aligned");
    return hip_status(pc::launch_stitch(coords, layout->n_regions / layout->chain_len, layout->n_guidance,
                                        layout->n_traj, chain_args(layout), chain, residual, proper,
                                        static_cast<hipStream_t>(stream)),
                      "stitch launch");
}

}  // namespace

extern "C" {

pc_status pc_kabsch_stitch(const float *coords, const pc_layout *layout, float *chain, float *residual,
                           void *stream) {
    return stitch(coords, layout, chain, residual, false, stream);
}

pc_status pc_kabsch_stitch_proper(const float *coords, const pc_layout *layout, float *chain, float *residual,
                                  void *stream) {
    return stitch(coords, layout, chain, residual, true, stream);
}

pc_status pc_philox_block(uint32_t out[4], const uint32_t ctr[4], uint64_t seed) {
    if (!out || !ctr) return fail(PC_ERR_NULL, "out and ctr are required");
    const pc::Words4 r = pc::philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], static_cast<uint32_t>(seed),
                                          static_cast<uint32_t>(seed >> 32));
    out[0] = r.v0;
    out[1] = r.v1;
    out[2] = r.v2;
    out[3] = r.v3;
    return ok();
}

pc_status pc_seam_index_map(int32_t *out, int32_t overlap) {
    if (!out) return fail(PC_ERR_NULL, "out is NULL");
    if (overlap < 2 || overlap > pc::kMaxOverlap) return fail(PC_ERR_PARAM, "overlap %d outside 2..%d", overlap,
                                                             pc::kMaxOverlap);
    const int off = pc::kBeads - overlap;
    int k = 0;
    for (int p = 0; p < overlap; ++p)
        for (int q = p + 1; q < overlap; ++q, ++k) {
            out[2 * k] = pc::packed_index(off + p, off + q);
            out[2 * k + 1] = pc::packed_index(p, q);
        }
    return ok();
}

}  // extern "C"
