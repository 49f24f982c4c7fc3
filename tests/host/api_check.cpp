// Host test of the C ABI (include/pc.h), built with the library's host code and
// the HIP stand-ins of hip_stub.cpp under the address and undefined-behaviour
// sanitizers (tests/test_host_sanitized.py).  No GPU: kernel launches are
// recorded, not run, and device pointers are never dereferenced.  Checks:
//   * the slice plan of dispatch.hpp covers any grid in order within the cap;
//   * every argument error returns its status with nothing launched;
//   * every launch of every entry point stays within one dispatch's work-item
//     cap, and its slices cover exactly the kernel's logical grid, up to the
//     largest layout the boundary accepts (2^31 - 1 maps);
//   * a failed launch stops the slices and returns PC_ERR_HIP;
//   * the host helpers (schedules, seam index map, Philox) run clean.
// Prints one line per failed check; exit status 0 when all pass.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "dispatch.hpp"
#include "hip_stub.hpp"
#include "pc.h"

namespace {

int g_fails = 0;
#define CHECK(cond)                                                           \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fails;                                                        \
        }                                                                     \
    } while (0)

constexpr uint64_t kCap = 0xFFFFFFFFull;
constexpr int64_t kMaxMaps = 0x7FFFFFFFLL;

// Fake device pointers: 16-byte aligned, never dereferenced.
float *const F = reinterpret_cast<float *>(uintptr_t(1) << 20);
float *const F2 = reinterpret_cast<float *>((uintptr_t(1) << 20) + 4096);
float *const MIS = reinterpret_cast<float *>((uintptr_t(1) << 20) + 4);  // misaligned
const float W2[2] = {0.f, 1.f};
const float W16[16] = {0.f, 1.f, 2.f, 3.f, 0.5f, 1.5f, -1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 2.f};

pc_layout lay(int R, int G, int S, int L = 1, int O = 0) { return pc_layout{R, G, S, L, O}; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One logical grid of a kernel: a run of recorded slices starting at workgroup 0.
struct Grid {
    int64_t blocks = 0;   // workgroups covered
    int slices = 0;
    uint32_t threads = 0;
    bool contiguous = true;
    bool within_cap = true;
};

std::vector<Grid> grids(const char *kernel, uint64_t cap) {
    std::vector<Grid> out;
    for (const auto &l : stub::launches) {
        if (l.kernel.find(kernel) == std::string::npos) continue;
        if (l.block0 <= 0) {  // 0 starts a grid; -1 (no offset argument) is a grid of its own
            out.push_back(Grid{});
            out.back().threads = l.block;
        }
        Grid &g = out.back();
        if (l.block0 >= 0 && l.block0 != g.blocks) g.contiguous = false;
        if (l.grid == 0 || l.grid_yz != 1 || l.block != g.threads) g.contiguous = false;
        if (static_cast<uint64_t>(l.grid) * l.block > cap) g.within_cap = false;
        g.blocks += l.grid;
        ++g.slices;
    }
    return out;
}

// Exactly `count` grids of `kernel`, each covering `blocks` workgroups of
// `threads` lanes in contiguous slices within the cap.
void expect_grids(const char *kernel, int64_t blocks, uint32_t threads, size_t count, uint64_t cap, int line) {
    const auto gs = grids(kernel, cap);
    bool ok = gs.size() == count;
    for (const auto &g : gs)
        ok = ok && g.blocks == blocks && g.threads == threads && g.contiguous && g.within_cap;
    if (!ok) {
        fprintf(stderr, "line %d: %s: want %zu grid(s) of %lld x %u within cap %llu; got %zu:", line, kernel, count,
                static_cast<long long>(blocks), threads, static_cast<unsigned long long>(cap), gs.size());
        for (const auto &g : gs)
            fprintf(stderr, " [%lld blocks x %u, %d slices%s%s]", static_cast<long long>(g.blocks), g.threads,
                    g.slices, g.contiguous ? "" : ", broken", g.within_cap ? "" : ", over cap");
        fprintf(stderr, "\n");
        ++g_fails;
    }
}
#define EXPECT_GRIDS(kernel, blocks, threads, count, cap) expect_grids(kernel, blocks, threads, count, cap, __LINE__)

// ---------------------------------------------------------------------------
void slice_plan() {
    const int threads[] = {64, 256, 512, 1024};
    const uint64_t caps[] = {1024, 1500, 4096, 65539, 3 * 512 + 17, kCap};
    for (int t : threads)
        for (uint64_t cap : caps) {
            const int64_t per = pc::slice_blocks(cap, t);
            CHECK(per >= 1 && static_cast<uint64_t>(per) * t <= cap && static_cast<uint64_t>(per + 1) * t > cap);
            const int64_t ns[] = {0, 1, 2, per - 1, per, per + 1, 2 * per, 2 * per + 1, 10 * per + 7, 12345,
                                  kMaxMaps};
            for (int64_t n : ns) {
                if (n < 0 || n / per > 2000000) continue;
                int64_t next = 0;
                int slices = 0;
                bool ok = true;
                const int st = pc::for_each_slice(n, t, cap, 0, [&](int64_t first, uint32_t count) {
                    ok = ok && first == next && count >= 1 && static_cast<int64_t>(count) <= per &&
                         static_cast<uint64_t>(count) * t <= cap;
                    next = first + count;
                    ++slices;
                    return 0;
                });
                CHECK(st == 0 && ok && next == n);
                CHECK(slices == (n == 0 ? 0 : ceil_div(n, per)));
            }
            // the first failing slice stops the plan and its status comes back
            int calls = 0;
            const int st = pc::for_each_slice(3 * per, t, cap, 0, [&](int64_t, uint32_t) { return ++calls == 2 ? 7 : 0; });
            CHECK(st == 7 && calls == 2);
        }
    // the hardware cap: the independent step's 512-lane workgroups, 8,388,607 per dispatch
    CHECK(pc::slice_blocks(kCap, 512) == 8388607);
    CHECK(pc::slice_blocks(kCap, 64) == 67108863);
}

// ---------------------------------------------------------------------------
int step(float *state, const pc_layout &L, double a, double an, double eta, int proj, float *disc,
         const float *w = W2) {
    return pc_ddim_cfg_step(state, F, F2, w, &L, a, an, eta, 7, 3, proj, disc, nullptr);
}

void validation() {
    const pc_layout ok = lay(1, 2, 8);
    struct Case {
        pc_layout L;
        float *state;
        double a, an, eta;
        int proj;
        float *disc;
        int want;
    } cases[] = {
        {ok, nullptr, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_NULL},
        {lay(0, 2, 8), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(1, 0, 8), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(1, 2, 0), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(1, 17, 8), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(32, 2, 8, 5, 12), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(32, 2, 8, 0, 12), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(32, 2, 8, 32, 1), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(32, 2, 8, 32, 33), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(1 << 20, 16, 1 << 12), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},
        {lay(0x7FFFFFFF, 1, 2), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},  // 2^32 - 2 maps
        {lay(1 << 16, 1 << 4, 1 << 11), F, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_SHAPE},  // exactly 2^31
        {ok, MIS, 0.3, 0.5, 1.0, 0, nullptr, PC_ERR_ALIGN},
        {ok, F, 0.0, 0.5, 1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 1.0, 1.0, 1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, NAN, 0.5, 1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 1.5, 1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 0.0, 1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.5, 0.4, 1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 0.5, -1.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 0.5, NAN, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 0.5, INFINITY, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 0.5, 5.0, 0, nullptr, PC_ERR_PARAM},
        {ok, F, 0.3, 0.5, 1.0, 1, nullptr, PC_ERR_PARAM},      // projection without chains
        {ok, F, 0.3, 0.5, 1.0, 0, F2, PC_ERR_PARAM},           // discrepancy without chains
        {lay(4, 1, 3, 2, 12), F, 0.3, 0.5, 1.0, 1, MIS, PC_ERR_ALIGN},
    };
    for (const auto &c : cases) {
        stub::reset();
        const int st = step(c.state, c.L, c.a, c.an, c.eta, c.proj, c.disc);
        if (st != c.want) fprintf(stderr, "step case R=%d G=%d S=%d: status %d, want %d\n", c.L.n_regions,
                                  c.L.n_guidance, c.L.n_traj, st, c.want);
        CHECK(st == c.want);
        CHECK(stub::launches.empty());
        CHECK(strlen(pc_last_error()) > 0);
    }
    stub::reset();
    CHECK(pc_ddim_cfg_step(F, nullptr, F2, W2, &ok, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_ddim_cfg_step(F, F, F2, nullptr, &ok, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_ddim_cfg_step(F, F, F2, W2, nullptr, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_ddim_cfg_step(F, MIS, F2, W2, &ok, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_ALIGN);
    const float wbad[2] = {0.f, INFINITY};
    CHECK(pc_ddim_cfg_step(F, F, F2, wbad, &ok, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_cfg_step_eps(F, nullptr, F2, W2, &ok, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_ddim_cfg_step_eps(F, F, MIS, W2, &ok, 0.3, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_ddim_cfg_step_eps(F, F, F2, W2, &ok, 0.6, 0.5, 1.0, 0, 1, 0, nullptr, nullptr) == PC_ERR_PARAM);
    CHECK(pc_init_state(nullptr, &ok, 0, nullptr) == PC_ERR_NULL);
    CHECK(pc_init_state(MIS, &ok, 0, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_normal_fill(F, nullptr, 0, 0, nullptr) == PC_ERR_NULL);
    CHECK(pc_philox_fill(reinterpret_cast<uint32_t *>(MIS), &ok, 0, 0, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_seam_project(F, &ok, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_seam_project(nullptr, &ok, nullptr) == PC_ERR_NULL);
    const pc_layout ch = lay(8, 2, 5, 4, 12);
    CHECK(pc_seam_project(MIS, &ch, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_seam_discrepancy(F, &ok, F2, nullptr, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_seam_discrepancy(F, &ch, nullptr, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_seam_discrepancy(F, &ch, F2, MIS, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_seam_mean_abs(F, &ok, F2, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_seam_mean_abs(F, &ch, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_mds_recover(F, -1, F2, nullptr, 0, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_mds_recover(F, kMaxMaps + 1, F2, nullptr, 0, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_mds_recover(F, 10, F2, nullptr, 257, nullptr) == PC_ERR_PARAM);
    CHECK(pc_mds_recover(F, 10, F2, nullptr, -3, nullptr) == PC_ERR_PARAM);
    CHECK(pc_mds_recover(nullptr, 10, F2, nullptr, 0, nullptr) == PC_ERR_NULL);
    CHECK(pc_mds_recover(F, 10, F2, MIS, 0, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_mds_recover(nullptr, 0, nullptr, nullptr, 0, nullptr) == PC_OK);  // empty batch: a no-op
    CHECK(pc_kabsch_stitch(F, &ok, F2, F2, nullptr) == PC_ERR_SHAPE);
    const pc_layout long_chain = lay(2048, 1, 1, 2048, 12);
    CHECK(pc_kabsch_stitch(F, &long_chain, F2, F2, nullptr) == PC_ERR_SHAPE);
    const pc_layout coplanar = lay(4, 1, 1, 4, 3);
    CHECK(pc_kabsch_stitch(F, &coplanar, F2, F2, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_kabsch_stitch(F, &ch, nullptr, F2, nullptr) == PC_ERR_NULL);
    CHECK(pc_kabsch_stitch_proper(F, &ok, F2, F2, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_kabsch_stitch_proper(F, &long_chain, F2, F2, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_kabsch_stitch_proper(F, &coplanar, F2, F2, nullptr) == PC_ERR_SHAPE);
    CHECK(pc_kabsch_stitch_proper(F, &ch, F2, nullptr, nullptr) == PC_ERR_NULL);
    CHECK(pc_kabsch_stitch_proper(F, &ch, F2, MIS, nullptr) == PC_ERR_ALIGN);
    CHECK(pc_set_max_dispatch_items(1023) == PC_ERR_PARAM);
    CHECK(pc_set_max_dispatch_items(kCap + 1) == PC_ERR_PARAM);
    CHECK(pc_seam_index_map(nullptr, 12) == PC_ERR_NULL);
    int32_t idx[2 * 496];
    CHECK(pc_seam_index_map(idx, 1) == PC_ERR_PARAM);
    CHECK(pc_seam_index_map(idx, 33) == PC_ERR_PARAM);
    uint32_t out4[4], ctr[4] = {0, 0, 0, 0};
    CHECK(pc_philox_block(nullptr, ctr, 0) == PC_ERR_NULL);
    CHECK(pc_philox_block(out4, nullptr, 0) == PC_ERR_NULL);
    // the whole chain is validated before anything is enqueued
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 7, 1000, 1e-4, 0.02, 1.0, 0, 0, 1, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 50, 1000, 1e-4, 0.02, 1.0, 0, 1, 1, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 50, 1000, 1e-4, 0.02, 9.0, 0, 0, 1, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 50, 1000, 1e-4, 0.02, 1.0, 0, -1, 1, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 0, 1000, 1e-4, 0.02, 1.0, 0, 0, 1, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 50, 1000, 0.0, 0.02, 1.0, 0, 0, 1, nullptr) == PC_ERR_PARAM);
    CHECK(pc_ddim_sample(F, F, F2, W2, &ok, 50, 1000, 1e-4, 0.02, 1.0, 0, 0, 1, nullptr) == PC_OK);
    CHECK(stub::launches.size() == 50);  // only the valid call enqueued anything
}

// ---------------------------------------------------------------------------
// Launch geometry of every entry point, at a given cap.
void geometry(const pc_layout &L, uint64_t cap) {
    const int64_t R = L.n_regions, G = L.n_guidance, S = L.n_traj, n = R * G * S;
    const bool chains = L.chain_len > 1;
    const float *w = G == 2 ? W2 : W16;
    CHECK(pc_set_max_dispatch_items(cap == kCap ? 0 : cap) == PC_OK);

    stub::reset();
    CHECK(pc_init_state(F, &L, 5, nullptr) == PC_OK);
    EXPECT_GRIDS("k_fill", ceil_div(n, 4), 512, 1, cap);

    stub::reset();
    CHECK(pc_ddim_cfg_step(F, F, F2, w, &L, 0.3, 0.5, 1.0, 1, 2, 0, nullptr, nullptr) == PC_OK);
    EXPECT_GRIDS("k_step_indep", R * G * ceil_div(S, 2), 512, 1, cap);

    stub::reset();
    CHECK(pc_ddim_cfg_step_eps(F, F, F2, w, &L, 0.3, 0.5, 1.0, 1, 2, 0, nullptr, nullptr) == PC_OK);
    EXPECT_GRIDS("k_step_indep", R * G * S, 512, 1, cap);

    stub::reset();
    CHECK(pc_mds_recover(F, n, F2, F2, 0, nullptr) == PC_OK);
    // two maps per wavefront, persistent grid of at most 2048 wavefronts
    EXPECT_GRIDS("k_mds", ceil_div(n, 2) < 2048 ? ceil_div(n, 2) : 2048, 64, 1, cap);
    if (!chains) return;

    const int64_t n_chains = R / L.chain_len, n_seams = n_chains * (L.chain_len - 1);
    const int64_t NP = L.overlap * (L.overlap - 1) / 2;
    stub::reset();
    CHECK(pc_ddim_cfg_step(F, F, F2, w, &L, 0.3, 0.5, 1.0, 1, 2, 1, F2, nullptr) == PC_OK);
    EXPECT_GRIDS("k_step_chain", R * G * ceil_div(S, 8), 512, 1, cap);  // with the discrepancy: 8 maps each
    stub::reset();
    CHECK(pc_ddim_cfg_step(F, F, F2, w, &L, 0.3, 0.5, 1.0, 1, 2, 1, nullptr, nullptr) == PC_OK);
    EXPECT_GRIDS("k_step_chain", R * G * ceil_div(S, 6), 512, 1, cap);

    stub::reset();
    CHECK(pc_ddim_cfg_step_eps(F, F, F2, w, &L, 0.3, 0.5, 1.0, 1, 2, 1, nullptr, nullptr) == PC_OK);
    EXPECT_GRIDS("k_step_chain", R * G * ceil_div(S, 6), 512, 1, cap);

    stub::reset();
    CHECK(pc_seam_project(F, &L, nullptr) == PC_OK);
    EXPECT_GRIDS("k_seam_project", ceil_div(n_seams * G * S * NP, 256), 256, 1, cap);

    stub::reset();
    CHECK(pc_seam_discrepancy(F, &L, F2, F, nullptr) == PC_OK);
    EXPECT_GRIDS("k_seam_disc", ceil_div(n_seams * G * S, 4), 256, 1, cap);
    EXPECT_GRIDS("k_mean_max", 1, 1024, 1, cap);

    stub::reset();
    CHECK(pc_seam_mean_abs(F, &L, F2, nullptr) == PC_OK);
    EXPECT_GRIDS("k_seam_mean_abs", n_seams * G, 1024, 1, cap);

    if (L.overlap >= 4 && L.chain_len <= 1024) {
        stub::reset();
        CHECK(pc_kabsch_stitch(F, &L, F2, F, nullptr) == PC_OK);
        EXPECT_GRIDS("k_stitch", n_chains * G * S, 256, 1, cap);
        for (const auto &l : stub::launches) CHECK(l.kernel.find("k_stitchILb0E") != std::string::npos);
        stub::reset();
        CHECK(pc_kabsch_stitch_proper(F, &L, F2, F, nullptr) == PC_OK);
        EXPECT_GRIDS("k_stitch", n_chains * G * S, 256, 1, cap);
        for (const auto &l : stub::launches) CHECK(l.kernel.find("k_stitchILb1E") != std::string::npos);
    }
}

void launches() {
    // workload shapes, small caps (several slices each) and the hardware cap
    const pc_layout shapes[] = {lay(1, 2, 8), lay(1, 2, 1000), lay(2658, 2, 100), lay(32, 2, 256, 32, 12),
                                lay(32, 1, 1000, 32, 12), lay(14, 2, 5, 7, 12), lay(6, 2, 5, 3, 32),
                                lay(10, 2, 5, 5, 2), lay(3, 16, 7)};
    const uint64_t caps[] = {kCap, 1024, 3 * 512, 4096 + 64, 1 << 20};
    for (const auto &L : shapes)
        for (uint64_t cap : caps) geometry(L, cap);

    // the largest layouts the boundary accepts, at the hardware cap
    geometry(lay(0x7FFFFFFF, 1, 1), kCap);                    // 2^31 - 1 maps, one per region
    geometry(lay(1 << 14, 2, (1 << 16) - 1), kCap);           // 2^31 - 2^15 maps
    geometry(lay(65536, 2, 128), kCap);                       // 2^24 maps: just past one step dispatch
    geometry(lay(1 << 30, 1, 1, 2, 32), kCap);                // 2^29 seams, 496 pairs each
    geometry(lay(1 << 20, 16, 127, 2, 12), kCap);             // 2,130,706,432 maps in two-tile chains
    geometry(lay(1023 * 2048, 1, 1024, 1023, 12), kCap);      // 2048 chains of 1023 tiles
    CHECK(pc_set_max_dispatch_items(0) == PC_OK);

    // one dispatch of the independent step holds 16,777,214 maps; one more map needs two
    stub::reset();
    pc_layout L = lay(1, 1, 16777214);
    CHECK(step(F, L, 0.3, 0.5, 1.0, 0, nullptr) == PC_OK);
    CHECK(stub::launches.size() == 1);
    stub::reset();
    L = lay(1, 1, 16777215);
    CHECK(step(F, L, 0.3, 0.5, 1.0, 0, nullptr) == PC_OK);
    CHECK(stub::launches.size() == 2 && stub::launches[1].block0 == 8388607 && stub::launches[1].grid == 1);

    // the whole chain: one grid per step (and the x_T fill where the first step cannot draw it)
    stub::reset();
    L = lay(4, 2, 9, 2, 12);
    CHECK(pc_set_max_dispatch_items(2048) == PC_OK);
    CHECK(pc_ddim_sample(F, F, F2, W2, &L, 250, 1000, 1e-4, 0.02, 1.0, 3, 5, 1, nullptr) == PC_OK);
    const auto chain_grids = grids("k_step_chain", 2048);
    const auto indep_grids = grids("k_step_indep", 2048);
    CHECK(chain_grids.size() == 50 && indep_grids.size() == 200);  // projection after every 5th step
    for (const auto &g : chain_grids) CHECK(g.blocks == 4 * 2 * 2 && g.contiguous && g.within_cap && g.slices == 4);
    for (const auto &g : indep_grids) CHECK(g.blocks == 4 * 2 * 5 && g.contiguous && g.within_cap);
    CHECK(grids("k_fill", 2048).empty());
    CHECK(pc_set_max_dispatch_items(0) == PC_OK);
}

void errors() {
    // a failing launch returns PC_ERR_HIP and no further slice is enqueued
    CHECK(pc_set_max_dispatch_items(1024) == PC_OK);
    pc_layout L = lay(1, 2, 40);
    stub::reset();
    stub::fail_on_call = 1;
    CHECK(step(F, L, 0.3, 0.5, 1.0, 0, nullptr) == PC_ERR_HIP);
    CHECK(stub::launches.size() == 1);
    CHECK(strstr(pc_last_error(), "injected") != nullptr);
    stub::reset();
    stub::fail_on_call = 3;
    CHECK(pc_mds_recover(F, 1000, F2, nullptr, 0, nullptr) == PC_ERR_HIP);  // 500 wavefronts, 16 per slice
    CHECK(stub::launches.size() == 3);
    stub::reset();
    stub::fail_on_call = 4;  // the fourth slice of the first step
    CHECK(pc_ddim_sample(F, F, F2, W2, &L, 50, 1000, 1e-4, 0.02, 1.0, 0, 0, 1, nullptr) == PC_ERR_HIP);
    CHECK(stub::launches.size() == 4);
    stub::reset();
    L = lay(4, 2, 10, 2, 12);
    stub::fail_on_call = 1;  // the discrepancy's first slice
    CHECK(pc_seam_discrepancy(F, &L, F2, F, nullptr) == PC_ERR_HIP);
    CHECK(stub::launches.size() == 1);
    CHECK(pc_set_max_dispatch_items(0) == PC_OK);
    stub::reset();
    CHECK(step(F, L, 0.3, 0.5, 1.0, 1, nullptr) == PC_OK);
    CHECK(strlen(pc_last_error()) == 0);  // a success clears the message
}

void host_helpers() {
    static double a[100000], b[100000];
    const int ns[] = {1, 2, 50, 250, 500, 1000};
    for (int n : ns) {
        CHECK(pc_ddim_schedule(n, 1000, 1e-4, 0.02, a, b) == PC_OK);
        for (int i = 0; i < n; ++i) CHECK(a[i] > 0.0 && a[i] < 1.0 && a[i] <= b[i] && b[i] <= 1.0);
        CHECK(b[n - 1] == 1.0);
        CHECK(pc_ddim_schedule_cosine(n, 1000, 0.008, 0.999, a, b) == PC_OK);
        for (int i = 0; i < n; ++i) CHECK(a[i] > 0.0 && a[i] < 1.0 && a[i] <= b[i] && b[i] <= 1.0);
    }
    CHECK(pc_ddim_schedule(100000, 100000, 1e-6, 1e-4, a, b) == PC_OK);
    CHECK(pc_ddim_schedule(3, 1000, 1e-4, 0.02, a, b) == PC_ERR_PARAM);
    CHECK(pc_ddim_schedule(50, 1, 1e-4, 0.02, a, b) == PC_ERR_PARAM);
    CHECK(pc_ddim_schedule(50, 1000, 1e-4, 1.0, a, b) == PC_ERR_PARAM);
    CHECK(pc_ddim_schedule(50, 1000, 1e-4, 0.02, nullptr, b) == PC_ERR_NULL);
    CHECK(pc_ddim_schedule_cosine(50, 1000, -0.1, 0.999, a, b) == PC_ERR_PARAM);
    CHECK(pc_ddim_schedule_cosine(50, 1000, 0.008, 1.0, a, b) == PC_ERR_PARAM);
    int32_t idx[2 * 496];
    for (int o = 2; o <= 32; ++o) {
        CHECK(pc_seam_index_map(idx, o) == PC_OK);
        const int np = o * (o - 1) / 2;
        for (int k = 0; k < np; ++k) CHECK(idx[2 * k] >= 0 && idx[2 * k] < 2016 && idx[2 * k + 1] >= 0 &&
                                           idx[2 * k + 1] < 2016);
        CHECK(idx[2 * (np - 1)] == 2015);  // the last pair of the right seam block is the map's last entry
    }
    uint32_t out[4], ctr[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    CHECK(pc_philox_block(out, ctr, ~0ull) == PC_OK);
    for (int s = -6; s <= 1; ++s) CHECK(strlen(pc_status_string(s)) > 0);
    CHECK(strstr(pc_version(), "gfx950") != nullptr);
}

}  // namespace

int main() {
    slice_plan();
    validation();
    launches();
    errors();
    host_helpers();
    if (g_fails) {
        fprintf(stderr, "%d check(s) failed\n", g_fails);
        return 1;
    }
    printf("host checks passed\n");
    return 0;
}
