// Guided DDIM step over tiled chains with the seam projection fused in.
#include "launch.hpp"
#include "stream.hpp"

namespace pc {
namespace {

constexpr int kChainU = 1;           // maps per lane per barrier, chain layout (measured best on MI355X)
// Maps of one (tile, weight) per workgroup, chain layout: enough to amortise
// the per-workgroup set-up and barriers.  Measured on MI355X with settled
// clocks: 6 is best for both the 16,384-map and the 32,000-map chain (41.8 and
// 76.2 us per step; 8 maps: 41.8 and 78.8; 4: 44 and 80; 10: 44.8 and 80.6).
constexpr int kChainMaps = 6;
// With the pre-projection discrepancy output, 8 (measured: 46.9 and 85.1 us against 48.2 and
// 87.1 with 6; 10 and 12 maps: 50.0 / 84.7 and 49.6 / 84.9).
constexpr int kChainMapsDisc = 8;
// The wavefront that sums the pre-projection discrepancy: the last one, which
// holds the right-seam lines and the idle lanes past the map's 504 quads.
constexpr uint32_t kDiscWave = kThreads / 64 - 1;

// Workgroups are laid out as for independent maps: one workgroup
// steps a.maps_per_block maps of one tile k (region r = c L + k) and weight g.
// Ownership is by 128-byte line (8 quads; a map is 63 lines): a line is a
// "seam line" if it holds any element of the left seam (pairs of beads
// 0..O-1).  Seam k, shared by tiles k and k+1, is resolved entirely by tile
// k's workgroup:
//   * lanes of plain and right-seam lines step tile k's quads; right-seam
//     values (beads 64-O..63) go to LDS;
//   * lanes of seam lines step tile k+1's quads instead (with tile k+1's
//     noise and references) and put its left-seam values in LDS; tile k+1's
//     workgroup skips those lines;
//   * tile 0's seam lines, which no left neighbour covers, are stepped by the
//     seam-line lanes of the chain's last tile, which have no right
//     neighbour to cover (tile 0's left seam is not shared: plain stores);
//   * after one barrier both sides form the float32 mean (left + right) * 0.5
//     (with PROJECT; otherwise each copy keeps its stepped value) and store
//     whole float4 quads.
// Every quad is stepped once, every store is a full float4, no cache line is
// written by two workgroups, and every lane runs exactly one stepping task
// per map.  With DISC the last wavefront sums the squared seam differences,
// pairs strided over its lanes and a fixed DPP tree across them, and stores
// the RMS per (seam, g, s) of its maps after the loop.  LDS is
// double-buffered by iteration parity, so one barrier per iteration
// suffices.  INIT (the projecting first step of a run) draws x_T in
// registers instead of reading a filled state.
template <int U, bool PROJECT, bool DISC, bool NOISE, bool NT, bool EPS, bool INIT = false>
__global__ __launch_bounds__(kThreads) void k_step_chain(float *__restrict__ state, const float *__restrict__ x0c,
                                                         const float *__restrict__ x0u,
                                                         const float *__restrict__ eps_c,
                                                         const float *__restrict__ eps_u, StepArgs a, ChainArgs ch,
                                                         float *__restrict__ pre_disc, int64_t block0) {
    __shared__ float s_right[2][U][kMaxPairs];  // tile k's stepped right-seam values
    __shared__ float s_left[2][U][kMaxPairs];   // tile k+1's stepped left-seam values

    const uint32_t q = threadIdx.x;
    const bool active = q < kQuads;
    const uint32_t b = static_cast<uint32_t>(block0) + xcd_remap(blockIdx.x, gridDim.x);  // logical workgroup
    const int rg = static_cast<int>(b) / a.blocks_per_rg;
    const int chunk = static_cast<int>(b) - rg * a.blocks_per_rg;
    const int r = rg / a.G;
    const int g = rg - r * a.G;
    const float w = a.w[g];
    const int L = ch.chain_len, O = ch.overlap, NP = ch.n_pairs;
    const int c = r / L;
    const int k = r - c * L;
    const int n_cols = a.G * a.S;
    const bool owns_seam = k < L - 1;
    const int off = kBeads - O;

    // Seam membership of this lane's four elements (pair index or -1), and
    // whether its 128-byte line (elements 32 m .. 32 m + 31) holds a
    // left-seam element.  A line spans at most two rows of the map.  Only
    // wavefronts whose 256 elements reach a seam row work it out (rows
    // 0..O-2 hold the left seam, rows 64-O.. the right one): it costs as
    // much VALU as stepping a map, and most wavefronts hold no seam element.
    int lp[4] = {-1, -1, -1, -1}, rp[4] = {-1, -1, -1, -1};
    bool seam_line = false;
    const int wave_e0 = __builtin_amdgcn_readfirstlane(static_cast<int>(q >> 6)) * 256;
    const bool may_left = wave_e0 <= packed_index(O - 2, O - 1);
    const bool may_right = wave_e0 + 255 >= packed_index(off, off + 1);
    if (active && (may_left || may_right)) {
        int i = 0, j = 1;
        packed_row_col(static_cast<int>(4 * q), i, j);
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            if (l > 0 && ++j == kBeads) {  // next element: next column, or the next row's first
                ++i;
                j = i + 1;
            }
            lp[l] = j < O ? block_pair_index(i, j, O) : -1;
            rp[l] = i >= off ? block_pair_index(i - off, j - off, O) : -1;
        }
        const int e0 = static_cast<int>(q / 8) * 32, e1 = e0 + 31;
        int i0, j0, i1, j1;
        packed_row_col(e0, i0, j0);
        packed_row_col(e1, i1, j1);
        // row i0 from column j0 on, row i1 up to column j1: left-seam columns are < O
        seam_line = (i0 <= O - 2 && j0 < O) || (i1 <= O - 2 && i1 > i0);
    }
    const bool right_quad = rp[0] >= 0 || rp[1] >= 0 || rp[2] >= 0 || rp[3] >= 0;
    const bool left_quad = lp[0] >= 0 || lp[1] >= 0 || lp[2] >= 0 || lp[3] >= 0;
    // The lane's one task: tile k's quad (plain and right-seam lines), tile
    // k+1's (seam lines, k < L-1) or tile 0's (seam lines of the last tile).
    const bool own = active && !seam_line;
    const bool halo = active && seam_line && owns_seam;
    const int dt = own ? 0 : (owns_seam ? 1 : -(L - 1));  // tile offset of the task
    const size_t off0 = static_cast<size_t>(static_cast<ptrdiff_t>(dt) * n_cols);  // map offset (wraps for dt < 0)

    float4 rc0 = make_float4(0.f, 0.f, 0.f, 0.f), ru0 = rc0;
    if (active && !EPS) {
        const size_t rr = static_cast<size_t>(r + dt);
        rc0 = ld4(x0c, rr * kQuads + q);
        ru0 = ld4(x0u, rr * kQuads + q);
    }

    const int s0 = chunk * a.maps_per_block;
    const int s1 = s0 + a.maps_per_block < a.S ? s0 + a.maps_per_block : a.S;
    const size_t t_base = static_cast<size_t>(rg) * a.S;
    // DISC: lane j of the last wavefront keeps map s0 + j's discrepancy, stored after the loop (a
    // store inside the loop makes every map wait for the previous map's stores to complete)
    float disc_keep = 0.f;
    int par = 0;
    for (int sb = s0; sb < s1; sb += U, par ^= 1) {
        const int nu = s1 - sb < U ? s1 - sb : U;
        float4 y0[U];
        {
            float4 x0[U], e0c[U], e0u[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u < nu && active) {
                    const size_t m0 = (t_base + sb + u + off0) * kQuads + q;
                    // INIT: first step of a run, x_T drawn here (Philox slot 0) instead of read
                    x0[u] = INIT ? philox_normals(q, static_cast<uint32_t>(t_base + sb + u + off0), 0u, a.k0, a.k1)
                                 : ld_state<NT>(state, m0);
                    if (EPS) {
                        e0c[u] = ld_state<NT>(eps_c, m0);
                        e0u[u] = ld_state<NT>(eps_u, m0);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u >= nu) break;
                if (!active) continue;
                const uint32_t m0 = static_cast<uint32_t>(t_base + sb + u + off0);
                const float4 z = NOISE ? philox_normals(q, m0, a.slot, a.k0, a.k1)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
                y0[u] = EPS ? step4<true>(x0[u], e0c[u], e0u[u], w, a.c, z)
                            : step4<false>(x0[u], rc0, ru0, w, a.c, z);
                // right-seam values of tile k (own lanes)
                if (own && owns_seam && right_quad) {
                    if (rp[0] >= 0) s_right[par][u][rp[0]] = y0[u].x;
                    if (rp[1] >= 0) s_right[par][u][rp[1]] = y0[u].y;
                    if (rp[2] >= 0) s_right[par][u][rp[2]] = y0[u].z;
                    if (rp[3] >= 0) s_right[par][u][rp[3]] = y0[u].w;
                }
                // left-seam values of tile k+1 (halo lanes)
                if (halo && left_quad) {
                    if (lp[0] >= 0) s_left[par][u][lp[0]] = y0[u].x;
                    if (lp[1] >= 0) s_left[par][u][lp[1]] = y0[u].y;
                    if (lp[2] >= 0) s_left[par][u][lp[2]] = y0[u].z;
                    if (lp[3] >= 0) s_left[par][u][lp[3]] = y0[u].w;
                }
            }
        }
        if (owns_seam) __syncthreads();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u >= nu) break;
            const size_t map = t_base + sb + u;
            if (PROJECT && owns_seam) {
                if (own && right_quad) {  // left copy (tile k) + right copy (tile k+1)
                    if (rp[0] >= 0) y0[u].x = (y0[u].x + s_left[par][u][rp[0]]) * 0.5f;
                    if (rp[1] >= 0) y0[u].y = (y0[u].y + s_left[par][u][rp[1]]) * 0.5f;
                    if (rp[2] >= 0) y0[u].z = (y0[u].z + s_left[par][u][rp[2]]) * 0.5f;
                    if (rp[3] >= 0) y0[u].w = (y0[u].w + s_left[par][u][rp[3]]) * 0.5f;
                }
                if (halo && left_quad) {
                    if (lp[0] >= 0) y0[u].x = (s_right[par][u][lp[0]] + y0[u].x) * 0.5f;
                    if (lp[1] >= 0) y0[u].y = (s_right[par][u][lp[1]] + y0[u].y) * 0.5f;
                    if (lp[2] >= 0) y0[u].z = (s_right[par][u][lp[2]] + y0[u].z) * 0.5f;
                    if (lp[3] >= 0) y0[u].w = (s_right[par][u][lp[3]] + y0[u].w) * 0.5f;
                }
            }
            if (active) st_state<NT>(state, (map + off0) * kQuads + q, y0[u]);
            if (DISC && owns_seam && (q >> 6) == kDiscWave) {  // wave-uniform: the last wavefront
                const int lane = static_cast<int>(q & 63);
                float acc = 0.f;
                for (int p = lane; p < NP; p += 64) {
                    const float d = s_right[par][u][p] - s_left[par][u][p];
                    acc = fmaf(d, d, acc);
                }
                const float sum = wave_sum(acc);
                disc_keep = lane == sb + u - s0 ? sqrtf(sum / static_cast<float>(NP)) : disc_keep;
            }
        }
    }
    if (DISC && owns_seam && (q >> 6) == kDiscWave && static_cast<int>(q & 63) < s1 - s0)
        pre_disc[(static_cast<size_t>(c) * (L - 1) + k) * n_cols + static_cast<size_t>(g) * a.S + s0 + (q & 63)] =
            disc_keep;
}

}  // namespace

hipError_t launch_step_chain(float *state, const float *x0c, const float *x0u, const float *eps_c, const float *eps_u,
                             StepArgs a, ChainArgs ch, bool project, float *pre_disc, bool noise, bool init,
                             hipStream_t stream) {
    const int64_t n_maps = static_cast<int64_t>(a.R) * a.G * a.S;
    const bool disc = pre_disc != nullptr;
    a.maps_per_block = disc ? kChainMapsDisc : kChainMaps;
    a.blocks_per_rg = (a.S + a.maps_per_block - 1) / a.maps_per_block;
    const int64_t blocks = static_cast<int64_t>(a.R) * a.G * a.blocks_per_rg;
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
    const bool eps = eps_c != nullptr;
    return launch_slices(blocks, kThreads, [&](int64_t first, uint32_t count) {
        const dim3 grid(count);
#define PC_CHAIN(P, D, N, T, E)                                                                                 \
    hipLaunchKernelGGL((k_step_chain<kChainU, P, D, N, T, E>), grid, dim3(kThreads), 0, stream, state, x0c, x0u, \
                       eps_c, eps_u, a, ch, pre_disc, first)
#define PC_CHAIN_E(P, D, N, T) \
    if (eps) PC_CHAIN(P, D, N, T, true); else PC_CHAIN(P, D, N, T, false)
#define PC_CHAIN_NT(P, D, N) \
    if (nt) PC_CHAIN_E(P, D, N, true); else PC_CHAIN_E(P, D, N, false)
        if (init) {  // the whole-loop entry point's first step: projecting, no discrepancy, references
#define PC_CHAIN_INIT(N, T)                                                                                    \
    hipLaunchKernelGGL((k_step_chain<kChainU, true, false, N, T, false, true>), grid, dim3(kThreads), 0, stream, \
                       state, x0c, x0u, eps_c, eps_u, a, ch, pre_disc, first)
            if (noise) {
                if (nt) PC_CHAIN_INIT(true, true); else PC_CHAIN_INIT(true, false);
            } else {
                if (nt) PC_CHAIN_INIT(false, true); else PC_CHAIN_INIT(false, false);
            }
#undef PC_CHAIN_INIT
        } else if (project) {
            if (disc) {
                if (noise) PC_CHAIN_NT(true, true, true); else PC_CHAIN_NT(true, true, false);
            } else {
                if (noise) PC_CHAIN_NT(true, false, true); else PC_CHAIN_NT(true, false, false);
            }
        } else {
            if (noise) PC_CHAIN_NT(false, true, true); else PC_CHAIN_NT(false, true, false);
        }
#undef PC_CHAIN_NT
#undef PC_CHAIN_E
#undef PC_CHAIN
    });
}

}  // namespace pc
