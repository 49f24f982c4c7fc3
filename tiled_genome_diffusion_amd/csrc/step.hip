// Guided DDIM step kernels and the Philox fills.
//
// Thread mapping: a workgroup has 512 lanes; lane q < 504 owns float4 quad q
// (packed elements 4q .. 4q+3) of every map the workgroup visits, so a
// wavefront streams 1 KB of contiguous state per map.  Because q is fixed
// per lane, the lane's reference values and the q-dependent part of its
// Philox counter stay in registers across maps.  Lanes 504..511 only take
// part in barriers.
#include "common.hpp"
#include "launch.hpp"

namespace pc {
namespace {

constexpr int kThreads = 512;
constexpr int kIndepU = 2;           // maps in flight per lane, independent layout
constexpr int kIndepMaps = 2;        // maps of one (region, weight) per workgroup
constexpr int kChainCh = 8;          // tiles per barrier interval, chain layout
// States well beyond the 256 MB Infinity Cache are streamed with
// non-temporal loads and stores: each value is touched once per step, so
// caching it only evicts the references.  Smaller states stay cacheable, so
// consecutive steps can hit in the Infinity Cache (measured: a 258 MB chain
// state steps 8% faster cached than streamed).
constexpr size_t kStreamBytes = size_t(512) << 20;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld4(const float *p, size_t quad) {
    return reinterpret_cast<const float4 *>(p)[quad];
}
__device__ __forceinline__ void st4(float *p, size_t quad, float4 v) {
    reinterpret_cast<float4 *>(p)[quad] = v;
}
template <bool NT>
__device__ __forceinline__ float4 ld_state(const float *p, size_t quad) {
    if (!NT) return ld4(p, quad);
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + quad);
    return make_float4(v.x, v.y, v.z, v.w);
}
template <bool NT>
__device__ __forceinline__ void st_state(float *p, size_t quad, float4 v) {
    if (!NT) return st4(p, quad, v);
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(p) + quad);
}

__device__ __forceinline__ float4 step4(float4 x, float4 xc, float4 xu, float w, const StepCoef &c, float4 z) {
    float4 y;
    y.x = ddim_cfg_element(x.x, xc.x, xu.x, w, c, z.x);
    y.y = ddim_cfg_element(x.y, xc.y, xu.y, w, c, z.y);
    y.z = ddim_cfg_element(x.z, xc.z, xu.z, w, c, z.z);
    y.w = ddim_cfg_element(x.w, xc.w, xu.w, w, c, z.w);
    return y;
}

// ---------------------------------------------------------------------------
// Fills: raw Philox words or normals of one slot for maps [m0, m1) of a
// workgroup.  MODE 0 writes normals (float4), MODE 1 raw words (uint4).
template <int MODE, bool NT>
__global__ __launch_bounds__(kThreads) void k_fill(void *__restrict__ out, int64_t n_maps, int32_t maps_per_block,
                                                   uint32_t k0, uint32_t k1, uint32_t slot) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    const int64_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t m0 = b * maps_per_block;
    const int64_t m1 = m0 + maps_per_block < n_maps ? m0 + maps_per_block : n_maps;
    for (int64_t m = m0; m < m1; ++m) {
        const size_t quad = static_cast<size_t>(m) * kQuads + q;
        if (MODE == 0) {
            st_state<NT>(static_cast<float *>(out), quad, philox_normals(q, static_cast<uint32_t>(m), slot, k0, k1));
        } else {
            const Words4 r = philox4x32_10(q, static_cast<uint32_t>(m), slot, 0u, k0, k1);
            reinterpret_cast<uint4 *>(out)[quad] = make_uint4(r.v0, r.v1, r.v2, r.v3);
        }
    }
}

// ---------------------------------------------------------------------------
// Independent maps: workgroup -> (region r, weight g, chunk of trajectories).
// U maps are loaded before any is computed, to keep U loads in flight.
template <int U, bool NOISE, bool NT>
__device__ __forceinline__ void step_maps(float *__restrict__ state, size_t map0, uint32_t t0, uint32_t q, float4 xc,
                                          float4 xu, float w, const StepArgs &a) {
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = ld_state<NT>(state, (map0 + u) * kQuads + q);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float4 z = NOISE ? philox_normals(q, t0 + u, a.slot, a.k0, a.k1) : make_float4(0.f, 0.f, 0.f, 0.f);
        st_state<NT>(state, (map0 + u) * kQuads + q, step4(x[u], xc, xu, w, a.c, z));
    }
}

template <int U, bool NOISE, bool NT>
__global__ __launch_bounds__(kThreads) void k_step_indep(float *__restrict__ state, const float *__restrict__ x0c,
                                                         const float *__restrict__ x0u, StepArgs a) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int rg = static_cast<int>(b) / a.blocks_per_rg;
    const int chunk = static_cast<int>(b) - rg * a.blocks_per_rg;
    const int r = rg / a.G;
    const int g = rg - r * a.G;
    const float w = a.w[g];
    const float4 xc = ld4(x0c, static_cast<size_t>(r) * kQuads + q);
    const float4 xu = ld4(x0u, static_cast<size_t>(r) * kQuads + q);
    const int s0 = chunk * a.maps_per_block;
    const int s1 = s0 + a.maps_per_block < a.S ? s0 + a.maps_per_block : a.S;
    const uint32_t t_base = static_cast<uint32_t>(rg) * static_cast<uint32_t>(a.S);
    int s = s0;
    for (; s + U <= s1; s += U) step_maps<U, NOISE, NT>(state, t_base + s, t_base + s, q, xc, xu, w, a);
    for (; s < s1; ++s) step_maps<1, NOISE, NT>(state, t_base + s, t_base + s, q, xc, xu, w, a);
}

// ---------------------------------------------------------------------------
// Chains: one workgroup per joint sample (chain c, weight g, trajectory s),
// walking the chain's tiles CH at a time.  Stepped values of seam entries go
// to LDS instead of memory; after a barrier, seam j (tiles j, j+1) is
// resolved from both copies: with PROJECT the float32 mean is written to both
// tiles, otherwise each copy is written back unchanged.  With DISC the RMS of
// (left - right) over the seam's pairs is stored per (seam, g, s), summed in
// pair order by one lane.
template <int CH, bool PROJECT, bool DISC, bool NOISE, bool NT>
__global__ __launch_bounds__(kThreads) void k_step_chain(float *__restrict__ state, const float *__restrict__ x0c,
                                                         const float *__restrict__ x0u, StepArgs a, ChainArgs ch,
                                                         float *__restrict__ pre_disc) {
    __shared__ float s_right[CH + 1][kMaxPairs];  // right-seam copies, slot = tile % (CH + 1)
    __shared__ float s_left[CH + 1][kMaxPairs];   // left-seam copies
    __shared__ int16_t s_lidx[kMaxPairs];         // packed index of pair p in the left tile
    __shared__ int16_t s_ridx[kMaxPairs];         // ... in the right tile

    const uint32_t q = threadIdx.x;
    const bool active = q < kQuads;
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int n_cols = a.G * a.S;
    const int c = static_cast<int>(b) / n_cols;
    const int gs = static_cast<int>(b) - c * n_cols;
    const int g = gs / a.S;
    const float w = a.w[g];
    const int L = ch.chain_len, O = ch.overlap, NP = ch.n_pairs;
    const int off = kBeads - O;

    for (int p = q; p < NP; p += kThreads) {
        int pp = 0;
        while (block_pair_index(pp + 1, pp + 2, O) <= p && pp + 2 < O) ++pp;
        const int qq = p - block_pair_index(pp, pp + 1, O) + pp + 1;
        s_lidx[p] = static_cast<int16_t>(packed_index(off + pp, off + qq));
        s_ridx[p] = static_cast<int16_t>(packed_index(pp, qq));
    }

    // Seam membership of this lane's four elements: pair index or -1.
    int lp[4], rp[4];
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        int i = 0, j = 1;
        if (active) packed_row_col(static_cast<int>(4 * q) + l, i, j);
        lp[l] = (active && j < O) ? block_pair_index(i, j, O) : -1;
        rp[l] = (active && i >= off) ? block_pair_index(i - off, j - off, O) : -1;
    }
    const bool has_left = lp[0] >= 0 || lp[1] >= 0 || lp[2] >= 0 || lp[3] >= 0;
    const bool has_right = rp[0] >= 0 || rp[1] >= 0 || rp[2] >= 0 || rp[3] >= 0;

    // map (tile k) = ((c L + k) G + g) S + s = (c L + k) G S + gs
    const size_t col_map0 = static_cast<size_t>(c) * L * n_cols + gs;
    __syncthreads();

    for (int k0 = 0; k0 < L; k0 += CH) {
        const int nk = L - k0 < CH ? L - k0 : CH;
        if (active) {
            float4 x[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u)
                if (u < nk) x[u] = ld_state<NT>(state, (col_map0 + static_cast<size_t>(k0 + u) * n_cols) * kQuads + q);
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                if (u >= nk) break;
                const int k = k0 + u;
                const int reg = c * L + k;
                const size_t map = col_map0 + static_cast<size_t>(k) * n_cols;
                const float4 xc = ld4(x0c, static_cast<size_t>(reg) * kQuads + q);
                const float4 xu = ld4(x0u, static_cast<size_t>(reg) * kQuads + q);
                const float4 z = NOISE ? philox_normals(q, static_cast<uint32_t>(map), a.slot, a.k0, a.k1)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
                const float4 y = step4(x[u], xc, xu, w, a.c, z);
                const bool lft = has_left && k > 0;
                const bool rgt = has_right && k < L - 1;
                if (!lft && !rgt) {
                    st_state<NT>(state, map * kQuads + q, y);
                } else {
                    const float v[4] = {y.x, y.y, y.z, y.w};
                    const int slot = k % (CH + 1);
                    float *dst = state + map * kPacked + 4 * q;
#pragma unroll
                    for (int l = 0; l < 4; ++l) {
                        const bool in_l = lft && lp[l] >= 0;
                        const bool in_r = rgt && rp[l] >= 0;
                        if (in_l) s_left[slot][lp[l]] = v[l];
                        if (in_r) s_right[slot][rp[l]] = v[l];
                        if (!in_l && !in_r) dst[l] = v[l];
                    }
                }
            }
        }
        __syncthreads();
        // Seams j = jlo .. jhi join tiles j and j+1, both stepped by now.
        const int jlo = k0 > 0 ? k0 - 1 : 0;
        const int jhi = k0 + nk - 2;
        const int n_seams = jhi - jlo + 1;
        if (n_seams > 0) {
            for (int it = q; it < n_seams * NP; it += kThreads) {
                const int j = jlo + it / NP;
                const int p = it - (j - jlo) * NP;
                const float lv = s_right[j % (CH + 1)][p];      // copy in the left tile
                const float rv = s_left[(j + 1) % (CH + 1)][p];  // copy in the right tile
                const size_t map_l = col_map0 + static_cast<size_t>(j) * n_cols;
                const size_t map_r = map_l + n_cols;
                if (PROJECT) {
                    const float m = (lv + rv) * 0.5f;
                    state[map_l * kPacked + s_lidx[p]] = m;
                    state[map_r * kPacked + s_ridx[p]] = m;
                } else {
                    state[map_l * kPacked + s_lidx[p]] = lv;
                    state[map_r * kPacked + s_ridx[p]] = rv;
                }
            }
            if (DISC && static_cast<int>(q) < n_seams) {
                const int j = jlo + static_cast<int>(q);
                const float *lv = s_right[j % (CH + 1)];
                const float *rv = s_left[(j + 1) % (CH + 1)];
                float acc = 0.f;
                for (int p = 0; p < NP; ++p) {
                    const float d = lv[p] - rv[p];
                    acc = fmaf(d, d, acc);
                }
                pre_disc[static_cast<size_t>(c * (L - 1) + j) * n_cols + gs] = sqrtf(acc / static_cast<float>(NP));
            }
        }
        __syncthreads();
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (host).  Shapes and pointers are validated by the C ABI layer.

hipError_t launch_fill(void *out, int64_t n_maps, uint32_t k0, uint32_t k1, uint32_t slot, bool raw,
                       hipStream_t stream) {
    constexpr int kMpb = 4;
    const int64_t blocks = (n_maps + kMpb - 1) / kMpb;
    const dim3 grid(static_cast<uint32_t>(blocks));
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
    if (raw)
        hipLaunchKernelGGL((k_fill<1, false>), grid, dim3(kThreads), 0, stream, out, n_maps, kMpb, k0, k1, slot);
    else if (nt)
        hipLaunchKernelGGL((k_fill<0, true>), grid, dim3(kThreads), 0, stream, out, n_maps, kMpb, k0, k1, slot);
    else
        hipLaunchKernelGGL((k_fill<0, false>), grid, dim3(kThreads), 0, stream, out, n_maps, kMpb, k0, k1, slot);
    return hipGetLastError();
}

hipError_t launch_step_indep(float *state, const float *x0c, const float *x0u, StepArgs a, bool noise,
                             hipStream_t stream) {
    a.maps_per_block = kIndepMaps;
    a.blocks_per_rg = (a.S + a.maps_per_block - 1) / a.maps_per_block;
    const int64_t n_maps = static_cast<int64_t>(a.R) * a.G * a.S;
    const int64_t blocks = static_cast<int64_t>(a.R) * a.G * a.blocks_per_rg;
    const dim3 grid(static_cast<uint32_t>(blocks));
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
#define PC_INDEP(N, T) \
    hipLaunchKernelGGL((k_step_indep<kIndepU, N, T>), grid, dim3(kThreads), 0, stream, state, x0c, x0u, a)
    if (noise) {
        if (nt) PC_INDEP(true, true); else PC_INDEP(true, false);
    } else {
        if (nt) PC_INDEP(false, true); else PC_INDEP(false, false);
    }
#undef PC_INDEP
    return hipGetLastError();
}

hipError_t launch_step_chain(float *state, const float *x0c, const float *x0u, StepArgs a, ChainArgs ch,
                             bool project, float *pre_disc, bool noise, hipStream_t stream) {
    const int64_t n_maps = static_cast<int64_t>(a.R) * a.G * a.S;
    const int64_t blocks = static_cast<int64_t>(a.R / ch.chain_len) * a.G * a.S;
    const dim3 grid(static_cast<uint32_t>(blocks));
    const bool disc = pre_disc != nullptr;
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
#define PC_CHAIN(P, D, N, T)                                                                                    \
    hipLaunchKernelGGL((k_step_chain<kChainCh, P, D, N, T>), grid, dim3(kThreads), 0, stream, state, x0c, x0u, a, \
                       ch, pre_disc)
#define PC_CHAIN_NT(P, D, N) \
    if (nt) PC_CHAIN(P, D, N, true); else PC_CHAIN(P, D, N, false)
    if (project) {
        if (disc) {
            if (noise) PC_CHAIN_NT(true, true, true); else PC_CHAIN_NT(true, true, false);
        } else {
            if (noise) PC_CHAIN_NT(true, false, true); else PC_CHAIN_NT(true, false, false);
        }
    } else {
        if (noise) PC_CHAIN_NT(false, true, true); else PC_CHAIN_NT(false, true, false);
    }
#undef PC_CHAIN_NT
#undef PC_CHAIN
    return hipGetLastError();
}

}  // namespace pc
