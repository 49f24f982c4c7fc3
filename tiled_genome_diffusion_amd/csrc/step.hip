// Guided DDIM step over independent maps, and the Philox fills.
#include "launch.hpp"
#include "stream.hpp"

namespace pc {
namespace {

constexpr int kIndepU = 2;           // maps in flight per lane, independent layout
// With noise predictions from buffers there are no references to amortise,
// and one map per workgroup streams fastest (measured on MI355X: 6.17 against
// 5.95 TB/s for two maps).
constexpr int kIndepUEps = 1, kIndepMapsEps = 1;

// ---------------------------------------------------------------------------
// Fills: raw Philox words or normals of one slot for maps [m0, m1) of a
// workgroup.  MODE 0 writes normals (float4), MODE 1 raw words (uint4).
template <int MODE, bool NT>
__global__ __launch_bounds__(kThreads) void k_fill(void *__restrict__ out, int64_t n_maps, int32_t maps_per_block,
                                                   uint32_t k0, uint32_t k1, uint32_t slot, int64_t block0) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    const int64_t b = block0 + xcd_remap(blockIdx.x, gridDim.x);  // logical workgroup (grid slices)
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
// Independent maps: workgroup -> (region r, weight g, chunk of trajectories),
// each lane stepping its quad of the chunk's maps (step_maps, stream.hpp).
template <int U, bool NOISE, bool NT, bool EPS>
__global__ __launch_bounds__(kThreads) void k_step_indep(float *__restrict__ state, const float *__restrict__ x0c,
                                                         const float *__restrict__ x0u,
                                                         const float *__restrict__ eps_c,
                                                         const float *__restrict__ eps_u, StepArgs a,
                                                         int64_t block0) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    // one map per workgroup (noise predictions from buffers) streams fastest with one
    // contiguous range per XCD; two maps per workgroup with chunks dealt in turn.  block0:
    // the slice's first logical workgroup (fewer than 2^31 in all: one or two maps each)
    const uint32_t b = static_cast<uint32_t>(block0) +
                       (EPS ? xcd_remap(blockIdx.x, gridDim.x) : xcd_remap_chunked(blockIdx.x, gridDim.x, kIndepChunk));
    const int rg = static_cast<int>(b) / a.blocks_per_rg;
    const int chunk = static_cast<int>(b) - rg * a.blocks_per_rg;
    const int r = rg / a.G;
    const int g = rg - r * a.G;
    const float w = a.w[g];
    float4 xc = make_float4(0.f, 0.f, 0.f, 0.f), xu = xc;
    if (!EPS) {
        xc = ld4(x0c, static_cast<size_t>(r) * kQuads + q);
        xu = ld4(x0u, static_cast<size_t>(r) * kQuads + q);
    }
    const int s0 = chunk * a.maps_per_block;
    const int s1 = s0 + a.maps_per_block < a.S ? s0 + a.maps_per_block : a.S;
    const uint32_t t_base = static_cast<uint32_t>(rg) * static_cast<uint32_t>(a.S);
    int s = s0;
    for (; s + U <= s1; s += U)
        step_maps<U, NOISE, NT, EPS>(state, eps_c, eps_u, t_base + s, t_base + s, q, xc, xu, w, a);
    for (; s < s1; ++s) step_maps<1, NOISE, NT, EPS>(state, eps_c, eps_u, t_base + s, t_base + s, q, xc, xu, w, a);
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (host).  Shapes and pointers are validated by the C ABI layer.

hipError_t launch_fill(void *out, int64_t n_maps, uint32_t k0, uint32_t k1, uint32_t slot, bool raw,
                       hipStream_t stream) {
    constexpr int kMpb = 4;
    const int64_t blocks = (n_maps + kMpb - 1) / kMpb;
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
    return launch_slices(blocks, kThreads, [&](int64_t first, uint32_t count) {
        const dim3 grid(count);
        if (raw)
            hipLaunchKernelGGL((k_fill<1, false>), grid, dim3(kThreads), 0, stream, out, n_maps, kMpb, k0, k1, slot,
                               first);
        else if (nt)
            hipLaunchKernelGGL((k_fill<0, true>), grid, dim3(kThreads), 0, stream, out, n_maps, kMpb, k0, k1, slot,
                               first);
        else
            hipLaunchKernelGGL((k_fill<0, false>), grid, dim3(kThreads), 0, stream, out, n_maps, kMpb, k0, k1, slot,
                               first);
    });
}

hipError_t launch_step_indep(float *state, const float *x0c, const float *x0u, const float *eps_c, const float *eps_u,
                             StepArgs a, bool noise, hipStream_t stream) {
    const bool eps = eps_c != nullptr;
    a.maps_per_block = eps ? kIndepMapsEps : kIndepMaps;
    a.blocks_per_rg = (a.S + a.maps_per_block - 1) / a.maps_per_block;
    const int64_t n_maps = static_cast<int64_t>(a.R) * a.G * a.S;
    const int64_t blocks = static_cast<int64_t>(a.R) * a.G * a.blocks_per_rg;
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
    return launch_slices(blocks, kThreads, [&](int64_t first, uint32_t count) {
        const dim3 grid(count);
#define PC_INDEP(U, N, T, E)                                                                                    \
    hipLaunchKernelGGL((k_step_indep<U, N, T, E>), grid, dim3(kThreads), 0, stream, state, x0c, x0u, eps_c, eps_u, \
                       a, first)
#define PC_INDEP_E(N, T) \
    if (eps) PC_INDEP(kIndepUEps, N, T, true); else PC_INDEP(kIndepU, N, T, false)
        if (noise) {
            if (nt) PC_INDEP_E(true, true); else PC_INDEP_E(true, false);
        } else {
            if (nt) PC_INDEP_E(false, true); else PC_INDEP_E(false, false);
        }
#undef PC_INDEP_E
#undef PC_INDEP
    });
}

}  // namespace pc
