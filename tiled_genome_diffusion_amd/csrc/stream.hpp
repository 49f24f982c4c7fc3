// Shared pieces of the step kernels: the thread mapping, state streaming
// (cached or non-temporal float4 loads and stores) and the four-element
// guided DDIM update.
//
// Thread mapping: a workgroup has 512 lanes; lane q < 504 owns float4 quad q
// (packed elements 4q .. 4q+3) of every map the workgroup visits, so a
// wavefront streams 1 KB of contiguous state per map.  Because q is fixed
// per lane, the lane's reference values and the q-dependent part of its
// Philox counter stay in registers across maps.
#pragma once

#include "common.hpp"

namespace pc {

constexpr int kThreads = 512;
// States well beyond the 256 MB Infinity Cache are streamed with
// non-temporal loads and stores: each value is touched once per step, so
// caching it only evicts the references.  Smaller states stay cacheable, so
// consecutive steps can hit in the Infinity Cache (measured: a 258 MB chain
// state steps 8% faster cached than streamed).
constexpr size_t kStreamBytes = size_t(512) << 20;

// Independent-map step: maps of one (region, weight) per workgroup, and the
// chunks of consecutive workgroups dealt to the XCDs in turn
// (xcd_remap_chunked).  Measured on MI355X over the 531,600-map slab: 1.38 ms
// per step against 1.43 ms with one contiguous range per XCD (chunks of 40,
// 60, 90, 100 and 125 workgroups: 1.40-1.43 ms).
constexpr int kIndepMaps = 2;
constexpr uint32_t kIndepChunk = 75;

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

// Step four elements.  EPS: (dc, du) are the network's conditional and
// unconditional noise predictions; otherwise they are the reference maps of
// the point-mass stand-in.
template <bool EPS>
__device__ __forceinline__ float4 step4(float4 x, float4 dc, float4 du, float w, const StepCoef &c, float4 z) {
    float4 y;
    if (EPS) {
        y.x = ddim_guided_update(x.x, dc.x, du.x, w, c, z.x);
        y.y = ddim_guided_update(x.y, dc.y, du.y, w, c, z.y);
        y.z = ddim_guided_update(x.z, dc.z, du.z, w, c, z.z);
        y.w = ddim_guided_update(x.w, dc.w, du.w, w, c, z.w);
    } else {
        y.x = ddim_cfg_element(x.x, dc.x, du.x, w, c, z.x);
        y.y = ddim_cfg_element(x.y, dc.y, du.y, w, c, z.y);
        y.z = ddim_cfg_element(x.z, dc.z, du.z, w, c, z.z);
        y.w = ddim_cfg_element(x.w, dc.w, du.w, w, c, z.w);
    }
    return y;
}

// Steps quad q of maps map0 .. map0 + U - 1 (trajectory ids t0 ..), U loads
// in flight before any is computed.  EPS: the noise predictions of each map
// are read from eps_c / eps_u (same layout as the state) instead of being
// formed from the region's references xc / xu.  With a.init (the first step
// of a run, wave-uniform) x_T is drawn from Philox slot 0 instead of read.
template <int U, bool NOISE, bool NT, bool EPS>
__device__ __forceinline__ void step_maps(float *__restrict__ state, const float *__restrict__ eps_c,
                                          const float *__restrict__ eps_u, size_t map0, uint32_t t0, uint32_t q,
                                          float4 xc, float4 xu, float w, const StepArgs &a) {
    float4 x[U], ec[U], eu[U];
    if (a.init) {  // first step of a run: x_T is drawn here, not read (wave-uniform)
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = philox_normals(q, t0 + u, 0u, a.k0, a.k1);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = ld_state<NT>(state, (map0 + u) * kQuads + q);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (EPS) {
            ec[u] = ld_state<NT>(eps_c, (map0 + u) * kQuads + q);
            eu[u] = ld_state<NT>(eps_u, (map0 + u) * kQuads + q);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float4 z = NOISE ? philox_normals(q, t0 + u, a.slot, a.k0, a.k1) : make_float4(0.f, 0.f, 0.f, 0.f);
        st_state<NT>(state, (map0 + u) * kQuads + q,
                     EPS ? step4<true>(x[u], ec[u], eu[u], w, a.c, z) : step4<false>(x[u], xc, xu, w, a.c, z));
    }
}

}  // namespace pc
