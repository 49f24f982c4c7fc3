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

}  // namespace pc
