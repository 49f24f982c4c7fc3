// Bandwidth probes for the benchmark: the state access pattern of the
// independent-map DDIM step with no arithmetic beyond one FMA per element, to
// measure the HBM rate that pattern reaches on the device at hand (the ceiling
// the step kernel is judged against), plus read-only and write-only streams of
// the same size.  Not part of the C ABI of include/pc.h: built into
// libpc_ceiling.so next to libpc.so and loaded only by bench.py.
//
// Pattern (as in k_step_indep): 512-lane workgroups, lane q < 504 owns float4
// quad q of each of the workgroup's kIndepMaps maps, both maps' loads issued
// before either is stored, workgroups dealt to the XCDs in chunks of
// kIndepChunk, non-temporal loads and stores for states above kStreamBytes.
#include "launch.hpp"
#include "stream.hpp"

namespace pc {
namespace {

template <bool NT>
__global__ __launch_bounds__(kThreads) void k_probe_rmw(float *__restrict__ x, int64_t n_maps, float a, float b,
                                                        int64_t block0) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    const int64_t m0 = (block0 + xcd_remap_chunked(blockIdx.x, gridDim.x, kIndepChunk)) * kIndepMaps;
    float4 v[kIndepMaps];
#pragma unroll
    for (int u = 0; u < kIndepMaps; ++u)
        if (m0 + u < n_maps) v[u] = ld_state<NT>(x, static_cast<size_t>(m0 + u) * kQuads + q);
#pragma unroll
    for (int u = 0; u < kIndepMaps; ++u) {
        if (m0 + u >= n_maps) break;
        const float4 y = make_float4(fmaf(a, v[u].x, b), fmaf(a, v[u].y, b), fmaf(a, v[u].z, b), fmaf(a, v[u].w, b));
        st_state<NT>(x, static_cast<size_t>(m0 + u) * kQuads + q, y);
    }
}

// Reads every quad; the sum is stored only if it equals `never` (so the loads
// cannot be dropped).
template <bool NT>
__global__ __launch_bounds__(kThreads) void k_probe_read(const float *__restrict__ x, int64_t n_maps, float never,
                                                         float *__restrict__ sink, int64_t block0) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    const int64_t m0 = (block0 + xcd_remap_chunked(blockIdx.x, gridDim.x, kIndepChunk)) * kIndepMaps;
    float4 v[kIndepMaps];
#pragma unroll
    for (int u = 0; u < kIndepMaps; ++u)
        v[u] = m0 + u < n_maps ? ld_state<NT>(x, static_cast<size_t>(m0 + u) * kQuads + q)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < kIndepMaps; ++u) s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    if (s == never) sink[0] = s;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void k_probe_write(float *__restrict__ x, int64_t n_maps, float value,
                                                          int64_t block0) {
    const uint32_t q = threadIdx.x;
    if (q >= kQuads) return;
    const int64_t m0 = (block0 + xcd_remap_chunked(blockIdx.x, gridDim.x, kIndepChunk)) * kIndepMaps;
    const float4 v = make_float4(value, value, value, value);
#pragma unroll
    for (int u = 0; u < kIndepMaps; ++u)
        if (m0 + u < n_maps) st_state<NT>(x, static_cast<size_t>(m0 + u) * kQuads + q, v);
}

template <class F>
int probe(int64_t n_maps, F &&launch) {
    if (n_maps < 0) return static_cast<int>(hipErrorInvalidValue);
    const int64_t blocks = (n_maps + kIndepMaps - 1) / kIndepMaps;
    const bool nt = static_cast<size_t>(n_maps) * kPacked * 4 > kStreamBytes;
    return static_cast<int>(launch_slices(blocks, kThreads, [&](int64_t first, uint32_t count) {
        launch(nt, dim3(count), first);
    }));
}

}  // namespace

uint64_t dispatch_items() { return kDispatchItemLimit; }

}  // namespace pc

// Each returns a hipError_t value (0 on success).  x: device float [n_maps][2016], 16-byte aligned.
extern "C" {

// x <- a x + b over every element, in place.
__attribute__((visibility("default"))) int pcc_probe_rmw(float *x, int64_t n_maps, float a, float b, void *stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return pc::probe(n_maps, [&](bool nt, dim3 grid, int64_t first) {
        if (nt)
            hipLaunchKernelGGL(pc::k_probe_rmw<true>, grid, dim3(pc::kThreads), 0, s, x, n_maps, a, b, first);
        else
            hipLaunchKernelGGL(pc::k_probe_rmw<false>, grid, dim3(pc::kThreads), 0, s, x, n_maps, a, b, first);
    });
}

// Reads every element; sink (device float [1]) is written only if the sum of a
// lane's elements equals `never`.
__attribute__((visibility("default"))) int pcc_probe_read(const float *x, int64_t n_maps, float never, float *sink,
                                                          void *stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return pc::probe(n_maps, [&](bool nt, dim3 grid, int64_t first) {
        if (nt)
            hipLaunchKernelGGL(pc::k_probe_read<true>, grid, dim3(pc::kThreads), 0, s, x, n_maps, never, sink, first);
        else
            hipLaunchKernelGGL(pc::k_probe_read<false>, grid, dim3(pc::kThreads), 0, s, x, n_maps, never, sink,
                               first);
    });
}

// x <- value everywhere.
__attribute__((visibility("default"))) int pcc_probe_write(float *x, int64_t n_maps, float value, void *stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return pc::probe(n_maps, [&](bool nt, dim3 grid, int64_t first) {
        if (nt)
            hipLaunchKernelGGL(pc::k_probe_write<true>, grid, dim3(pc::kThreads), 0, s, x, n_maps, value, first);
        else
            hipLaunchKernelGGL(pc::k_probe_write<false>, grid, dim3(pc::kThreads), 0, s, x, n_maps, value, first);
    });
}

}  // extern "C"
