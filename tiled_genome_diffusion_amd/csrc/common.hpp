// Shared definitions of the gfx950 kernels: map layout, Philox4x32-10,
// Box-Muller, and the workgroup -> XCD remapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pc {

constexpr int kBeads = 64;
constexpr int kPacked = 2016;           // 64 * 63 / 2 distances per map
constexpr int kQuads = kPacked / 4;     // 504 float4 per map; one Philox block each
constexpr int kMaxGuidance = 16;
constexpr int kMaxOverlap = 32;
constexpr int kMaxPairs = kMaxOverlap * (kMaxOverlap - 1) / 2;

// Packed index of bead pair (i, j), i < j: rows of the strict upper triangle.
__host__ __device__ constexpr int packed_index(int i, int j) {
    return i * (2 * kBeads - i - 1) / 2 + (j - i - 1);
}

// Row and column of packed element e (inverse of packed_index).  Row i starts
// at i (2n - i - 1) / 2, so i is the floor of the smaller root of that
// quadratic; a float estimate (the hardware square root, within a few ulp of
// a root below 128) is corrected by at most one step each way.
__device__ inline void packed_row_col(int e, int &i, int &j) {
    constexpr int b = 2 * kBeads - 1;
    int r = static_cast<int>((b - __builtin_amdgcn_sqrtf(static_cast<float>(b * b - 8 * e))) * 0.5f);
    r = r < 0 ? 0 : (r > kBeads - 2 ? kBeads - 2 : r);
    if (r < kBeads - 2 && packed_index(r + 1, r + 2) <= e) ++r;
    if (r > 0 && packed_index(r, r + 1) > e) --r;
    i = r;
    j = e - packed_index(r, r + 1) + r + 1;
}

// Inverse of block_pair_index: pair p of an O-bead block -> (pp, qq).
__host__ __device__ inline void block_pair_row_col(int p, int O, int &pp, int &qq) {
    const int b = 2 * O - 1;
    int r = static_cast<int>((b - sqrtf(static_cast<float>(b * b - 8 * p))) * 0.5f);
    r = r < 0 ? 0 : (r > O - 2 ? O - 2 : r);
    if (r < O - 2 && (r + 1) * (2 * O - r - 2) / 2 <= p) ++r;
    if (r > 0 && r * (2 * O - r - 1) / 2 > p) --r;
    pp = r;
    qq = p - r * (2 * O - r - 1) / 2 + r + 1;
}

// Index of pair (p, q), p < q, among the O(O-1)/2 pairs of an O-bead block.
__host__ __device__ constexpr int block_pair_index(int p, int q, int O) {
    return p * (2 * O - p - 1) / 2 + (q - p - 1);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  One round maps counter
// (c0, c1, c2, c3) with key (k0, k1) to
//   (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
// the key advances by the Weyl constants between rounds.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct Words4 {
    uint32_t v0, v1, v2, v3;
};

// Three-way XOR: one v_bitop3_b32 (truth table 0x96) on gfx950.
__host__ __device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
    return a ^ b ^ c;
#endif
}

__host__ __device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                        uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c0;
        const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c2;
        const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k1);
        c1 = static_cast<uint32_t>(p1);
        c3 = static_cast<uint32_t>(p0);
        c0 = n0;
        c2 = n2;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
    return Words4{c0, c1, c2, c3};
}

// Box-Muller (1958) on 24-bit uniforms u1 = ((ra >> 8) + 1) 2^-24 in (0, 1] and
// u2 = (rb >> 8) 2^-24 in [0, 1), both exact in float32:
//   zc = sqrt(-2 ln u1) cos(2 pi u2),  zs = sqrt(-2 ln u1) sin(2 pi u2).
// gfx950's transcendental unit evaluates it directly: v_log_f32 gives log2
// (-2 ln u1 = -2 ln 2 log2 u1), and v_sin_f32 / v_cos_f32 take their argument
// in revolutions, so 2 pi u2 needs no range reduction.  Measured over all
// 2^24 inputs: |sin, cos error| <= 1.3e-7 and radius relative error
// <= 1.4e-7, so |z error| <= 1.6e-6 for |z| <= sqrt(48 ln 2).
__device__ __forceinline__ void box_muller(uint32_t ra, uint32_t rb, float &zc, float &zs) {
    const float u1 = static_cast<float>((ra >> 8) + 1u) * 0x1p-24f;
    const float u2 = static_cast<float>(rb >> 8) * 0x1p-24f;
    const float rad = __builtin_amdgcn_sqrtf(-1.38629436111989061f * __builtin_amdgcn_logf(u1));
    zc = rad * __builtin_amdgcn_cosf(u2);
    zs = rad * __builtin_amdgcn_sinf(u2);
}

// Four standard normals of packed elements 4q .. 4q+3 of trajectory t.
__device__ __forceinline__ float4 philox_normals(uint32_t q, uint32_t t, uint32_t slot, uint32_t k0, uint32_t k1) {
    const Words4 r = philox4x32_10(q, t, slot, 0u, k0, k1);
    float4 z;
    box_muller(r.v0, r.v1, z.x, z.y);
    box_muller(r.v2, r.v3, z.z, z.w);
    return z;
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  This bijection gives each XCD a contiguous range of logical
// workgroup ids, so neighbouring logical work (the same region's references)
// shares one XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t n) {
    constexpr uint32_t kXcd = 8;
    const uint32_t per = n / kXcd, rem = n % kXcd;
    const uint32_t x = b % kXcd, i = b / kXcd;
    return x * per + (x < rem ? x : rem) + i;
}

// Chunked variant: XCD x works through chunks x, x + 8, x + 16, ... of C
// consecutive logical workgroups, so the eight XCDs stream neighbouring
// address ranges at any moment.  Workgroups past the last whole round of
// 8 C keep their order.  A bijection on [0, n).
__device__ __forceinline__ uint32_t xcd_remap_chunked(uint32_t b, uint32_t n, uint32_t C) {
    constexpr uint32_t kXcd = 8;
    const uint32_t full = n / (kXcd * C) * (kXcd * C);
    if (b >= full) return b;
    const uint32_t x = b % kXcd, i = b / kXcd;
    return ((i / C) * kXcd + x) * C + i % C;
}

// Wavefront sum by DPP: quad permutes, then the half-row and row mirrors
// leave every lane of a 16-lane row holding the row total (each step adds a
// value to its mirror image, so the lanes of a row round identically); row
// broadcasts 15 and 31 fold the four rows into lane 63, which is read back
// as a wave-uniform value.  Six full-rate DPP adds and one readlane, in a
// fixed order.  Only lane 63 is read, so the broadcasts run on every row
// (rows 0-2 end with partial sums nobody reads): with full row masks each
// folds into a single v_add_f32_dpp.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);         // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);         // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);        // row_half_mirror
    v += dpp<0x140>(v);        // row_mirror
    v += dpp<0x142>(v);        // row_bcast:15: row r += row r - 1 (rows 1 and 3 matter)
    v += dpp<0x143>(v);        // row_bcast:31: rows 2 and 3 += row 1
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// N independent wavefront sums, stage by stage: each value takes exactly the
// steps of wave_sum (same bits), and the DPP adds of different values fill
// each other's wait states instead of leaving one dependent chain to stall.
template <int N>
__device__ __forceinline__ void wave_sums(float (&v)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0xB1>(v[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x4E>(v[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x141>(v[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x140>(v[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x142>(v[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x143>(v[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[n]), 63));
}

// Coefficients of one guided DDIM step, rounded to float32 from float64 on
// the host.  With a = abar_t, a' = abar_next:
struct StepCoef {
    float sa;       // sqrt(a)
    float inv_s1a;  // 1 / sqrt(1 - a)
    float s1a;      // sqrt(1 - a)
    float inv_sa;   // 1 / sqrt(a)
    float sap;      // sqrt(a')
    float cdir;     // sqrt(max(0, 1 - a' - sigma^2))
    float sigma;    // eta sqrt((1 - a') / (1 - a)) sqrt(1 - a / a')
};

struct StepArgs {
    StepCoef c;
    float w[kMaxGuidance];
    int32_t R, G, S;
    int32_t maps_per_block;   // independent layout: maps of one (r, g) per workgroup
    int32_t blocks_per_rg;
    uint32_t k0, k1, slot;    // Philox key words and step slot
    uint32_t init;            // 1: the state holds no x_T yet; draw it from slot 0 instead of reading it
                              // (independent-map kernel only)
};

struct ChainArgs {
    int32_t chain_len;
    int32_t overlap;
    int32_t n_pairs;          // overlap (overlap - 1) / 2
};

// Guidance combine + DDIM update of one element from its two noise
// predictions.  Every rounding is spelled out (explicit fmaf, and the library
// is built with -ffp-contract=off), so every kernel that steps an element
// produces the same bits.
__device__ __forceinline__ float ddim_guided_update(float x, float eps_c, float eps_u, float w, const StepCoef &c,
                                                   float z) {
    const float eps = fmaf(w, eps_c - eps_u, eps_u);       // classifier-free guidance
    const float x0_hat = fmaf(-c.s1a, eps, x) * c.inv_sa;  // predicted clean map
    return fmaf(c.sigma, z, fmaf(c.cdir, eps, c.sap * x0_hat));
}

// The same with the point-mass stand-in denoiser: the noise predictions are
// (x - sqrt(a) x0) / sqrt(1 - a) for the conditional and unconditional
// reference maps.
__device__ __forceinline__ float ddim_cfg_element(float x, float x0c, float x0u, float w, const StepCoef &c, float z) {
    const float eps_c = fmaf(-c.sa, x0c, x) * c.inv_s1a;
    const float eps_u = fmaf(-c.sa, x0u, x) * c.inv_s1a;
    return ddim_guided_update(x, eps_c, eps_u, w, c, z);
}

}  // namespace pc
