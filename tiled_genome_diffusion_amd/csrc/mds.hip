// Batched classical (Torgerson) MDS: two maps per 64-lane wavefront.  Half h
// = lane / 32 of wavefront w works on map 2w + h; lane l = lane % 32 of a half
// owns beads l and l + 32 (rows l and l + 32 of the map's matrices).
//
//   1. The two packed maps (16 KB, contiguous) are copied from HBM straight
//      into LDS (global_load_lds: 16-byte loads that bypass the registers);
//      lane l gathers rows l and l + 32 of A = D o D into 128 VGPRs (two
//      constant-offset LDS reads per entry; for column j only one of the two
//      rows needs a select between the packed row and the packed column).
//   2. B = -1/2 J A J is never formed: for Q orthogonal to the all-ones
//      vector, B Q = -1/2 J (A Q), so each product subtracts the column means
//      of A Q (a half-wave sum per column) instead of centring A.
//   3. Block-4 subspace iteration with Rayleigh-Ritz: Q <- orth(Z) by
//      modified Gram-Schmidt (a column that cancels is projected twice),
//      Z = B Q on the matrix cores (v_mfma_f32_4x4x1f32: lane 4 blk + r
//      supplies q_kr from Q^T in LDS, lane l its own A_lk, so output register
//      r of lane l accumulates (A Q)_lr; two passes cover both rows), H =
//      Q^T Z by half-wave sums, a 4x4 Jacobi eigensolve (values uniform per
//      half, so one instruction stream serves both maps), Ritz vectors V =
//      Q W, Z W = B V and the residuals ||B V_k - theta_k V_k|| of the three
//      largest.  A map stops when each is small against its pair's gap
//      (eigenvector error ~ residual / gap) or after max_iters Rayleigh-Ritz
//      steps in all; a wavefront runs until both of its maps have stopped.
//   4. The iteration finds the eigenvalues of largest magnitude.  If negative
//      ones could hide a positive eigenvalue (the third largest Ritz value is
//      below the smallest magnitude found), the negative Ritz vectors that
//      outrank it are projected out (held in the map's LDS buffer, dead once A
//      is in registers) and that map's iteration restarts on the complement,
//      at most kPasses passes in all, so the largest magnitudes left are the
//      wanted positive eigenvalues.
//   5. X = V_3 diag(sqrt(max(theta, 0))), each column signed so that its
//      largest-magnitude entry is positive (lowest bead on ties), written as
//      soon as the map stops.
// Sums over a map's 64 beads are half-wave sums: DPP adds inside 16-lane
// rows, then rows 0 + 1 and 2 + 3 exchanged by v_permlane16_swap, so every
// lane of a half holds its map's total with identical bits.  The wave-uniform
// work of a one-map-per-wavefront design (the 4x4 eigensolves, the reductions,
// the convergence logic) is shared by two maps here, at two waves per SIMD
// (256 VGPRs) instead of four.
#include "common.hpp"
#include "launch.hpp"
#include "mds_start.hpp"

namespace pc {
namespace {

constexpr int kLanes = 64;
constexpr int kHalf = 32;
constexpr int kBlk = 4;

// Column k of the start block for bead i (orthonormal, orthogonal to the
// all-ones vector; mds_start.hpp).
__device__ __forceinline__ float start_vec(int i, int k) { return kMdsStart[i][k]; }

__device__ __forceinline__ float swap_rows_add(float v) {
    // rows 1 <-> 0 and 3 <-> 2 of the two copies: (r0, r0, r2, r2) + (r1, r1, r3, r3)
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// N independent sums over each half-wave, stage by stage (the DPP adds of
// different values fill each other's wait states).  After the four DPP stages
// every lane of a 16-lane row holds the row total (each stage adds a value to
// its mirror image, so a row's lanes round identically); the swap then adds
// the other row of the half.
template <int N>
__device__ __forceinline__ void half_sums(float (&v)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0xB1>(v[n]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x4E>(v[n]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x141>(v[n]);  // row_half_mirror
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] += dpp<0x140>(v[n]);  // row_mirror
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = swap_rows_add(v[n]);
}

__device__ __forceinline__ float half_sum(float v) {
    float a[1] = {v};
    half_sums(a);
    return a[0];
}

// Largest values over each half-wave of N non-negative values, stage by stage.
template <int N>
__device__ __forceinline__ void half_maxes_nonneg(float (&v)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = fmaxf(v[n], dpp<0xB1>(v[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = fmaxf(v[n], dpp<0x4E>(v[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = fmaxf(v[n], dpp<0x141>(v[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = fmaxf(v[n], dpp<0x140>(v[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[n]), __float_as_uint(v[n]), false, false);
        v[n] = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
}

__device__ __forceinline__ bool any(bool p) { return __ballot(p) != 0; }

// Orders LDS accesses between the lanes of the (one-wavefront) workgroup: the
// LDS executes a wavefront's instructions in issue order, so a write is seen
// by every later read of any lane, and only the compiler must be kept from
// reordering them.  (A workgroup barrier would also wait for the next maps'
// loads into LDS in flight.)
__device__ __forceinline__ void lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Jacobi on the symmetric 4x4 of each half (values uniform within a half),
// in round-robin order: each sweep is three rounds of two rotations on
// disjoint index pairs, (0,1)+(2,3), (0,2)+(1,3), (0,3)+(1,2).  The angles of
// a round come from the same matrix (a rotation leaves the other pair's
// 2x2 block untouched), so the two rotations are independent chains.  The
// rotation that zeroes h_pq uses t = sgn(th) / (|th| + sqrt(th^2 + 1)) with
// th = (h_qq - h_pp) / (2 h_pq) (formed as 2 h_pq sgn(d) / (|d| + sqrt(d^2 +
// 4 h_pq^2)), d = h_qq - h_pp), c = 1 / sqrt(1 + t^2), s = t c.  t needs no
// correct rounding: c and s are formed from it, so the rotation stays
// orthogonal, and the hardware rcp / rsq / sqrt are used.  The eigenvector
// matrix W is spread over lanes: lanes r and 32 + r (r < 4) hold row r of
// their map's W in wl.  A rotation whose h_pq^2 is below `skip2` (1e-15 of
// the squared diagonal norm, under float32 resolution of the largest
// eigenvalue) is carried out as the identity; a round whose four rotations
// (two per map) all skip is left out.
struct Rot {
    float t, c, s, apq;
    bool skip;
};

template <int P, int Q>
__device__ __forceinline__ Rot rotation(const float (&h)[kBlk][kBlk], float skip2) {
    Rot r;
    r.apq = h[P][Q];
    r.skip = r.apq * r.apq <= skip2;
    const float d = h[Q][Q] - h[P][P];
    const float den = fabsf(d) + __builtin_amdgcn_sqrtf(fmaf(d, d, 4.f * r.apq * r.apq));
    const float tr = copysignf(2.f, d) * r.apq * __builtin_amdgcn_rcpf(den);
    r.t = r.skip ? 0.f : tr;
    r.c = r.skip ? 1.f : __builtin_amdgcn_rsqf(fmaf(r.t, r.t, 1.f));
    r.s = r.t * r.c;
    return r;
}

// h <- J^T h J for the rotation J in the (P, Q) plane.
template <int P, int Q>
__device__ __forceinline__ void rotate(float (&h)[kBlk][kBlk], float (&wl)[kBlk], const Rot &r) {
    h[P][P] = fmaf(-r.t, r.apq, h[P][P]);
    h[Q][Q] = fmaf(r.t, r.apq, h[Q][Q]);
    h[P][Q] = h[Q][P] = r.skip ? r.apq : 0.f;
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
        if (k == P || k == Q) continue;
        const float hp = h[k][P], hq = h[k][Q];
        h[k][P] = h[P][k] = fmaf(r.c, hp, -r.s * hq);
        h[k][Q] = h[Q][k] = fmaf(r.s, hp, r.c * hq);
    }
    const float wp = wl[P], wq = wl[Q];
    wl[P] = fmaf(r.c, wp, -r.s * wq);
    wl[Q] = fmaf(r.s, wp, r.c * wq);
}

template <int P1, int Q1, int P2, int Q2>
__device__ __forceinline__ void jacobi_round(float (&h)[kBlk][kBlk], float (&wl)[kBlk], float skip2) {
    const Rot r1 = rotation<P1, Q1>(h, skip2);
    const Rot r2 = rotation<P2, Q2>(h, skip2);
    if (!any(!r1.skip || !r2.skip)) return;
    rotate<P1, Q1>(h, wl, r1);
    rotate<P2, Q2>(h, wl, r2);
}

// On return h is diagonal to float32 precision in both halves and lanes r,
// 32 + r (r < 4) hold row r of their eigenvector matrix (columns are
// eigenvectors) in wl.
__device__ __forceinline__ void jacobi4(float (&h)[kBlk][kBlk], float (&wl)[kBlk], int l) {
#pragma unroll
    for (int c = 0; c < kBlk; ++c) wl[c] = l == c ? 1.f : 0.f;
    for (int sweep = 0; sweep < 8; ++sweep) {
        float off = h[0][1] * h[0][1], dia = h[0][0] * h[0][0];
        off = fmaf(h[0][2], h[0][2], off);
        off = fmaf(h[0][3], h[0][3], off);
        off = fmaf(h[1][2], h[1][2], off);
        off = fmaf(h[1][3], h[1][3], off);
        off = fmaf(h[2][3], h[2][3], off);
        dia = fmaf(h[1][1], h[1][1], dia);
        dia = fmaf(h[2][2], h[2][2], dia);
        dia = fmaf(h[3][3], h[3][3], dia);
        if (!any(off > 1e-14f * dia)) break;
        const float skip2 = 1e-15f * dia;
        jacobi_round<0, 1, 2, 3>(h, wl, skip2);
        jacobi_round<0, 2, 1, 3>(h, wl, skip2);
        jacobi_round<0, 3, 1, 2>(h, wl, skip2);
    }
}

// lo in lanes whose l (lane % 32) is at most j, hi in lanes with l > j, for
// 0 <= j < 31 and all 64 lanes active.  The lane mask is the low half of the
// execution mask shifted by j + 1, copied into both halves (scalar
// operations); inverse_ballot hands it to a single v_cndmask as its condition,
// with no vector compare, and leaves the compiler free to schedule the LDS
// reads around it.  (The mask is not written as a 64-bit constant: hipcc
// encodes such a constant as a 32-bit literal that gfx950 zero-extends, which
// loses the upper 32 lanes.)
__device__ __forceinline__ float select_above(float lo, float hi, int j) {
    const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_read_exec()) << (j + 1);
    const uint64_t above = static_cast<uint64_t>(m) | (static_cast<uint64_t>(m) << 32);
    return __builtin_amdgcn_inverse_ballot_w64(above) ? hi : lo;
}

// Gram-Schmidt of the four columns y (rows l and l + 32 in y0, y1) into q,
// against the all-ones vector first: the products rely on every column of Q
// being orthogonal to it (B q = -1/2 J A q), and a column that cancels to
// rounding noise is not, until projected.  Each column is projected twice
// ("twice is enough": classical Gram-Schmidt with one reorthogonalisation),
// all coefficients of a pass from one batch of sums, so a column costs three
// dependent reductions, not one per previous column.  The second pass
// restores orthogonality to float32 precision even when the column cancels
// almost completely (the fourth column of B Q when B has rank 3).  A column
// that vanishes is replaced by its start vector, projected, and by zero if
// that vanishes too.
template <int K>
__device__ __forceinline__ void project_pass(const float (&q0)[kBlk], const float (&q1)[kBlk], float &v0,
                                             float &v1) {
    float c[K + 1];
    c[K] = v0 + v1;  // against the all-ones vector
#pragma unroll
    for (int m = 0; m < K; ++m) c[m] = fmaf(q0[m], v0, q1[m] * v1);
    half_sums(c);
    const float mean = c[K] * (1.f / kBeads);
    v0 -= mean;
    v1 -= mean;
#pragma unroll
    for (int m = 0; m < K; ++m) {
        v0 = fmaf(-c[m], q0[m], v0);
        v1 = fmaf(-c[m], q1[m], v1);
    }
}

template <int K>
__device__ __forceinline__ void orthonormalise_column(int l, const float (&y0)[kBlk], const float (&y1)[kBlk],
                                                      float (&q0)[kBlk], float (&q1)[kBlk]) {
    float v0 = y0[K], v1 = y1[K];
    project_pass<K>(q0, q1, v0, v1);
    project_pass<K>(q0, q1, v0, v1);
    float n2 = half_sum(fmaf(v0, v0, v1 * v1));
    const bool vanished = !(n2 > 1e-30f);
    if (any(vanished)) {  // rare: start over from the start vector where the column vanished
        float w0 = start_vec(l, K), w1 = start_vec(l + kHalf, K);
        project_pass<K>(q0, q1, w0, w1);
        project_pass<K>(q0, q1, w0, w1);
        const float m2 = half_sum(fmaf(w0, w0, w1 * w1));
        const bool gone = !(m2 > 1e-30f);
        v0 = vanished ? (gone ? 0.f : w0) : v0;
        v1 = vanished ? (gone ? 0.f : w1) : v1;
        n2 = vanished ? (gone ? 1.f : m2) : n2;
    }
    const float s = __builtin_amdgcn_rsqf(n2);
    q0[K] = v0 * s;
    q1[K] = v1 * s;
}

__device__ __forceinline__ void orthonormalise(int l, const float (&y0)[kBlk], const float (&y1)[kBlk],
                                               float (&q0)[kBlk], float (&q1)[kBlk]) {
    orthonormalise_column<0>(l, y0, y1, q0, q1);
    orthonormalise_column<1>(l, y0, y1, q0, q1);
    orthonormalise_column<2>(l, y0, y1, q0, q1);
    orthonormalise_column<3>(l, y0, y1, q0, q1);
}

constexpr int kPasses = 4;                      // iteration passes per map, at most
constexpr int kMaxDefl = (kPasses - 1) * kBlk;  // deflated vectors per map, at most
static_assert(kMaxDefl * kBeads <= kPacked, "deflated vectors are kept in the map's LDS buffer");

// Removes from the columns z their components along the first n (per half)
// deflated vectors of the half's map, one vector after the other; vector d's
// component for bead b is at dfl[d * 64 + b].  nmax bounds n over both halves.
__device__ __forceinline__ void project_out(const float *dfl, int n, int nmax, int l, float (&z0)[kBlk],
                                            float (&z1)[kBlk]) {
    for (int d = 0; d < nmax; ++d) {
        const float v0 = dfl[d * kBeads + l], v1 = dfl[d * kBeads + l + kHalf];
        float c[kBlk];
#pragma unroll
        for (int k = 0; k < kBlk; ++k) c[k] = fmaf(v0, z0[k], v1 * z1[k]);
        half_sums(c);
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            const float ck = d < n ? c[k] : 0.f;
            z0[k] = fmaf(-ck, v0, z0[k]);
            z1[k] = fmaf(-ck, v1, z1[k]);
        }
    }
}

// z = B q for the four columns q of each half's map (rows l and l + 32):
// A q on the matrix cores, minus the stand-in squared on the diagonal
// (g0sq, g1sq), then centred: B q = -1/2 (A q - 1 (mean over beads of A q)).
// 64 rank-1 steps of v_mfma_f32_4x4x1f32 per row set (16 blocks of 4x4):
// block blk multiplies A = (q_k0 .. q_k3) (lane 4 blk + r supplies q_kr of
// its half's map, read from Q^T in LDS) by B = (a_{4 blk + c, k})_c (lane l
// supplies its own row's a_k), so output register r of lane l accumulates
// sum_k q_kr a_lk = (A q)_lr.  Four accumulators per row set take the steps in
// turn, so consecutive steps do not wait on each other.
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void block_matvec(const float (&a0)[kBeads], const float (&a1)[kBeads], float g0sq,
                                             float g1sq, int half, int l, const float (&q0)[kBlk],
                                             const float (&q1)[kBlk], float *s_qt, float (&z0)[kBlk],
                                             float (&z1)[kBlk]) {
    float *my_qt = s_qt + half * (kBlk * kBeads);  // this half's Q^T: column c at my_qt[c * 64 + bead]
#pragma unroll
    for (int c = 0; c < kBlk; ++c) {
        my_qt[c * kBeads + l] = q0[c];
        my_qt[c * kBeads + l + kHalf] = q1[c];
    }
    lds_order();
    const float4 *qa = reinterpret_cast<const float4 *>(my_qt + (l & 3) * kBeads);
    f32x4v acc0[4], acc1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc0[e] = acc1[e] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k4 = 0; k4 < kBeads / 4; ++k4) {
        const float4 a = qa[k4];  // q_{4 k4 + e, l & 3}
        acc0[0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.x, a0[4 * k4 + 0], acc0[0], 0, 0, 0);
        acc1[0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.x, a1[4 * k4 + 0], acc1[0], 0, 0, 0);
        acc0[1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.y, a0[4 * k4 + 1], acc0[1], 0, 0, 0);
        acc1[1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.y, a1[4 * k4 + 1], acc1[1], 0, 0, 0);
        acc0[2] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.z, a0[4 * k4 + 2], acc0[2], 0, 0, 0);
        acc1[2] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.z, a1[4 * k4 + 2], acc1[2], 0, 0, 0);
        acc0[3] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.w, a0[4 * k4 + 3], acc0[3], 0, 0, 0);
        acc1[3] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.w, a1[4 * k4 + 3], acc1[3], 0, 0, 0);
        // keep at most two rows of Q^T in flight (hoisting all 16 LDS reads
        // would overflow the register file)
        if (k4 % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    float m[kBlk];
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
        z0[k] = fmaf(-g0sq, q0[k], (acc0[0][k] + acc0[1][k]) + (acc0[2][k] + acc0[3][k]));
        z1[k] = fmaf(-g1sq, q1[k], (acc1[0][k] + acc1[1][k]) + (acc1[2][k] + acc1[3][k]));
        m[k] = z0[k] + z1[k];
    }
    half_sums(m);
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
        const float mean = m[k] * (1.f / kBeads);
        z0[k] = (z0[k] - mean) * -0.5f;
        z1[k] = (z1[k] - mean) * -0.5f;
    }
    lds_order();  // Q^T is read before the next product rewrites it
}

// True when negative eigenvalues may hide a wanted one: the third largest Ritz
// value is below the smallest Ritz magnitude, so an eigenvalue the iteration
// missed (magnitude <= that smallest one) could outrank it.  Below 1e-6 of the
// largest Ritz value the spectrum is float32 noise and never counts.
__device__ __forceinline__ bool may_hide(const float (&d)[kBlk], float rho) {
    return d[2] < rho && rho > 1e-6f * fabsf(d[0]);
}

// Coordinates of the maps whose iteration has just stopped (`finish`, per
// half): each column of V_3 signed by its largest-magnitude entry (lowest bead
// on ties) and scaled by sqrt(max(theta, 0)).
__device__ __forceinline__ void write_coords(bool finish, bool write, int half, int l, size_t m,
                                             const float (&theta)[kBlk], const float (&v0)[kBlk],
                                             const float (&v1)[kBlk], float *__restrict__ coords,
                                             float *__restrict__ eigvals) {
    float out0[3], out1[3], best[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) best[k] = fmaxf(fabsf(v0[k]), fabsf(v1[k]));
    half_maxes_nonneg(best);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float b0 = fabsf(v0[k]), b1 = fabsf(v1[k]);
        const uint64_t m0 = __ballot(b0 == best[k]), m1 = __ballot(b1 == best[k]);
        // lowest bead of each half holding the largest magnitude: beads 0..31 are row 0 of lanes 0..31
        const uint32_t lo0 = static_cast<uint32_t>(m0), lo1 = static_cast<uint32_t>(m1);
        const uint32_t hi0 = static_cast<uint32_t>(m0 >> 32), hi1 = static_cast<uint32_t>(m1 >> 32);
        const int la = lo0 ? __builtin_ctz(lo0) : __builtin_ctz(lo1 | 0x80000000u);
        const int lb = hi0 ? __builtin_ctz(hi0) : __builtin_ctz(hi1 | 0x80000000u);
        const float sa0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v0[k]), la));
        const float sa1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v1[k]), la));
        const float sb0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v0[k]), kHalf + lb));
        const float sb1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v1[k]), kHalf + lb));
        const float sa = lo0 ? sa0 : sa1, sb = hi0 ? sb0 : sb1;
        const float sv = half ? sb : sa;
        const float scale = __builtin_amdgcn_sqrtf(fmaxf(theta[k], 0.f));
        out0[k] = (sv < 0.f ? -v0[k] : v0[k]) * scale;
        out1[k] = (sv < 0.f ? -v1[k] : v1[k]) * scale;
    }
    if (finish && write) {
        float *dst0 = coords + (m * kBeads + l) * 3;
        float *dst1 = coords + (m * kBeads + l + kHalf) * 3;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            dst0[k] = out0[k];
            dst1[k] = out1[k];
        }
        if (eigvals && l == 0) {
#pragma unroll
            for (int k = 0; k < 3; ++k) eigvals[m * 3 + k] = theta[k];
        }
    }
}

// Copies `quads` float4 of packed maps starting at src into LDS at dst with
// global_load_lds (each instruction writes lane l's 16 bytes at dst + 16 l),
// without passing through registers.  Asynchronous: wait_loads() before the
// first read of dst.
__device__ __forceinline__ void stage(const float *src_maps, float4 *dst, int quads, int lane) {
    typedef __attribute__((address_space(1))) void *gptr;
    typedef __attribute__((address_space(3))) void *lptr;
    const char *src = reinterpret_cast<const char *>(src_maps);  // wave-uniform
    const uint32_t off = static_cast<uint32_t>(lane) * 16u;
    const int full = quads / kLanes, tail = quads % kLanes;
    for (int c = 0; c < full; ++c)
        __builtin_amdgcn_global_load_lds((gptr)(src + c * kLanes * 16 + off), (lptr)(dst + c * kLanes), 16, 0, 0);
    if (lane < tail)
        __builtin_amdgcn_global_load_lds((gptr)(src + full * kLanes * 16 + off), (lptr)(dst + full * kLanes), 16, 0,
                                         0);
}

// The two maps of pair p (maps 2p and 2p + 1, consecutive in memory) into the
// two halves of s_map; with an odd map count the last pair holds map 2p twice.
__device__ __forceinline__ void stage_pair(const float *maps, int64_t n_maps, int64_t p, float4 *s_map, int lane) {
    const float *src = maps + static_cast<size_t>(2 * p) * kPacked;
    if (2 * p + 1 < n_maps) {
        stage(src, s_map, 2 * kQuads, lane);
    } else {
        stage(src, s_map, kQuads, lane);
        stage(src, s_map + kQuads, kQuads, lane);
    }
}

// Waits for this wavefront's loads into LDS (and its stores) to complete.
__device__ __forceinline__ void wait_loads() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt(7), lgkmcnt(15): gfx9 encoding
    lds_order();
}

// Waits for this wavefront's LDS reads to complete (before the buffer they
// read is refilled by loads that bypass the LDS queue).
__device__ __forceinline__ void wait_lds_reads() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt(63), expcnt(7)
    lds_order();
}

// Start block of the iteration: u_k = e_s - e_t for beads (s, t) = (0, 16),
// (16, 32), (32, 48), (48, 63), the ends of four disjoint stretches of the
// chain.  Each is orthogonal to the all-ones vector, so B u = -1/2 J (a_s -
// a_t) comes from two columns of A that the lanes hold already (the first
// product is free); for a map that is Euclidean its span is that of the four
// displacements x_s - x_t, independent sums of steps of the walk.
constexpr int kSeedS[kBlk] = {0, 16, 32, 48};
constexpr int kSeedT[kBlk] = {16, 32, 48, 63};

// Column j of a lane's row of A, with the stand-in on the diagonal taken out.
__device__ __forceinline__ float a_entry(const float (&a)[kBeads], int row, int j) { return row == j ? 0.f : a[j]; }

// Iteration of one pair (rows l, l + 32 of A in a0, a1) to coordinates;
// returns false if deflated vectors overwrote the LDS buffer (the next pair's
// maps, prefetched into it, must then be loaded again).
__device__ __forceinline__ bool solve_pair(const float (&a0)[kBeads], const float (&a1)[kBeads], float g0sq,
                                           float g1sq, int half, int l, size_t m, bool write, int32_t max_iters,
                                           float *dfl, float *s_qt, float *s_w, float *__restrict__ coords,
                                           float *__restrict__ eigvals) {
    const int i0 = l, i1 = l + kHalf;
    bool buffer_kept = true;
    // Per-half iteration state (uniform within a half).
    int it = 1, pass = 0, steps = 0, n_dfl = 0;
    bool fin = false;
    float q0[kBlk], q1[kBlk], z0[kBlk], z1[kBlk];
    {
        float mz[kBlk];
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            z0[k] = a_entry(a0, i0, kSeedS[k]) - a_entry(a0, i0, kSeedT[k]);
            z1[k] = a_entry(a1, i1, kSeedS[k]) - a_entry(a1, i1, kSeedT[k]);
            mz[k] = z0[k] + z1[k];
        }
        half_sums(mz);
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            const float mean = mz[k] * (1.f / kBeads);
            z0[k] = (z0[k] - mean) * -0.5f;
            z1[k] = (z1[k] - mean) * -0.5f;
        }
    }
    for (;;) {
        orthonormalise(l, z0, z1, q0, q1);
        block_matvec(a0, a1, g0sq, g1sq, half, l, q0, q1, s_qt, z0, z1);
        const int nmax = max(__builtin_amdgcn_readlane(n_dfl, 0), __builtin_amdgcn_readlane(n_dfl, kHalf));
        project_out(dfl, n_dfl, nmax, l, z0, z1);
        const bool rr = !fin && it > 0;  // this half takes a Rayleigh-Ritz step (not after a restart)
        if (!any(rr)) {
            it += fin ? 0 : 1;
            continue;
        }
        float h[kBlk][kBlk], wl[kBlk], hs[kBlk * (kBlk + 1) / 2];
        {
            int n = 0;
#pragma unroll
            for (int r = 0; r < kBlk; ++r)
#pragma unroll
                for (int c = r; c < kBlk; ++c, ++n)
                    hs[n] = fmaf(q0[r], z0[c], fmaf(q0[c], z0[r], fmaf(q1[r], z1[c], q1[c] * z1[r])));
            half_sums(hs);
            n = 0;
#pragma unroll
            for (int r = 0; r < kBlk; ++r)
#pragma unroll
                for (int c = r; c < kBlk; ++c) {
                    const float sm = hs[n++] * 0.5f;
                    h[r][c] = sm;
                    h[c][r] = sm;
                }
        }
        jacobi4(h, wl, l);
        float d[kBlk] = {h[0][0], h[1][1], h[2][2], h[3][3]};
        // Sort descending, carrying the eigenvector columns (selects only).
#pragma unroll
        for (int x = 0; x < kBlk - 1; ++x)
#pragma unroll
            for (int y = 0; y < kBlk - 1 - x; ++y) {
                const bool sw = d[y + 1] > d[y];
                const float t = d[y];
                d[y] = sw ? d[y + 1] : d[y];
                d[y + 1] = sw ? t : d[y + 1];
                const float u = wl[y];
                wl[y] = sw ? wl[y + 1] : u;
                wl[y + 1] = sw ? u : wl[y + 1];
            }
        // W to every lane of the half (row r from lane r of the half).
        float *my_w = s_w + half * (kBlk * kBlk);
        if (l < kBlk) *reinterpret_cast<float4 *>(my_w + l * kBlk) = make_float4(wl[0], wl[1], wl[2], wl[3]);
        lds_order();
        float w[kBlk][kBlk];
#pragma unroll
        for (int r = 0; r < kBlk; ++r) {
            const float4 wr = *reinterpret_cast<const float4 *>(my_w + r * kBlk);
            w[r][0] = wr.x;
            w[r][1] = wr.y;
            w[r][2] = wr.z;
            w[r][3] = wr.w;
        }
        lds_order();
        float vec0[kBlk], vec1[kBlk], yv0[kBlk], yv1[kBlk];
        float thmax = 0.f, rho = 3.4e38f;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            vec0[k] = fmaf(q0[3], w[3][k], fmaf(q0[2], w[2][k], fmaf(q0[1], w[1][k], q0[0] * w[0][k])));
            vec1[k] = fmaf(q1[3], w[3][k], fmaf(q1[2], w[2][k], fmaf(q1[1], w[1][k], q1[0] * w[0][k])));
            yv0[k] = fmaf(z0[3], w[3][k], fmaf(z0[2], w[2][k], fmaf(z0[1], w[1][k], z0[0] * w[0][k])));
            yv1[k] = fmaf(z1[3], w[3][k], fmaf(z1[2], w[2][k], fmaf(z1[1], w[1][k], z1[0] * w[0][k])));
            thmax = fmaxf(thmax, fabsf(d[k]));
            rho = fminf(rho, fabsf(d[k]));
        }
        // A wanted pair has converged when its residual would move its
        // coordinate column (vec sqrt(theta)) by ~4e-6 of the largest one: an
        // eigenvector error is about residual / gap, so the tolerance scales
        // with the pair's gap to the other Ritz values (and, for the third, to
        // the largest magnitude the block may have missed), clamped to
        // [5e-7, 4e-6] of the largest magnitude (5e-7: float32 floor).  Pairs
        // to deflate take 4e-6.
        const bool hide = may_hide(d, rho);
        const float cap = 4e-6f * thmax, floor_tol = 5e-7f * thmax;
        float r2s[kBlk];  // squared residual norms, all four in one batch of sums
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            const float e0 = fmaf(-d[k], vec0[k], yv0[k]), e1 = fmaf(-d[k], vec1[k], yv1[k]);
            r2s[k] = fmaf(e0, e0, e1 * e1);
        }
        half_sums(r2s);
        bool done = true;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            float tk = cap;
            if (d[k] > 0.f) {
                float g = k == 2 ? d[k] - rho : 3.4e38f;
#pragma unroll
                for (int j = 0; j < kBlk; ++j)
                    if (j != k) g = fminf(g, fabsf(d[k] - d[j]));
                // sqrt(thmax / theta_k) by the hardware: a tolerance needs no correct rounding
                const float ratio = __builtin_amdgcn_sqrtf(thmax * __builtin_amdgcn_rcpf(d[k]));
                tk = hide ? cap : fminf(cap, fmaxf(floor_tol, 4e-6f * fmaxf(g, 0.f) * ratio));
            }
            const bool considered = hide || k < 3;
            const bool counted = !hide || fabsf(d[k]) >= 1e-3f * thmax;
            done = done && (!considered || !counted || r2s[k] <= tk * tk);
        }
        steps += rr ? 1 : 0;
        const bool spent = steps >= max_iters;
        const bool stop = rr && (done || spent);
        const bool finish = stop && (!hide || pass == kPasses - 1 || spent);
        const bool restart = stop && !finish;
        if (any(finish)) write_coords(finish, write, half, l, m, d, vec0, vec1, coords, eigvals);
        fin = fin || finish;
        if (!any(!fin)) break;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {  // the rotated product seeds the next step
            z0[k] = rr ? yv0[k] : z0[k];
            z1[k] = rr ? yv1[k] : z1[k];
        }
        if (any(restart)) {
            // deflate the negative Ritz vectors that outrank the third Ritz value, then start
            // over from the start block projected onto their complement.  The vectors go to the
            // LDS buffer of the packed maps, which may be receiving the next pair: let that
            // land first (it is loaded again afterwards).
            if (buffer_kept) wait_loads();
            buffer_kept = false;
            const float floor = fmaxf(d[2], 0.f);
#pragma unroll
            for (int k = 0; k < kBlk; ++k) {
                const bool add = restart && d[k] < 0.f && -d[k] > floor;
                if (add) {
                    dfl[n_dfl * kBeads + l] = vec0[k];
                    dfl[n_dfl * kBeads + l + kHalf] = vec1[k];
                }
                n_dfl += add ? 1 : 0;
            }
            lds_order();
            const int nmax2 = max(__builtin_amdgcn_readlane(n_dfl, 0), __builtin_amdgcn_readlane(n_dfl, kHalf));
            float zs0[kBlk], zs1[kBlk];
#pragma unroll
            for (int k = 0; k < kBlk; ++k) {
                zs0[k] = start_vec(i0, k);
                zs1[k] = start_vec(i1, k);
            }
            project_out(dfl, n_dfl, nmax2, l, zs0, zs1);
#pragma unroll
            for (int k = 0; k < kBlk; ++k) {
                z0[k] = restart ? zs0[k] : z0[k];
                z1[k] = restart ? zs1[k] : z1[k];
            }
        }
        pass += restart ? 1 : 0;
        it = restart ? 0 : (fin ? it : it + 1);
    }
    return buffer_kept;
}

// Persistent wavefronts: logical workgroup b (one wavefront; block0 +
// blockIdx.x when the grid is launched in slices) solves pairs b, b + G,
// b + 2G, ... of maps (G = n_blocks, pair p = maps 2p, 2p + 1).  Once a
// pair's rows are in registers, the next pair's maps are loaded into the
// same LDS buffer while the current pair iterates, so the HBM latency hides
// behind the arithmetic.
__global__ __launch_bounds__(kLanes, 2) void k_mds(const float *__restrict__ maps, int64_t n_maps,
                                                   float *__restrict__ coords, float *__restrict__ eigvals,
                                                   int32_t max_iters, int64_t n_blocks, int64_t block0) {
    __shared__ float4 s_map[2 * kQuads];              // two packed maps; deflated vectors after a restart
    __shared__ __align__(16) float s_qt[2 * kBlk * kBeads];  // Q^T of each half's map
    __shared__ __align__(16) float s_w[2 * kBlk * kBlk];     // Ritz rotation W of each half's map
    const int lane = threadIdx.x;
    const int half = lane >> 5, l = lane & (kHalf - 1);
    const int64_t n_pairs = (n_maps + 1) / 2;
    int64_t p = block0 + blockIdx.x;
    if (p >= n_pairs) return;  // wave-uniform
    stage_pair(maps, n_maps, p, s_map, lane);
    bool staged = true;  // s_map holds, or is receiving, pair p
    const float *xs = reinterpret_cast<const float *>(s_map) + half * kPacked;
    float *dfl = reinterpret_cast<float *>(s_map) + half * kPacked;
    const int i0 = l, i1 = l + kHalf;
    for (; p < n_pairs; p += n_blocks) {
        if (!staged) stage_pair(maps, n_maps, p, s_map, lane);
        wait_loads();
        const bool pair = 2 * p + 1 < n_maps;
        const size_t m = static_cast<size_t>(pair ? 2 * p + half : 2 * p);
        const bool write = pair || half == 0;

        // Rows i0 = l and i1 = l + 32 of A = D o D.  Entry (i, j) is packed
        // (i, j) for j > i, i.e. row_i[j - 1] with row_i = xs + idx(i, i + 1) -
        // i, and packed (j, i) for j < i, i.e. col_i[c_j] with col_i = xs + i and
        // c_j = idx(j, j + 1) - j - 1: reads at a per-lane base plus a constant
        // offset.  For j < 32 row i1 is always past j (column read) and row i0
        // needs the select; for j >= 32 row i0 is always before j (row read)
        // and row i1 needs it.  Every read stays inside the map's 2016 entries.
        // At j = i the loop squares a stand-in g (the entry before row i's
        // first) instead of the diagonal 0; g^2 is taken back out of every
        // product (block_matvec) and of the start block (a_entry).
        float a0[kBeads], a1[kBeads];
        const float *row0 = xs + packed_index(i0, i0 + 1) - i0, *col0 = xs + i0;
        const float *row1 = xs + packed_index(i1, i1 + 1) - i1, *col1 = xs + i1;
#pragma unroll
        for (int j = 0; j < kBeads; ++j) {
            const int cj = packed_index(j, j + 1) - j - 1;
            float d0, d1;
            if (j == 0) {
                d0 = xs[i0 > 0 ? i0 - 1 : 0];  // packed (0, i0) = i0 - 1
                d1 = col1[cj];
            } else if (j < kHalf) {
                d0 = j < kHalf - 1 ? select_above(row0[j - 1], col0[cj], j) : row0[j - 1];
                d1 = col1[cj];
            } else {
                d0 = row0[j - 1];
                d1 = j < kBeads - 1 ? select_above(row1[j - 1], col1[cj], j - kHalf) : row1[j - 1];
            }
            a0[j] = d0 * d0;
            a1[j] = d1 * d1;
        }
        const float g0 = xs[i0 > 0 ? packed_index(i0, i0 + 1) - 1 : 0];
        const float g1 = xs[packed_index(i1, i1 + 1) - 1];
        const float g0sq = g0 * g0, g1sq = g1 * g1;

        // The packed maps are in registers: refill the buffer with the next pair.
        wait_lds_reads();
        staged = p + n_blocks < n_pairs;
        if (staged) stage_pair(maps, n_maps, p + n_blocks, s_map, lane);
        staged = solve_pair(a0, a1, g0sq, g1sq, half, l, m, write, max_iters, dfl, s_qt, s_w, coords, eigvals) &&
                 staged;
    }
}

// Workgroups of the persistent MDS grid: MI355X's 256 compute units hold
// eight of the kernel's wavefronts each (two per SIMD, by LDS and registers).
constexpr int64_t kMdsGrid = 256 * 8;

}  // namespace

hipError_t launch_mds(const float *maps, int64_t n_maps, float *coords, float *eigvals, int32_t max_iters,
                      hipStream_t stream) {
    const int64_t n_pairs = (n_maps + 1) / 2;
    const int64_t n_blocks = n_pairs < kMdsGrid ? n_pairs : kMdsGrid;
    return launch_slices(n_blocks, kLanes, [&](int64_t first, uint32_t count) {
        hipLaunchKernelGGL(k_mds, dim3(count), dim3(kLanes), 0, stream, maps, n_maps, coords, eigvals, max_iters,
                           n_blocks, first);
    });
}

}  // namespace pc
