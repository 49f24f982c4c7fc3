// Batched classical (Torgerson) MDS: one 64-lane workgroup per map, lane i
// owning bead i.
//
//   1. The packed map is copied from HBM straight into LDS (global_load_lds,
//      eight 16-byte loads per lane that bypass the registers); lane i
//      gathers row i of A = D o D into 64 VGPRs (two constant-offset LDS
//      reads and a select on a constant lane mask per entry).
//   2. Double centring B = J A J (times -1/2) from the row means (LDS) and the
//      grand mean (wavefront reduction); row i of B stays in VGPRs.
//   3. Block-4 subspace iteration with Rayleigh-Ritz: Q <- orth(Z) by
//      modified Gram-Schmidt (a column that cancels is projected twice),
//      Z = B Q (64 4x4x1 MFMA steps, Q^T read from LDS), H = Q^T Z by DPP
//      wavefront reductions, a 4x4 Jacobi eigensolve (wave-uniform values,
//      eigenvector rows spread over lanes 0..3), Ritz vectors V = Q W,
//      Z W = B V and the residuals ||B V_k - theta_k V_k|| of the three
//      largest.  Stops when each is small against its pair's gap
//      (eigenvector error ~ residual / gap) or after max_iters Rayleigh-Ritz
//      steps in all.  The workgroup is capped at 128 VGPRs so four maps run
//      per SIMD (the kernel is VALU-bound; on MI355X four waves beat three by
//      12%, and five need 96 VGPRs, spill and run 14% slower).
//   4. The iteration finds the eigenvalues of largest magnitude.  If negative
//      ones could hide a positive eigenvalue (the third largest Ritz value is
//      below the smallest magnitude found), the negative Ritz vectors that
//      outrank it are projected out (held in LDS) and the iteration restarts
//      on the complement, at most kPasses passes in all, so the largest
//      magnitudes left are the wanted positive eigenvalues.
//   5. X = V_3 diag(sqrt(max(theta, 0))), each column signed so that its
//      largest-magnitude entry is positive (lowest index on ties).
#include "common.hpp"
#include "launch.hpp"
#include "mds_start.hpp"

namespace pc {
namespace {

constexpr int kLanes = 64;
constexpr int kBlk = 4;

// Column k of the start block for bead i (orthonormal, orthogonal to the
// all-ones vector; mds_start.hpp).
__device__ __forceinline__ float start_vec(int i, int k) { return kMdsStart[i][k]; }

// Cyclic Jacobi on a symmetric 4x4 (values identical in every lane).  The
// rotation that zeroes h_pq uses t = sgn(th) / (|th| + sqrt(th^2 + 1)) with
// th = (h_qq - h_pp) / (2 h_pq) (formed as 2 h_pq sgn(d) / (|d| + sqrt(d^2 +
// 4 h_pq^2)), d = h_qq - h_pp), c = 1 / sqrt(1 + t^2), s = t c; only the
// entries it changes are updated (h_pp -= t h_pq, h_qq += t h_pq, rows r != p,
// q rotate).  t needs no correct rounding: c and s are formed from it, so the
// rotation stays orthogonal, and the hardware rcp / rsq / sqrt are used.  The
// eigenvector matrix W is spread over lanes: lane r < 4 holds row r in wl, so
// a rotation costs each lane two columns of one row.  Rotations whose h_pq^2
// is below `skip2` (1e-15 of the squared diagonal norm, under float32
// resolution of the largest eigenvalue) are skipped.  (Carrying skipped
// rotations out as identities with selects instead of a branch measured 4%
// slower over the whole kernel.)
template <int P, int Q>
__device__ __forceinline__ void jacobi_rotate(float (&h)[kBlk][kBlk], float (&wl)[kBlk], float skip2) {
    const float apq = h[P][Q];
    if (apq * apq <= skip2) return;  // wave-uniform
    // t = sgn(th) / (|th| + sqrt(th^2 + 1)) with th = d / (2 h_pq), d = h_qq - h_pp,
    // multiplied through by 2 |h_pq|: one transcendental fewer, and no overflow of th
    const float d = h[Q][Q] - h[P][P];
    const float den = fabsf(d) + __builtin_amdgcn_sqrtf(fmaf(d, d, 4.f * apq * apq));
    const float t = copysignf(2.f, d) * apq * __builtin_amdgcn_rcpf(den);
    const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f));
    const float sn = t * c;
    h[P][P] = fmaf(-t, apq, h[P][P]);
    h[Q][Q] = fmaf(t, apq, h[Q][Q]);
    h[P][Q] = h[Q][P] = 0.f;
#pragma unroll
    for (int r = 0; r < kBlk; ++r) {
        if (r == P || r == Q) continue;
        const float hp = h[r][P], hq = h[r][Q];
        h[r][P] = h[P][r] = fmaf(c, hp, -sn * hq);
        h[r][Q] = h[Q][r] = fmaf(sn, hp, c * hq);
    }
    const float wp = wl[P], wq = wl[Q];
    wl[P] = fmaf(c, wp, -sn * wq);
    wl[Q] = fmaf(sn, wp, c * wq);
}

// On return h is diagonal to float32 precision and lane r < 4 holds row r of
// the eigenvector matrix (eigenvectors as columns) in wl.
__device__ __forceinline__ void jacobi4(float (&h)[kBlk][kBlk], float (&wl)[kBlk], int lane) {
#pragma unroll
    for (int c = 0; c < kBlk; ++c) wl[c] = lane == c ? 1.f : 0.f;
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
        if (off <= 1e-14f * dia) break;
        const float skip2 = 1e-15f * dia;
        jacobi_rotate<0, 1>(h, wl, skip2);
        jacobi_rotate<0, 2>(h, wl, skip2);
        jacobi_rotate<0, 3>(h, wl, skip2);
        jacobi_rotate<1, 2>(h, wl, skip2);
        jacobi_rotate<1, 3>(h, wl, skip2);
        jacobi_rotate<2, 3>(h, wl, skip2);
    }
}

// hi in lanes above lane j (lane id > j), lo in lanes 0 .. j, for a wavefront
// with all 64 lanes active.  The lane mask is the execution mask shifted by
// j + 1 (one scalar shift once the caller's loop over j is unrolled), and the
// select a single v_cndmask on that SGPR pair, with no vector compare.  (The
// mask is not written as a 64-bit constant: hipcc encodes such a constant as
// a 32-bit literal that gfx950 zero-extends, which loses the upper 32 lanes;
// measured.  The asm is one ALU instruction on ordinary registers, so the
// compiler places every wait before it.)
__device__ __forceinline__ float select_above(float lo, float hi, int j) {
    const uint64_t above = j < kLanes - 1 ? __builtin_amdgcn_read_exec() << (j + 1) : 0ull;
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(lo), "v"(hi), "s"(above));
    return r;
}

// Largest value over the wavefront of a non-negative v (DPP, as wave_sum).
__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, dpp<0x142>(v));  // only lane 63 is read (as in wave_sum)
    v = fmaxf(v, dpp<0x143>(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Modified Gram-Schmidt of the four per-lane columns y into q.  A column that
// loses more than 4 decimal digits of its norm to the projections (the fourth
// column of B Q when B has rank 3) is projected a second time, which restores
// orthogonality to float32 precision; a column that vanishes is replaced by
// its start vector.  (Classical Gram-Schmidt, whose coefficients come from one
// batch of sums, measured 5% slower over the whole kernel: it issues more
// instructions, and the kernel is bound by instruction issue, not by the
// latency of the reductions.)
__device__ __forceinline__ void orthonormalise(int lane, const float (&y)[kBlk], float (&q)[kBlk]) {
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
        float v = y[k];
        for (int attempt = 0; attempt < 2; ++attempt) {
            const float n0 = k > 0 ? wave_sum(v * v) : 0.f;
#pragma unroll
            for (int l = 0; l < k; ++l) v = fmaf(-wave_sum(q[l] * v), q[l], v);
            float n2 = wave_sum(v * v);
            if (k > 0 && n2 < 1e-4f * n0) {  // cancellation: project once more
#pragma unroll
                for (int l = 0; l < k; ++l) v = fmaf(-wave_sum(q[l] * v), q[l], v);
                n2 = wave_sum(v * v);
            }
            if (n2 > 1e-30f) {
                v *= __builtin_amdgcn_rsqf(n2);
                break;
            }
            v = start_vec(lane, k);
            if (attempt == 1) v = 0.f;
        }
        q[k] = v;
    }
}

constexpr int kPasses = 4;                     // iteration passes per map, at most
constexpr int kMaxDefl = (kPasses - 1) * kBlk;  // deflated vectors, at most
static_assert(kMaxDefl * kBeads <= kPacked, "deflated vectors are kept in the map's LDS buffer");

// Deflated Ritz vectors: n of them in LDS, vector d's component for bead l at
// v[d * kBeads + l].  They are orthonormal to float32 rounding.
struct Deflation {
    float *v;
    int n;
};

// Removes from the four per-lane columns z their components along the deflated
// vectors, one vector after the other.
__device__ __forceinline__ void project_out(const Deflation &dfl, int lane, float (&z)[kBlk]) {
    for (int d = 0; d < dfl.n; ++d) {
        const float v = dfl.v[d * kBeads + lane];
#pragma unroll
        for (int k = 0; k < kBlk; ++k) z[k] = fmaf(-wave_sum(v * z[k]), v, z[k]);
    }
}

// z = B q for the four per-lane columns q (row `lane` of B in b, whose
// diagonal entry is off by diag_err), on the matrix cores: 64 rank-1 steps of
// v_mfma_f32_4x4x1f32 (16 blocks of 4x4).  Block c / 4 of step k multiplies
// A = (q_k0 .. q_k3) (lane 4 blk + r supplies q_kr, read from Q^T in LDS) by
// B = (b_{4 blk + j, k})_j (lane l supplies its own b[k] = B_lk = B_kl), so
// output register r of lane l accumulates sum_k q_kr B_kl = (B q)_lr: lane l
// ends with row l of B Q.  Four accumulators take the steps in turn, so
// consecutive steps do not wait on each other.
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void block_matvec(const float (&b)[kBeads], float diag_err, int lane,
                                             const float (&q)[kBlk], float4 *s_q, float (&z)[kBlk]) {
    float *s_qt = reinterpret_cast<float *>(s_q);  // Q^T: column c at s_qt[c * 64 + bead]
#pragma unroll
    for (int c = 0; c < kBlk; ++c) s_qt[c * kBeads + lane] = q[c];
    __syncthreads();
    const float4 *qa = reinterpret_cast<const float4 *>(s_qt + (lane & 3) * kBeads);
    f32x4v acc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k4 = 0; k4 < kBeads / 4; ++k4) {
        const float4 a = qa[k4];  // q_{4 k4 + e, lane & 3}
        acc[0] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.x, b[4 * k4 + 0], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.y, b[4 * k4 + 1], acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.z, b[4 * k4 + 2], acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_4x4x1f32(a.w, b[4 * k4 + 3], acc[3], 0, 0, 0);
        // keep at most two rows of Q^T in flight (hoisting all 16 LDS reads
        // would overflow the register file)
        if (k4 % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k = 0; k < kBlk; ++k) z[k] = fmaf(-diag_err, q[k], (acc[0][k] + acc[1][k]) + (acc[2][k] + acc[3][k]));
    __syncthreads();
}

// True when negative eigenvalues may hide a wanted one: the third largest Ritz
// value is below the smallest Ritz magnitude, so an eigenvalue the iteration
// missed (magnitude <= that smallest one) could outrank it.  Below 1e-6 of the
// largest Ritz value the spectrum is float32 noise and never counts.
__device__ __forceinline__ bool may_hide(const float (&d)[kBlk], float rho) {
    return d[2] < rho && rho > 1e-6f * fabsf(d[0]);
}

// Block-4 subspace iteration on P B P, P the projector onto the complement of
// the deflated vectors (none at first).  Each iteration orthonormalises the
// last product (q <- MGS(z); the first pass starts from the fixed orthonormal
// start block, later passes from its projection onto the complement),
// multiplies again (z <- P B q), and from the second product on takes the
// Rayleigh-Ritz pairs of (q, z): H = q^T z, H = W diag(theta) W^T, vec = q W,
// residual ||z W - theta vec||.
//
// A pass ends when the three largest pairs have converged (the result).  If
// negative eigenvalues may hide a wanted one, it ends instead once every pair
// above 1e-3 of the largest magnitude has converged; the negative pairs that
// outrank the third largest Ritz value are then deflated and a new pass
// starts on the complement, whose largest magnitudes move toward the wanted
// positive eigenvalues.  The whole iteration stops after max_iters
// Rayleigh-Ritz steps over all passes.  (B has
// eigenvalue 0 on the all-ones vector, so its third largest eigenvalue is
// never negative, and projecting directions out, which leaves 0 in their
// place, cannot change the three largest.)  On return theta (descending) and
// vec (lane = bead) hold the last Ritz pairs.
__device__ __forceinline__ void subspace(const float (&b)[kBeads], float diag_err, Deflation &dfl, int32_t max_iters,
                                         int lane, float4 *s_q, float (&theta)[kBlk], float (&vec)[kBlk]) {
    float q[kBlk], z[kBlk];
    int pass = 0, steps = 0;
    for (int it = 0;; ++it) {
        if (it == 0 && pass == 0) {  // the start block is orthonormal already
#pragma unroll
            for (int k = 0; k < kBlk; ++k) q[k] = start_vec(lane, k);
        } else {
            orthonormalise(lane, z, q);
        }
        block_matvec(b, diag_err, lane, q, s_q, z);
        project_out(dfl, lane, z);
        if (it == 0) continue;  // the first product only seeds the subspace
        float h[kBlk][kBlk], wl[kBlk], hs[kBlk * (kBlk + 1) / 2];
        {
            int n = 0;
#pragma unroll
            for (int r = 0; r < kBlk; ++r)
#pragma unroll
                for (int c = r; c < kBlk; ++c) hs[n++] = fmaf(q[r], z[c], q[c] * z[r]);
            wave_sums(hs);
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
        jacobi4(h, wl, lane);
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
        // W to every lane (row r from lane r).
        float w[kBlk][kBlk];
#pragma unroll
        for (int r = 0; r < kBlk; ++r)
#pragma unroll
            for (int c = 0; c < kBlk; ++c) w[r][c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl[c]), r));
        float yv[kBlk];
        float thmax = 0.f, rho = 3.4e38f;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            vec[k] = fmaf(q[3], w[3][k], fmaf(q[2], w[2][k], fmaf(q[1], w[1][k], q[0] * w[0][k])));
            yv[k] = fmaf(z[3], w[3][k], fmaf(z[2], w[2][k], fmaf(z[1], w[1][k], z[0] * w[0][k])));
            theta[k] = d[k];
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
            const float r = fmaf(-d[k], vec[k], yv[k]);
            r2s[k] = r * r;
        }
        wave_sums(r2s);
        bool done = true;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            if (!done || (!hide && k == 3)) break;  // wave-uniform
            const float r2 = r2s[k];
            float tk = cap;
            if (!hide && d[k] > 0.f) {
                float g = k == 2 ? d[k] - rho : 3.4e38f;
#pragma unroll
                for (int j = 0; j < kBlk; ++j)
                    if (j != k) g = fminf(g, fabsf(d[k] - d[j]));
                tk = fminf(cap, fmaxf(floor_tol, 4e-6f * fmaxf(g, 0.f) * sqrtf(thmax / d[k])));
            }
            if (!hide || fabsf(d[k]) >= 1e-3f * thmax) done = r2 <= tk * tk;
        }
        const bool spent = ++steps >= max_iters;
        if (done || spent) {
            if (!hide || pass == kPasses - 1 || spent) break;
            const float floor = fmaxf(d[2], 0.f);
#pragma unroll
            for (int k = 0; k < kBlk; ++k) {
                if (d[k] < 0.f && -d[k] > floor) {  // wave-uniform
                    dfl.v[dfl.n * kBeads + lane] = vec[k];
                    ++dfl.n;
                }
            }
            ++pass;
            it = -1;
#pragma unroll
            for (int k = 0; k < kBlk; ++k) z[k] = start_vec(lane, k);
            project_out(dfl, lane, z);
            continue;
        }
#pragma unroll
        for (int k = 0; k < kBlk; ++k) z[k] = yv[k];
    }
}

// Copies packed map m from HBM straight into LDS with global_load_lds (each
// instruction writes lane l's 16 bytes at s_map + 16 l), without passing
// through registers.  Asynchronous: the compiler waits for it before the
// first LDS read of s_map.
__device__ __forceinline__ void stage_map(const float *maps, size_t m, float4 *s_map, int lane) {
    typedef __attribute__((address_space(1))) void *gptr;
    typedef __attribute__((address_space(3))) void *lptr;
    const char *src = reinterpret_cast<const char *>(maps + m * kPacked);  // wave-uniform
    const uint32_t off = static_cast<uint32_t>(lane) * 16u;                 // the lane's bytes in a chunk
#pragma unroll
    for (int c = 0; c < kQuads / kLanes; ++c)
        __builtin_amdgcn_global_load_lds((gptr)(src + c * kLanes * 16 + off), (lptr)(s_map + c * kLanes), 16, 0, 0);
    constexpr int kTail = kQuads % kLanes;  // 56 quads in the last chunk
    if (lane < kTail) {
        constexpr int c = kQuads / kLanes;
        __builtin_amdgcn_global_load_lds((gptr)(src + c * kLanes * 16 + off), (lptr)(s_map + c * kLanes), 16, 0, 0);
    }
}

// One map per 64-lane workgroup, lane i owning bead i.
__global__ __launch_bounds__(kLanes, 4) void k_mds(const float *__restrict__ maps, float *__restrict__ coords,
                                                float *__restrict__ eigvals, int32_t max_iters, int64_t block0) {
    __shared__ float4 s_map[kQuads];
    __shared__ float4 s_q[kBeads];
    __shared__ __align__(16) float s_mean[kBeads];
    const int i = threadIdx.x;
    const size_t m = static_cast<size_t>(block0) + blockIdx.x;
    stage_map(maps, m, s_map, i);
    __syncthreads();
    const float *xs = reinterpret_cast<const float *>(s_map);

    // Row i of A = D o D.  Entry (i, j) is packed (i, j) for j > i, i.e.
    // row[j - 1] of lane i's contiguous packed row, and packed (j, i) for j < i,
    // i.e. col[c_j] with c_j = idx(j, j + 1) - j - 1; both are reads at a
    // per-lane base plus a constant offset, and a select keeps the valid one.
    // Every read stays inside the 2016 entries.  At j = i the loop squares a
    // stand-in g (the entry before lane i's row) instead of the diagonal 0;
    // g^2 is taken back out of the row sum here and out of every product B q
    // (block_matvec's diag_err), which is cheaper than a select per entry.
    float b[kBeads];
    const float *row = xs + packed_index(i, i + 1) - i;
    const float *col = xs + i;
    float rsum = 0.f;
#pragma unroll
    for (int j = 0; j < kBeads; ++j) {
        float d;
        if (j == 0) {
            d = xs[i > 0 ? i - 1 : 0];  // packed (0, i) = i - 1
        } else {
            const float dr = row[j - 1];
            const float dc = col[packed_index(j, j + 1) - j - 1];
            d = select_above(dr, dc, j);  // j < i ? dc : dr
        }
        b[j] = d * d;
        rsum += b[j];
    }
    const float g = xs[i > 0 ? packed_index(i, i + 1) - 1 : 0];
    const float g2 = g * g;
    rsum -= g2;
    // B = -1/2 J A J: b_ij = -a_ij / 2 + u_i + u_j with u_i = mean_i / 2 - grand mean / 4.
    const float gmean = wave_sum(rsum) * (1.f / (kBeads * kBeads));
    const float u_i = 0.5f * (rsum * (1.f / kBeads)) - 0.25f * gmean;
    const float diag_err = fmaf(g2, -0.5f, u_i + u_i) - (u_i + u_i);  // stored b_ii minus the true one
    s_mean[i] = u_i;
    __syncthreads();
    const float4 *s_u = reinterpret_cast<const float4 *>(s_mean);
#pragma unroll
    for (int j4 = 0; j4 < kBeads / 4; ++j4) {
        const float4 u = s_u[j4];
        b[4 * j4 + 0] = fmaf(b[4 * j4 + 0], -0.5f, u_i + u.x);
        b[4 * j4 + 1] = fmaf(b[4 * j4 + 1], -0.5f, u_i + u.y);
        b[4 * j4 + 2] = fmaf(b[4 * j4 + 2], -0.5f, u_i + u.z);
        b[4 * j4 + 3] = fmaf(b[4 * j4 + 3], -0.5f, u_i + u.w);
    }

    float theta[kBlk], vec[kBlk];
    Deflation dfl{reinterpret_cast<float *>(s_map), 0};  // the packed map is dead once B is in registers
    subspace(b, diag_err, dfl, max_iters, i, s_q, theta, vec);

    // Sign each column by its largest-magnitude entry (lowest bead on ties).
    float out[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float a = fabsf(vec[k]);
        const float best = wave_max_nonneg(a);
        const int first = __builtin_ctzll(__ballot(a == best));
        const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vec[k]), first));
        out[k] = (sv < 0.f ? -vec[k] : vec[k]) * sqrtf(fmaxf(theta[k], 0.f));
    }
    float *dst = coords + (m * kBeads + i) * 3;
    dst[0] = out[0];
    dst[1] = out[1];
    dst[2] = out[2];
    if (eigvals && i == 0) {
        eigvals[m * 3 + 0] = theta[0];
        eigvals[m * 3 + 1] = theta[1];
        eigvals[m * 3 + 2] = theta[2];
    }
}

}  // namespace

hipError_t launch_mds(const float *maps, int64_t n_maps, float *coords, float *eigvals, int32_t max_iters,
                      hipStream_t stream) {
    return launch_slices(n_maps, kLanes, [&](int64_t first, uint32_t count) {
        hipLaunchKernelGGL(k_mds, dim3(count), dim3(kLanes), 0, stream, maps, coords, eigvals, max_iters, first);
    });
}

}  // namespace pc
