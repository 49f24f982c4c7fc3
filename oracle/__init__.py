"""Float64 CPU oracle of the tiled ensemble-diffusion hot path — TEST INFRASTRUCTURE.

This package is the slow, plain reference that the HIP library is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does, and it imports nothing from the
HIP library or its binding.  Inputs come from ``workloads`` (seeded walks),
which holds none of the method's arithmetic.

What it computes, in the order the method runs (ParaChromo, sections 3.1 and
4.3.2, over ChromoGen's sampler):

* ``philox``   Philox4x32-10 counter-based generator (Salmon et al., SC'11),
               keyed by (seed) and counted by (quad, trajectory, step slot).
* ``normals``  Box-Muller transform of Philox words into N(0, 1) samples.
* ``schedule`` linear-beta schedule, its cumulative products and the DDIM
               timestep grid (Song et al., ref. [7] of the paper).
* ``ddim``     point-mass stand-in denoiser, classifier-free guidance combine
               (Ho & Salimans, ref. [15]) and the DDIM reverse step.
* ``layout``   packed strict-upper-triangle distance-map layout.
* ``seam``     overlap-consistency projection of adjacent tiles and the seam
               discrepancy (ParaChromo, sections 4.3.2 and 5.5, Eq. (6)).
* ``mds``      classical (Torgerson) MDS: double centring and the top-3
               eigenpairs, by numpy's symmetric eigensolver or by cyclic Jacobi.
* ``sampler``  the whole trajectory loop for independent regions and chains.

Every function is float64 unless it states otherwise.  No function here is
"parity unpinned": each one is pinned by tests against closed forms,
invariants, brute force or an independent implementation.
"""
