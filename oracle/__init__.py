"""CPU oracle for the edge-conditioned Clebsch-Gordan tensor-product convolution.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 restatement
of what the convolution computes, written from the source pages:

* "Sobek: Streaming Equivariant Tensor Product Convolutions" (sections 2-4,
  Eqs. 3-12, 15-22, 32-36), and
* "LunaTP: Enabling Efficient and Scalable Tensor Product for Equivariant
  MLIPs" (section 2.1, Eq. 1; section 2.2, Algorithm 1).

Only the tests, the smoke entry point and the CPU-baseline leg of the
benchmark may import it.  It shares no code with the HIP library and never
imports it; the two meet only through the seeded inputs of ``workloads``.

Modules: ``cg`` (real Clebsch-Gordan tensors), ``sh`` (real spherical
harmonics), ``irreps`` (irreps strings and path enumeration), ``csr``
(receiver and source CSR), ``conv`` (forward in both schedules, backward,
double backward).
"""
