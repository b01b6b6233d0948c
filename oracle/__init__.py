"""CPU oracle for the NeRF forward-render hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the method computes, written from the method's published
description (the blog post "Spatial Intelligence - Part 1: NeRF", the
notebook "Instant-NGP - Visual Experiments (a 2D multiresolution hash grid)"
and the KiloNeRF abstract).  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``volume_rendering_amd``) never imports, links or calls anything here, and
nothing here imports the product: the two share no code.  Their only common
dependency is ``seeded_inputs`` (seeded fixtures, none of the method's
arithmetic).

Floating point is float64 except where a step is defined as a sequence of
float32 operations so that an integer decision it feeds (a floor, a bin, a
comparison) is bit-reproducible; those steps say so.

Modules
  philox     counter-based generator for the random numbers the method draws
  rays       pinhole ray generation
  sampling   stratified samples, sample points, inverse-CDF resampling, merge
  encoding   frequency encoding, 3D/2D multiresolution hash grid, spherical harmonics
  mlp        radiance-field networks (float64 and bf16-emulating)
  composite  alpha compositing by transmittance
  render     end-to-end pipelines: hierarchical NeRF, hash-grid field, many tiny MLPs
"""
