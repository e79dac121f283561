"""CPU oracle for the DualQuant dual-scale block-coordinate-descent solver.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with
the HIP library (no kernels, headers, helpers, tables or constant generators)
and never imports it.

What it is: a plain, slow, float64 numpy implementation of what the method
computes, written from the pages that describe it:

* "DualQuant: Dual-scale Calibration-free Weight-and-Activation Quantization
  for LLMs" (paper summary at paperlayer.ai, arXiv 2610.13767v1), cited here
  as [DQ summary] with its section numbers;
* "DualQuant: Calibration-Free Dual-Scale Weight and Activation Quantization"
  (third-party reproduction README at daiwk.github.io), cited as
  [DQ repro] with its section titles -- the only page whose update equations
  survived ("Core equations");
* "SQuant: On-the-Fly Data-Free Quantization" (tutorial at
  engineermaxxing.com), cited as [SQuant tutorial] with its chapter;
* "Round-to-Nearest & Basic Weight Quantization" (tutorial at
  14cs17.netlify.app), cited as [RTN tutorial] with its section.

Modules:
  formats   -- element grids, legal scale sets, projections, encodings
  dualquant -- init, the BCD iteration, packing, activation quantization,
               diagnostics

Every function says which passage it follows. Where the pages are silent
the reading taken is stated in the docstring.
"""

from . import formats, dualquant  # noqa: F401
