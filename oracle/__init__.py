"""CPU oracle for the fused weight-gradient + optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library, its Python
binding) may import, call, link or execute anything under ``oracle/``; only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path: it was written from
the FORGE paper (arXiv 2606.22932) and from the published definitions it names,
not from the kernels.

Everything is plain NumPy.  Floating-point arithmetic is fp64 unless a step is
defined in a storage precision (bf16 / fp32 rounding, the int8 quantiser's
fp32 scale arithmetic), in which case that step is spelled out in that
precision.  See ``forge_oracle`` for the per-function citations and the list of
readings taken where the pages leave a step open.
"""

from .forge_oracle import *  # noqa: F401,F403
