"""CPU oracle for the DSA decode/prefill path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package imports nothing from the product path.

The oracle is a plain, slow, obviously-correct NumPy implementation written
from the source pages, in float64 except where a step's result is a bit
pattern (the INT8 row), which follows its fp32 formula exactly.  Page
citations use these short names:

  [Flash]   "GLM-5.3-Flash" (pypto-lib model staging page)
  [Kernels] "GLM-5.3 Kernels" (store_int8 / sparse MLA kernel release)
  [Ref]     "Module glm5next_dsa_ref" (the DSA + kpool indexer CPU reference docs)
  [TF402]   TensorFold issue #402 (full GLM-5.3 on three DGX Sparks)

Pinning status of each function is stated in its docstring; functions whose
result rests only on a reading of silent or ambiguous text say
"parity unpinned" for that part.
"""
from .dsa import *  # noqa: F401,F403
