"""Plain, slow CPU oracle for the NVFP4 block-scaled linear, the grouped linear of the
attention output projection, the router gate, the fused RMSNorm + quantization and the
MoE grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, tables or helpers) and imports nothing
from ``fp4_block_scaled_route_amd``.

Sources.  The method is described on three pages of the public repository
``biondizzle/nvfp4-megamoe-kernel`` (commit listings):

* "commit 1121cd7 - single_shot_inference.py"  (page P1 below)
* "commit efe63ca - single_shot_inference.py"  (page P2)
* "commit 4c6464e - vllm"                       (page P3)

The pages have no numbered sections; each function cites the page and the
commit note (by topic) that defines what it computes.  Number formats follow
the OCP Microscaling Formats (MX) specification v1.0 (E2M1 and E4M3), which
the pages rely on without restating.

Precision.  Matrix products and dequantization run in float64.  The
activation quantizer runs in float32 in a fixed operation order, because
there floating point decides integer codes and both sides must take that
decision in the same precision (the GPU kernel's float32).

Modules:
  codec   E2M1 / E4M3FN decode and round-to-nearest-even encode, nibble unpack,
          weight dequantization.
  quant   activation global scale and NVFP4 block quantization.
  linear  dense block-scaled linear (bf16 or NVFP4 activations).
  moe     permute / segment offsets, expert FFN with SwiGLU, weighted combine.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against values fixed independently of this code (spec tables, hand-worked
examples under ``tests/golden/``, exact rational brute force, closed forms,
library routines and invariants).  No function is left "parity unpinned".
"""

from . import codec, quant, linear, moe  # noqa: F401
