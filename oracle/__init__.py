"""CPU oracle for the compressed sparse KV decode path. TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code, tables or helpers with the HIP library
and never imports it; the library never imports this package.

What it computes is the plain definition of each step, written out with numpy
in float64 (the codec encoders take their rounding decisions in float32, the
precision the encoded caches are defined in):

* ``formats``   - bf16, E4M3 (OCP "E4M3FN") and E2M1 value tables from the
  formats' public definitions, the fp8-row / fp4-group-of-16 encoders, and the
  mixed rows that keep the rotary channels in bf16 and the rest in fp8.
* ``method``    - compression into c4a / c128a entries, indexer scores, exact
  top-k, shared-K/V softmax attention over gathered entries plus the window,
  the inverse rotary embedding of the output, and the streaming decode step
  that appends one state per sequence to a ring of the newest W states and
  emits each entry when its window completes.
* ``accounting`` - bytes per token and per sequence for the cache layouts whose
  sizes the pages print.

Sources (cited by page title and section):
  [P1] "How DeepSeek V4 Uses Less Memory: KV Cache Explained" (aitoolsreview.co.uk)
  [P2] "DeepSeek V4 KV Cache" visual walkthrough (vizuaraai.github.io), Steps 1-7
  [P3] "KV cache at 890 bytes per token: how DeepSeek squeezed attention memory" (flash24.org)

Pinning: every function is checked in ``tests/test_oracle_pins.py`` against
something other than itself (the pages' worked examples and printed figures,
closed forms, library routines such as torch's float8 conversion and
scaled-dot-product attention, integer arithmetic, brute force). The one
result without such a pin is the end-to-end output at the full workload sizes
(the pages print no output values): parity unpinned beyond the step pins.
"""
from . import accounting, formats, method  # noqa: F401
