"""CPU oracle of the DSpark draft pass (float64, numpy).

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import, call or run anything in this
package.  It shares no code with the GPU library: the only module both sides
use is ``synth`` (seeded generator, no arithmetic of the method).

Modules:
  codecs  -- exact decoding of bf16 / Q8_0 / FP8 E4M3FN stored weights
  dspark  -- the draft pass: fc, MLA layers (absorbed and decompressed),
             SwiGLU, final norm + lm_head, Markov rollout, confidence,
             acceptance length, throughput closed forms

Parity unpinned end to end: the pages print no worked example of a whole
draft pass; every step is pinned separately (tests/test_oracle_*.py).
"""
from . import codecs, dspark  # noqa: F401
