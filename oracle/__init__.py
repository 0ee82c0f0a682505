"""CPU oracle for segment attention (test infrastructure only).

This package is the slow, plain, fp64 statement of what the segment-attention
hot path computes. It exists to check the HIP library, and only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path never calls it, and it shares no code, constants
or helpers with the HIP library: every formula here is written out from the
source pages (cited per function) or from the plain mathematical definition.

Sources (web pages about the Hy-Nomas world model):

* "Hy-Nomas: an 8.6B world model whose memory is a KV cache, and what it takes
  to fit a 4090" (ai.thesatyajit.com), sections "How one segment is made"
  (token grid, 16 heads of 128, 3D RoPE split [16, 56, 56], segment-wise
  attention), "What 'world memory' stores" (per-layer K/V of past segments,
  byte arithmetic) and "The 4090 preset" (power-spaced frame selection
  equation and its worked example for 360 past frames).
* "Hy-Nomas en una RTX 4090" (inferencekey.com), section "El preset de una
  GPU" (KV stored low-precision, computed in BF16).

Modules
-------
``numerics``   bf16 and OCP e4m3fn rounding / decoding, by definition.
``rope``       3D rotary position embedding over (t, h, w).
``select``     history frame selection policies (ALL, RECENT, POWER,
               ANCHOR_RECENT).
``attention``  dense softmax attention in fp64 (two-pass, exact max) and the
               segment key-set assembly.
``cache``      cache-plane layout offsets, byte counts and the expected plane
               contents after an append (bf16 and e4m3 + scales).

Pins: every function is checked by ``tests/test_oracle_*.py`` against
something other than itself (printed values of the pages, closed forms,
invariants, independent library routines, brute force). None is left
"parity unpinned".
"""

from . import numerics, rope, select, attention, cache  # noqa: F401
