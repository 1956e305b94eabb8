"""CPU oracle for the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never calls it, links it or falls back to it, and it shares no code
with the GPU library: it consumes the same seeded inputs (``workload``) and
nothing else.

Everything here is plain NumPy in fp64, written to be checked by eye against
the pages it cites:

* ``philox``   -- Philox4x32-10 counter-based generator (Salmon, Moraes,
                  Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
                  SC'11) and the two uniform conversions.
* ``forward``  -- the synthetic target forward: pre-norm residual MLP blocks
                  (RMSNorm, up, SiLU, down) and a final RMSNorm + LM head, all
                  positions at once.
* ``verify``   -- modified rejection sampling per request: accept with
                  min(1, p/q), resample the first rejection from
                  normalize(max(0, p - q)), bonus token after full acceptance;
                  greedy mode at temperature 0.
* ``laws``     -- closed forms and exact laws used to pin the above.
* ``attention`` -- causal attention of the verified positions over a paged
                  KV cache, the append, the commit of the accepted positions
                  and a block free list.
* ``moe``      -- the verification forward of a mixture-of-experts target
                  (top-k routing, SiLU experts, rank-order combine).
* ``cycle``    -- the draft loop and the whole draft-then-verify cycle.
* ``dsd``      -- the draft-length choice (goodput-optimal K per batch size)
                  and the running-average window rule.

Pins (what each function is checked against, outside itself) are listed in
each module's docstring; none is "parity unpinned".
"""
from . import philox, forward, verify, laws  # noqa: F401
