"""CPU oracle for the Switch-Transformer MoE layer forward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark may import or run anything in
this directory.  The product path (the HIP library and its Python binding)
never imports it, and this directory imports nothing from the product path:
the two share no code.  Inputs come from the seeded generator in `datagen`,
which holds none of the layer's arithmetic.

Modules
  moe    -- the vectorised NumPy oracle, one function per step of the layer,
            in float64 unless the pages fix the precision (the router's
            logits are fp32, as the pages' selective-precision recipe asks).
  brute  -- pure-Python per-token loops for tiny inputs; an independent
            second statement of the same definitions, used to pin `moe`.

Every function cites the page passage it follows.  Readings of passages that
are silent, garbled or in conflict are stated where they are used.

Parity pins (tests/test_oracle_pins.py and tests/test_oracle_brute.py):
every step of `moe` is pinned by a page-printed value, a closed form, an
invariant or the brute force.  No function is parity-unpinned.
"""
from . import moe  # noqa: F401
from . import brute  # noqa: F401
