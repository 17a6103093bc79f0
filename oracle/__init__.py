"""CPU oracle of the QSA hot path (numpy, float64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of the
benchmark are the only code that may import, call or run anything in this package.  It shares
no code with the HIP library, and the library never falls back to it.

Every function here is pinned by CPU tests against something other than itself: torch's own
bf16 / float8_e4m3fn casts (exhaustively), torch's rms_norm and scaled_dot_product_attention
in float64, closed forms, brute-force sorting, exact integer arithmetic, and invariants of the
method (budget >= context reproduces full causal attention; cache bytes do not depend on how
a prefill is chunked).  No function is "parity unpinned".
"""

from . import numerics, qsa  # noqa: F401
