"""CPU oracle for exact softmax attention (float64).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the bench's
CPU-baseline leg may import it; the product path never does. It shares no code
with the HIP path.

Every function is pinned by tests/test_oracle_pins.py to values and properties the
pages and the mathematics fix; no function here is left "parity unpinned".
"""
from . import attention, backward, online  # noqa: F401  (modules; call attention.attention(...))
