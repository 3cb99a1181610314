"""CPU oracle of the routing front-end. Test infrastructure only: imported by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
product path."""
from . import rgt_oracle  # noqa: F401
