"""CPU oracle for the compression path -- test infrastructure only (tests, smoke check,
CPU-baseline leg of the benchmark).  The product path never imports it."""
from . import bkv_oracle  # noqa: F401
