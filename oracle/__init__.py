"""Plain fp64 CPU oracle for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path never does, and this package
never imports the product package.

The arithmetic lives in ``sdpa_oracle.c`` (plain C, fp64, one query row at a time); this
module only builds it with gcc and marshals numpy arrays through ctypes.
"""

from .oracle import Oracle, build_oracle, load_oracle, oracle_lib_path

__all__ = ["Oracle", "build_oracle", "load_oracle", "oracle_lib_path"]
