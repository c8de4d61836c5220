"""CPU oracle for the sparse-attention step (DSA indexer -> exact top-k -> sparse MLA).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this package never
imports the product path: the two share no code.
"""

from .ml4_oracle import *  # noqa: F401,F403
