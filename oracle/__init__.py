"""CPU oracle for the CSA/HCA hybrid-attention hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
statement of what the hot path computes.  It exists to check the HIP
implementation; nothing in the product path may import or call it.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark use it.

It shares no code with the HIP path and imports nothing from
``sparse_attention_csa_amd``.  Stored inputs (bf16 and OCP e4m3fn bytes) are
decoded by the oracle's own decoders in ``oracle.formats``.

Sources (cited by page title and section in each function):

* "DeepSeek-V4" book (slop-6tp.pages.dev/papers-html/dsv4), chapters 5-8 and 13.
* "2026 DeepSeek-V4" research note (awesome.papernotes.org), sections
  "Method Deep Dive", "Key design 1" and "Key design 2" with their equations.
* Anthology note 361 (dmarx.github.io), configuration list.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against worked
examples printed on the pages, closed forms, special cases that reduce to a
library routine, and brute force on tiny inputs.  No function is left
parity-unpinned.
"""

from . import formats  # noqa: F401
from . import csa  # noqa: F401
