"""fp64 CPU oracle for the frozen-NF4-base LoRA linear and its blockwise-streamed stack.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything here. The product path
(``nf4_weight_streamed_amd`` and its HIP library) never imports, calls or links
this package, and this package imports nothing from the product path; the two
share no code, tables or constants.

Pinning status of every function is listed in the module header of
``oracle/nf4_oracle.py``.
"""

from .nf4_oracle import *  # noqa: F401,F403
