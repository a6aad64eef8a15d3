"""Independent fp64 CPU oracle for sparse, head-ragged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers, tables or constants) and imports
nothing but the Python standard library and numpy.

Sources (the pages, cited by title and section):
  * "Tangram: Unlocking Non-Uniform KV Cache Compression for Efficient
    Multi-turn LLM Serving" (paper review) -- 3.1 Budget Reservation,
    3.2 Ragged Paging, 3.3 AOT Load Balancing.
  * "FlexiCache: Leveraging Temporal Stability of Attention Heads for
    Efficient KV Cache Management (MLSys 2026)" (paper summary) -- Core method
    (sparse decode, Quest-style min-max page bound), System engineering
    (per-head block table with null entries), Key observations (assumption 2,
    GPU-resident MinMax cache), tiered placement.
  * "CacheGen -- KV Cache Compression and Streaming" (paper notes) --
    sections 3 and 7: change-based encoding over token groups, layer-wise
    quantization, arithmetic coding per (channel, layer) (codec_oracle.py).

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, brute force or invariants; none is "parity unpinned" except the
relation of ``plan_split`` to Tangram's unprinted Algorithm 1 (only its
stated goal is pinned).
"""

from .kvs_oracle import *  # noqa: F401,F403
from .codec_oracle import *  # noqa: F401,F403
