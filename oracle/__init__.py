"""CPU oracle for score-and-select prompt KV-cache compression.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test-suite, the smoke check and the bench's
``cpu_baseline`` leg use it.  It shares no code, table or helper with the HIP
library under ``kv_cache_compression_bf16_amd/``; the only thing both sides
consume is the seeded synthetic data from ``kv_cache_compression_bf16_amd.workload``
(which holds none of the method's arithmetic).

Everything here is plain numpy in float64 (bf16 inputs are exact in float64),
written in the order and notation of the pages it cites:

* ``score``   -- observation-window attention, softmax over the prefix, window
                 mean, grouped-query sum (SnapKV section of the ZigZagKV blog);
                 Keyformer's Gumbel noise and temperature.
* ``philox``  -- Philox4x32-10 / Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
                 "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), the
                 uniform mapping and the Gumbel(0,1) transform.
* ``budget``  -- MBA, LMBA and ZigZag's proportional per-layer allocation with
                 a floor (ZigZagKV blog, observation and allocation sections).
* ``pool``    -- SnapKV's 1D pooling of the importance along the keys.
* ``select``  -- per-head top-k plus the recent window.
* ``threshold`` -- KVzap's threshold rule with a sliding window (variable
                 kept count per head, packed output) and the packed gather.
* ``compact`` -- gather of the kept K/V rows.
* ``decode``  -- Keyformer's decode phase: per-step score accumulation over the
                 compressed cache and eviction of the lowest-scoring old token.
* ``think``   -- ThinK key-channel pruning, magnitude-based and query-driven.
* ``sizes``   -- the KV-cache size formula and ThinK's kept-channel count.

Parity status of each function (what pins it) is listed in each module's
docstring; every function here has at least one pin in ``tests/``.
"""

from . import budget, compact, decode, philox, pool, score, select, sizes, think, threshold  # noqa: F401
