"""CPU float64 oracle of unified paged varlen attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The GPU library (``paged_varlen_attention_ua_amd``)
and its C ABI never import, link or execute anything here, and this package
imports nothing from them.

Parity pins: every function here is pinned by ``tests/test_oracle.py`` against
facts that do not come from this code (closed forms, a hand-worked example in
``tests/golden/``, a brute-force loop implementation on tiny inputs, torch's
float64 SDPA for the dense special case, format definitions, torch's fp8
casts for both e4m3 dialects).  Pinned: ``formats.decode_*``, ``attention``
(including per-token K/V scales), ``merge_partials_base2``,
``partition_states_base2``.  Parity unpinned (no case of the pages combines
them, so only the plainest reading is implemented): ALiBi together with sinks,
and the order of softcap relative to ALiBi.
"""

from .attention import attention, merge_partials_base2, partition_states_base2  # noqa: F401
from .formats import (decode, decode_bf16, decode_e4m3fn, decode_e4m3fnuz,  # noqa: F401
                      decode_fp16)
