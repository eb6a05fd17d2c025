"""CPU oracle for paged attention: plain fp64 numpy, test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library
(``paged_kv_cache_48_amd``) and never imports it.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
the worked examples the pages print (``tests/golden/``), closed forms, the
invariances the pages state, and the independent brute force in
``brute_force.py``.  No function is parity-unpinned.
"""

from .paged_attention import (  # noqa: F401
    widen,
    ref_slot_mapping,
    ref_reshape_and_cache,
    ref_copy_blocks,
    ref_gather,
    ref_decode,
    ref_prefill,
)
from .brute_force import brute_decode, brute_prefill, contiguous_cache  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    ref_dequantize,
    ref_quantize,
    ref_reshape_and_cache_fp8,
)
