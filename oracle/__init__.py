"""Plain fp64 CPU oracle for paged-KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import or call it.  It shares no code with the HIP
library (``paged_kv_cache_436_amd``) and imports nothing from it.

The oracle is the *definition* of what the method computes, written out slowly
and obviously:

* ``sizing``        - the KV-cache size formula ("KV Cache 原理与 PagedAttention",
                      §一 显存占用公式) and the paged-pool byte count.
* ``codecs``        - bf16 widening, FP8-e5m2 and per-token-head INT8 codecs
                      (same page, §四 KV Cache 量化 table; bjdmk.com.cn article,
                      §5.2 量化粒度).
* ``layout``        - the documented pool tile layout, as an index function.
* ``cache_ops``     - expected pool after the cache write and after a
                      copy-on-write block copy.
* ``attention``     - slot mapping, block-table gather, naive softmax attention
                      (bjdmk.com.cn article §2.1; "KV Cache 原理与 PagedAttention"
                      §三 工作方式 step 4).
* ``block_manager`` - a Python model of the host block manager: fixed-size
                      blocks, per-sequence tables, on-demand allocation, forks
                      and copy-on-write (§三 of the first page; §3.1-3.2 of the
                      bjdmk.com.cn article).

Every floating-point computation is done in float64 unless the quantity is
defined in float32 (quantiser arithmetic, fp32 scales), where numpy float32
with IEEE rounding is used on purpose.

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: library routines, closed forms, the pages' worked size examples,
brute force, permutation/aliasing invariants.  No function here is
"parity unpinned".
"""

from . import sizing, codecs, layout, cache_ops, attention, block_manager  # noqa: F401
