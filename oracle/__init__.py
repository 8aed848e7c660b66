"""CPU oracle for the paged grouped-query decode attention engine.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it.
It shares no code with the HIP path: no kernels, headers, helpers, tables or
pre/post-processing.  Everything here is a plain, slow, fp64 restatement of
what the PersistentKV summary pages define:

* ``attention``  -- grouped-query decode attention over a paged KV pool read
  through a block table (sections "Methodology / 1. Native block-table decode
  engine": GQA with G = Hq/Hkv query heads per KV head; "Layout": runs on the
  paged layout without repacking).
* ``split_state`` / ``merge`` -- partial online-softmax state of one disjoint
  sequence range and the exact combination of such states ("Sequence
  splitting" bullet of the same section).
* ``planner`` -- row-local split bounds, the compact workqueue and exact-length
  buckets ("Row-local bounds" and "Compact workqueue" bullets; "Results":
  launches per step).
* ``policy`` -- first-match calibrated threshold table keyed on (B, N_max)
  ("2. Calibrated adaptive policy").
* ``append_kv`` -- storing a step's new key/value through the block table
  (the input side of the decode step; not described on the pages).
* ``cost`` -- plan features and the argmin choice of a learned per-path
  linear cost model (future work on the pages: es page,
  "Significado y Reivindicaciones" / "Direcciones Futuras").
"""
from .attention import (  # noqa: F401
    attention,
    decode_values,
    gather_row,
    merge,
    round_to_bf16,
    round_to_f16,
    split_state,
    split_states_for_plan,
)
from .append import append_kv  # noqa: F401
from . import cost  # noqa: F401
from .planner import plan, pages_of  # noqa: F401
from .policy import choose  # noqa: F401
