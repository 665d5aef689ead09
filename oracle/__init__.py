"""CPU oracle for cached GQA attention with append.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package imports
nothing from the product path: the two share no code.

The oracle is the plain definition of what the hot path computes, written in
float64 NumPy with explicit masks and no cache at all:

* every real token's raw (pre-RoPE) key and value are kept in a list per
  layer and row;
* on every step every cached key is rotated again at its absolute position
  (nothing is stored rotated), the new queries are rotated at theirs;
* each query attends, with a float64 max-subtracted softmax, to exactly the
  keys the offset causal mask (clamped by the sliding window) allows.

Modules
-------
rope       rotary embedding, half-split pairing
mask       the offset causal mask, the sliding-window clamp, left padding
attention  softmax attention over an explicit key selection; single-sequence
           full forward
cache      the incremental definition (``OracleCache``), the integer slot
           addressing model, and an explicit ring-buffer model used only to
           check the oracle against itself
sizes      KV-cache byte counts

Parity status of each function is stated in its module header.
"""

from . import rope, mask, attention, cache, sizes  # noqa: F401
from .cache import OracleCache, CacheFull, slot_indices, RingModel  # noqa: F401
from .attention import full_forward, softmax_attend  # noqa: F401
from .mask import offset_mask  # noqa: F401
from .sizes import kv_nbytes  # noqa: F401
