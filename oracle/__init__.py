"""Float64 CPU oracle for banded sliding-window attention with global tokens.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP library never routes through it, and it imports nothing
from the HIP side (no kernels, no headers, no helpers, no shared constants).

Source of the definition: the Longformer summary page (velog.io/@lainshower,
"Longformer"), section 3-1 "Attention Pattern" -- sliding window, dilated
sliding window, global attention, separate projections for global attention --
and section 7 "Longformer-Encoder-Decoder" for the left-only (causal) mask.
Every reading taken where the page is silent is listed in ``masked_softmax.py``.

Every function here is pinned by ``tests/test_oracle_*.py`` against brute
force, closed forms, library reductions and hand-derived golden values;
``attention_banded`` (the same definition over each row's enumerated keys,
O(n*w*d)) is pinned against those pinned functions and brute force.
"""

from .masked_softmax import (  # noqa: F401
    allowed_mask,
    attention,
    attention_backward,
    band_mask,
    global_row_mask,
)
from .banded import attention_banded  # noqa: F401
from .projection import project  # noqa: F401
