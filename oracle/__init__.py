"""Oracle package: plain float64 CPU attention, used by tests, the smoke check
and the benchmark's CPU-baseline leg only. TEST INFRASTRUCTURE ONLY; the
library never imports it."""

from .attention import (  # noqa: F401
    attention_reference,
    attention_rows,
    attention_weights,
    causal_keep_mask,
    default_scale,
)
from .prefix import (  # noqa: F401
    attention_prefix,
    merge_reference,
    prefix_keep_mask,
)
from .backward import attention_backward, attention_delta  # noqa: F401
