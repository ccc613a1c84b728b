"""fp64 CPU oracle for relative attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""

from .relattn_oracle import (  # noqa: F401
    attention_weights,
    brute_force_prefill,
    cache_rows,
    decode,
    extend,
    logit_rows,
    prefill,
    rel_logits,
    scale_factor,
    sheared_bias,
)
from .prologue_oracle import (  # noqa: F401
    STATE_ROWS,
    cache_positions,
    prologue,
    rms_norm,
    short_conv,
)
from .mx_oracle import (  # noqa: F401
    E4M3_MAX,
    MX_BLOCK,
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    e8m0_value,
    mx_dequantize,
    mx_quantize,
    mx_round,
)
from .backward_oracle import (  # noqa: F401
    prefill_backward,
)
