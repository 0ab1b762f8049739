"""Independent fp64 CPU oracle for the QK-norm + RoPE + causal / sliding-window attention path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never calls it, and it shares no code with it.
"""

from .attention import (  # noqa: F401
    EPS_DEFAULT,
    ROPE_BASE_DEFAULT,
    attention,
    attention_layer,
    decode_attention,
    kv_head,
    qknorm_rope,
    rms_norm,
    rope_apply,
    rope_cos_sin,
    sssl_windows,
    visible,
)
from .backward import (  # noqa: F401
    attention_backward,
    attention_layer_backward,
    qknorm_rope_backward,
    rms_norm_backward,
    rope_apply_backward,
)
from .value_gate import (  # noqa: F401
    attention_layer_ve,
    attention_layer_ve_backward,
    gate_of,
    value_gate,
    value_gate_backward,
)
