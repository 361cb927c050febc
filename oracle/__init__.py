"""CPU float64 oracle for the RIB windowed-attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the HIP
library (``windowed_attention_implicit_amd``) and imports nothing from it.

Every function here is the plain definition of a step written out in numpy
float64 (the explicit N x N score matrix included), each citing the passage it
follows. The source tags are defined in ``oracle/rib.py``.
"""

from .rib import (  # noqa: F401
    window_coords,
    fourier_features,
    gelu,
    mlp_param_count,
    posgen,
    window_partition,
    window_unpartition,
    concat_scores,
    attention_window_fwd,
    attention_window_bwd,
    rib_window_attn_fwd,
    rib_window_attn_bwd,
    default_scale,
    gelu_grad,
    posgen_bwd,
    rpb_bias,
    rpb_attention_window_fwd,
    rpb_window_attn_fwd,
    cla_depthwise3x3,
    cla_gate,
    cla_apply,
)
