"""MI355X-native Kimi Delta Attention (KDA) decode step.

The product is ``libkda.so`` (HIP for gfx950, C ABI in ``include/kda.h``);
this package holds its sources (``csrc/``), its build script (``build.py``)
and a thin ctypes binding (``kda.py``) with the same entry-point names.
"""
from .kda import (  # noqa: F401
    EXPORTS,
    KDA_GATE_BOUNDED,
    KDA_GATE_SOFTPLUS,
    KDA_STATE_BF16,
    KDA_STATE_F32,
    KdaError,
    kda_conv_step,
    kda_decode_layer_step,
    kda_decode_multi,
    kda_decode_step,
    kda_decode_step_gated,
    kda_prefill_gated,
    kda_prefill_workspace_bytes,
    kda_recurrent_step,
    kda_status_string,
    kda_version,
    load,
)
