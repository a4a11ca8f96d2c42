"""fp64 CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python
binding) never imports it and shares no code with it.
"""

from .attention import (  # noqa: F401
    attention_probs,
    attn_backward,
    attn_backward_delta,
    attn_forward,
    attn_forward_rows,
    band_mask,
    kv_head,
    qknorm,
    rms_norm,
    rms_norm_backward,
    rope_angles,
    rope_rotate,
    rope_rotate_back,
    rope_tables,
    sssl_windows,
    ve_backward,
    ve_gate,
    ve_layers,
    ve_mix,
)
from .muon import POLAR_EXPRESS_COEFFS, polar_express, polar_step  # noqa: F401,E402
