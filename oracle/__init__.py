"""CPU oracle for the bitwise-deterministic MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import anything in this package.  The
HIP library never calls it, and it shares no code, headers, tables or
helpers with the HIP path; both sides only consume the same seeded inputs
(package ``synth``).
"""
from .moe import (  # noqa: F401
    decode, route, permute, expert_forward, expert_backward, forward, backward,
    combine_rows, layer_loss,
)
from .fingerprint import fingerprint, mix64, DTYPE_CODE  # noqa: F401
from .router import (  # noqa: F401
    router_logits, router_probs, router_dlogits, router_backward, router_loss,
)
from .mx import (  # noqa: F401,E402
    e4m3_decode, e4m3_encode, e8m0_decode, mx_quantize, mx_quantize_fast, mx_dequantize, mx_grouped_rows,
    MXW_PAD, mx_pad_offsets, mx_quantize_expert_rows, act_p_f32, mx_wgrad,
)
from .nvfp4 import e2m1_decode, e2m1_encode, nvfp4_quantize, nvfp4_dequantize  # noqa: F401,E402
