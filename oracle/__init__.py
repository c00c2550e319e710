"""Reference oracle for the sparse Mixture-of-Experts layer forward pass.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 CPU
implementation of what the layer computes, written from the page
"How Mixture of Experts Scales Model Parameters" (zhangchitc.github.io).
Only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The GPU product path
never calls it and shares no code with it: it decodes the same raw input
bytes with its own decoders and computes every expert densely before
masking.
"""

from .moe_oracle import (  # noqa: F401
    decode_bf16,
    decode_f32,
    decode_e2m1,
    decode_e8m0,
    decode_mxfp4,
    decode_e4m3,
    round_e4m3,
    encode_e4m3,
    quantize_mxfp8,
    decode_mxfp8,
    mxfp8_round,
    decode_matrix,
    router_logits,
    softmax_rows,
    topk_select,
    topk_weights,
    swiglu_expert,
    forward,
    dispatch,
    aux_loss,
    active_experts,
    resolve_slots,
)
