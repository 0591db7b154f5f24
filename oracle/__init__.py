"""CPU oracle for the Qwen3 attention-sublayer core: QK-Norm, rotate-half RoPE,
causal grouped-query softmax attention (prefill over packed sequences, and
appending new tokens against a cache of already-normed, already-rotated keys);
(``oracle.layer``) the sublayer around it: the bias-free q/k/v projections
before the core and o_proj after it; and (``oracle.gated``) the gated
global-attention layer of Qwen3-Next / Qwen3.5: zero-centred norm, partial
RoPE, per-head sigmoid output gate, and its sublayer with the projections.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library under ``attention_qk_norm_amd/``, and imports
nothing from there.

Everything is plain numpy in float64, written from the definitions on the
pages (cited per function by page title and section).  Inputs are converted
exactly to float64; nothing is rounded on the way.  Pinning: every function is
pinned by closed forms, invariants, special cases and brute force in
``tests/test_oracle_pins.py``; no function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    kv_head_for_q_head,
    rms_norm_heads,
    rope_inv_freq,
    rope_rotate_half,
    qk_norm_rope,
    causal_softmax,
    attention_prefill,
    attention_prefill_rows,
    attention_append,
    attention_decode,
)
from .layer import (  # noqa: F401
    linear,
    split_heads,
    merge_heads,
    qkv_projection,
    attention_layer_prefill,
    attention_layer_prefill_rows,
    attention_layer_append,
)
from .gated import (  # noqa: F401
    rotary_dim,
    rms_norm_zero_centred,
    rope_partial,
    gated_qk_norm_rope,
    split_query_gate,
    sigmoid,
    gated_attention_prefill,
    gated_attention_prefill_rows,
    gated_attention_append,
    gated_qkv_projection,
    gated_attention_layer_prefill,
    gated_attention_layer_prefill_rows,
    gated_attention_layer_append,
)
