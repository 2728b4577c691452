"""CPU oracle for the padding-removed GPT decoder-layer forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import or call this package; the product path never does.
It shares no code with the HIP library: no kernels, headers, helpers, tables
or pre/post-processing.  Its inputs come from ``workloads`` (seeded
generators) and every value it computes is its own.

What it computes, and where that comes from:
  * Energon-AI announcement article (Colossal-AI team), "Runtime" section:
    for variable-length NLP inputs the runtime adds ``transpose_padding_remove``
    and ``transpose_padding_rebuild`` ops so that the layer's work is done on
    the valid tokens only (redundant-computation elimination, RCE).
  * EnergonAI README, "Scaling Ability": RCE as first raised by
    EffectiveTransformer; GPT-3 layers in FP16; sequence length half the
    padding length.
  * The same article, "Ease of use" listing: the MLP chain is GEMM, add bias +
    GELU, GEMM, add bias + residual (then LayerNorm in that post-LN listing).

Readings where the pages are silent (each is listed with its reason in the
design notes of this repository):
  * pre-LN GPT block: a = LN1(x); h = x + Out(Attn(QKV(a))); y = h + FC2(gelu(FC1(LN2(h))));
  * LayerNorm with biased variance and eps inside the square root;
  * GeLU in the tanh form (the erf form on request);
  * attention scale 1/sqrt(head_dim), causal, keys restricted to the
    sequence's valid tokens; masked keys are skipped, never added as -inf;
  * right padding (valid tokens first); pads of the output are +0.0;
  * "transpose" in the op names: a plain gather/scatter between
    [batch, pad_len, hidden] and [valid_tokens, hidden];
  * fused QKV weight [3*H', H] laid out as q | k | v blocks, each head-major;
    every weight in nn.Linear [out, in] layout.

Precision: float64 throughout, on the exact (fp16- or fp32-stored) input
values.  Parity pins: see tests/test_oracle_*.py.
"""
from .layer import (  # noqa: F401
    offsets_from_lengths, offsets_from_mask, remove_padding, rebuild_padding,
    layer_norm, gelu, linear, causal_attention_packed, causal_attention_query, causal_attention_padded,
    layer_forward_packed, layer_forward_padded, stack_forward_padded, stack_forward_packed,
    to_f64_params, transpose_padding_rebuild_heads, transpose_padding_remove_heads, attention_padded_heads,
    add_bias_residual_layernorm, attention_packed_bidirectional, attention_via_padded_heads,
    encoder_layer_forward_packed, encoder_layer_forward_padded,
)
from .batching import (  # noqa: F401
    Cost, batch_cost, token_seconds, fifo_batches, length_order, dp_runs, dynamic_batches, padded_rows,
)
from .decode import SequenceCache, extend_sequence, extend_batch, prefill_first_layer_cache  # noqa: F401
