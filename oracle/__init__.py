"""CPU oracle (float64, NumPy) for speculative-verify MLA attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the product path.  See ``mla_oracle`` for what is
computed and which passages each function follows.
"""
from .mla_oracle import (  # noqa: F401
    absorb_query, attend_chunk, bf16_to_f64, fp8_e4m3_to_f64, gated_output, kv_decoder,
    lse_merge, request_keys,
    sigmoid, softmax_attend, split_pages, token_bound, verify_attention_latent,
    verify_attention_mla,
)
