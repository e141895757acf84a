"""fp64 CPU oracle for MLA absorbed decode, the latent down-projection and
explicit-form prefill.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may import, call or execute anything under oracle/.  It shares no
code with the HIP path, and the HIP path never imports it.
"""
from .codecs import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode_satfinite, f64_to_bf16_bits  # noqa: F401
from .mla_oracle import (  # noqa: F401
    absorb_query, cache_rows, fp8_cache_codes, decode_absorbed, decode_explicit, fp8_quantize_rows,
    latent_attention, mha_cache_elements_per_token, mla_cache_bytes_per_token,
    mla_cache_elements_per_token, out_projection, prefill_explicit, project_latent, reference_decode,
    reference_decode_multi, reference_prefill, rope,
    sequence_rows, softmax_with_lse,
)
