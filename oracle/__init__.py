"""CPU oracle (test infrastructure only; the library never imports it)."""
from .pq_oracle import (  # noqa: F401
    attention_weights, chunk_partials, codebook_update, decode_attention, decode_attention_paged,
    default_scale, encode, fp8_e4m3_to_float64, kmeans, merge_partials, paged_slots, reconstruct,
)
