"""CPU oracle for paged-KV attention (test infrastructure only; see pagedkv_oracle)."""
from .pagedkv_oracle import (  # noqa: F401
    BLOCK_SIZE,
    attention_contiguous,
    gather,
    kv_write,
    paged_attention,
    step,
    to_f64,
)
