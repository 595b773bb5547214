"""fp64 CPU oracle for paged-KV attention (test infrastructure only)."""
from .ref import attention, decode, gather, kv_write, softmax_attention, to_f64
from .qkv import derive_slots, qkv_rope_write, rms_norm, rope, to_stored, token_positions

__all__ = ["attention", "decode", "gather", "kv_write", "softmax_attention", "to_f64",
           "derive_slots", "qkv_rope_write", "rms_norm", "rope", "to_stored", "token_positions"]
