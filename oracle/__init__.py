"""fp64 CPU oracle for paged-KV attention (test infrastructure only)."""
from .ref import attention, decode, gather, kv_write, softmax_attention, to_f64

__all__ = ["attention", "decode", "gather", "kv_write", "softmax_attention", "to_f64"]
