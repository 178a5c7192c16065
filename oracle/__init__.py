"""fp64 CPU oracle (test infrastructure only; never on the product path).

Importable by the tests, the package entry's ``smoke()`` check and the
benchmark's CPU-baseline leg, and by nothing else.
"""
from . import blocksparse, dropout, fp8, varlen
from .attention import attention_backward, attention_forward, attention_forward_kv, attention_probs

__all__ = ["attention_forward", "attention_forward_kv", "attention_backward", "attention_probs", "blocksparse", "dropout", "fp8", "varlen"]
