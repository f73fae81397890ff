"""KV cache sizing and utilisation (closed forms).

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, batch: int,
                   bytes_per_elem: float) -> float:
    """KV cache bytes = 2 x layers x kv_heads x head_dim x seq_len x batch x
    bytes per element, the 2 counting K and V ("KV Cache优化实战" §2.1;
    "企业官网建设流程全解析" §2.1).  For multi-head attention kv_heads x head_dim
    equals the hidden size, which is the form "KV Cache 和 vLLM" §1.3 uses."""
    return 2 * layers * kv_heads * head_dim * seq_len * batch * bytes_per_elem


def prealloc_utilisation(lengths, max_len: int) -> float:
    """Share of a max-length preallocation that holds tokens:
    sum_b L_b / (B * max_len) ("KV Cache 和 vLLM" §2.2)."""
    lengths = list(lengths)
    return sum(lengths) / (len(lengths) * max_len) if lengths else 0.0


def paged_utilisation(lengths, block_tokens: int = 16) -> float:
    """Share of allocated block slots that hold tokens when every sequence
    owns ceil(L_b / 16) private blocks: sum_b L_b / (16 * sum_b ceil(L_b/16))."""
    lengths = list(lengths)
    blocks = sum(-(-L // block_tokens) for L in lengths)
    return sum(lengths) / (block_tokens * blocks) if blocks else 0.0
