"""Closed forms for KV-cache sizes and pre-allocation waste.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
  (pwwt.cn/news/3010209), section "KV Cache 的内存开销与分页机制": the KV
  size is 2 (K and V) x layers x sequence length x KV heads x head size x
  bytes per element x batch; the 70B example (80 layers, 8 KV heads, 128,
  fp16); and the waste of reserving 4096 slots for short requests.
* "端侧 SLM 显存保活术…" (sheratonhq.com/news/141880), sections
  "KV Cache 的物理膨胀账本" (bytes per token per layer for 2 KV heads of 128
  in fp16, and over 24 layers) and "嵌入式轻量 Block 分配器设计" (16-token
  blocks, bytes per block, pool of 512 blocks).
"""
from __future__ import annotations


def kv_cache_bytes(num_layers: int, seq_len: int, num_kv_heads: int, head_dim: int,
                   dtype_bytes: int, batch: int = 1) -> int:
    return 2 * num_layers * seq_len * num_kv_heads * head_dim * dtype_bytes * batch


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return kv_cache_bytes(num_layers, 1, num_kv_heads, head_dim, dtype_bytes)


def block_bytes(tokens_per_block: int, bytes_per_token: int) -> int:
    return tokens_per_block * bytes_per_token


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: ceil(n / block_size)."""
    return -(-num_tokens // block_size)


def preallocation_waste(used_tokens: int, reserved_tokens: int) -> float:
    """Fraction of a fixed reservation left idle; an overflow has no waste."""
    if used_tokens >= reserved_tokens:
        return 0.0
    return 1.0 - used_tokens / reserved_tokens
