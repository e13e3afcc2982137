"""Work and byte accounting for the roofline figures, and the MI355X peaks.

Bytes per token follow the KV-cache memory function on page 4, section 2.1
(2 * H_kv * D * dtype bytes per token per layer; the page prints 16.0 GB for
Llama-3-8B and 40.0 GB for Llama-3-70B at 131072 tokens, in units of 2^30
bytes).  FLOP counts are those of the attention definition (page 2, section
2.1): a score is a D-long dot product and the output a weighted sum of D-long
rows, 2*D multiply-adds per (query, key) pair, 4*D flops.
"""
from __future__ import annotations

from typing import Iterable

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# MI355X published peaks (dense; no sparsity).
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "f32": 157.3}
VALU_F32_PEAK_TFLOPS = 157.3


def kv_bytes_per_token_layer(num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K plus V bytes one token stores in one layer: 2 * H_kv * D * bytes."""
    return 2 * num_kv_heads * head_dim * dtype_bytes


def kv_cache_gib(num_layers: int, num_kv_heads: int, head_dim: int, seq_len: int,
                 dtype_bytes: int = 2) -> float:
    """Whole-model KV-cache size of one sequence in GiB (2^30 bytes)."""
    per = kv_bytes_per_token_layer(num_kv_heads, head_dim, dtype_bytes)
    return per * num_layers * seq_len / float(1 << 30)


def decode_kv_bytes(context_lens: Iterable[int], num_kv_heads: int, head_dim: int,
                    dtype: str) -> int:
    """Algorithmic HBM bytes of one decode call: every stored K and V row of
    every sequence is read once (once per KV head, not per query head)."""
    per = kv_bytes_per_token_layer(num_kv_heads, head_dim, DTYPE_BYTES[dtype])
    return sum(int(l) for l in context_lens) * per


def append_bytes(n_tokens: int, num_kv_heads: int, head_dim: int, dtype: str) -> int:
    """HBM bytes of storing n_tokens new K and V rows of the same type: each
    row is read from the new-token buffer and written to its page slot."""
    return 2 * n_tokens * num_kv_heads * head_dim * DTYPE_BYTES[dtype] * 2


def decode_unique_kv_bytes(page_lists, context_lens, num_kv_heads: int, head_dim: int,
                           page_size: int, dtype: str) -> int:
    """Bytes of distinct physical pages touched (shared-prefix pages once)."""
    seen = set()
    for pl, n in zip(page_lists, context_lens):
        for i in range((int(n) + page_size - 1) // page_size):
            seen.add(pl[i])
    return len(seen) * page_size * kv_bytes_per_token_layer(num_kv_heads, head_dim,
                                                            DTYPE_BYTES[dtype])


def prefill_pairs(kv_lens: Iterable[int], chunk_lens: Iterable[int]) -> int:
    """(query, key) pairs per query head of a causal chunk at the end of each
    sequence: row i of C sees kv_len - C + i + 1 keys."""
    total = 0
    for L, c in zip(kv_lens, chunk_lens):
        L, c = int(L), int(c)
        hist = L - c
        total += c * hist + c * (c + 1) // 2
    return total


def prefill_flops(kv_lens, chunk_lens, num_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * num_q_heads * prefill_pairs(kv_lens, chunk_lens)
