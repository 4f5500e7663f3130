"""Algorithmic work counts for roofline reporting (what the method must move or compute).

Sources (cited by page and section):
  P1  "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576)
  P2  "大模型推理性能优化：Prefill与Decode瓶颈及KV缓存显存管理" (wmrh.cn/news/64708)
  P3  prefill/decode article on the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127)

* Attention FLOPs: P3 §2.2 counts 2*2*L*S^2*d for a dense (non-causal) prefill -- one
  multiply-add per (query, key, channel) for Q K^T and again for P V.  Over causal visible pairs
  only, a request with q_len q over seq_len s has q*(s-q) + q*(q+1)/2 visible (query, key) pairs,
  so FLOPs = 4 * d * Hq * sum_b visible_pairs_b (softmax exponentials not counted).
* KV bytes: P3 §2.3 gives bytes = 2 * L * n_kv_heads * d_head * S * B * bytes_per_elem; a decode
  step reads every cached key and value once per KV head (P3 §3.2).  GQA sharing means a KV row is
  counted once per KV head, never per query head.
* Sliding window W (P2 §5.2, P3 §6.3): the row at position p sees min(p + 1, W) keys, and a request
  needs its keys from max(0, ctx - W + 1) on, ctx = s - q; W = 0 means no window.
"""
from __future__ import annotations

import numpy as np

MI355X_HBM_BYTES_PER_S = 8.0e12        # published HBM3E peak
MI355X_BF16_DENSE_FLOPS = 2.5166e15    # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense (no sparsity)
MI355X_FP32_VECTOR_FLOPS = 157.3e12


def _tri(n):
    """1 + 2 + ... + n for n >= 0."""
    return n * (n + 1) // 2


def visible_pairs(q_lens, seq_lens, window: int = 0) -> int:
    """Visible (query row, key) pairs: sum over rows p = ctx .. s-1 of min(p + 1, W)."""
    q = np.asarray(q_lens, dtype=np.int64)
    s = np.asarray(seq_lens, dtype=np.int64)
    if window <= 0:
        return int(np.sum(q * (s - q) + q * (q + 1) // 2))
    lo, hi = s - q + 1, s                       # u = p + 1 runs over lo .. hi
    a = np.minimum(hi, window)                  # u <= W contribute u
    below = np.where(a >= lo, _tri(a) - _tri(lo - 1), 0)
    above = (hi - np.maximum(lo, window + 1) + 1).clip(min=0) * window
    return int(np.sum(below + above))


def attention_flops(q_lens, seq_lens, num_q_heads: int, head_dim: int, window: int = 0) -> int:
    """Visible-pair FLOPs of Q K^T and P V (causal, optionally windowed)."""
    return 4 * head_dim * num_q_heads * visible_pairs(q_lens, seq_lens, window)


def needed_keys(q_lens, seq_lens, window: int = 0) -> int:
    """Keys a pass must read per KV head: s for each request, or s - max(0, s - q - W + 1) with a window."""
    q = np.asarray(q_lens, dtype=np.int64)
    s = np.asarray(seq_lens, dtype=np.int64)
    if window <= 0:
        return int(np.sum(s))
    return int(np.sum(s - np.maximum(0, s - q - window + 1)))


def dense_prefill_attention_flops(num_layers: int, seq_len: int, hidden: int) -> float:
    """P3 §2.2's dense count 2 * 2 * L * S^2 * d (hidden size d, all S x S pairs)."""
    return 2.0 * 2.0 * num_layers * float(seq_len) ** 2 * hidden


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, esz: int) -> int:
    """P3 §2.3: 2 (K and V) * L * n_kv_heads * d_head * bytes_per_elem."""
    return 2 * num_layers * num_kv_heads * head_dim * esz


def kv_read_bytes(seq_lens, num_kv_heads: int, head_dim: int, esz: int, q_lens=None, window: int = 0) -> int:
    """Bytes of K and V one attention pass must read: every visible key once per KV head."""
    if window > 0:
        n = needed_keys(q_lens, seq_lens, window)
    else:
        n = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    return n * 2 * num_kv_heads * head_dim * esz


def append_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, esz: int) -> int:
    """KV append: each token's K and V rows read once and written once."""
    return 2 * 2 * num_tokens * num_kv_heads * head_dim * esz


def blocks_needed(num_tokens: int, block_size: int = 16) -> int:
    return -(-int(num_tokens) // block_size)
