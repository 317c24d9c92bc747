"""Algorithmic work and byte counts used to price a launch against its roofline.

Only counts that the method itself requires are used: masked score products,
padding, softmax arithmetic and re-reads are not counted.

* Prefill FLOPs: each visible (query row, key) pair of each query head costs a
  D-long dot product for QK^T and a D-long multiply-add into O for PV, i.e.
  4 * D flops ("Attention kernels", section "Memory round trips of standard
  attention": S = QK^T and O = PV are the two matrix products).
* Decode bytes: every cached K and V element of every KV head is read once
  ("Attention kernels", section "Prefill and decode attention": a decode token
  reads its request's whole KV cache, once for all query heads of a group);
  per token per KV head that is 2 * D * element_bytes, the per-layer term of
  the KV-cache size formula of the talk summary (aitrends.kr, 37:00).
"""

import numpy as np


def visible_pairs(q_len, kv_len, causal, window=0):
    """Number of (row, key) pairs a request's rows see: row i of q_len rows over
    kv_len keys sees keys [lo_i, hi_i] with hi_i = kv_len - q_len + i when causal
    (bottom-right alignment, else kv_len - 1) and lo_i = kv_len - q_len + i - window + 1
    with a sliding window (else 0), both clipped to [0, kv_len - 1]."""
    q_len, kv_len = int(q_len), int(kv_len)
    rows = np.arange(q_len, dtype=np.int64)
    hi = np.clip(kv_len - q_len + rows, -1, kv_len - 1) if causal else np.full(q_len, kv_len - 1)
    lo = np.clip(kv_len - q_len + rows - window + 1, 0, kv_len) if window > 0 else np.zeros(q_len, dtype=np.int64)
    return int(np.maximum(hi - lo + 1, 0).sum())


def prefill_flops(q_lens, kv_lens, num_q_heads, head_dim, causal=True, window=0):
    """4 * D * Hq * sum of visible pairs over requests."""
    pairs = sum(visible_pairs(a, b, causal, window) for a, b in zip(q_lens, kv_lens))
    return 4 * int(head_dim) * int(num_q_heads) * pairs


def kv_bytes(kv_lens, num_kv_heads, head_dim, elt_bytes):
    """Bytes of K and V a decode pass must read: sum(len) * 2 * Hkv * D * elt."""
    return sum(int(x) for x in kv_lens) * 2 * int(num_kv_heads) * int(head_dim) * int(elt_bytes)


def score_matrix_bytes(n, elt_bytes=2):
    """Size of one materialised N x N score matrix (what a fused kernel never writes)."""
    return int(n) * int(n) * int(elt_bytes)


def kv_cache_bytes_per_seq(seq_len, num_kv_heads, head_dim, num_layers, elt_bytes=2):
    """The talk summary's formula: S * (K * H) * L * 2 (K and V) * bytes."""
    return int(seq_len) * int(num_kv_heads) * int(head_dim) * int(num_layers) * 2 * int(elt_bytes)


def decode_intensity(group_size, elt_bytes=2):
    """Flops per KV byte for one decode token: (4 * D * g) / (2 * D * elt)."""
    return 4.0 * group_size / (2.0 * elt_bytes)
