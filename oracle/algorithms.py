"""The pages' tiled attention algorithms, written step by step in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These exist to pin the pages' claims that the tiled methods reach the plain
definition exactly (up to rounding order), so that the GPU kernels may be
compared against ``attention.attend``:

* online softmax ("Attention kernels", section "FlashAttention"): walk the K
  blocks one at a time; per block update each row's running maximum and
  running exponential sum, and when the maximum moves, multiply what has been
  accumulated so far by the correction factor; after the last block the result
  equals attention over the whole row;
* split-KV decode ("Attention kernels", section "Prefill and decode
  attention"): cut the KV axis into pieces, attend within each piece, and
  combine the pieces "the same way as online softmax" -- here, weighting each
  piece by exp(its log-sum-exp minus the largest one).
"""

import numpy as np


def _visible(lq, lk, causal):
    """Bottom-right causal visibility [Lq, Lk] in global key positions."""
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= (lk - lq) + i


def online_softmax_attend(q, k, v, scale, causal, tile):
    """Online-softmax attention over K/V blocks of ``tile`` keys. Returns (o, lse)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    vis = _visible(lq, lk, causal)
    m = np.full(lq, -np.inf)            # running row maximum
    l = np.zeros(lq)                    # running sum of exp(s - m)
    acc = np.zeros((lq, v.shape[1]))    # running un-normalised output
    for start in range(0, lk, tile):
        stop = min(start + tile, lk)
        s = scale * (q @ k[start:stop].T)
        s = np.where(vis[:, start:stop], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        base = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - base)        # correction factor for what was accumulated
        p = np.exp(s - base[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[start:stop]
        m = m_new
    empty = l == 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        o = acc / l[:, None]
        lse = m + np.log(l)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine per-piece results: o_parts [S, Lq, D] (each normalised by its own
    sum), lse_parts [S, Lq] (-inf for a piece with no visible key)."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    big = lse_parts.max(axis=0)
    empty = ~np.isfinite(big)
    base = np.where(empty, 0.0, big)
    w = np.exp(lse_parts - base[None, :])                  # exp(-inf) = 0 for empty pieces
    total = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (w[:, :, None] * o_parts).sum(axis=0) / total[:, None]
        lse = base + np.log(total)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def split_kv_attend(q, k, v, scale, causal, num_splits):
    """Split-KV attention: ``num_splits`` contiguous key pieces of
    ceil(Lk / num_splits) keys (trailing pieces may be empty), merged by LSE."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    vis = _visible(lq, lk, causal)
    chunk = -(-lk // num_splits) if lk else 0
    o_parts = np.zeros((num_splits, lq, v.shape[1]))
    lse_parts = np.full((num_splits, lq), -np.inf)
    for sp in range(num_splits):
        start, stop = sp * chunk, min((sp + 1) * chunk, lk)
        if stop <= start:
            continue
        s = scale * (q @ k[start:stop].T)
        s = np.where(vis[:, start:stop], s, -np.inf)
        m = s.max(axis=1)
        ok = np.isfinite(m)
        base = np.where(ok, m, 0.0)
        e = np.exp(s - base[:, None])
        l = e.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            o_parts[sp] = np.where(ok[:, None], (e @ v[start:stop]) / l[:, None], 0.0)
            lse_parts[sp] = np.where(ok, base + np.log(l), -np.inf)
    return merge_partials(o_parts, lse_parts)
