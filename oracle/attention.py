"""The plain definition of exact GQA softmax attention, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition ("Attention kernels", section "Memory round trips of standard
attention"): for one head, S = Q K^T (an Lq x Lk score matrix), P = softmax(S)
normalised row by row, O = P V. Here S is materialised in full, masked entries
are set to -inf, the softmax subtracts the row maximum before exponentiating,
and the per-row statistic written beside O is the natural-log
log-sum-exp of the scaled scores.

Readings where the pages say nothing:
  * scores are multiplied by a caller-supplied ``scale`` (1/sqrt(D) in every
    workload);
  * GQA head mapping is contiguous: query head h reads KV head h // g with
    g = Hq / Hkv ("Optimization 1", sections 2.2 and 2.4);
  * causal masking is bottom-right aligned: query row i of a request with Lq
    new tokens over Lk keys sees keys j <= Lk - Lq + i (so a chunk sees its
    whole cached prefix; with Lq == Lk this is the ordinary causal mask);
  * a row with no visible key has output 0 and lse = -inf;
  * paged caches: K pages are [num_blocks, Hkv, block_size, D] and V pages are
    [num_blocks, Hkv, D, block_size] (tokens innermost); token t of request b
    sits in physical block block_table[b, t // block_size], slot
    t % block_size ("Optimization 1", section 3.4; "Attention kernels",
    section "Paged KV and kernels");
  * decode seq_lens count every cached token including the current one;
  * sliding window W > 0 (a lower bound on the visible keys, "Optimization 1", section 2 on
    shrinking the effective KV; the NVIDIA guideline summary, principle 3): row i drops the keys
    j < (Lk - Lq) + i - W + 1, the same bottom-right alignment as the causal bound.
"""

import numpy as np

from .formats import decode_bf16_bits, decode_e4m3fn


def attend(q, k, v, scale, causal, window=0):
    """One (request, query head): q [Lq, D], k [Lk, D], v [Lk, D] float64.

    Returns (o [Lq, D], lse [Lq]). Bottom-right causal alignment when ``causal``.
    window > 0 (sliding window): row i also drops the keys j < (Lk - Lq) + i - window + 1,
    i.e. with ``causal`` it sees its own position and the window - 1 keys before it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    dv = v.shape[1] if v.ndim == 2 else q.shape[1]
    if lk == 0:
        return np.zeros((lq, dv)), np.full(lq, -np.inf)
    s = scale * (q @ k.T)                                   # S = scale * Q K^T, [Lq, Lk]
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    if causal:
        s = np.where(j <= (lk - lq) + i, s, -np.inf)
    if window > 0:
        s = np.where(j >= (lk - lq) + i - window + 1, s, -np.inf)
    m = s.max(axis=1)                                       # row maximum
    empty = ~np.isfinite(m)                                 # rows with no visible key
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])                         # masked entries -> exp(-inf) = 0
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = e / l[:, None]                                  # P = softmax(S), row by row
        lse = m_safe + np.log(l)
    p[empty] = 0.0
    lse[empty] = -np.inf
    o = p @ v                                               # O = P V
    return o, lse


def _units(num_requests, num_q_heads, units):
    if units is None:
        return [(b, h) for b in range(num_requests) for h in range(num_q_heads)]
    return [(int(b), int(h)) for b, h in units]


def prefill_varlen(q, k, v, cu_seqlens, causal, scale, units=None, window=0):
    """Varlen self-attention over contiguous K/V.

    q [T, Hq, D], k/v [T, Hkv, D] float64; cu_seqlens [B+1] (request b owns
    rows cu_seqlens[b]:cu_seqlens[b+1] of q, k and v). Returns out [T, Hq, D]
    and lse [T, Hq]; with ``units`` (a list of (request, head)) only those are
    computed and every other entry is NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    t, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = hq // hkv
    out = np.full((t, hq, v.shape[2]), np.nan)
    lse = np.full((t, hq), np.nan)
    for b, h in _units(len(cu) - 1, hq, units):
        lo, hi = cu[b], cu[b + 1]
        kvh = h // g
        o_bh, lse_bh = attend(q[lo:hi, h], k[lo:hi, kvh], v[lo:hi, kvh], scale, causal, window)
        out[lo:hi, h] = o_bh
        lse[lo:hi, h] = lse_bh
    return out, lse


def prefill_varlen_fp8(q_codes, k_codes, v_codes, q_scale, k_scale, v_scale, cu_seqlens, causal, scale,
                       units=None, window=0):
    """FP8 varlen prefill ("Attention kernels", section "FlashAttention", the third version's FP8
    variant): the exact attention of the decoded inputs.

    q_codes [T, Hq, D], k_codes / v_codes [T, Hkv, D] uint8 OCP e4m3fn codes; q_scale [Hq],
    k_scale / v_scale [Hkv]. Each input is its decoded code times its head's scale, in fp64; the
    attention itself is ``prefill_varlen`` (materialised S, softmax, P V). Rounding P to fp8 on
    the way into the P V product is the kernel's approximation of this result, not part of it.
    """
    q = decode_e4m3fn(q_codes) * np.asarray(q_scale, dtype=np.float64)[None, :, None]
    k = decode_e4m3fn(k_codes) * np.asarray(k_scale, dtype=np.float64)[None, :, None]
    v = decode_e4m3fn(v_codes) * np.asarray(v_scale, dtype=np.float64)[None, :, None]
    return prefill_varlen(q, k, v, cu_seqlens, causal, scale, units=units, window=window)


def gather_paged(k_cache, v_cache, table_row, length, kv_head):
    """Naive page gather for one request and one KV head.

    k_cache [num_blocks, Hkv, bs, D], v_cache [num_blocks, Hkv, D, bs] in any
    element type. Logical block i of the request lives in physical block
    table_row[i]; its slots 0 .. bs-1 hold tokens i*bs .. i*bs+bs-1. Returns
    K [length, D] and V [length, D] in the caches' element type.
    """
    bs = k_cache.shape[2]
    d_k = k_cache.shape[3]
    d_v = v_cache.shape[2]
    k_rows = np.empty((length, d_k), dtype=k_cache.dtype)
    v_rows = np.empty((length, d_v), dtype=v_cache.dtype)
    for logical in range((length + bs - 1) // bs):
        phys = int(table_row[logical])
        first = logical * bs
        used = min(bs, length - first)                      # the last block may be partly filled
        k_rows[first:first + used] = k_cache[phys, kv_head, :used, :]
        v_rows[first:first + used] = v_cache[phys, kv_head, :, :used].T
    return k_rows, v_rows


def _decode_rows(raw, kv_format, head_scale):
    if kv_format == "bf16":
        return decode_bf16_bits(raw)
    if kv_format == "e4m3fn":
        return decode_e4m3fn(raw) * float(head_scale)
    if kv_format == "f64":
        return np.asarray(raw, dtype=np.float64)
    raise ValueError(f"unknown kv_format {kv_format!r}")


def varlen_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, causal, scale,
                 kv_format="bf16", k_scale=None, v_scale=None, units=None, window=0):
    """Mixed varlen batch over a paged KV cache (prefill chunks and decode rows alike).

    q [Tq, Hq, D] float64; request b owns query rows cu_seqlens_q[b]:cu_seqlens_q[b+1]
    and seq_lens_k[b] cached keys (its new tokens included, at the end).
    kv_format: "bf16" (uint16 bit patterns), "e4m3fn" (uint8 codes; value =
    decoded code * k_scale[kv_head] or v_scale[kv_head]) or "f64" (float values).
    Returns out [Tq, Hq, D], lse [Tq, Hq]; entries outside ``units`` are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    cuq = [int(x) for x in cu_seqlens_q]
    lens = [int(x) for x in seq_lens_k]
    tq, hq, d = q.shape
    hkv = k_cache.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = hq // hkv
    ks = np.ones(hkv) if k_scale is None else np.asarray(k_scale, dtype=np.float64)
    vs = np.ones(hkv) if v_scale is None else np.asarray(v_scale, dtype=np.float64)
    out = np.full((tq, hq, v_cache.shape[2]), np.nan)
    lse = np.full((tq, hq), np.nan)
    gathered = {}
    for b, h in _units(len(cuq) - 1, hq, units):
        kvh = h // g
        key = (b, kvh)
        if key not in gathered:
            k_raw, v_raw = gather_paged(k_cache, v_cache, block_table[b], lens[b], kvh)
            gathered = {key: (_decode_rows(k_raw, kv_format, ks[kvh]),
                              _decode_rows(v_raw, kv_format, vs[kvh]))}
        k_rows, v_rows = gathered[key]
        lo, hi = cuq[b], cuq[b + 1]
        o_bh, lse_bh = attend(q[lo:hi, h], k_rows, v_rows, scale, causal, window)
        out[lo:hi, h] = o_bh
        lse[lo:hi, h] = lse_bh
    return out, lse


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale,
                 kv_format="bf16", k_scale=None, v_scale=None, units=None, window=0):
    """One query token per request over its paged cache: q [B, Hq, D] -> out [B, Hq, D], lse [B, Hq].

    The query is the newest cached token, so it sees all seq_lens[b] keys
    ("Attention kernels", section "Prefill and decode attention").
    """
    q = np.asarray(q, dtype=np.float64)
    nb = q.shape[0]
    cu = np.arange(nb + 1)
    return varlen_paged(q, k_cache, v_cache, block_table, cu, seq_lens, True, scale,
                        kv_format, k_scale, v_scale, units, window)
