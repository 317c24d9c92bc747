"""Appending new tokens to a paged KV cache, written as a naive token-by-token scatter.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes ("Optimization 1: batching and attention", section 3.4 PagedAttention: the
cache is a pool of fixed-size blocks and a block table maps a request's logical blocks to
physical ones; "Attention kernels", section "Paged KV and kernels": the kernel turns block
numbers into addresses, and an FP8 cache is read directly): request b's new tokens (rows
cu_seqlens_new[b] .. cu_seqlens_new[b+1]-1 of k_new / v_new, n_b of them) become its last n_b
cached tokens, i.e. positions t = seq_lens_k[b] - n_b + i (seq_lens_k counts them, as the
attention calls do). Token t lands in physical block block_table[b, t // bs], slot t % bs:
K row [block, h, slot, :], V column [block, h, :, slot] (the layouts the attention oracle
gathers from). Nothing else changes.

Readings where the pages say nothing: a bf16 cache stores the bf16 bits unchanged; an fp8 cache
stores e4m3fn(x / scale[h]) -- the quotient computed in fp32, the precision the kernel divides
in, then rounded to the nearest code (ties to even) and saturated at 448 (``encode_e4m3fn``).
"""

import numpy as np

from .formats import encode_e4m3fn


def quantize_e4m3fn(bf16_bits, scale):
    """bf16 bit patterns [..., D] and one fp32 scale -> e4m3fn codes of x / scale (fp32 quotient)."""
    x = (np.asarray(bf16_bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    q = (x / np.float32(scale)).astype(np.float32)        # IEEE fp32 division, correctly rounded
    return encode_e4m3fn(q)


def kv_append_paged(k_cache, v_cache, k_new, v_new, block_table, cu_seqlens_new, seq_lens_k,
                    kv_format="bf16", k_scale=None, v_scale=None):
    """Return copies of the caches with the new tokens written in.

    k_cache [N, Hkv, bs, D], v_cache [N, Hkv, D, bs]: uint16 bf16 bits or uint8 e4m3fn codes.
    k_new, v_new [T_new, Hkv, D]: uint16 bf16 bits. block_table [B, max_blocks] int;
    cu_seqlens_new [B + 1]; seq_lens_k [B] (cached tokens after the append).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    hkv, bs = kc.shape[1], kc.shape[2]
    cu = np.asarray(cu_seqlens_new)
    for b in range(len(cu) - 1):
        n = int(cu[b + 1] - cu[b])
        first = int(seq_lens_k[b]) - n
        for i in range(n):
            row = int(cu[b]) + i
            t = first + i
            block = int(block_table[b][t // bs])
            slot = t % bs
            for h in range(hkv):
                if kv_format == "bf16":
                    kc[block, h, slot, :] = k_new[row, h, :]
                    vc[block, h, :, slot] = v_new[row, h, :]
                else:
                    kc[block, h, slot, :] = quantize_e4m3fn(k_new[row, h, :], k_scale[h])
                    vc[block, h, :, slot] = quantize_e4m3fn(v_new[row, h, :], v_scale[h])
    return kc, vc
