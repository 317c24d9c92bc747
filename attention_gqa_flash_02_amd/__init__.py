"""Exact grouped-query softmax attention over a KV cache on AMD MI355X (gfx950).

A thin Python binding of the C ABI declared in include/attn_gqa.h: each
function below has the name of the C entry point it calls and only marshals
arguments (torch tensors -> device pointers and sizes, the current HIP stream).
Every step of the computation runs in the HIP kernels of lib/libattn_gqa.so;
there is no fallback: if the library is not built, calls raise.

PyTorch is used for device memory (outputs, workspace) and streams only.
"""

import torch

from . import _lib
from .workmodel import visible_pairs, prefill_flops, kv_bytes

__all__ = [
    "AttnError",
    "ATTN_KV_BF16",
    "ATTN_KV_FP8_E4M3FN",
    "attn_status_string",
    "attn_prefill_varlen",
    "attn_prefill_varlen_fp8",
    "attn_decode_num_splits",
    "attn_decode_workspace_bytes",
    "attn_decode_paged",
    "attn_decode_paged_noalloc",
    "ATTN_DECODE_NOALLOC_MAX_BYTES",
    "attn_varlen_workspace_bytes",
    "attn_varlen_paged",
    "attn_kv_append_paged",
    "library_path",
]

ATTN_KV_BF16 = 0
ATTN_KV_FP8_E4M3FN = 1
ATTN_DECODE_NOALLOC_MAX_BYTES = 16 << 20


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = int(status)
        super().__init__(f"{where}: {attn_status_string(status)}")


def library_path():
    return _lib.LIB_PATH


def attn_status_string(status):
    return _lib.load().attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(t, name, dtype, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_ndim(t, name, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _check_out(out, lse, out_shape, lse_shape, dev):
    if out is not None:
        _check(out, "out", torch.bfloat16, dev, out_shape)
    if lse is not None:
        _check(lse, "lse", torch.float32, dev, lse_shape)


def _kv_dtype(cache):
    if cache.dtype == torch.bfloat16:
        return ATTN_KV_BF16
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return ATTN_KV_FP8_E4M3FN
    raise TypeError(f"unsupported KV cache dtype {cache.dtype}")


def _check_caches(k_cache, v_cache, head_dim, dev, k_scale, v_scale):
    """k_cache [N, Hkv, bs, D], v_cache [N, Hkv, D, bs] (tokens innermost), same dtype, on dev; fp8
    caches need k_scale / v_scale fp32 [Hkv]. Returns (kv dtype code, N, Hkv, bs)."""
    kvt = _kv_dtype(k_cache)
    if _kv_dtype(v_cache) != kvt or k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must have the same dtype")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check_ndim(t, name, 4)
        if not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be contiguous on {dev}")
    nblk, hkv, bs, d = k_cache.shape
    if d != head_dim:
        raise ValueError(f"k_cache head_dim {d} does not match the queries' {head_dim}")
    if tuple(v_cache.shape) != (nblk, hkv, d, bs):
        raise ValueError(f"v_cache must be [num_blocks, Hkv, head_dim, block_size] = {(nblk, hkv, d, bs)} "
                         f"(tokens innermost), got {tuple(v_cache.shape)}")
    if kvt == ATTN_KV_FP8_E4M3FN:
        _check(k_scale, "k_scale", torch.float32, dev, (hkv,))
        _check(v_scale, "v_scale", torch.float32, dev, (hkv,))
    return kvt, nblk, hkv, bs


def _max_len(cu):
    cu = cu.cpu()
    return int((cu[1:] - cu[:-1]).max()) if cu.numel() > 1 else 0


def attn_prefill_varlen(q, k, v, cu_seqlens, causal, scale, out=None, lse=None, max_seqlen=None,
                        return_lse=True, stream=None, window=0):
    """q [T, Hq, D], k/v [T, Hkv, D] bf16; cu_seqlens int32 [B+1] on the same device; window > 0 = a
    sliding window of that many keys. Returns (out [T, Hq, D] bf16, lse [T, Hq] fp32 or None)."""
    dev = q.device
    _check(q, "q", torch.bfloat16, dev)
    _check_ndim(q, "q", 3)
    total, hq, d = q.shape
    _check(k, "k", torch.bfloat16, dev)
    _check_ndim(k, "k", 3)
    hkv = k.shape[1]
    _check(k, "k", torch.bfloat16, dev, (total, hkv, d))
    _check(v, "v", torch.bfloat16, dev, (total, hkv, d))
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _check_ndim(cu_seqlens, "cu_seqlens", 1)
    _check_out(out, lse, (total, hq, d), (total, hq), dev)
    if max_seqlen is None:
        max_seqlen = _max_len(cu_seqlens)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((total, hq), dtype=torch.float32, device=dev)
    st = _lib.load().attn_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), int(bool(causal)), float(scale), _ptr(out), _ptr(lse),
        cu_seqlens.numel() - 1, total, int(max_seqlen), hq, hkv, d, int(window), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_prefill_varlen")
    return out, lse


def attn_prefill_varlen_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens, causal, scale, out=None, lse=None,
                            max_seqlen=None, return_lse=True, stream=None, window=0):
    """q [T, Hq, 128], k/v [T, Hkv, 128] e4m3fn codes (torch.uint8 or torch.float8_e4m3fn); q_scale [Hq],
    k_scale/v_scale [Hkv] fp32; cu_seqlens int32 [B+1]; all on one device. Returns (out [T, Hq, 128] bf16,
    lse [T, Hq] fp32 or None)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name} must hold e4m3fn codes (uint8 or float8_e4m3fn)")
        _check(t, name, t.dtype, dev)
        _check_ndim(t, name, 3)
    total, hq, d = q.shape
    hkv = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (total, hkv, d):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(total, hkv, d)}")
    _check(q_scale, "q_scale", torch.float32, dev, (hq,))
    _check(k_scale, "k_scale", torch.float32, dev, (hkv,))
    _check(v_scale, "v_scale", torch.float32, dev, (hkv,))
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _check_ndim(cu_seqlens, "cu_seqlens", 1)
    _check_out(out, lse, (total, hq, d), (total, hq), dev)
    if max_seqlen is None:
        max_seqlen = _max_len(cu_seqlens)
    if out is None:
        out = torch.empty((total, hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((total, hq), dtype=torch.float32, device=dev)
    st = _lib.load().attn_prefill_varlen_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(cu_seqlens),
        int(bool(causal)), float(scale), _ptr(out), _ptr(lse),
        cu_seqlens.numel() - 1, total, int(max_seqlen), hq, hkv, d, int(window), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_prefill_varlen_fp8")
    return out, lse


def attn_decode_num_splits(num_seqs, num_kv_heads, head_dim, kv_dtype, block_size, max_blocks_per_seq,
                           requested=0):
    return int(_lib.load().attn_decode_num_splits(num_seqs, num_kv_heads, head_dim, kv_dtype, block_size,
                                                  max_blocks_per_seq, requested))


def attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits):
    return int(_lib.load().attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits))


def attn_varlen_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits):
    return int(_lib.load().attn_varlen_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits))


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return workspace
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() or workspace.device != device:
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale=None, v_scale=None,
                      out=None, lse=None, num_splits=0, workspace=None, return_lse=True, stream=None, window=0):
    """q [B, Hq, D] bf16; k_cache [N, Hkv, bs, D], v_cache [N, Hkv, D, bs] (bf16, or uint8 e4m3fn codes
    with k_scale/v_scale fp32 [Hkv]); block_table int32 [B, max_blocks]; seq_lens int32 [B]."""
    dev = q.device
    _check(q, "q", torch.bfloat16, dev)
    _check_ndim(q, "q", 3)
    b, hq, d = q.shape
    kvt, nblk, hkv, bs = _check_caches(k_cache, v_cache, d, dev, k_scale, v_scale)
    _check(block_table, "block_table", torch.int32, dev)
    _check_ndim(block_table, "block_table", 2)
    if block_table.shape[0] != b:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {b} requests")
    _check(seq_lens, "seq_lens", torch.int32, dev, (b,))
    _check_out(out, lse, (b, hq, d), (b, hq), dev)
    maxblk = block_table.shape[1]
    splits = attn_decode_num_splits(b, hkv, d, kvt, bs, maxblk, num_splits)
    ws = _workspace(attn_decode_workspace_bytes(b, hq, d, splits), dev, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, hq), dtype=torch.float32, device=dev)
    st = _lib.load().attn_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), float(scale), _ptr(out),
        b, hq, hkv, d, bs, nblk, maxblk, splits, _ptr(lse),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        kvt, _ptr(k_scale), _ptr(v_scale), int(window), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged")
    return out, lse


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale=None, v_scale=None,
                              out=None, lse=None, num_splits=0, return_lse=True, stream=None, window=0):
    """attn_decode_paged without a workspace: the partials go to the library's own fixed device
    array (ATTN_DECODE_NOALLOC_MAX_BYTES per GPU). With out (and lse, or return_lse=False) given,
    nothing is allocated on this path either."""
    dev = q.device
    _check(q, "q", torch.bfloat16, dev)
    _check_ndim(q, "q", 3)
    b, hq, d = q.shape
    kvt, nblk, hkv, bs = _check_caches(k_cache, v_cache, d, dev, k_scale, v_scale)
    _check(block_table, "block_table", torch.int32, dev)
    _check_ndim(block_table, "block_table", 2)
    if block_table.shape[0] != b:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {b} requests")
    _check(seq_lens, "seq_lens", torch.int32, dev, (b,))
    _check_out(out, lse, (b, hq, d), (b, hq), dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, hq), dtype=torch.float32, device=dev)
    st = _lib.load().attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), float(scale), _ptr(out),
        b, hq, hkv, d, bs, nblk, block_table.shape[1], int(num_splits), _ptr(lse),
        kvt, _ptr(k_scale), _ptr(v_scale), int(window), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_noalloc")
    return out, lse


def attn_varlen_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, causal, scale,
                      k_scale=None, v_scale=None, out=None, lse=None, max_q_len=None, num_splits=0,
                      workspace=None, return_lse=True, stream=None, window=0):
    """Mixed varlen batch (prefill chunks over cached prefixes and decode tokens) over a paged cache:
    q [Tq, Hq, D] bf16, caches as for attn_decode_paged, cu_seqlens_q int32 [B+1], seq_lens_k int32 [B]."""
    dev = q.device
    _check(q, "q", torch.bfloat16, dev)
    _check_ndim(q, "q", 3)
    tq, hq, d = q.shape
    kvt, nblk, hkv, bs = _check_caches(k_cache, v_cache, d, dev, k_scale, v_scale)
    _check(seq_lens_k, "seq_lens_k", torch.int32, dev)
    _check_ndim(seq_lens_k, "seq_lens_k", 1)
    b = seq_lens_k.numel()
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, (b + 1,))
    _check(block_table, "block_table", torch.int32, dev)
    _check_ndim(block_table, "block_table", 2)
    if block_table.shape[0] != b:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {b} requests")
    _check_out(out, lse, (tq, hq, d), (tq, hq), dev)
    maxblk = block_table.shape[1]
    if max_q_len is None:
        max_q_len = _max_len(cu_seqlens_q)
    splits = attn_decode_num_splits(b, hkv, d, kvt, bs, maxblk, num_splits)
    ws = _workspace(attn_varlen_workspace_bytes(b, hq, d, splits), dev, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=dev)
    st = _lib.load().attn_varlen_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), kvt, _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(cu_seqlens_q), _ptr(seq_lens_k), int(bool(causal)), float(scale), _ptr(out), _ptr(lse),
        b, tq, int(max_q_len), hq, hkv, d, bs, nblk, maxblk, splits, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), int(window), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_varlen_paged")
    return out, lse


def attn_kv_append_paged(k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_new, seq_lens_k,
                         k_scale=None, v_scale=None, stream=None):
    """Write new tokens' K/V (k_new, v_new [T_new, Hkv, D] bf16) into a paged cache in place:
    request b's rows cu_seqlens_new[b] .. cu_seqlens_new[b+1]-1 become its last cached tokens
    (seq_lens_k counts them). k_cache [N, Hkv, bs, D] / v_cache [N, Hkv, D, bs] are bf16, or uint8 /
    float8_e4m3fn codes quantised with k_scale / v_scale [Hkv] fp32."""
    dev = k_new.device
    _check(k_new, "k_new", torch.bfloat16, dev)
    _check_ndim(k_new, "k_new", 3)
    t_new, hkv, d = k_new.shape
    _check(v_new, "v_new", torch.bfloat16, dev, (t_new, hkv, d))
    kvt, nblk, hkv_c, bs = _check_caches(k_cache, v_cache, d, dev, k_scale, v_scale)
    if hkv_c != hkv:
        raise ValueError(f"the caches hold {hkv_c} KV heads, k_new {hkv}")
    _check(seq_lens_k, "seq_lens_k", torch.int32, dev)
    _check_ndim(seq_lens_k, "seq_lens_k", 1)
    b = seq_lens_k.numel()
    _check(cu_seqlens_new, "cu_seqlens_new", torch.int32, dev, (b + 1,))
    _check(block_table, "block_table", torch.int32, dev)
    _check_ndim(block_table, "block_table", 2)
    if block_table.shape[0] != b:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {b} requests")
    st = _lib.load().attn_kv_append_paged(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), kvt, _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(cu_seqlens_new), _ptr(seq_lens_k), seq_lens_k.numel(), t_new, hkv, d, bs,
        nblk, block_table.shape[1], _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_kv_append_paged")
