"""ctypes declarations of the C ABI in include/attn_gqa.h (argument types only)."""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_GQA_LIBRARY names another build of the same library to load instead (the host-ASan build of
# the validation tests).
LIB_PATH = os.environ.get("ATTN_GQA_LIBRARY") or os.path.join(_PKG, "lib", "libattn_gqa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "attn_gqa.h")

c_void_p = ctypes.c_void_p
c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float
c_size = ctypes.c_size_t
c_fp = ctypes.POINTER(ctypes.c_float)
c_ip = ctypes.POINTER(ctypes.c_int32)

SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [c_i32]),
    # q, k, v, cu_seqlens, causal, scale, out, lse, num_seqs, total_tokens, max_seqlen, Hq, Hkv, D, window, stream
    "attn_prefill_varlen": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32, c_f32, c_void_p, c_void_p,
                                    c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_void_p]),
    # q, k, v, q_scale, k_scale, v_scale, cu_seqlens, causal, scale, out, lse, num_seqs, total_tokens,
    # max_seqlen, Hq, Hkv, D, window, stream
    "attn_prefill_varlen_fp8": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_i32, c_f32, c_void_p, c_void_p, c_i32, c_i32, c_i32, c_i32,
                                        c_i32, c_i32, c_i32, c_void_p]),
    "attn_decode_num_splits": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "attn_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    # q, k_cache, v_cache, block_table, seq_lens, scale, out, num_seqs, Hq, Hkv, D, block_size, num_blocks,
    # max_blocks_per_seq, num_splits, lse, workspace, workspace_bytes, kv_dtype, k_scale, v_scale, window, stream
    "attn_decode_paged": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_f32, c_void_p,
                                  c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_void_p,
                                  c_void_p, c_size, c_i32, c_void_p, c_void_p, c_i32, c_void_p]),
    # attn_decode_paged without workspace / workspace_bytes
    "attn_decode_paged_noalloc": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_f32, c_void_p,
                                          c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_void_p,
                                          c_i32, c_void_p, c_void_p, c_i32, c_void_p]),
    "attn_varlen_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    # q, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, cu_seqlens_q, seq_lens_k, causal, scale,
    # out, lse, num_seqs, total_q, max_q_len, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
    # num_splits, workspace, workspace_bytes, window, stream
    "attn_varlen_paged": (c_i32, [c_void_p, c_void_p, c_void_p, c_i32, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_i32, c_f32, c_void_p, c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                  c_i32, c_i32, c_i32, c_i32, c_i32, c_void_p, c_size, c_i32, c_void_p]),
    "attn_kv_append_paged": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                     c_void_p]),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load():
    """Load lib/libattn_gqa.so once and declare every entry point; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run `python -m attention_gqa_flash_02_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
