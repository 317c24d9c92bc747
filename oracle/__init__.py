"""Plain fp64 CPU oracle for exact grouped-query softmax attention over a KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``attention_gqa_flash_02_amd``) never imports it and shares no code with it.

Sources (web pages; cited by title and section):

* "Attention kernels", LLM serving book (froggydisk.github.io): sections
  "Memory round trips of standard attention" (S = QK^T, P = softmax(S) row by
  row, O = PV), "FlashAttention" (tiling + online softmax is exact, only O and
  per-row statistics are written), "Prefill and decode attention" (split-KV
  decode merged like online softmax; GQA heads share one KV read), "Paged KV
  and kernels" (block table turns block numbers into addresses; varlen batch).
* "Optimization 1: batching and attention" (beengineer500.github.io):
  section 2.2 (MHA / GQA / MQA), section 2.4 (num_key_value_heads; Llama 3
  shares one KV head among 32/8 = 4 query heads), section 3.4 (PagedAttention:
  fixed-size blocks, block table, worked example 7 -> 1 -> 3 with 4-token
  blocks).

Modules:
  formats    -- exact decoders: bf16 bit patterns and OCP fp8 e4m3fn codes.
  attention  -- the plain definition (materialised S, max-subtracted softmax,
                PV, natural-log LSE), naive token-by-token page gather, and the
                paged decode / mixed varlen / fp8 prefill entry points built on them.
  algorithms -- the pages' tiled algorithms written step by step (online
                softmax over K blocks, split-KV + LSE merge), used only to pin
                the pages' claim that they reach the plain definition exactly.
  cache      -- appending new tokens to a paged cache: a token-by-token scatter, with the
                e4m3fn quantiser for fp8 caches.
  parallel   -- a process pool over (request, head) units, for timing only.

Pins: every public function is checked in ``tests/test_oracle_*.py`` against
closed forms, brute force, a library routine or the pages' worked example.
"""

from .formats import decode_bf16_bits, decode_e4m3fn, encode_e4m3fn, E4M3FN_MAX
from .cache import kv_append_paged, quantize_e4m3fn
from .attention import (
    attend,
    prefill_varlen,
    prefill_varlen_fp8,
    gather_paged,
    decode_paged,
    varlen_paged,
)
from .algorithms import online_softmax_attend, split_kv_attend, merge_partials

__all__ = [
    "decode_bf16_bits",
    "decode_e4m3fn",
    "encode_e4m3fn",
    "quantize_e4m3fn",
    "kv_append_paged",
    "E4M3FN_MAX",
    "attend",
    "prefill_varlen",
    "prefill_varlen_fp8",
    "gather_paged",
    "decode_paged",
    "varlen_paged",
    "online_softmax_attend",
    "split_kv_attend",
    "merge_partials",
]
