"""GPU parity at the full workload sizes, in the launch configuration the bench times: the
batch-32 paged decode, the 4 x 8192 causal prefill (bf16; the fp8 one is in test_gpu_fp8_prefill),
the 2 x 131072 split-KV decode at 16, 64 and the library's partition count, and the mixed fp8
step. The oracle computes sampled (request, query head) units one by one; every other output is
left out of the comparison."""

import numpy as np
import pytest
import torch

import attention_gqa_flash_02_amd as lib
import synth
from helpers import compare, oracle_paged, oracle_prefill

pytestmark = pytest.mark.gpu


def _to(case, dev):
    for name, val in list(vars(case).items()):
        if isinstance(val, torch.Tensor):
            setattr(case, name, val.to(dev))
    return case


def _decode(case, splits):
    out, lse = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                     case.scale, k_scale=case.k_scale, v_scale=case.v_scale, num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


def test_decode_batch32_full(gpu):
    """32 requests, lengths U[1024, 8192], 32/8 heads, 16-token shuffled pages: 64 sampled units
    plus every head of the shortest and the longest request."""
    case = _to(synth.config_case("c2"), gpu)
    out, lse = _decode(case, 0)
    rng = np.random.default_rng(2)
    lens = case.seq_lens_k.cpu().numpy()
    units = {(int(b), int(h)) for b, h in zip(rng.integers(0, 32, 64), rng.integers(0, 32, 64))}
    units |= {(int(lens.argmin()), h) for h in range(32)} | {(int(lens.argmax()), h) for h in range(32)}
    ref_o, ref_l = oracle_paged(case, units=sorted(units))
    compare(out, lse, ref_o, ref_l, label=f"decode batch 32 full ({len(units)} units)")


def test_prefill_4x8192_full(gpu):
    """The causal 4 x 8192 prefill (32/8 heads, head_dim 128): one (sequence, head) unit per
    sequence, spread over the KV groups and the heads inside a group."""
    case = _to(synth.config_case("c3"), gpu)
    out, lse = lib.attn_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens, case.causal, case.scale,
                                       max_seqlen=case.max_seqlen)
    torch.cuda.synchronize()
    units = [(0, 0), (1, 7), (2, 19), (3, 30)]
    ref_o, ref_l = oracle_prefill(case, units=units)
    compare(out, lse, ref_o, ref_l, label="prefill 4x8192 full (4 units)")


@pytest.mark.parametrize("q_len", [4, 8])
def test_multi_token_decode_batch32_full(gpu, q_len):
    """Speculative verification on the batch-32 decode cache, as the bench times it: each request's
    last q_len cached tokens are new query rows (causal), 32/8 heads, so 16 or 32 rows per KV head
    take the split-KV decode path in one or two 16-row blocks, with the library's partition count;
    checked on sampled (request, head) units."""
    case = _to(synth.config_case("c2"), gpu)
    b, hq, d = case.q.shape
    g = torch.Generator().manual_seed(21)
    case.q = torch.randn((b * q_len, hq, d), generator=g).to(torch.bfloat16).to(gpu)
    case.cu_seqlens_q = torch.arange(0, b * q_len + 1, q_len, dtype=torch.int32, device=gpu)
    case.causal = True
    s = lib.attn_decode_num_splits(b, case.num_kv_heads, d, 0, case.block_size, case.block_table.shape[1], 0)
    out, lse = lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                                     case.seq_lens_k, True, case.scale, max_q_len=q_len, num_splits=s)
    torch.cuda.synchronize()
    units = [(0, 0), (9, 6), (17, 13), (25, 22), (31, 31)]
    ref_o, ref_l = oracle_paged(case, units=units)
    compare(out, lse, ref_o, ref_l, label=f"multi-token q_len={q_len} batch-32 full (5 units)")


@pytest.mark.parametrize("splits", [16, 64, 0])
def test_splitkv_2x131072_full(gpu, splits):
    """2 requests of 131072 cached tokens, 32/2 heads (group 16), 64-token pages: the partition
    counts of the workload (16 and 64) and the library's own choice."""
    case = _to(synth.config_case("c4"), gpu)
    out, lse = _decode(case, splits)
    units = [(0, 0), (0, 15), (1, 16), (1, 31), (0, 22)]
    ref_o, ref_l = oracle_paged(case, units=units)
    compare(out, lse, ref_o, ref_l, label=f"split-KV 2x131072 full splits={splits}")


def test_mixed_step_full(gpu):
    """The mixed fp8 step in one call: 8 prefill chunks of 2048 over prefixes U[0, 32768] and 120
    decodes over U[512, 32768], 16/4 heads, head_dim 256, e4m3fn KV with per-head scales."""
    case = _to(synth.config_case("c5"), gpu)
    out, lse = lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                                     case.seq_lens_k, case.causal, case.scale, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    torch.cuda.synchronize()
    n_pre = sum(1 for x in case.q_lens if x > 1)
    n = len(case.q_lens)
    # prefill chunks: first, middle and last chunk; decodes: first, two in the middle, last
    units = [(0, 0), (n_pre // 2, 5), (n_pre - 1, 15), (n_pre, 3), (n_pre + 50, 9), (n_pre + 90, 14), (n - 1, 12)]
    ref_o, ref_l = oracle_paged(case, units=units)
    compare(out, lse, ref_o, ref_l, beyond_rounding=True, label="mixed step full (7 units)")
