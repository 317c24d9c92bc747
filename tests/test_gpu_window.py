"""Sliding-window attention (window W > 0: row i drops keys j < Lk - Lq + i - W + 1) on every
path -- contiguous prefill, paged split-KV decode, the mixed varlen batch, fp8 KV -- against the
fp64 oracle with the same window."""

import numpy as np
import pytest
import torch

import attention_gqa_flash_02_amd as lib
import synth
from helpers import compare, oracle_paged, oracle_prefill

pytestmark = pytest.mark.gpu


def _to(case, dev):
    for k, v in list(vars(case).items()):
        if isinstance(v, torch.Tensor):
            setattr(case, k, v.to(dev))
    return case


@pytest.mark.parametrize("window", [1, 17, 64, 200])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d,hq,hkv", [(128, 8, 2), (256, 4, 4), (128, 6, 2)])
def test_prefill_window(gpu, window, causal, d, hq, hkv):
    lens = [1, 17, 64, 100, 33, 300]
    case = _to(synth.make_prefill(500 + window + d + hq, lens, hq, hkv, d, causal=causal), gpu)
    out, lse = lib.attn_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens, case.causal, case.scale,
                                       max_seqlen=case.max_seqlen, window=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_prefill(case, window=window)
    compare(out, lse, ref_o, ref_l, label=f"prefill window={window} causal={causal} d={d} hq={hq} hkv={hkv}")


def test_prefill_window_4x8192_full(gpu):
    """The windowed prefill the bench times: causal 4 x 8192, 32/8 heads, head_dim 128, a 4096-key
    window, checked on sampled (sequence, head) units; rows past 4096 see exactly 4096 keys."""
    case = _to(synth.config_case("c3"), gpu)
    out, lse = lib.attn_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens, case.causal, case.scale,
                                       max_seqlen=case.max_seqlen, window=4096)
    torch.cuda.synchronize()
    units = [(0, 3), (1, 12), (2, 21), (3, 29)]
    ref_o, ref_l = oracle_prefill(case, units=units, window=4096)
    compare(out, lse, ref_o, ref_l, label="prefill 4x8192 window=4096 full (4 units)")


@pytest.mark.parametrize("window", [1, 100, 1000, 5000])
@pytest.mark.parametrize("splits", [0, 3, 16])
def test_decode_window(gpu, window, splits):
    case = _to(synth.config_case("c2", shrink=4), gpu)      # 8 requests, lengths U[256, 2048]
    out, lse = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                     case.scale, num_splits=splits, window=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_paged(case, window=window)
    compare(out, lse, ref_o, ref_l, label=f"decode window={window} splits={splits}")


@pytest.mark.parametrize("window", [300, 2500])
def test_decode_window_long_context(gpu, window):
    case = _to(synth.config_case("c4", shrink=32), gpu)     # 2 x 4096 tokens, g = 16, bs 64
    for splits in (16, 64):
        out, lse = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                         case.scale, num_splits=splits, window=window)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_paged(case, window=window)
        compare(out, lse, ref_o, ref_l, label=f"c4/32 window={window} splits={splits}")


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("window", [5, 64, 333])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_window(gpu, kv_format, window, causal):
    q_lens = [1, 3, 37, 64, 0, 130, 1, 5]
    kv_lens = [1, 300, 37, 64 + 500, 17, 130 + 33, 2000, 5]
    gen = torch.Generator().manual_seed(600 + window)
    case = _to(synth.make_paged(600 + window, kv_lens, q_lens, 8, 2, 128, 16, kv_format=kv_format, causal=causal,
                                lengths_drawn=gen), gpu)
    for splits in (0, 3):
        out, lse = lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                                         case.seq_lens_k, case.causal, case.scale, k_scale=case.k_scale,
                                         v_scale=case.v_scale, num_splits=splits, window=window)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_paged(case, window=window)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"varlen {kv_format} window={window} causal={causal} splits={splits}")


def test_varlen_window_mixed_step_d256(gpu):
    case = _to(synth.config_case("c5", shrink=16), gpu)    # 1 chunk of 128 over a prefix + 7 decodes
    out, lse = lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                                     case.seq_lens_k, True, case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                                     window=700)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_paged(case, window=700)
    compare(out, lse, ref_o, ref_l, beyond_rounding=True, label="c5/16 window=700")
