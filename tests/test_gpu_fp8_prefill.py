"""FP8 prefill (e4m3fn Q/K/V with per-head scales, fp8 MFMA, P rounded to e4m3) against the fp64
oracle of the decoded inputs: ragged varlen batches, causal and not, sliding windows, group sizes
1-8, the 4 x 8192 workload on sampled (request, head) units, and the edge cases."""

import numpy as np
import pytest
import torch

import attention_gqa_flash_02_amd as lib
import synth
from helpers import compare, oracle_prefill_fp8, MAX_ABS_FP8, MEAN_ABS_FP8

pytestmark = pytest.mark.gpu


def _to(case, dev):
    for k, v in list(vars(case).items()):
        if isinstance(v, torch.Tensor):
            setattr(case, k, v.to(dev))
    return case


def _run(case, window=0):
    out, lse = lib.attn_prefill_varlen_fp8(case.q, case.k, case.v, case.q_scale, case.k_scale, case.v_scale,
                                           case.cu_seqlens, case.causal, case.scale,
                                           max_seqlen=max(case.seqlens), window=window)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 4), (16, 2), (6, 2), (32, 2)])
def test_fp8_prefill_ragged(gpu, causal, hq, hkv):
    lens = [1, 17, 64, 65, 200, 1000, 31]
    case = _to(synth.make_prefill_fp8(900 + hq * 10 + hkv, lens, hq, hkv, 128, causal=causal), gpu)
    out, lse = _run(case)
    ref_o, ref_l = oracle_prefill_fp8(case)
    compare(out, lse, ref_o, ref_l, max_abs=MAX_ABS_FP8, mean_abs=MEAN_ABS_FP8,
            label=f"fp8 prefill causal={causal} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("window", [1, 17, 64, 300])
def test_fp8_prefill_window(gpu, window):
    lens = [700, 129, 33]
    case = _to(synth.make_prefill_fp8(950 + window, lens, 8, 2, 128), gpu)
    out, lse = _run(case, window=window)
    ref_o, ref_l = oracle_prefill_fp8(case, window=window)
    if window == 1:
        # Every row sees one key (P = 1 exactly), so the output is that key's decoded V row: an O(1)
        # value (not an average), whose bf16 rounding alone comes to a mean-abs of about 1e-3. Against
        # the oracle's result rounded to bf16 as the kernel rounds its fp32 result, the kernel must
        # be exact.
        compare(out, lse, ref_o, ref_l, max_abs=0.0, mean_abs=0.0, label="fp8 prefill window=1 vs bf16(oracle)",
                rounded_ref=True)
    else:
        compare(out, lse, ref_o, ref_l, max_abs=MAX_ABS_FP8, mean_abs=MEAN_ABS_FP8,
                label=f"fp8 prefill window={window}")


def test_fp8_prefill_long_sampled(gpu):
    """The 4 x 8192 causal workload (32/8 heads) in the launch the bench times, checked on sampled
    (request, head) units the oracle computes one by one."""
    case = _to(synth.make_prefill_fp8(3, [8192] * 4, 32, 8, 128), gpu)
    out, lse = _run(case)
    units = [(0, 0), (1, 7), (2, 19), (3, 31)]
    ref_o, ref_l = oracle_prefill_fp8(case, units=units)
    compare(out, lse, ref_o, ref_l, max_abs=MAX_ABS_FP8, mean_abs=MEAN_ABS_FP8, label="fp8 prefill 4x8192 sampled")


def test_fp8_prefill_many_sequences(gpu):
    """800 short sequences (1 to 40 tokens, a few of 300) in one fp8 call."""
    g = np.random.default_rng(880)
    lens = [int(x) for x in g.integers(1, 41, 800)]
    for i in (3, 500, 799):
        lens[i] = 300
    case = _to(synth.make_prefill_fp8(880, lens, 8, 2, 128), gpu)
    out, lse = _run(case)
    ref_o, ref_l = oracle_prefill_fp8(case)
    compare(out, lse, ref_o, ref_l, max_abs=MAX_ABS_FP8, mean_abs=MEAN_ABS_FP8, label="fp8 prefill 800 sequences")


def test_fp8_prefill_edges(gpu):
    # empty batch: nothing launched, nothing written
    case = _to(synth.make_prefill_fp8(7, [3], 4, 2, 128), gpu)
    out = torch.full((0, 4, 128), 1.0, dtype=torch.bfloat16, device=gpu)
    e = torch.zeros(0, 4, 128, dtype=torch.uint8, device=gpu)
    e2 = torch.zeros(0, 2, 128, dtype=torch.uint8, device=gpu)
    cu = torch.tensor([0, 0], dtype=torch.int32, device=gpu)
    lib.attn_prefill_varlen_fp8(e, e2, e2, case.q_scale, case.k_scale, case.v_scale, cu, True, 0.1, out=out,
                                max_seqlen=0)
    # single-token requests see only themselves: out = decoded v (times v_scale), lse = its score
    # (P = 1 exactly: against the oracle rounded to bf16 as the kernel rounds its fp32 result, exact)
    case = _to(synth.make_prefill_fp8(8, [1, 1, 1], 4, 2, 128), gpu)
    out, lse = _run(case)
    ref_o, ref_l = oracle_prefill_fp8(case)
    compare(out, lse, ref_o, ref_l, max_abs=0.0, mean_abs=0.0, rounded_ref=True, label="fp8 prefill single tokens")
    # head_dim 256 is not supported by the fp8 path
    q = torch.zeros(4, 2, 256, dtype=torch.uint8, device=gpu)
    s = torch.ones(2, dtype=torch.float32, device=gpu)
    with pytest.raises(lib.AttnError):
        lib.attn_prefill_varlen_fp8(q, q, q, s, s, s, torch.tensor([0, 4], dtype=torch.int32, device=gpu),
                                    True, 0.1, max_seqlen=4)
