"""Shared test helpers: move seeded cases to the oracle's numpy types and compare results."""

import numpy as np
import torch

import oracle

MAX_ABS = 1e-2      # bf16 outputs vs the fp64 oracle
MEAN_ABS = 1e-3
LSE_ABS = 1e-3
# fp8 prefill rounds P to e4m3 (the kernel's approximation, not part of the definition): max-abs
# 3e-2 is the fp8 bar; the mean-abs bar stays the bf16 one (1e-3). The fp8-KV attention calls
# consume the same codes as the oracle, so they are held to the bf16 bars.
MAX_ABS_FP8 = 3e-2
MEAN_ABS_FP8 = 1e-3


def bf16_np(t):
    """bf16 tensor (any device) -> float64 numpy via the oracle's own bit decoder."""
    bits = t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return oracle.decode_bf16_bits(bits)


def cache_np(t):
    """Paged cache tensor -> the raw numpy form the oracle decodes (uint16 bf16 bits or uint8 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def oracle_prefill(case, units=None, window=0):
    return oracle.prefill_varlen(bf16_np(case.q), bf16_np(case.k), bf16_np(case.v),
                                 case.cu_seqlens.cpu().numpy(), case.causal, case.scale, units=units, window=window)


def oracle_prefill_fp8(case, units=None, window=0):
    np_ = lambda t: t.detach().cpu().numpy()
    return oracle.prefill_varlen_fp8(np_(case.q), np_(case.k), np_(case.v), np_(case.q_scale).astype(np.float64),
                                     np_(case.k_scale).astype(np.float64), np_(case.v_scale).astype(np.float64),
                                     np_(case.cu_seqlens), case.causal, case.scale, units=units, window=window)


def oracle_paged(case, units=None, window=0):
    fmt = "bf16" if case.kv_format == "bf16" else "e4m3fn"
    ks = None if case.k_scale is None else case.k_scale.cpu().numpy().astype(np.float64)
    vs = None if case.v_scale is None else case.v_scale.cpu().numpy().astype(np.float64)
    return oracle.varlen_paged(bf16_np(case.q), cache_np(case.k_cache), cache_np(case.v_cache),
                               case.block_table.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(),
                               case.seq_lens_k.cpu().numpy(), case.causal, case.scale,
                               kv_format=fmt, k_scale=ks, v_scale=vs, units=units, window=window)


def compare(out, lse, ref_out, ref_lse, max_abs=MAX_ABS, mean_abs=MEAN_ABS, lse_abs=LSE_ABS, label=""):
    """out/lse: GPU tensors; ref_*: oracle numpy (NaN marks entries the oracle did not compute)."""
    o = bf16_np(out)
    mask = ~np.isnan(ref_out)
    assert mask.any(), "nothing to compare"
    err = np.abs(o[mask] - ref_out[mask])
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "max_ref": float(np.abs(ref_out[mask]).max())}
    if lse is not None:
        l = lse.detach().cpu().numpy().astype(np.float64)
        lm = ~np.isnan(ref_lse)
        both_inf = np.isneginf(l[lm]) & np.isneginf(ref_lse[lm])
        with np.errstate(invalid="ignore"):
            lerr = np.where(both_inf, 0.0, np.abs(l[lm] - ref_lse[lm]))
        stats["lse_max_abs"] = float(lerr.max()) if lerr.size else 0.0
    print(f"[parity] {label} {stats}", flush=True)
    assert np.isfinite(o[mask]).all(), f"{label}: non-finite outputs"
    assert stats["max_abs"] <= max_abs, f"{label}: max-abs {stats['max_abs']} > {max_abs}"
    assert stats["mean_abs"] <= mean_abs, f"{label}: mean-abs {stats['mean_abs']} > {mean_abs}"
    if lse is not None:
        assert stats["lse_max_abs"] <= lse_abs, f"{label}: lse {stats['lse_max_abs']} > {lse_abs}"
    return stats
