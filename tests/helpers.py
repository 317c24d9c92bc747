"""Shared test helpers: move seeded cases to the oracle's numpy types and compare results."""

import numpy as np
import torch

import oracle

MAX_ABS = 1e-2      # bf16 outputs vs the fp64 oracle
MEAN_ABS = 1e-3
LSE_ABS = 1e-3
# fp8 prefill rounds P to e4m3 (the kernel's approximation, not part of the definition): max-abs
# 3e-2 is the fp8 bar; the mean-abs bar stays the bf16 one (1e-3). The fp8-KV attention calls
# consume the same codes as the oracle, so they are held to the bf16 bars, counting what exceeds the
# output's own bf16 rounding (code * scale is not a bf16 value, so a row that sees one key outputs an
# O(1) value that no bf16 output can match to 1e-2 when it is above 4 in magnitude).
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


def round_bf16(x):
    """float64 -> the float64 value of bf16(fp32(x)) (round to nearest even at each step): the two
    roundings a kernel's fp32 result goes through on its way to a bf16 output."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def half_ulp_bf16(x):
    """Half the spacing of bf16 values at |x| (bf16 keeps 8 significant bits): the largest error a
    correctly rounded bf16 output of x can have."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 0.0)


def compare(out, lse, ref_out, ref_lse, max_abs=MAX_ABS, mean_abs=MEAN_ABS, lse_abs=LSE_ABS, label="",
            rounded_ref=False, beyond_rounding=False):
    """out/lse: GPU tensors; ref_*: oracle numpy (NaN marks entries the oracle did not compute).
    rounded_ref: measure the output error against the oracle's result rounded to bf16 as a kernel's
    fp32 result is (the output format's own rounding is then not counted as error).
    beyond_rounding: an element's error is what its distance to the oracle exceeds half a bf16 ulp of
    the oracle value by (the error a correctly rounded bf16 output may have is not counted)."""
    o = bf16_np(out)
    mask = ~np.isnan(ref_out)
    assert mask.any(), "nothing to compare"
    ref_c = round_bf16(ref_out[mask]) if rounded_ref else ref_out[mask]
    err = np.abs(o[mask] - ref_c)
    if beyond_rounding:
        err = np.maximum(err - half_ulp_bf16(ref_out[mask]), 0.0)
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
