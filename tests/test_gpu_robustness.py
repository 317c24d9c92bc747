"""Robustness and invariance of the HIP path on the GPU (through the C ABI):

  * NaN poison: spare pages and the unused tail slots of every last page hold NaN (bf16 NaN, or the
    e4m3fn NaN code 0x7F); no output may change or turn non-finite, because no kernel may let a
    slot past a request's end reach its arithmetic ("Optimization 1", section 3.4: the last block
    of a request is only partly filled).
  * Physical page permutation: the same logical cache stored under another shuffle of the physical
    blocks (block table permuted to match) gives bit-identical outputs ("Attention kernels",
    section "Paged KV and kernels": the kernel reaches blocks only through the table).
  * Repeat determinism: the same inputs give bit-identical outputs call after call (the prefill
    kernels order their tile loads by hand-placed waits and barriers; a race would show here).
  * Every finite e4m3fn code through the kernels' dequantisation: with one visible key a row's
    output is that key's V row and its LSE is its score, so the decoded values must come out exact.
"""

import numpy as np
import pytest
import torch

import attention_gqa_flash_02_amd as lib
import oracle
import synth
from helpers import compare, oracle_paged

pytestmark = pytest.mark.gpu

NAN = float("nan")


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


def _varlen(case, splits):
    out, lse = lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                                     case.seq_lens_k, case.causal, case.scale, k_scale=case.k_scale,
                                     v_scale=case.v_scale, num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


def _poison_is_there(case):
    """The NaN poison really is in the cache (spare blocks exist and hold NaN / 0x7F)."""
    kc = case.k_cache.cpu()
    if kc.dtype == torch.bfloat16:
        assert torch.isnan(kc.float()).any()
    else:
        assert (kc == 0x7F).any()


# ---------------------------------------------------------------------------------------------
# NaN poison
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs", [(128, 16), (128, 64), (256, 16), (256, 256)])
def test_nan_poison_decode(gpu, kv_format, d, bs):
    lens = [1, 2, 15, 17, 63, 65, 300, 1000]        # every length leaves part of its last page unused
    gen = torch.Generator().manual_seed(800 + d + bs)
    case = synth.make_paged(800 + d + bs, lens, [1] * len(lens), 16, 4, d, bs, kv_format=kv_format,
                            poison=NAN, lengths_drawn=gen)
    _poison_is_there(case)
    case = _to(case, gpu)
    for splits in (0, 1, 7):
        out, lse = _decode(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"NaN poison decode {kv_format} d={d} bs={bs} splits={splits}")


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs", [(128, 16), (256, 16), (256, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_nan_poison_mixed(gpu, kv_format, d, bs, causal):
    """Decode rows (at head_dim 128 also a request of 24 rows per KV head: two 16-row blocks) and
    paged prefill chunks (over prefixes and without) in one call."""
    q_lens = [1, 3, 37, 64, 130, 1, 70, 6]
    kv_lens = [5, 300, 37, 64 + 500, 130 + 33, 2000, 70 + 1, 6 + 251]
    gen = torch.Generator().manual_seed(820 + d + bs)
    case = synth.make_paged(820 + d + bs, kv_lens, q_lens, 8, 2, d, bs, kv_format=kv_format, causal=causal,
                            poison=NAN, lengths_drawn=gen)
    _poison_is_there(case)
    case = _to(case, gpu)
    for splits in (0, 3):
        out, lse = _varlen(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"NaN poison mixed {kv_format} d={d} bs={bs} causal={causal} splits={splits}")


def test_nan_poison_full_size_splitkv(gpu):
    """The 2 x 131072 split-KV workload with NaN in every spare page: sampled units against the oracle."""
    case = _to(synth.config_case("c4", poison=NAN), gpu)
    out, lse = _decode(case, 0)
    units = [(0, 0), (1, 31)]
    ref_o, ref_l = oracle_paged(case, units=units)
    compare(out, lse, ref_o, ref_l, label="NaN poison 2x131072")
    assert torch.isfinite(out.float()).all()


# ---------------------------------------------------------------------------------------------
# physical page permutation: bit-identical outputs
# ---------------------------------------------------------------------------------------------

def _repermuted(case, seed):
    """The same logical cache under another physical order: block i moves to perm[i]."""
    n = case.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed)).to(case.k_cache.device)
    kc = torch.empty_like(case.k_cache)
    vc = torch.empty_like(case.v_cache)
    kc[perm] = case.k_cache
    vc[perm] = case.v_cache
    table = perm[case.block_table.long()].to(torch.int32)
    new = synth.PagedCase(**{k: v for k, v in vars(case).items()})
    new.k_cache, new.v_cache, new.block_table = kc, vc, table
    return new


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs", [(128, 16), (256, 64)])
def test_page_permutation_bitwise(gpu, kv_format, d, bs):
    q_lens = [1, 1, 40, 1, 90, 2]
    kv_lens = [700, 33, 40 + 200, 1500, 90, 64]
    gen = torch.Generator().manual_seed(840 + d)
    base = _to(synth.make_paged(840 + d, kv_lens, q_lens, 8, 2, d, bs, kv_format=kv_format, lengths_drawn=gen),
               gpu)
    dec = _to(synth.make_paged(841 + d, [700, 33, 1500, 64], [1] * 4, 16, 4, d, bs, kv_format=kv_format,
                               lengths_drawn=torch.Generator().manual_seed(841 + d)), gpu)
    for seed in (1, 2):
        other = _repermuted(base, seed)
        assert not torch.equal(other.block_table, base.block_table)
        for splits in (0, 5):
            o1, l1 = _varlen(base, splits)
            o2, l2 = _varlen(other, splits)
            assert torch.equal(o1, o2) and torch.equal(l1, l2), f"mixed call differs under permutation {seed}"
        dother = _repermuted(dec, seed)
        for splits in (0, 1, 9):
            o1, l1 = _decode(dec, splits)
            o2, l2 = _decode(dother, splits)
            assert torch.equal(o1, o2) and torch.equal(l1, l2), f"decode differs under permutation {seed}"
    out, lse = _varlen(base, 0)
    ref_o, ref_l = oracle_paged(base)
    compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn", label=f"permutation base {kv_format} d={d}")


# ---------------------------------------------------------------------------------------------
# repeat determinism
# ---------------------------------------------------------------------------------------------

def _same_every_time(run, n=4, between=None):
    first = [t.clone() for t in run()]
    for i in range(n - 1):
        if between is not None:
            between()
        again = run()
        for a, b in zip(first, again):
            assert torch.equal(a, b), f"repeat {i + 1} differs from the first call"


def test_prefill_bf16_repeat_bitwise(gpu):
    """The head_dim-128 ping-pong kernel (causal and windowed) and the head_dim-256 kernel."""
    c = _to(synth.make_prefill(850, [2048, 1000, 3001, 64], 32, 8, 128), gpu)
    c256 = _to(synth.make_prefill(851, [700, 1300, 33], 16, 4, 256), gpu)
    noise = torch.randn(1 << 22, device=gpu)

    def busy():                                      # unrelated work between the calls
        noise.mul_(1.0001)

    for window in (0, 777):
        _same_every_time(lambda: lib.attn_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens, True, c.scale,
                                                         max_seqlen=c.max_seqlen, window=window), between=busy)
    _same_every_time(lambda: lib.attn_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens, False, c.scale,
                                                     max_seqlen=c.max_seqlen), between=busy)
    _same_every_time(lambda: lib.attn_prefill_varlen(c256.q, c256.k, c256.v, c256.cu_seqlens, True, c256.scale,
                                                     max_seqlen=c256.max_seqlen), between=busy)


def test_prefill_fp8_repeat_bitwise(gpu):
    c = _to(synth.make_prefill_fp8(852, [2048, 1000, 3001, 64], 32, 8, 128), gpu)
    for causal, window in ((True, 0), (False, 0), (True, 500)):
        _same_every_time(lambda: lib.attn_prefill_varlen_fp8(c.q, c.k, c.v, c.q_scale, c.k_scale, c.v_scale,
                                                             c.cu_seqlens, causal, c.scale, max_seqlen=3001,
                                                             window=window))


def test_mixed_and_decode_repeat_bitwise(gpu):
    case = _to(synth.config_case("c5", shrink=8), gpu)
    _same_every_time(lambda: _varlen(case, 0))
    dec = _to(synth.config_case("c2", shrink=4), gpu)
    _same_every_time(lambda: _decode(dec, 0))
    # several new tokens per request at group 4: the decode role's two 16-row blocks
    gen = torch.Generator().manual_seed(950)
    mt = _to(synth.make_paged(950, [900, 2000, 64, 1500], [6, 8, 5, 1], 16, 4, 128, 16, lengths_drawn=gen), gpu)
    _same_every_time(lambda: _varlen(mt, 0))


# ---------------------------------------------------------------------------------------------
# every finite e4m3fn code through the kernels' dequantisation, exactly
# ---------------------------------------------------------------------------------------------

FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 254 codes


def _codes_case(dev, d, bs, q_len):
    """254 requests, one KV head shared by 16 query heads. Request b holds q_len cached tokens; its
    token 0 has K codes FINITE_CODES[(b + i) % 254] and V codes FINITE_CODES[(b + 3 + i) % 254] at
    position i (later tokens: random finite codes). Query head h of every row is the one-hot vector
    at position h * d / 16 (bf16 1.0), the score scale is 1, k_scale = 1 and v_scale = 0.5. The
    remaining slots of each page hold the NaN code."""
    nb = len(FINITE_CODES)
    g = np.random.default_rng(d + bs + q_len)
    blocks_per = (q_len + bs - 1) // bs
    perm = g.permutation(nb * blocks_per + 3)
    kc = np.full((len(perm), 1, bs, d), 0x7F, dtype=np.uint8)
    vc = np.full((len(perm), 1, d, bs), 0x7F, dtype=np.uint8)
    table = np.zeros((nb, blocks_per), dtype=np.int32)
    idx = np.arange(d)
    for b in range(nb):
        table[b] = perm[b * blocks_per:(b + 1) * blocks_per]
        for t in range(q_len):
            if t == 0:
                krow = FINITE_CODES[(b + idx) % nb]
                vrow = FINITE_CODES[(b + 3 + idx) % nb]
            else:
                krow = g.choice(FINITE_CODES, d)
                vrow = g.choice(FINITE_CODES, d)
            blk, slot = table[b, t // bs], t % bs
            kc[blk, 0, slot, :] = krow
            vc[blk, 0, :, slot] = vrow
    q = torch.zeros((nb * q_len, 16, d), dtype=torch.bfloat16)
    for h in range(16):
        q[:, h, h * (d // 16)] = 1.0
    case = synth.PagedCase(
        q=q, k_cache=torch.from_numpy(kc), v_cache=torch.from_numpy(vc), block_table=torch.from_numpy(table),
        cu_seqlens_q=torch.arange(0, nb * q_len + 1, q_len, dtype=torch.int32),
        seq_lens_k=torch.full((nb,), q_len, dtype=torch.int32), q_lens=[q_len] * nb, kv_lens=[q_len] * nb,
        kv_format="e4m3fn", k_scale=torch.ones(1), v_scale=torch.full((1,), 0.5), causal=True, scale=1.0,
        num_q_heads=16, num_kv_heads=1, head_dim=d, block_size=bs, used_blocks=nb * blocks_per)
    return _to(case, dev), kc, vc, table


def _check_codes(case, kc, vc, table, out, lse, q_len, label):
    """Row 0 of every request sees only token 0: out = 0.5 * e4m3(V row), lse = e4m3(K at h*d/16)."""
    d = case.head_dim
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    nb = table.shape[0]
    for b in range(nb):
        blk = table[b, 0]
        v_exp = 0.5 * oracle.decode_e4m3fn(vc[blk, 0, :, 0])
        k_dec = oracle.decode_e4m3fn(kc[blk, 0, 0, :])
        row = b * q_len
        for h in range(16):
            got = o[row, h]
            assert np.array_equal(got, v_exp), (
                f"{label}: request {b} head {h}: V codes decoded wrong at "
                f"{np.flatnonzero(got != v_exp)[:4].tolist()}")
            s = k_dec[h * (d // 16)]
            assert abs(l[row, h] - s) <= 2e-6 * max(1.0, abs(s)), (
                f"{label}: request {b} head {h}: lse {l[row, h]} vs score {s} (K code "
                f"{kc[blk, 0, 0, h * (d // 16)]:#04x})")
    seen_k = {int(kc[table[b, 0], 0, 0, h * (d // 16)]) for b in range(nb) for h in range(16)}
    seen_v = {int(c) for b in range(nb) for c in vc[table[b, 0], 0, :, 0]}
    assert seen_k == set(FINITE_CODES.tolist()) and seen_v == set(FINITE_CODES.tolist())


@pytest.mark.parametrize("d,bs", [(128, 16), (256, 16), (128, 64)])
def test_fp8_every_code_decode(gpu, d, bs):
    case, kc, vc, table = _codes_case(gpu, d, bs, 1)
    for splits in (0, 1):
        out, lse = _decode(case, splits)
        _check_codes(case, kc, vc, table, out, lse, 1, f"decode d={d} bs={bs} splits={splits}")
        out, lse = _varlen(case, splits)
        _check_codes(case, kc, vc, table, out, lse, 1, f"mixed (decode path) d={d} bs={bs} splits={splits}")


@pytest.mark.parametrize("d,bs", [(128, 16), (256, 16)])
def test_fp8_every_code_paged_prefill(gpu, d, bs):
    """Two new rows per request (32 rows per KV head): the mixed call's prefill tiles; row 0 is exact,
    row 1 (two keys) is checked against the oracle."""
    case, kc, vc, table = _codes_case(gpu, d, bs, 2)
    out, lse = _varlen(case, 0)
    _check_codes(case, kc, vc, table, out, lse, 2, f"mixed (prefill path) d={d} bs={bs}")
    ref_o, ref_l = oracle_paged(case, units=[(b, h) for b in range(0, 254, 17) for h in (0, 7, 15)])
    # row 1 mixes two keys whose codes reach 448 (outputs up to 224, where a bf16 ulp is 1)
    compare(out, lse, ref_o, ref_l, beyond_rounding=True, label=f"every code, prefill path d={d}")
