"""Pins for the fp64 oracle: brute force, closed forms, invariances, a library
routine and the pages' worked example. CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from oracle import algorithms as alg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng_global = np.random.default_rng(12345)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------------------------
# Pin 1: brute force with pure-Python loops on tiny shapes.
# ---------------------------------------------------------------------------------------------

def _brute(q, k, v, scale, causal):
    lq, d = len(q), len(q[0])
    lk = len(k)
    out, lse = [], []
    for i in range(lq):
        scores = []
        for j in range(lk):
            if causal and j > lk - lq + i:
                continue
            scores.append((j, scale * sum(q[i][c] * k[j][c] for c in range(d))))
        if not scores:
            out.append([0.0] * len(v[0]) if lk else [0.0] * d)
            lse.append(-math.inf)
            continue
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        out.append([sum(x * v[j][c] for j, x in w) / tot for c in range(len(v[0]))])
        lse.append(mx + math.log(tot))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("lq,lk,d,causal", [(1, 1, 1, True), (3, 3, 4, True), (4, 7, 5, True),
                                            (5, 8, 8, False), (8, 8, 3, True), (2, 6, 8, False),
                                            (6, 4, 2, True)])
def test_pin1_bruteforce(lq, lk, d, causal):
    rng = np.random.default_rng(lq * 100 + lk * 10 + d)
    q, k, v = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d)
    scale = 0.7
    o, lse = oa.attend(q, k, v, scale, causal)
    ob, lseb = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lseb))
    fin = np.isfinite(lseb)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Pin 2: torch scaled_dot_product_attention (CPU, float64) with KV repeated per group and an
# explicit bottom-right mask.
# ---------------------------------------------------------------------------------------------

def _sdpa(q, k, v, scale, causal, g):
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, Lq, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    lq, lk = q.shape[0], k.shape[0]
    mask = None
    if causal:
        i = torch.arange(lq)[:, None]
        j = torch.arange(lk)[None, :]
        mask = j <= (lk - lq) + i
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("lq,lk,hq,hkv,causal", [(16, 16, 4, 1, True), (5, 40, 8, 2, True),
                                                 (33, 33, 6, 3, False), (1, 70, 4, 4, True)])
def test_pin2_sdpa_crosscheck(lq, lk, hq, hkv, causal):
    rng = np.random.default_rng(7 + lq + lk)
    d = 16
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    scale = 1 / math.sqrt(d)
    ref = _sdpa(q, k, v, scale, causal, hq // hkv)
    g = hq // hkv
    for h in range(hq):
        o, _ = oa.attend(q[:, h], k[:, h // g], v[:, h // g], scale, causal)
        np.testing.assert_allclose(o, ref[:, h], rtol=0, atol=1e-12)


def test_pin2_prefill_varlen_matches_sdpa_per_request():
    rng = np.random.default_rng(99)
    lens = [7, 1, 20]
    hq, hkv, d = 4, 2, 8
    t = sum(lens)
    q, k, v = _rand(rng, t, hq, d), _rand(rng, t, hkv, d), _rand(rng, t, hkv, d)
    cu = np.cumsum([0] + lens)
    out, lse = oa.prefill_varlen(q, k, v, cu, True, 0.3)
    for b in range(len(lens)):
        lo, hi = cu[b], cu[b + 1]
        ref = _sdpa(q[lo:hi], k[lo:hi], v[lo:hi], 0.3, True, hq // hkv)
        np.testing.assert_allclose(out[lo:hi], ref, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


# ---------------------------------------------------------------------------------------------
# Pins 3-6: closed forms.
# ---------------------------------------------------------------------------------------------

def test_pin3_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(3)
    lq, lk, d = 6, 9, 5
    q = _rand(rng, lq, d)
    key = _rand(rng, d)
    k = np.tile(key, (lk, 1))
    v = _rand(rng, lk, d)
    scale = 0.9
    o, lse = oa.attend(q, k, v, scale, True)
    for i in range(lq):
        n_vis = lk - lq + i + 1
        np.testing.assert_allclose(o[i], v[:n_vis].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[i], scale * q[i] @ key + math.log(n_vis), atol=1e-12)


def test_pin4_zero_query_causal():
    rng = np.random.default_rng(4)
    n, d = 12, 4
    q = np.zeros((n, d))
    k, v = _rand(rng, n, d), _rand(rng, n, d)
    o, lse = oa.attend(q, k, v, 0.5, True)
    for i in range(n):
        np.testing.assert_allclose(o[i], v[:i + 1].mean(axis=0), atol=1e-13)
        assert lse[i] == pytest.approx(math.log(i + 1), abs=1e-14)


def test_pin5_one_dominant_score_selects_its_value_row():
    rng = np.random.default_rng(5)
    lk, d = 30, 8
    jstar = 17
    q = np.zeros((1, d))
    q[0, 0] = 20.0
    k = _rand(rng, lk, d)
    k[:, 0] = 0.0                    # every other key orthogonal to e0
    k[jstar, 0] = 10.0               # score gap 200 * scale
    v = _rand(rng, lk, d)
    o, lse = oa.attend(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0], v[jstar], atol=1e-40 + 1e-13)
    assert lse[0] == pytest.approx(200.0, abs=1e-12)


def test_pin6_constant_values_and_identity_columns():
    rng = np.random.default_rng(6)
    lq, lk, d = 5, 5, 8
    q, k = _rand(rng, lq, d), _rand(rng, lk, d)
    v = np.full((lk, d), 2.5)
    o, _ = oa.attend(q, k, v, 0.8, True)
    np.testing.assert_allclose(o, 2.5, atol=1e-14)
    v_id = np.eye(lk, d)             # column j of V picks key j: O[:, :Lk] = P
    p, _ = oa.attend(q, k, v_id, 0.8, True)
    np.testing.assert_allclose(p[:, :lk].sum(axis=1), 1.0, atol=1e-14)
    for i in range(lq):
        assert np.all(p[i, i + 1:lk] == 0.0)      # masked entries exactly zero
        assert np.all(p[i, :i + 1] > 0.0)


def test_pin6_empty_rows_have_zero_output_and_minus_inf_lse():
    q = np.ones((3, 4))
    o, lse = oa.attend(q, np.zeros((0, 4)), np.zeros((0, 4)), 1.0, True)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    # more new rows than keys: the first rows see nothing under bottom-right alignment
    k = np.ones((2, 4))
    o, lse = oa.attend(np.ones((4, 4)), k, np.ones((2, 4)), 1.0, True)
    assert np.all(o[:2] == 0.0) and np.all(np.isneginf(lse[:2]))
    assert np.all(np.isfinite(lse[2:]))


# ---------------------------------------------------------------------------------------------
# Pins 7-8: the pages' exactness claims (tiles, splits).
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("tile", [1, 7, 16, 64, 100])
@pytest.mark.parametrize("causal", [True, False])
def test_pin7_online_softmax_tiles_equal_plain(tile, causal):
    rng = np.random.default_rng(70 + tile)
    lq, lk, d = 37, 100, 16
    q, k, v = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d)
    o, lse = oa.attend(q, k, v, 0.25, causal)
    o2, lse2 = alg.online_softmax_attend(q, k, v, 0.25, causal, tile)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 3, 16, 64])
def test_pin8_split_merge_equals_unsplit(splits):
    rng = np.random.default_rng(80 + splits)
    lq, lk, d = 4, 150, 16
    q, k, v = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d)
    o, lse = oa.attend(q, k, v, 0.25, True)
    o2, lse2 = alg.split_kv_attend(q, k, v, 0.25, True, splits)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


def test_pin8_merge_handles_empty_pieces():
    o_parts = np.zeros((3, 2, 4))
    o_parts[1] = 1.0
    lse_parts = np.array([[-np.inf, -np.inf], [0.5, -np.inf], [-np.inf, -np.inf]])
    o, lse = alg.merge_partials(o_parts, lse_parts)
    np.testing.assert_allclose(o[0], 1.0)
    assert lse[0] == pytest.approx(0.5)
    assert np.all(o[1] == 0.0) and np.isneginf(lse[1])


# ---------------------------------------------------------------------------------------------
# Pins 9-10: paging.
# ---------------------------------------------------------------------------------------------

def _paged_from_dense(k, v, bs, rng, spare=3, poison=1e4):
    """Scatter dense per-request K/V [L, Hkv, D] lists into shuffled pages."""
    lens = [x.shape[0] for x in k]
    hkv, d = k[0].shape[1], k[0].shape[2]
    nblk = [-(-n // bs) for n in lens]
    pool = sum(nblk) + spare
    perm = rng.permutation(pool)
    kc = np.full((pool, hkv, bs, d), poison)
    vc = np.full((pool, hkv, d, bs), poison)
    table = np.zeros((len(lens), max(nblk)), dtype=np.int64)
    pos = 0
    for b, n in enumerate(lens):
        for t in range(n):
            blk = perm[pos + t // bs]
            kc[blk, :, t % bs, :] = k[b][t]
            vc[blk, :, :, t % bs] = v[b][t]
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    return kc, vc, table


def test_pin9_page_permutation_block_size_and_poison_invariance():
    rng = np.random.default_rng(9)
    hq, hkv, d = 4, 2, 8
    lens = [13, 1, 40]
    k = [_rand(rng, n, hkv, d) for n in lens]
    v = [_rand(rng, n, hkv, d) for n in lens]
    q = _rand(rng, len(lens), hq, d)
    ref = None
    for bs in (4, 16, 64):
        for trial in range(2):
            kc, vc, table = _paged_from_dense(k, v, bs, np.random.default_rng(trial * 31 + bs))
            o, lse = oa.decode_paged(q, kc, vc, table, lens, 0.4, kv_format="f64")
            if ref is None:
                ref = (o, lse)
                # and against the dense definition
                for b in range(len(lens)):
                    for h in range(hq):
                        od, ld = oa.attend(q[b:b + 1, h], k[b][:, h // 2], v[b][:, h // 2], 0.4, True)
                        np.testing.assert_allclose(o[b, h], od[0], atol=1e-13)
            np.testing.assert_array_equal(o, ref[0])
            np.testing.assert_array_equal(lse, ref[1])


def test_pin10_worked_block_table_example():
    with open(os.path.join(GOLDEN, "paged_block_table_example.json")) as f:
        ex = json.load(f)
    bs = ex["block_size"]
    table = np.array(ex["block_table"])
    n = ex["num_tokens"]
    pool = 8
    # tag every slot with its (physical block, slot) address
    kc = np.zeros((pool, 1, bs, 2))
    vc = np.zeros((pool, 1, 2, bs))
    for blk in range(pool):
        for s in range(bs):
            kc[blk, 0, s] = (blk, s)
            vc[blk, 0, :, s] = (blk, s)
    k_rows, v_rows = oa.gather_paged(kc, vc, table, n, 0)
    np.testing.assert_array_equal(k_rows, np.array(ex["token_to_physical_slot"], dtype=float))
    np.testing.assert_array_equal(v_rows, np.array(ex["token_to_physical_slot"], dtype=float))
    used = {tuple(x) for x in ex["token_to_physical_slot"]}
    for blk, slot in ex["unused_slots"]:
        assert (blk, slot) not in used


# ---------------------------------------------------------------------------------------------
# Pins 11-13: head mapping, cross-path consistency, shift invariance.
# ---------------------------------------------------------------------------------------------

def test_pin11_gqa_equals_mha_on_repeated_kv_and_special_cases():
    rng = np.random.default_rng(11)
    t, hq, d = 10, 8, 8
    q = _rand(rng, t, hq, d)
    for hkv in (1, 2, 4, 8):                     # MQA, GQA g=4, GQA g=2, MHA
        g = hq // hkv
        k, v = _rand(rng, t, hkv, d), _rand(rng, t, hkv, d)
        o, lse = oa.prefill_varlen(q, k, v, [0, t], True, 0.5)
        o_mha, lse_mha = oa.prefill_varlen(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), [0, t], True, 0.5)
        np.testing.assert_array_equal(o, o_mha)
        np.testing.assert_array_equal(lse, lse_mha)
        # head h reads KV head h // g (contiguous groups)
        for h in range(hq):
            o_h, _ = oa.attend(q[:, h], k[:, h // g], v[:, h // g], 0.5, True)
            np.testing.assert_array_equal(o[:, h], o_h)


def test_pin12_decode_row_equals_prefill_row_and_chunks_equal_full():
    rng = np.random.default_rng(12)
    n, hq, hkv, d = 24, 4, 2, 8
    q, k, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    full_o, full_lse = oa.prefill_varlen(q, k, v, [0, n], True, 0.35)
    # decode of token t over keys 0..t equals prefill row t
    for t in (0, 5, n - 1):
        kc, vc, table = _paged_from_dense([k[:t + 1]], [v[:t + 1]], 4, np.random.default_rng(t))
        o, lse = oa.decode_paged(q[t:t + 1], kc, vc, table, [t + 1], 0.35, kv_format="f64")
        np.testing.assert_allclose(o[0], full_o[t], atol=1e-13)
        np.testing.assert_allclose(lse[0], full_lse[t], atol=1e-13)
    # a chunk of new rows over a cached prefix (bottom-right causal) equals the full-prefill rows
    prefix = 10
    kc, vc, table = _paged_from_dense([k], [v], 4, np.random.default_rng(1))
    o, lse = oa.varlen_paged(q[prefix:], kc, vc, table, [0, n - prefix], [n], True, 0.35, kv_format="f64")
    np.testing.assert_allclose(o, full_o[prefix:], atol=1e-13)
    np.testing.assert_allclose(lse, full_lse[prefix:], atol=1e-13)


def test_pin13_key_shift_invariance():
    rng = np.random.default_rng(13)
    lq, lk, d = 5, 12, 8
    q, k, v = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d)
    c = _rand(rng, d)
    scale = 0.6
    o, lse = oa.attend(q, k, v, scale, True)
    o2, lse2 = oa.attend(q, k + c[None, :], v, scale, True)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + scale * (q @ c), atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Pin 14: storage formats.
# ---------------------------------------------------------------------------------------------

def test_pin14_e4m3fn_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(mine), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert np.nanmax(mine) == oracle.E4M3FN_MAX == 448.0
    assert mine[0x01] == 2.0 ** -9                          # smallest subnormal
    assert mine[0x08] == 2.0 ** -6                          # smallest normal
    # every finite code is exactly representable in bf16
    fin = mine[~nan]
    as_bf16 = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(as_bf16, fin)


def test_pin14_bf16_decoder_against_torch():
    rng = np.random.default_rng(14)
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.decode_bf16_bits(bits), x.to(torch.float64).numpy())


def test_pin14_fp8_cache_decoding_with_scales():
    rng = np.random.default_rng(15)
    hkv, d, bs = 2, 4, 4
    kc = rng.integers(0, 256, size=(3, hkv, bs, d), dtype=np.uint8)
    kc[kc == 0x7F] = 0x7E
    kc[kc == 0xFF] = 0xFE
    vc = rng.integers(0, 256, size=(3, hkv, d, bs), dtype=np.uint8)
    vc[vc == 0x7F] = 0x00
    vc[vc == 0xFF] = 0x80
    ks, vs = np.array([0.5, 2.0]), np.array([0.25, 3.0])
    q = _rand(rng, 1, 4, d) * 0.01
    table = np.array([[2, 0]])
    o, lse = oa.decode_paged(q, kc, vc, table, [6], 1.0, kv_format="e4m3fn", k_scale=ks, v_scale=vs)
    kf = oracle.decode_e4m3fn(kc) * ks[None, :, None, None]
    vf = oracle.decode_e4m3fn(vc) * vs[None, :, None, None]
    o2, lse2 = oa.decode_paged(q, kf, vf, table, [6], 1.0, kv_format="f64")
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


# ---- sliding window (a lower bound on the visible keys, bottom-right aligned)

def test_window_covering_all_keys_equals_no_window():
    g = np.random.default_rng(41)
    q, k, v = g.normal(size=(7, 8)), g.normal(size=(19, 8)), g.normal(size=(19, 8))
    for causal in (True, False):
        o0, l0 = oa.attend(q, k, v, 0.3, causal)
        o1, l1 = oa.attend(q, k, v, 0.3, causal, window=19 + 7)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_one_sees_only_its_own_key():
    g = np.random.default_rng(42)
    q, k, v = g.normal(size=(6, 4)), g.normal(size=(10, 4)), g.normal(size=(10, 4))
    o, l = oa.attend(q, k, v, 0.5, True, window=1)
    own = np.arange(6) + 4                                   # bottom-right: row i's own key is 4 + i
    assert np.allclose(o, v[own], rtol=0, atol=1e-15)
    assert np.allclose(l, 0.5 * np.einsum("id,id->i", q, k[own]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [2, 5, 13])
@pytest.mark.parametrize("causal", [True, False])
def test_window_rows_equal_full_attention_over_their_key_range(window, causal):
    g = np.random.default_rng(43 + window)
    lq, lk = 9, 21
    q, k, v = g.normal(size=(lq, 6)), g.normal(size=(lk, 6)), g.normal(size=(lk, 6))
    o, l = oa.attend(q, k, v, 0.4, causal, window=window)
    for i in range(lq):
        lo = max(0, lk - lq + i - window + 1)
        hi = (lk - lq + i + 1) if causal else lk
        # brute force over the key range, written out
        s = [0.4 * float(q[i] @ k[j]) for j in range(lo, hi)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        ref = sum(wj * v[lo + n] for n, wj in enumerate(w)) / sum(w)
        assert np.allclose(o[i], ref, rtol=0, atol=1e-12)
        assert abs(l[i] - (m + math.log(sum(w)))) < 1e-12


def test_window_decode_row_equals_last_prefill_row_and_paged_equals_contiguous():
    g = np.random.default_rng(44)
    lk, d, hkv, g_ = 50, 8, 2, 2
    q = g.normal(size=(lk, hkv * g_, d))
    k, v = g.normal(size=(lk, hkv, d)), g.normal(size=(lk, hkv, d))
    o_p, l_p = oa.prefill_varlen(q, k, v, [0, lk], True, 0.25, window=7)
    bs = 16
    nblk = -(-lk // bs)
    table = np.array([list(np.random.default_rng(1).permutation(nblk))])
    kc = np.zeros((nblk, hkv, bs, d))
    vc = np.zeros((nblk, hkv, d, bs))
    for t in range(lk):
        kc[table[0][t // bs], :, t % bs, :] = k[t]
        vc[table[0][t // bs], :, :, t % bs] = v[t]
    o_d, l_d = oa.decode_paged(q[-1:], kc, vc, table, [lk], 0.25, kv_format="f64", window=7)
    assert np.allclose(o_d[0], o_p[-1], rtol=0, atol=1e-13) and np.allclose(l_d[0], l_p[-1], rtol=0, atol=1e-13)
