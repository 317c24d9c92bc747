"""Pins of the KV-cache append oracle and its e4m3fn encoder (no GPU).

The encoder is pinned by the OCP e4m3fn definition (every code round-trips, midpoints go to
the even code, saturation at 448, the subnormal range) and cross-checked against torch's
float8_e4m3fn cast; the append is pinned by the worked block-table example ("Optimization 1:
batching and attention", section 3.4) and by reading the tokens back with the attention
oracle's own page gather.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_block_table_example.json")
POS = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))     # +0 .. 448, increasing


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3fn(oracle.decode_e4m3fn(codes)), codes)


def test_encoder_midpoints_go_to_the_even_code_and_neighbours_to_the_nearest():
    lo, hi = POS[:-1], POS[1:]
    mid = (lo + hi) / 2                                  # exact in float64
    got = oracle.encode_e4m3fn(mid)
    even = np.where(np.arange(1, 0x7F) % 2 == 0, np.arange(1, 0x7F), np.arange(0, 0x7E)).astype(np.uint8)
    assert np.array_equal(got, even)
    eps = (hi - lo) * 1e-3
    assert np.array_equal(oracle.encode_e4m3fn(mid - eps), np.arange(0, 0x7E, dtype=np.uint8))
    assert np.array_equal(oracle.encode_e4m3fn(mid + eps), np.arange(1, 0x7F, dtype=np.uint8))
    # negative values mirror the positive ones with the sign bit set
    assert np.array_equal(oracle.encode_e4m3fn(-(mid + eps)), np.arange(1, 0x7F, dtype=np.uint8) | 0x80)


def test_encoder_saturates_and_keeps_the_sign_of_zero():
    assert oracle.encode_e4m3fn(np.array([448.0, 460.0, 1e6, -500.0])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.encode_e4m3fn(np.array([0.0, -0.0])).tolist() == [0x00, 0x80]
    # subnormals: the smallest is 2^-9; half of it is a tie between 0 and 2^-9 -> the even code 0
    assert oracle.encode_e4m3fn(np.array([2.0 ** -10, 2.0 ** -10 * 1.01, 3 * 2.0 ** -10])).tolist() == [0x00, 0x01, 0x02]


def test_encoder_matches_torch_float8_cast_in_range():
    g = np.random.default_rng(3)
    x = np.concatenate([g.normal(0, 40, 20000), g.uniform(-448, 448, 20000), g.normal(0, 0.01, 5000)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3fn(x), ref)


def test_quantize_divides_in_fp32():
    bits = (np.array([1.5, -3.0, 100.0], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    scale = np.float32(0.3)
    q = (np.array([1.5, -3.0, 100.0], dtype=np.float32) / scale).astype(np.float32)
    assert np.array_equal(oracle.quantize_e4m3fn(bits, scale), oracle.encode_e4m3fn(q))


def _bf16_bits(x):
    return (torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
            .view(np.uint16))


def test_append_follows_the_worked_block_table_example():
    g = json.load(open(GOLDEN))
    bs, table, n = g["block_size"], g["block_table"], g["num_tokens"]
    num_blocks, hkv, d = 8, 2, 4
    kc = np.full((num_blocks, hkv, bs, d), 0x7777, dtype=np.uint16)
    vc = np.full((num_blocks, hkv, d, bs), 0x7777, dtype=np.uint16)
    k_new = np.arange(n * hkv * d, dtype=np.uint16).reshape(n, hkv, d) + 1
    v_new = k_new + 1000
    kc2, vc2 = oracle.kv_append_paged(kc, vc, k_new, v_new, np.array([table]), np.array([0, n]), np.array([n]))
    for t, (blk, slot) in enumerate(g["token_to_physical_slot"]):
        assert np.array_equal(kc2[blk, :, slot, :], k_new[t])
        assert np.array_equal(vc2[blk, :, :, slot], v_new[t])
    for blk, slot in g["unused_slots"]:
        assert np.all(kc2[blk, :, slot, :] == 0x7777) and np.all(vc2[blk, :, :, slot] == 0x7777)
    touched = {tuple(x) for x in g["token_to_physical_slot"]}
    for blk in range(num_blocks):
        for slot in range(bs):
            if (blk, slot) not in touched:
                assert np.all(kc2[blk, :, slot, :] == kc[blk, :, slot, :])


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
def test_append_then_gather_returns_the_tokens_and_chunks_compose(kv_format):
    g = np.random.default_rng(11)
    bs, hkv, d, num_blocks = 16, 2, 32, 40
    prior = [5, 0, 31]                                   # cached before the append
    n_new = [3, 20, 1]
    lens = [p + n for p, n in zip(prior, n_new)]
    perm = g.permutation(num_blocks)
    table = np.zeros((3, 4), dtype=np.int64)
    used = 0
    for b, L in enumerate(lens):
        nb = -(-L // bs)
        table[b, :nb] = perm[used:used + nb]
        used += nb
    dt = np.uint16 if kv_format == "bf16" else np.uint8
    kc = g.integers(0, 60, size=(num_blocks, hkv, bs, d)).astype(dt)
    vc = g.integers(0, 60, size=(num_blocks, hkv, d, bs)).astype(dt)
    x = g.normal(0, 1, size=(sum(n_new), hkv, d))
    k_new, v_new = _bf16_bits(x), _bf16_bits(x * 2)
    cu = np.concatenate([[0], np.cumsum(n_new)])
    ks = np.array([0.01, 0.02], dtype=np.float32)
    vs = np.array([0.03, 0.005], dtype=np.float32)
    kw = dict(kv_format=kv_format, k_scale=ks, v_scale=vs)
    kc2, vc2 = oracle.kv_append_paged(kc, vc, k_new, v_new, table, cu, np.array(lens), **kw)
    for b in range(3):
        for h in range(hkv):
            kr, vr = oa.gather_paged(kc2, vc2, table[b], lens[b], h)
            new_k, new_v = kr[prior[b]:], vr[prior[b]:]
            rows = slice(cu[b], cu[b + 1])
            if kv_format == "bf16":
                assert np.array_equal(new_k, k_new[rows, h])
                assert np.array_equal(new_v, v_new[rows, h])
            else:
                # dequantised values sit within half an e4m3 step (2^-4 relative) of the input
                kx = oracle.decode_bf16_bits(k_new[rows, h])
                kd = oracle.decode_e4m3fn(new_k) * float(ks[h])
                assert np.all(np.abs(kd - kx) <= np.abs(kx) * 2.0 ** -4 + float(ks[h]) * 2.0 ** -10)
            # tokens cached before the append are untouched
            kr0, vr0 = oa.gather_paged(kc, vc, table[b], lens[b], h)
            assert np.array_equal(kr[:prior[b]], kr0[:prior[b]])
            assert np.array_equal(vr[:prior[b]], vr0[:prior[b]])
    # appending request 1's 20 tokens as 12 then 8 gives the same cache
    lens_a = [prior[0], prior[1] + 12, prior[2]]
    cu_a = np.array([0, 0, 12, 12])
    kca, vca = oracle.kv_append_paged(kc, vc, k_new[3:15], v_new[3:15], table, cu_a, np.array(lens_a), **kw)
    cu_b = np.array([0, 3, 11, 12])
    sel = np.r_[0:3, 15:23, 23:24]
    kcb, vcb = oracle.kv_append_paged(kca, vca, k_new[sel], v_new[sel], table, cu_b, np.array(lens), **kw)
    assert np.array_equal(kcb, kc2) and np.array_equal(vcb, vc2)


def test_synth_append_shared_prior_page():
    """The compact append case used at full size: blocks that receive new tokens get distinct
    pages 1 ..; every other logical block maps to page 0, which the oracle's scatter never writes
    (so a kernel write there shows up in the byte comparison)."""
    import synth
    prior, new = [0, 5, 16, 100, 7, 31, 250], [1, 3, 17, 64, 0, 1, 45]
    case = synth.make_append(9, prior, new, 2, 128, 16, "e4m3fn", shared_prior_page=True)
    table = case.block_table.numpy()
    pages = []
    for b, (p, n) in enumerate(zip(prior, new)):
        touched = set(range(p // 16, (p + n - 1) // 16 + 1)) if n else set()
        for lb in range(-(-(p + n) // 16)):
            if lb in touched:
                assert table[b, lb] >= 1
                pages.append(int(table[b, lb]))
            else:
                assert table[b, lb] == 0
    assert len(pages) == len(set(pages)) and max(pages) < case.k_cache.shape[0]

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.contiguous().view(torch.uint8).numpy()
    kc, vc = oracle.kv_append_paged(bits(case.k_cache), bits(case.v_cache), bits(case.k_new), bits(case.v_new),
                                    table, case.cu_seqlens_new.numpy(), case.seq_lens_k.numpy(), kv_format="e4m3fn",
                                    k_scale=case.k_scale.numpy(), v_scale=case.v_scale.numpy())
    assert np.array_equal(kc[0], bits(case.k_cache)[0]) and np.array_equal(vc[0], bits(case.v_cache)[0])
    assert not np.array_equal(kc[pages], bits(case.k_cache)[pages])
