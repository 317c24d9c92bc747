"""Pins of the fp8 prefill oracle (the exact attention of e4m3fn codes times per-head scales):
identical keys give the mean of the decoded V, the Q and K scales only enter as their product,
V's scale multiplies only its own heads' outputs, and a query head's scale touches only that head."""

import numpy as np

import oracle


def _case(seed, lens, hq, hkv, d=16):
    rng = np.random.default_rng(seed)
    t = sum(lens)
    # finite e4m3fn codes (exclude the NaN codes 0x7F and 0xFF)
    codes = lambda h: rng.choice(np.r_[0:0x7F, 0x80:0xFF], size=(t, h, d)).astype(np.uint8)
    cu = np.r_[0, np.cumsum(lens)].astype(np.int32)
    return codes(hq), codes(hkv), codes(hkv), cu


def test_identical_keys_give_mean_of_v():
    lens = [5, 9]
    q, _, v, cu = _case(1, lens, 4, 2)
    k = np.zeros_like(v)
    k[:] = v[0:1]                                     # one key row repeated everywhere
    qs, ks, vs = np.full(4, 0.01), np.full(2, 0.02), np.array([0.5, 0.25])
    out, _ = oracle.prefill_varlen_fp8(q, k, v, qs, ks, vs, cu, True, 0.3)
    dv = oracle.decode_e4m3fn(v) * vs[None, :, None]
    for b in range(2):
        lo = cu[b]
        for i in range(lens[b]):
            for h in range(4):
                want = dv[lo:lo + i + 1, h // 2].mean(axis=0)
                assert np.allclose(out[lo + i, h], want, rtol=0, atol=1e-12)


def test_q_and_k_scales_enter_as_a_product():
    q, k, v, cu = _case(2, [7, 12], 4, 2)
    vs = np.array([0.3, 0.7])
    a = oracle.prefill_varlen_fp8(q, k, v, np.full(4, 0.01), np.full(2, 0.02), vs, cu, True, 0.125)
    b = oracle.prefill_varlen_fp8(q, k, v, np.full(4, 0.04), np.full(2, 0.005), vs, cu, True, 0.125)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_v_scale_touches_only_its_heads():
    q, k, v, cu = _case(3, [10], 4, 2)
    qs, ks = np.full(4, 0.01), np.full(2, 0.02)
    o1, l1 = oracle.prefill_varlen_fp8(q, k, v, qs, ks, np.array([0.1, 0.2]), cu, True, 0.2)
    o2, l2 = oracle.prefill_varlen_fp8(q, k, v, qs, ks, np.array([0.1, 0.4]), cu, True, 0.2)
    assert np.array_equal(o1[:, :2], o2[:, :2])              # heads 0, 1 read KV head 0
    assert np.allclose(o2[:, 2:], 2 * o1[:, 2:], rtol=1e-14, atol=0)
    assert np.array_equal(l1, l2)


def test_q_scale_touches_only_its_head():
    q, k, v, cu = _case(4, [6, 11], 4, 2)
    ks, vs = np.full(2, 0.02), np.full(2, 0.3)
    o1, l1 = oracle.prefill_varlen_fp8(q, k, v, np.full(4, 0.01), ks, vs, cu, False, 0.2)
    qs = np.full(4, 0.01)
    qs[3] = 0.03
    o2, l2 = oracle.prefill_varlen_fp8(q, k, v, qs, ks, vs, cu, False, 0.2)
    assert np.array_equal(o1[:, :3], o2[:, :3]) and np.array_equal(l1[:, :3], l2[:, :3])
    assert not np.allclose(o1[:, 3], o2[:, 3])
