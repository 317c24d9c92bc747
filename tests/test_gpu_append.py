"""Paged KV-cache append on the GPU against the oracle's token-by-token scatter: every byte of
both caches must match (the appended slots bit-exactly, including the e4m3fn codes, and every
other byte unchanged)."""

import numpy as np
import pytest
import torch

import attention_gqa_flash_02_amd as lib
import oracle
import synth

pytestmark = pytest.mark.gpu


def _np_bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def _check(case, gpu):
    dev = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in vars(case).items()}
    kc, vc = dev["k_cache"].clone(), dev["v_cache"].clone()
    lib.attn_kv_append_paged(dev["k_new"], dev["v_new"], kc, vc, dev["block_table"], dev["cu_seqlens_new"],
                             dev["seq_lens_k"], k_scale=dev["k_scale"], v_scale=dev["v_scale"])
    torch.cuda.synchronize()
    fmt = "bf16" if case.kv_format == "bf16" else "e4m3fn"
    ks = None if case.k_scale is None else case.k_scale.numpy()
    vs = None if case.v_scale is None else case.v_scale.numpy()
    ref_k, ref_v = oracle.kv_append_paged(_np_bits(case.k_cache), _np_bits(case.v_cache), _np_bits(case.k_new),
                                          _np_bits(case.v_new), case.block_table.numpy(),
                                          case.cu_seqlens_new.numpy(), case.seq_lens_k.numpy(), kv_format=fmt,
                                          k_scale=ks, v_scale=vs)
    got_k, got_v = _np_bits(kc), _np_bits(vc)
    bad_k = np.argwhere(got_k != ref_k)
    bad_v = np.argwhere(got_v != ref_v)
    assert bad_k.size == 0, f"K differs at {bad_k[:5].tolist()} ({len(bad_k)} elements)"
    assert bad_v.size == 0, f"V differs at {bad_v[:5].tolist()} ({len(bad_v)} elements)"


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs,hkv", [(128, 16, 2), (256, 16, 4), (128, 64, 1), (256, 32, 2), (128, 256, 2),
                                      (256, 256, 1)])
def test_append_mixed_batch(gpu, kv_format, d, bs, hkv):
    # decode tokens, chunks crossing page boundaries, an empty request, a first fill
    prior = [0, 5, 16, 100, 7, 0, 31, 250]
    new = [1, 3, 17, 64, 0, 130, 1, 45]
    case = synth.make_append(200 + d + bs, prior, new, hkv, d, bs, kv_format, value_std=2.0)
    _check(case, gpu)


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs", [(128, 16), (256, 16), (128, 32), (256, 64), (128, 256)])
def test_append_chunks_cut_by_workgroups(gpu, kv_format, d, bs):
    """Long runs of new rows at every alignment to the 16-slot chunks of a page, so that the
    64-row ranges of the workgroups cut chunks inside a request (written whole by the first
    workgroup, partly from rows past its range), start or end a request inside a cut chunk, and
    end the batch in a short last range."""
    prior = [5, 16, 37, 0, 250, 1, 15, 94]
    new = [300, 200, 129, 64, 77, 63, 1, 95]
    case = synth.make_append(400 + d + bs, prior, new, 2, d, bs, kv_format, value_std=2.0)
    _check(case, gpu)


def test_append_mixed_step_full(gpu):
    """The append the bench times, at full size and in its launch configuration: the new tokens of
    one mixed step (8 prefill chunks of 2048 over prefixes U[0, 32768] and 120 decodes over
    contexts U[512, 32768]), 4 KV heads, head_dim 256, 16-token pages, e4m3fn codes. Only the
    pages that receive new tokens are distinct; every cached-only block shares page 0, which must
    stay unchanged like every other byte."""
    prior, new = synth.mixed_step_append_lengths()
    case = synth.make_append(5, prior, new, 4, 256, 16, "e4m3fn", shared_prior_page=True)
    _check(case, gpu)


def test_append_many_requests_and_rounding_ties(gpu):
    # 700 requests (the row -> request search crosses its LDS window), mostly single tokens with
    # runs of empty requests; one head's scale is 1 so that quotients hit e4m3 midpoints exactly
    g = np.random.default_rng(5)
    new = [int(x) for x in g.choice([0, 0, 0, 1, 1, 2, 40], size=700)]
    prior = [int(x) for x in g.integers(0, 300, size=700)]
    case = synth.make_append(77, prior, new, 2, 128, 16, "e4m3fn", value_std=40.0, scales=[1.0, 0.01, 1.0, 0.3])
    # overwrite some new values with exact e4m3 midpoints (representable in bf16) and saturating values
    vals = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    flat = case.k_new.view(-1, case.k_new.shape[-1])
    take = torch.from_numpy(np.concatenate([mids, -mids, [500.0, -1e4, 0.0]]).astype(np.float32)).to(torch.bfloat16)
    flat[: (take.numel() + 127) // 128].view(-1)[: take.numel()] = take
    _check(case, gpu)


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
def test_append_rows_past_the_search_window(gpu, kv_format):
    """1000 requests with 600 empty ones after the first: the first workgroup's rows 3 .. belong to
    requests 601 .., outside the 257-entry window of cu_seqlens_new it holds in LDS (requests
    0 .. 256), so their requests are found by the search in memory."""
    new = [3] + [0] * 600 + [2] + [1] * 398
    prior = [5 + (7 * b) % 40 for b in range(len(new))]
    case = synth.make_append(91, prior, new, 2, 128, 16, kv_format, value_std=2.0)
    _check(case, gpu)


def test_append_empty_is_a_noop(gpu):
    case = synth.make_append(3, [4, 9], [0, 0], 2, 128, 16, "bf16")
    _check(case, gpu)


def test_append_quotient_edges(gpu):
    """fp8 quotients x / scale at the edges of the quantiser's reciprocal path: heads whose scale
    or reciprocal is subnormal (those divide), a scale just below a power of two, inputs below
    2^-96 (bf16 subnormals, +-0), and inputs placed so that x / scale lands next to e4m3
    midpoints. Every quotient stays finite (the oracle's encoder takes finite values)."""
    d, hkv = 128, 4
    new = [40, 1, 23]
    scales = [1e-38, 1e38, 0.0123, float(np.nextafter(np.float32(2.0 ** -20), np.float32(0))),   # K heads
              2.0 ** -126, 3.0e37, 0.3, 1.0]                                                       # V heads
    case = synth.make_append(91, [3, 0, 17], new, hkv, d, 16, "e4m3fn", scales=scales)
    g = np.random.default_rng(91)
    rows = sum(new)
    vals = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float64)
    for t, sc in ((case.k_new, case.k_scale.numpy()), (case.v_new, case.v_scale.numpy())):
        x = np.empty((rows, hkv, d), dtype=np.float32)
        for h in range(hkv):
            s = np.float64(sc[h])
            # quotients near every e4m3 midpoint (one bf16 rounding away), random magnitudes, tiny
            # inputs: bf16 subnormals, values around 2^-96, signed zeros
            near = (g.choice(mids, rows * d // 2) * s * g.choice([-1, 1], rows * d // 2))
            wide = g.standard_normal(rows * d // 4) * 10.0 ** g.uniform(-30, 0, rows * d // 4)
            tiny = np.concatenate([g.uniform(-1, 1, rows * d // 8) * 2.0 ** -100,
                                   g.uniform(-1, 1, rows * d // 16) * 1e-39, [0.0, -0.0]])
            col = np.concatenate([near, wide, tiny])
            col = np.resize(col, rows * d)
            col = np.clip(col, -3.0, 3.0)                     # finite quotients for the 1e-38 scale
            x[:, h, :] = col.reshape(rows, d)
        t.copy_(torch.from_numpy(x).to(torch.bfloat16))
    _check(case, gpu)
