"""attn_decode_paged_noalloc (the paged decode for callers that cannot allocate: its partials go to
the library's fixed per-GPU array instead of a caller workspace) against attn_decode_paged on the
same inputs, through the C ABI. The two share their kernels, so with the same partition count the
outputs must be bit-identical. Two calls in a row, the second on a smaller batch (the array keeps the
first call's contents), then a shape whose partials exceed the array (rejected before any launch),
and the entry point captured in a graph and replayed with other no-alloc calls in between.
Validation of the new entry point is also checked without a GPU."""

import ctypes

import pytest
import torch

import attention_gqa_flash_02_amd as lib
from attention_gqa_flash_02_amd import _lib
import synth

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: the calls below fail validation


def _noalloc_raw(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, table=FAKE, lens=FAKE, scale=0.1, out=FAKE, nseq=2, hq=8, hkv=2, d=128,
             bs=16, nblk=10, maxblk=4, splits=1, lse=None, kvt=0, ks=None, vs=None, window=0)
    a.update(kw)
    return _lib.load().attn_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["table"], a["lens"], a["scale"],
                                                 a["out"], a["nseq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nblk"],
                                                 a["maxblk"], a["splits"], a["lse"], a["kvt"], a["ks"], a["vs"],
                                                 a["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(kvt=1), 1), (dict(d=96), 3), (dict(bs=48), 3), (dict(hq=7), 2),
    (dict(scale=-1.0), 2), (dict(window=-1), 2),
    # 4096 partitions x 2 x 16 x (256 + 1) x 4 bytes = 134 MB of partials > ATTN_DECODE_NOALLOC_MAX_BYTES
    (dict(d=256, bs=256, maxblk=4096, nseq=64, hkv=8, hq=32, splits=4096), 4),
])
def test_noalloc_validation(kw, code):
    assert _noalloc_raw(**kw) == code


def _to(case, dev):
    for name, val in list(vars(case).items()):
        if isinstance(val, torch.Tensor):
            setattr(case, name, val.to(dev))
    return case


def _both(case, splits):
    b, hq, d = case.q.shape
    out_ref, lse_ref = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                             case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                                             num_splits=splits)
    out = torch.empty_like(case.q)
    lse = torch.empty((b, hq), dtype=torch.float32, device=case.q.device)
    lib.attn_decode_paged_noalloc(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k, case.scale,
                                  k_scale=case.k_scale, v_scale=case.v_scale, out=out, lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    return out_ref, lse_ref, out, lse


@pytest.mark.gpu
def test_noalloc_matches_decode_two_calls(gpu):
    big = _to(synth.config_case("c2", shrink=2), gpu)          # 16 requests, lengths U[512, 4096]
    small = _to(synth.make_paged(91, [1, 300, 17], [1, 1, 1], 32, 8, 128, 16,
                                 lengths_drawn=torch.Generator().manual_seed(91)), gpu)
    for case, splits in ((big, 0), (small, 0), (big, 37), (small, 5)):
        out_ref, lse_ref, out, lse = _both(case, splits)
        assert torch.equal(out, out_ref), f"B={case.q.shape[0]} splits={splits}: out differs"
        assert torch.equal(lse, lse_ref), f"B={case.q.shape[0]} splits={splits}: lse differs"


@pytest.mark.gpu
def test_noalloc_fp8_head_dim_256(gpu):
    dec = _to(synth.make_paged(92, [5000, 33, 700], [1, 1, 1], 16, 4, 256, 16, kv_format="e4m3fn",
                               lengths_drawn=torch.Generator().manual_seed(92)), gpu)
    for splits in (0, 3):
        out_ref, lse_ref, out, lse = _both(dec, splits)
        assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)


@pytest.mark.gpu
def test_noalloc_rejects_oversized_partials(gpu):
    case = _to(synth.make_paged(93, [100, 50], [1, 1], 32, 2, 128, 64,
                                lengths_drawn=torch.Generator().manual_seed(93)), gpu)
    # a block table of 2048 columns (131072 tokens per request possible): up to 2048 useful partitions,
    # whose partials (2048 x 2 x 16 x 129 x 4 bytes = 33.8 MB) exceed the 16 MiB array
    table = torch.zeros((2, 2048), dtype=torch.int32, device=gpu)
    table[:, :case.block_table.shape[1]] = case.block_table
    out = torch.full_like(case.q, 7.0)
    with pytest.raises(lib.AttnError) as e:
        lib.attn_decode_paged_noalloc(case.q, case.k_cache, case.v_cache, table, case.seq_lens_k, case.scale,
                                      out=out, num_splits=100000)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote its output"
    # the same table with the automatic partition count fits
    out_ref, lse_ref = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, table, case.seq_lens_k, case.scale)
    out2, lse2 = lib.attn_decode_paged_noalloc(case.q, case.k_cache, case.v_cache, table, case.seq_lens_k,
                                               case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out2, out_ref) and torch.equal(lse2, lse_ref)


@pytest.mark.gpu
def test_noalloc_in_graph(gpu):
    """The callers the entry point is for: captured once in a graph and replayed. Between replays an
    eager no-alloc call on another batch overwrites the shared array; every replay, on new query
    values, must still equal attn_decode_paged on the same inputs bit for bit."""
    case = _to(synth.config_case("c2", shrink=4), gpu)
    other = _to(synth.make_paged(94, [2000, 9, 640], [1, 1, 1], 32, 8, 128, 16,
                                 lengths_drawn=torch.Generator().manual_seed(94)), gpu)
    b, hq, d = case.q.shape
    out = torch.empty_like(case.q)
    lse = torch.empty((b, hq), dtype=torch.float32, device=gpu)
    splits = lib.attn_decode_num_splits(b, case.num_kv_heads, d, 0, case.block_size, case.block_table.shape[1], 0)

    def call():
        lib.attn_decode_paged_noalloc(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                      case.scale, out=out, lse=lse, num_splits=splits)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(95)
    for rep in range(3):
        lib.attn_decode_paged_noalloc(other.q, other.k_cache, other.v_cache, other.block_table, other.seq_lens_k,
                                      other.scale, num_splits=7)
        torch.cuda.synchronize()
        case.q.copy_(torch.randn(case.q.shape, generator=gen).to(torch.bfloat16).to(gpu))
        graph.replay()
        torch.cuda.synchronize()
        out_ref, lse_ref = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table,
                                                 case.seq_lens_k, case.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"replay {rep}: out differs"
        assert torch.equal(lse, lse_ref), f"replay {rep}: lse differs"
