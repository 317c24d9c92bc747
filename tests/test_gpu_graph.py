"""The paged decode, the mixed varlen call and the KV append (with the decode after it) inside a
captured HIP graph: the library allocates nothing, never synchronises and records no memset, so a
serving loop can capture a step once and replay it. Each replay runs on new input values written
into the captured buffers, with eager work in between, and must equal the eager call on the same
inputs bit for bit."""

import pytest
import torch

import attention_gqa_flash_02_amd as lib
import synth

pytestmark = pytest.mark.gpu


def _to(case, dev):
    for name, val in list(vars(case).items()):
        if isinstance(val, torch.Tensor):
            setattr(case, name, val.to(dev))
    return case


def _replays_match(call, case, out, lse, gpu):
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
    gen = torch.Generator(device="cpu").manual_seed(9)
    for rep in range(4):
        case.q.copy_(torch.randn(case.q.shape, generator=gen).to(torch.bfloat16).to(gpu))
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        _ = torch.randn(1 << 20, device=gpu).sum()  # unrelated eager work between replays
        call()                                       # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_o, out), f"replay {rep}: output differs from the eager call"
        assert torch.equal(got_l, lse), f"replay {rep}: lse differs from the eager call"


def test_decode_in_graph(gpu):
    case = _to(synth.config_case("c2", shrink=4), gpu)
    b, hq, d = case.q.shape
    out = torch.empty_like(case.q)
    lse = torch.empty((b, hq), dtype=torch.float32, device=gpu)
    splits = lib.attn_decode_num_splits(b, case.num_kv_heads, d, 0, case.block_size, case.block_table.shape[1], 0)
    ws = torch.empty(lib.attn_decode_workspace_bytes(b, case.num_q_heads, d, splits), dtype=torch.uint8,
                     device=gpu)

    def call():
        lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k, case.scale,
                              out=out, lse=lse, num_splits=splits, workspace=ws)
    _replays_match(call, case, out, lse, gpu)


def test_mixed_in_graph(gpu):
    case = _to(synth.config_case("c5", shrink=8), gpu)
    t, hq, d = case.q.shape
    b = case.seq_lens_k.numel()
    out = torch.empty_like(case.q)
    lse = torch.empty((t, hq), dtype=torch.float32, device=gpu)
    splits = lib.attn_decode_num_splits(b, case.num_kv_heads, d, 1, case.block_size, case.block_table.shape[1], 0)
    ws = torch.empty(lib.attn_varlen_workspace_bytes(b, case.num_q_heads, d, splits), dtype=torch.uint8,
                     device=gpu)
    max_q = max(case.q_lens)

    def call():
        lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                              case.seq_lens_k, case.causal, case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                              out=out, lse=lse, max_q_len=max_q, num_splits=splits, workspace=ws)
    _replays_match(call, case, out, lse, gpu)


def test_append_then_decode_in_graph(gpu):
    """A decode step as a serving loop captures it: each request's new token's K and V appended to
    the paged cache, then the decode over the cache that now holds it, in one graph. Every replay
    takes new Q, K and V values; the outputs and both caches must equal the eager step's bit for
    bit, and the new rows must sit in their slots."""
    case = _to(synth.config_case("c2", shrink=4), gpu)
    b, hq, d = case.q.shape
    hkv, bs = case.num_kv_heads, case.block_size
    k_new = torch.zeros((b, hkv, d), dtype=torch.bfloat16, device=gpu)
    v_new = torch.zeros_like(k_new)
    cu = torch.arange(b + 1, dtype=torch.int32, device=gpu)
    out = torch.empty_like(case.q)
    lse = torch.empty((b, hq), dtype=torch.float32, device=gpu)
    splits = lib.attn_decode_num_splits(b, hkv, d, 0, bs, case.block_table.shape[1], 0)
    ws = torch.empty(lib.attn_decode_workspace_bytes(b, hq, d, splits), dtype=torch.uint8, device=gpu)

    def call():
        lib.attn_kv_append_paged(k_new, v_new, case.k_cache, case.v_cache, case.block_table, cu, case.seq_lens_k)
        lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k, case.scale,
                              out=out, lse=lse, num_splits=splits, workspace=ws)

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
    gen = torch.Generator(device="cpu").manual_seed(19)
    last = (case.seq_lens_k - 1).cpu()
    table = case.block_table.cpu()
    for rep in range(4):
        for t in (case.q, k_new, v_new):
            t.copy_(torch.randn(t.shape, generator=gen).to(torch.bfloat16).to(gpu))
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (out, lse, case.k_cache, case.v_cache)]
        _ = torch.randn(1 << 20, device=gpu).sum()  # unrelated eager work between replays
        call()                                       # eager, same inputs
        torch.cuda.synchronize()
        for name, g, e in zip(("out", "lse", "k_cache", "v_cache"), got, (out, lse, case.k_cache, case.v_cache)):
            assert torch.equal(g, e), f"replay {rep}: {name} differs from the eager step"
        for r in (0, b // 2, b - 1):                 # the new rows in their slots
            pos = int(last[r])
            blk = int(table[r, pos // bs])
            assert torch.equal(case.k_cache[blk, :, pos % bs, :], k_new[r]), f"replay {rep}: K of request {r}"
            assert torch.equal(case.v_cache[blk, :, :, pos % bs], v_new[r]), f"replay {rep}: V of request {r}"
