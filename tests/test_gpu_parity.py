"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on seeded inputs."""

import math

import numpy as np
import pytest
import torch

import attention_gqa_flash_02_amd as lib
import synth
from helpers import compare, oracle_paged, oracle_prefill

pytestmark = pytest.mark.gpu


def _to(case, dev):
    for name, val in list(vars(case).items()):
        if isinstance(val, torch.Tensor):
            setattr(case, name, val.to(dev))
    return case


def _run_prefill(case):
    out, lse = lib.attn_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens, case.causal, case.scale,
                                       max_seqlen=case.max_seqlen)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("d,hq,hkv,causal", [(128, 8, 2, True), (128, 4, 4, False), (256, 4, 2, True)])
def test_prefill_many_sequences(gpu, d, hq, hkv, causal):
    """800 short sequences (1 to 40 tokens, a few of 300) in one call: most q-tiles of the grid,
    sized by the longest sequence, find no rows of their sequence. Rows that see a few keys output
    values up to about 4.5, whose own bf16 rounding (up to 0.0156 past 4) exceeds 1e-2 whatever a
    kernel does, so the error is measured beyond that rounding."""
    g = np.random.default_rng(800 + d + hq)
    lens = [int(x) for x in g.integers(1, 41, 800)]
    for i in (17, 400, 799):
        lens[i] = 300
    case = _to(synth.make_prefill(800 + d + hq, lens, hq, hkv, d, causal=causal), gpu)
    out, lse = _run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    compare(out, lse, ref_o, ref_l, beyond_rounding=True,
            label=f"800 sequences d={d} hq={hq} hkv={hkv} causal={causal}")


@pytest.mark.parametrize("name", ["c1_prefill"])
def test_prefill_c1_full(gpu, name):
    case = _to(synth.config_case(name), gpu)
    out, lse = _run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    compare(out, lse, ref_o, ref_l, label=name)


def test_prefill_c3_shrunk(gpu):
    case = _to(synth.config_case("c3", shrink=16), gpu)     # 4 x 512 tokens, 32/8 heads
    out, lse = _run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    compare(out, lse, ref_o, ref_l, label="c3/16")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2), (6, 2), (32, 2)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [128, 256])
def test_prefill_varlen_ragged(gpu, hq, hkv, causal, d):
    lens = [1, 17, 64, 100, 33, 130]
    case = _to(synth.make_prefill(11 + hq + hkv + d, lens, hq, hkv, d, causal=causal), gpu)
    out, lse = _run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    compare(out, lse, ref_o, ref_l, label=f"ragged hq={hq} hkv={hkv} causal={causal} d={d}")


def _run_decode(case, splits=0):
    out, lse = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                     case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                                     num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


def test_decode_c1(gpu):
    case = _to(synth.config_case("c1_decode"), gpu)
    for splits in (0, 1, 2, 5):
        out, lse = _run_decode(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, label=f"c1_decode splits={splits}")


@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_decode_c2_shrunk(gpu, splits):
    case = _to(synth.config_case("c2", shrink=4), gpu)       # 8 requests, lengths U[256, 2048]
    out, lse = _run_decode(case, splits)
    ref_o, ref_l = oracle_paged(case)
    compare(out, lse, ref_o, ref_l, label=f"c2/4 splits={splits}")


@pytest.mark.parametrize("splits", [1, 16, 64])
def test_decode_c4_shrunk(gpu, splits):
    case = _to(synth.config_case("c4", shrink=32), gpu)      # 2 x 4096 tokens, g = 16, bs 64
    out, lse = _run_decode(case, splits)
    ref_o, ref_l = oracle_paged(case)
    compare(out, lse, ref_o, ref_l, label=f"c4/32 splits={splits}")


def test_decode_workspace_reuse(gpu):
    """One workspace, filled with arbitrary bytes first, serves calls of different shapes and split
    counts in a row; every call matches the oracle (the workspace needs no initialisation)."""
    gen = torch.Generator().manual_seed(77)
    cases = [_to(synth.config_case("c2", shrink=4), gpu),
             _to(synth.make_paged(78, [1, 40, 700, 3000, 0, 129], [1] * 6, 8, 2, 128, 16, lengths_drawn=gen), gpu),
             _to(synth.config_case("c4", shrink=32), gpu)]
    ws = torch.randint(0, 256, (1 << 23,), dtype=torch.uint8, generator=gen).to(gpu)
    for case, splits in [(cases[0], 16), (cases[0], 16), (cases[1], 8), (cases[0], 64), (cases[2], 16),
                         (cases[2], 64), (cases[1], 3), (cases[0], 0)]:
        out, lse = lib.attn_decode_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_k,
                                         case.scale, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, label=f"workspace reuse B={case.q.shape[0]} splits={splits}")


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs", [(128, 16), (128, 64), (128, 256), (256, 16), (256, 64), (256, 128), (256, 256)])
def test_decode_every_variant(gpu, kv_format, d, bs):
    """Every decode kernel instantiation: head_dim 128/256 x bf16/e4m3fn pages x page rows of at
    most 32 tokens (nontemporal V loads per half) and longer ones (loads issued in pairs), up to
    the largest block size the library takes (256). The oracle reads the same fp8 codes, so fp8
    pages are held to the bf16 bar."""
    lens = [1, 31, 64, 65, 200, 700, 1500]
    gen = torch.Generator().manual_seed(60 + d + bs)
    case = _to(synth.make_paged(60 + d + bs, lens, [1] * len(lens), 16, 4, d, bs, kv_format=kv_format,
                                lengths_drawn=gen), gpu)
    for splits in (0, 1, 5):
        out, lse = _run_decode(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"decode {kv_format} d={d} bs={bs} splits={splits}")


@pytest.mark.parametrize("d,bs", [(256, 16), (128, 32), (128, 16)])
def test_decode_fp8(gpu, d, bs):
    lens = [1, 15, 16, 17, 300, 1000]
    gen = torch.Generator().manual_seed(31)
    case = _to(synth.make_paged(31, lens, [1] * len(lens), 16, 4, d, bs, kv_format="e4m3fn",
                                lengths_drawn=gen), gpu)
    for splits in (1, 4):
        out, lse = _run_decode(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, beyond_rounding=True, label=f"fp8 d={d} bs={bs} splits={splits}")


@pytest.mark.parametrize("d,kv_format", [(128, "bf16"), (256, "e4m3fn")])
def test_decode_planned_shares(gpu, d, kv_format):
    """The share plan charges (request, kv head) units of fewer than 256 chunks two extra places
    for starting a piece. Units at 254-257 chunks sit on both sides of that threshold, short units
    between them, and partition counts up to one share per 4 places make shares that hold only a
    unit's extra places (no piece of it) next to shares that start inside one."""
    ch = 64 if d == 128 else 32                      # tokens per chunk of the decode kernel
    lens = [1, 254 * ch, 2, 255 * ch, 255 * ch + 1, 65, 257 * ch, 3 * ch, 130]
    gen = torch.Generator().manual_seed(77 + d)
    case = _to(synth.make_paged(77 + d, lens, [1] * len(lens), 8, 2, d, 16, kv_format=kv_format,
                                lengths_drawn=gen), gpu)
    ref_o, ref_l = oracle_paged(case)
    for splits in (0, 5, 200, 1000):
        out, lse = _run_decode(case, splits)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"planned shares d={d} {kv_format} splits={splits}")


@pytest.mark.parametrize("d,kv_format", [(128, "bf16"), (256, "e4m3fn")])
def test_decode_many_requests(gpu, d, kv_format):
    """600 requests (more than the 256 threads of the plan's prefix, so each sums several), a
    tenth of them empty, lengths up to 300: the plan, the shares and the merge over many short
    units, at the library's partition count and at a few others."""
    g = np.random.default_rng(600 + d)
    lens = [0 if x < 0.1 else int(y) for x, y in zip(g.random(600), g.integers(1, 301, 600))]
    case = _to(synth.make_paged(600 + d, lens, [1] * len(lens), 8, 2, d, 16, kv_format=kv_format), gpu)
    ref_o, ref_l = oracle_paged(case)
    for splits in (0, 7, 300, 2000):
        out, lse = _run_decode(case, splits)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"600 requests d={d} {kv_format} splits={splits}")


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_decode_group_sizes_and_edges(gpu, g):
    lens = [0, 1, 2, 63, 64, 65, 257, 1000]
    hkv = 2
    gen = torch.Generator().manual_seed(40 + g)
    case = _to(synth.make_paged(40 + g, lens, [1] * len(lens), g * hkv, hkv, 128, 16, lengths_drawn=gen), gpu)
    for splits in (1, 3):
        out, lse = _run_decode(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, label=f"edges g={g} splits={splits}")


# ---------------------------------------------------------------------------------------------
# Mixed varlen batch over a paged cache (prefill chunks over cached prefixes + decode tokens in
# one call), bf16 and fp8 e4m3fn KV.
# ---------------------------------------------------------------------------------------------

def _run_varlen(case, splits=0):
    out, lse = lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                                     case.seq_lens_k, case.causal, case.scale, k_scale=case.k_scale,
                                     v_scale=case.v_scale, num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


def test_varlen_many_requests(gpu):
    """300 requests in one mixed call: mostly single decode tokens, some multi-token requests and
    prefill chunks of up to 100 rows over cached prefixes, and empty caches."""
    g = np.random.default_rng(300)
    q_lens = [int(x) for x in g.choice([1, 1, 1, 1, 2, 4, 33, 100], size=300)]
    kv_lens = [q + int(p) for q, p in zip(q_lens, g.integers(0, 400, 300))]
    case = _to(synth.make_paged(301, kv_lens, q_lens, 8, 2, 128, 16), gpu)
    ref_o, ref_l = oracle_paged(case)
    for splits in (0, 5):
        out, lse = _run_varlen(case, splits)
        compare(out, lse, ref_o, ref_l, label=f"300 requests mixed splits={splits}")


def test_varlen_c5_shrunk(gpu):
    case = _to(synth.config_case("c5", shrink=16), gpu)   # 1 chunk of 128 over a prefix + 7 decodes
    out, lse = _run_varlen(case)
    ref_o, ref_l = oracle_paged(case)
    compare(out, lse, ref_o, ref_l, beyond_rounding=True, label="c5/16")


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("d,bs", [(128, 16), (256, 16), (128, 64), (256, 64), (128, 256), (256, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_mixed(gpu, kv_format, d, bs, causal):
    # decode rows (q_len 1..4 with g = 4 stay on the decode path), prefill chunks over prefixes,
    # a chunk with no prefix, a request with no new rows
    q_lens = [1, 3, 37, 64, 0, 130, 1, 5]
    kv_lens = [1, 300, 37, 64 + 500, 17, 130 + 33, 2000, 5]
    gen = torch.Generator().manual_seed(70 + d + bs)
    case = _to(synth.make_paged(70 + d + bs, kv_lens, q_lens, 8, 2, d, bs, kv_format=kv_format, causal=causal,
                                lengths_drawn=gen), gpu)
    for splits in (0, 3):
        out, lse = _run_varlen(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, beyond_rounding=kv_format == "e4m3fn",
                label=f"mixed {kv_format} d={d} bs={bs} causal={causal} splits={splits}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (16, 1), (32, 2)])
def test_varlen_group_sizes(gpu, hq, hkv):
    q_lens = [2, 1, 40, 17]
    kv_lens = [100, 64, 40 + 90, 17]
    gen = torch.Generator().manual_seed(90 + hq)
    case = _to(synth.make_paged(90 + hq, kv_lens, q_lens, hq, hkv, 128, 16, lengths_drawn=gen), gpu)
    out, lse = _run_varlen(case)
    ref_o, ref_l = oracle_paged(case)
    compare(out, lse, ref_o, ref_l, label=f"varlen hq={hq} hkv={hkv}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (16, 4), (16, 2)])
def test_varlen_multi_token_decode(gpu, hq, hkv):
    """Speculative verification: 2-8 new query rows per request over a long cache; rows that fit
    32 per KV head (head_dim 128) go through the split-KV decode path, in one or two 16-row blocks,
    the others through the prefill path."""
    q_lens = [2, 3, 4, 5, 6, 7, 8, 1]
    kv_lens = [900, 2000, 64, 17, 3000, 33, 1500, 700]
    gen = torch.Generator().manual_seed(300 + hq + hkv)
    case = _to(synth.make_paged(300 + hq + hkv, kv_lens, q_lens, hq, hkv, 128, 16, lengths_drawn=gen), gpu)
    for splits in (0, 5):
        out, lse = _run_varlen(case, splits)
        ref_o, ref_l = oracle_paged(case)
        compare(out, lse, ref_o, ref_l, label=f"multi-token hq={hq} hkv={hkv} splits={splits}")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_many_key_tiles(gpu, hq, hkv, causal):
    """Requests of 4 to 12 key tiles of 64, so that the ping-pong loop (unrolled by three over its
    three tile buffers) ends at every position of its unroll, with and without the causal mask, for
    query tiles of 64 rows (4 heads per workgroup) and 256 rows (one head per workgroup)."""
    lens = [257, 300, 384, 449, 520, 640, 700, 767]
    case = _to(synth.make_prefill(500 + hq + int(causal), lens, hq, hkv, 128, causal=causal), gpu)
    out, lse = _run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    compare(out, lse, ref_o, ref_l, label=f"many tiles hq={hq} hkv={hkv} causal={causal}")
