"""The C-ABI library loads, exports every declared symbol, and rejects invalid calls before any
HIP call (these run without a GPU: validation returns first)."""

import ctypes
import re

import pytest

from attention_gqa_flash_02_amd import _lib

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def declared_functions():
    text = open(_lib.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 7
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings():
    lib = _lib.load()
    for code in range(6):
        assert lib.attn_status_string(code).startswith(b"ATTN_")
    assert lib.attn_status_string(99) == b"ATTN_ERR_UNKNOWN"


def _prefill(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, causal=1, scale=0.1, window=0, out=FAKE, lse=None, nseq=1,
                total=16, maxlen=16, hq=4, hkv=1, d=128)
    args.update(kw)
    return _lib.load().attn_prefill_varlen(args["q"], args["k"], args["v"], args["cu"], args["causal"],
                                           args["scale"], args["out"], args["lse"], args["nseq"], args["total"],
                                           args["maxlen"], args["hq"], args["hkv"], args["d"], args["window"],
                                           None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(cu=None), 1), (dict(out=None), 1),
    (dict(nseq=0), 2), (dict(hq=6, hkv=4), 2), (dict(hkv=0), 2), (dict(total=-1), 2), (dict(maxlen=17), 2),
    (dict(causal=2), 2), (dict(scale=float("nan")), 2), (dict(scale=-0.5), 2), (dict(window=-1), 2),
    (dict(d=64), 3), (dict(d=192), 3),
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code


def test_prefill_empty_batch_is_a_noop():
    assert _prefill(total=0, maxlen=0) == 0


def _prefill_fp8(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, qs=FAKE, ks=FAKE, vs=FAKE, cu=FAKE, causal=1, scale=0.1, window=0, out=FAKE,
                lse=None, nseq=1, total=16, maxlen=16, hq=4, hkv=1, d=128)
    args.update(kw)
    return _lib.load().attn_prefill_varlen_fp8(args["q"], args["k"], args["v"], args["qs"], args["ks"], args["vs"],
                                               args["cu"], args["causal"], args["scale"], args["out"], args["lse"],
                                               args["nseq"], args["total"], args["maxlen"], args["hq"], args["hkv"],
                                               args["d"], args["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(qs=None), 1), (dict(ks=None), 1),
    (dict(vs=None), 1), (dict(cu=None), 1), (dict(out=None), 1),
    (dict(nseq=0), 2), (dict(hq=6, hkv=4), 2), (dict(total=-1), 2), (dict(maxlen=17), 2), (dict(causal=2), 2),
    (dict(scale=float("inf")), 2), (dict(window=-1), 2),
    (dict(d=256), 3), (dict(d=64), 3),
])
def test_prefill_fp8_validation(kw, code):
    assert _prefill_fp8(**kw) == code


def test_prefill_fp8_empty_batch_is_a_noop():
    assert _prefill_fp8(total=0, maxlen=0) == 0


def _decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kvt=0, ks=None, vs=None, table=FAKE, lens=FAKE, scale=0.1, window=0,
             out=FAKE, lse=None, nseq=2, hq=8, hkv=2, d=128, bs=16, nblk=10, maxblk=4, splits=1, ws=None, wsb=0)
    a.update(kw)
    return _lib.load().attn_decode_paged(a["q"], a["kc"], a["vc"], a["table"], a["lens"], a["scale"], a["out"],
                                         a["nseq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nblk"], a["maxblk"],
                                         a["splits"], a["lse"], a["ws"], a["wsb"], a["kvt"], a["ks"], a["vs"],
                                         a["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(table=None), 1), (dict(lens=None), 1), (dict(out=None), 1),
    (dict(kvt=1), 1),                               # fp8 without scales
    (dict(kvt=7), 3), (dict(d=96), 3), (dict(bs=8), 3), (dict(bs=48), 3), (dict(hq=64, hkv=2), 3),
    (dict(nseq=-1), 2), (dict(nseq=16385), 3), (dict(hq=7), 2), (dict(nblk=0), 2), (dict(maxblk=0), 2), (dict(splits=-2), 2),
    (dict(window=-3), 2),
    (dict(splits=2, maxblk=40), 4),                 # partials need a workspace
    (dict(splits=2, maxblk=40, ws=FAKE, wsb=16), 4),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def test_split_planning_and_workspace_sizes():
    lib = _lib.load()
    # (num_seqs, num_kv_heads, head_dim, kv_dtype, block_size, max_blocks_per_seq, requested)
    assert lib.attn_decode_num_splits(2, 2, 128, 0, 64, 2048, 64) == 64
    assert lib.attn_decode_num_splits(2, 2, 128, 0, 64, 2048, 100000) == 2048   # one share per 4 chunks
    assert lib.attn_decode_num_splits(2, 2, 128, 0, 16, 8, 100000) == 2         # 4 units x 2 chunks
    assert lib.attn_decode_num_splits(1, 1, 128, 1, 16, 1, 8) == 1
    assert lib.attn_decode_num_splits(64, 8, 256, 0, 256, 4096, 100000) == 4096  # at most 4096
    assert lib.attn_decode_num_splits(0, 1, 128, 0, 16, 1, 8) == 0
    assert lib.attn_decode_num_splits(1, 1, 96, 0, 16, 1, 8) == 0               # head_dim
    assert lib.attn_decode_num_splits(1, 1, 128, 5, 16, 1, 8) == 0              # kv dtype
    assert lib.attn_decode_workspace_bytes(2, 2, 128, 1) == 2 * 16 * 129 * 4 + 3 * 4
    assert lib.attn_decode_workspace_bytes(2, 2, 128, 64) == 64 * 2 * 16 * 129 * 4 + 3 * 4
    assert lib.attn_decode_workspace_bytes(2, 2, 128, 0) == 0
    # (num_seqs, num_q_heads, head_dim, num_splits): the size does not depend on the head count
    assert lib.attn_decode_workspace_bytes(2, 32, 128, 4) == lib.attn_decode_workspace_bytes(2, 1, 128, 4)
    assert lib.attn_decode_workspace_bytes(2, 0, 128, 4) == 0


def test_varlen_validation():
    lib = _lib.load()
    st = lib.attn_varlen_paged(FAKE, FAKE, FAKE, 0, None, None, FAKE, None, FAKE, 1, 0.1, FAKE, None, 2,
                               10, 5, 8, 2, 128, 16, 10, 4, 1, None, 0, 0, None)
    assert st == 1                                   # cu_seqlens_q missing
    st = lib.attn_varlen_paged(FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, 1, 0.1, FAKE, None, 2,
                               10, 11, 8, 2, 128, 16, 10, 4, 1, None, 0, 0, None)
    assert st == 2                                   # max_q_len > total_q
    st = lib.attn_varlen_paged(FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, 1, 0.1, FAKE, None, 2,
                               10, 5, 8, 2, 128, 16, 10, 4, 1, None, 0, -1, None)
    assert st == 2                                   # negative window
    # head_dim 256: the mixed kernel's LDS (129 KB for the 8-wave decode combine buffer + one int per request) caps
    # num_seqs at 7927
    st = lib.attn_varlen_paged(FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, 1, 0.1, FAKE, None, 7928,
                               6000, 5, 8, 2, 256, 16, 10, 4, 1, None, 0, 0, None)
    assert st == 3
    st = lib.attn_varlen_paged(FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, 1, 0.1, FAKE, None, 7927,
                               6000, 5, 8, 2, 256, 16, 10, 4, 1, None, 0, 0, None)
    assert st == 4                                   # passes the cap, then no workspace
    st = lib.attn_varlen_paged(FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, 1, 0.1, FAKE, None, 16384,
                               20000, 5, 8, 2, 128, 16, 10, 4, 1, None, 0, 0, None)
    assert st == 4                                   # head_dim 128: no cap below the request limit


def _append(**kw):
    a = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, kvt=0, ks=None, vs=None, table=FAKE, cu=FAKE, lens=FAKE,
             nseq=2, total=5, hkv=2, d=128, bs=16, nblk=10, maxblk=4)
    a.update(kw)
    return _lib.load().attn_kv_append_paged(a["kn"], a["vn"], a["kc"], a["vc"], a["kvt"], a["ks"], a["vs"],
                                            a["table"], a["cu"], a["lens"], a["nseq"], a["total"], a["hkv"],
                                            a["d"], a["bs"], a["nblk"], a["maxblk"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), 1), (dict(vc=None), 1), (dict(cu=None), 1), (dict(lens=None), 1), (dict(table=None), 1),
    (dict(kvt=1), 1),                               # fp8 without scales
    (dict(kvt=3), 3), (dict(d=64), 3), (dict(bs=8), 3), (dict(nseq=16385), 3),
    (dict(nseq=0), 2), (dict(total=-1), 2), (dict(hkv=0), 2), (dict(nblk=0), 2), (dict(maxblk=0), 2),
])
def test_append_validation(kw, code):
    assert _append(**kw) == code


def test_append_nothing_is_a_noop():
    assert _append(total=0) == 0
    assert _append(total=0, kn=None, vn=None) == 0


def test_missing_library_raises_and_nothing_falls_back(monkeypatch, tmp_path):
    """Without the built library every entry point raises; no other implementation answers."""
    import torch
    import attention_gqa_flash_02_amd as attn

    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libattn_gqa.so"))
    with pytest.raises(_lib.LibraryMissing):
        _lib.load()
    q = torch.zeros(16, 4, 128, dtype=torch.bfloat16)
    kv = torch.zeros(16, 1, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 16], dtype=torch.int32)
    with pytest.raises(_lib.LibraryMissing):
        attn.attn_prefill_varlen(q, kv, kv, cu, True, 128 ** -0.5, max_seqlen=16)
    with pytest.raises(_lib.LibraryMissing):
        attn.attn_decode_workspace_bytes(2, 2, 128, 4)
