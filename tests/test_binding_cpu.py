"""The Python binding rejects mismatched shapes before anything reaches the C ABI (CPU tensors: every
call below raises ValueError from the binding's own checks, so no kernel is launched and no device
pointer is formed)."""

import pytest
import torch

import attention_gqa_flash_02_amd as attn

BF = torch.bfloat16
I32 = torch.int32


def _paged(b=2, hq=8, hkv=2, d=128, bs=16, nblk=6, maxblk=3, dtype=BF):
    return dict(q=torch.zeros(b, hq, d, dtype=BF),
                k_cache=torch.zeros(nblk, hkv, bs, d, dtype=dtype),
                v_cache=torch.zeros(nblk, hkv, d, bs, dtype=dtype),
                block_table=torch.zeros(b, maxblk, dtype=I32),
                seq_lens=torch.zeros(b, dtype=I32))


def _decode(**kw):
    a = _paged()
    a.update(kw)
    return attn.attn_decode_paged(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], 0.1,
                                  k_scale=a.get("k_scale"), v_scale=a.get("v_scale"), out=a.get("out"),
                                  lse=a.get("lse"))


@pytest.mark.parametrize("kw", [
    dict(v_cache=torch.zeros(6, 2, 16, 128, dtype=BF)),          # V in the K order (bs != D: detectable)
    dict(k_cache=torch.zeros(6, 2, 16, 256, dtype=BF)),          # head_dim differs from q
    dict(v_cache=torch.zeros(6, 4, 128, 16, dtype=BF)),          # KV head count differs
    dict(block_table=torch.zeros(3, 3, dtype=I32)),              # rows != requests
    dict(seq_lens=torch.zeros(3, dtype=I32)),                    # lengths != requests
    dict(out=torch.zeros(2, 8, 64, dtype=BF)),                   # out shape
    dict(lse=torch.zeros(2, 4, dtype=torch.float32)),            # lse shape
    dict(k_cache=torch.zeros(6, 2, 16, 128, dtype=torch.uint8),  # fp8 with a wrong scale count
         v_cache=torch.zeros(6, 2, 128, 16, dtype=torch.uint8),
         k_scale=torch.ones(3), v_scale=torch.ones(2)),
])
def test_decode_binding_rejects_shapes(kw):
    with pytest.raises(ValueError):
        _decode(**kw)


def test_decode_binding_rejects_mixed_dtypes():
    with pytest.raises(TypeError):
        _decode(v_cache=torch.zeros(6, 2, 128, 16, dtype=torch.uint8))


def _varlen(**kw):
    a = _paged()
    a["q"] = torch.zeros(5, 8, 128, dtype=BF)
    a["cu"] = torch.tensor([0, 1, 5], dtype=I32)
    a.update(kw)
    return attn.attn_varlen_paged(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["cu"], a["seq_lens"],
                                  True, 0.1, out=a.get("out"), max_q_len=4)


@pytest.mark.parametrize("kw", [
    dict(cu=torch.tensor([0, 5], dtype=I32)),                    # cu_seqlens_q needs num_seqs + 1 entries
    dict(block_table=torch.zeros(1, 3, dtype=I32)),
    dict(v_cache=torch.zeros(6, 2, 16, 128, dtype=BF)),
    dict(out=torch.zeros(4, 8, 128, dtype=BF)),
])
def test_varlen_binding_rejects_shapes(kw):
    with pytest.raises(ValueError):
        _varlen(**kw)


@pytest.mark.parametrize("which", ["k", "v", "out"])
def test_prefill_binding_rejects_shapes(which):
    q = torch.zeros(16, 4, 128, dtype=BF)
    k = torch.zeros(16, 1, 128, dtype=BF)
    v = torch.zeros(16, 1, 128, dtype=BF)
    out = None
    if which == "k":
        k = torch.zeros(16, 1, 256, dtype=BF)
    elif which == "v":
        v = torch.zeros(15, 1, 128, dtype=BF)
    else:
        out = torch.zeros(16, 4, 64, dtype=BF)
    with pytest.raises(ValueError):
        attn.attn_prefill_varlen(q, k, v, torch.tensor([0, 16], dtype=I32), True, 0.1, out=out, max_seqlen=16)


def test_prefill_fp8_binding_rejects_scale_counts():
    q = torch.zeros(16, 4, 128, dtype=torch.uint8)
    kv = torch.zeros(16, 1, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        attn.attn_prefill_varlen_fp8(q, kv, kv, torch.ones(3), torch.ones(1), torch.ones(1),
                                     torch.tensor([0, 16], dtype=I32), True, 0.1, max_seqlen=16)


def test_append_binding_rejects_shapes():
    a = _paged()
    kn = torch.zeros(3, 2, 128, dtype=BF)
    with pytest.raises(ValueError):   # cu_seqlens_new needs num_seqs + 1 entries
        attn.attn_kv_append_paged(kn, kn, a["k_cache"], a["v_cache"], a["block_table"],
                                  torch.tensor([0, 3], dtype=I32), a["seq_lens"])
    with pytest.raises(ValueError):   # V in the K order
        attn.attn_kv_append_paged(kn, kn, a["k_cache"], torch.zeros(6, 2, 16, 128, dtype=BF), a["block_table"],
                                  torch.tensor([0, 1, 3], dtype=I32), a["seq_lens"])
