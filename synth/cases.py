"""Seeded case builders (see the package docstring for the recipe)."""

from dataclasses import dataclass, field
import math

import torch

POISON_FINITE = 1.0e4


@dataclass
class PrefillCase:
    """Varlen self-attention over contiguous K/V (token-major)."""
    q: torch.Tensor            # bf16 [T, Hq, D]
    k: torch.Tensor            # bf16 [T, Hkv, D]
    v: torch.Tensor            # bf16 [T, Hkv, D]
    cu_seqlens: torch.Tensor   # int32 [B + 1]
    seqlens: list
    causal: bool
    scale: float
    num_q_heads: int
    num_kv_heads: int
    head_dim: int

    @property
    def total_tokens(self):
        return int(self.q.shape[0])

    @property
    def max_seqlen(self):
        return max(self.seqlens) if self.seqlens else 0


@dataclass
class PagedCase:
    """Queries over a paged KV cache: decode (q_len 1) or a mixed varlen batch."""
    q: torch.Tensor              # bf16 [Tq, Hq, D]
    k_cache: torch.Tensor        # bf16 or uint8 (e4m3fn codes) [num_blocks, Hkv, bs, D]
    v_cache: torch.Tensor        # bf16 or uint8 [num_blocks, Hkv, D, bs]
    block_table: torch.Tensor    # int32 [B, max_blocks_per_seq]
    cu_seqlens_q: torch.Tensor   # int32 [B + 1]
    seq_lens_k: torch.Tensor     # int32 [B]
    q_lens: list
    kv_lens: list
    kv_format: str               # "bf16" | "e4m3fn"
    k_scale: torch.Tensor = None  # fp32 [Hkv] (e4m3fn only)
    v_scale: torch.Tensor = None
    causal: bool = True
    scale: float = 1.0
    num_q_heads: int = 0
    num_kv_heads: int = 0
    head_dim: int = 0
    block_size: int = 16
    used_blocks: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.kv_lens)

    @property
    def num_blocks(self):
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])

    @property
    def is_decode(self):
        return all(x == 1 for x in self.q_lens)


def _cu(lengths, device):
    cu = [0]
    for x in lengths:
        cu.append(cu[-1] + int(x))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def _randn_bf16(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_prefill(seed, seqlens, num_q_heads, num_kv_heads, head_dim, causal=True, scale=None,
                 device="cpu"):
    """Contiguous varlen prefill case; draws Q, then K, then V."""
    gen = torch.Generator(device=device).manual_seed(seed)
    total = int(sum(seqlens))
    q = _randn_bf16(gen, (total, num_q_heads, head_dim), device)
    k = _randn_bf16(gen, (total, num_kv_heads, head_dim), device)
    v = _randn_bf16(gen, (total, num_kv_heads, head_dim), device)
    return PrefillCase(q=q, k=k, v=v, cu_seqlens=_cu(seqlens, device), seqlens=[int(x) for x in seqlens],
                       causal=causal, scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
                       num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim)


@dataclass
class Fp8PrefillCase:
    """Varlen self-attention over contiguous e4m3fn-coded Q/K/V with per-head fp32 scales."""
    q: torch.Tensor            # uint8 codes [T, Hq, D]
    k: torch.Tensor            # uint8 codes [T, Hkv, D]
    v: torch.Tensor            # uint8 codes [T, Hkv, D]
    q_scale: torch.Tensor      # fp32 [Hq]
    k_scale: torch.Tensor      # fp32 [Hkv]
    v_scale: torch.Tensor      # fp32 [Hkv]
    cu_seqlens: torch.Tensor   # int32 [B + 1]
    seqlens: list
    causal: bool
    scale: float
    num_q_heads: int
    num_kv_heads: int
    head_dim: int


def _fp8_codes(x):
    """fp32 [T, H, D] -> (per-head scale amax_h / 448, e4m3fn codes of x / scale via torch's cast)."""
    amax = x.abs().amax(dim=(0, 2))
    head_scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / head_scale.view(1, -1, 1)).clamp(-448.0, 448.0)
    return head_scale.to(torch.float32), y.to(torch.float8_e4m3fn).view(torch.uint8)


def make_prefill_fp8(seed, seqlens, num_q_heads, num_kv_heads, head_dim, causal=True, scale=None, device="cpu"):
    """FP8 varlen prefill case: Q, then K, then V drawn N(0, 1) in fp32 and cast to e4m3fn codes
    with per-head scales amax / 448 (the same recipe as the fp8 KV cache)."""
    gen = torch.Generator(device=device).manual_seed(seed)
    total = int(sum(seqlens))
    draws = [torch.randn((total, h, head_dim), generator=gen, device=device, dtype=torch.float32)
             for h in (num_q_heads, num_kv_heads, num_kv_heads)]
    (qs, qc), (ks, kc), (vs, vc) = (_fp8_codes(x) for x in draws)
    return Fp8PrefillCase(q=qc, k=kc, v=vc, q_scale=qs, k_scale=ks, v_scale=vs, cu_seqlens=_cu(seqlens, device),
                          seqlens=[int(x) for x in seqlens], causal=causal,
                          scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
                          num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim)


def _kv_draws(gen, kv_lens, num_kv_heads, head_dim, device, chunk_tokens):
    """Yield (request, first_token, values [n, Hkv, D] float32) in a fixed call order,
    so that a second pass from the same generator state repeats the same numbers."""
    for b, length in enumerate(kv_lens):
        t = 0
        while t < int(length):
            n = min(chunk_tokens, int(length) - t)
            yield b, t, torch.randn((n, num_kv_heads, head_dim), generator=gen, device=device,
                                    dtype=torch.float32)
            t += n


def _fp8_scale_pass(gen, kv_lens, num_kv_heads, head_dim, device, chunk_tokens):
    """First pass over the draws: per-head scale = amax_h / 448."""
    amax = torch.zeros(num_kv_heads, dtype=torch.float32, device=device)
    for _, _, x in _kv_draws(gen, kv_lens, num_kv_heads, head_dim, device, chunk_tokens):
        amax = torch.maximum(amax, x.abs().amax(dim=(0, 2)))
    return torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))


def make_paged(seed, kv_lens, q_lens, num_q_heads, num_kv_heads, head_dim, block_size,
               kv_format="bf16", causal=True, scale=None, spare_frac=0.05, poison=POISON_FINITE,
               device="cpu", chunk_tokens=1 << 16, lengths_drawn=None):
    """Paged-cache case. ``kv_lens[b]`` cached tokens per request (its ``q_lens[b]``
    new tokens are the last ones). Draw order: page permutation, Q, K, V (the
    lengths are drawn by the caller first, from the same generator, and passed
    in through ``lengths_drawn`` = the generator to continue from)."""
    if len(kv_lens) != len(q_lens):
        raise ValueError("kv_lens and q_lens must have one entry per request")
    gen = lengths_drawn if lengths_drawn is not None else torch.Generator(device="cpu").manual_seed(seed)
    nb = len(kv_lens)
    blocks_per = [(int(x) + block_size - 1) // block_size for x in kv_lens]
    used = sum(blocks_per)
    pool = used + max(1, int(math.ceil(spare_frac * used)))
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    max_blocks = max(1, max(blocks_per) if blocks_per else 1)
    table = torch.zeros((nb, max_blocks), dtype=torch.int32)
    pos = 0
    for b, nblk in enumerate(blocks_per):
        table[b, :nblk] = perm[pos:pos + nblk]
        pos += nblk

    # Q and K/V values come from a generator on the target device (seeded from the same seed).
    dgen = torch.Generator(device=device).manual_seed(seed * 7919 + 17)
    total_q = int(sum(q_lens))
    q = _randn_bf16(dgen, (total_q, num_q_heads, head_dim), device)

    if kv_format == "bf16":
        kc = torch.full((pool, num_kv_heads, block_size, head_dim), poison, dtype=torch.bfloat16, device=device)
        vc = torch.full((pool, num_kv_heads, head_dim, block_size), poison, dtype=torch.bfloat16, device=device)
        k_scale = v_scale = None
        state_k = dgen.get_state()
    elif kv_format == "e4m3fn":
        poison_code = 0x7F if (isinstance(poison, float) and math.isnan(poison)) else 0x7E
        kc = torch.full((pool, num_kv_heads, block_size, head_dim), poison_code, dtype=torch.uint8, device=device)
        vc = torch.full((pool, num_kv_heads, head_dim, block_size), poison_code, dtype=torch.uint8, device=device)
        state_k = dgen.get_state()
        k_scale = _fp8_scale_pass(dgen, kv_lens, num_kv_heads, head_dim, device, chunk_tokens)
    else:
        raise ValueError(f"unknown kv_format {kv_format!r}")

    table_dev = table.to(device)

    def fill(cache, is_v, head_scale, gen_state):
        dgen.set_state(gen_state)
        for b, t, x in _kv_draws(dgen, kv_lens, num_kv_heads, head_dim, device, chunk_tokens):
            n = x.shape[0]
            if kv_format == "bf16":
                vals = x.to(torch.bfloat16)
            else:
                y = (x / head_scale.view(1, -1, 1)).clamp(-448.0, 448.0)
                vals = y.to(torch.float8_e4m3fn).view(torch.uint8)
            tok = torch.arange(t, t + n, device=device)
            phys = table_dev[b, tok // block_size].long()
            slot = tok % block_size
            if is_v:
                cache[phys, :, :, slot] = vals          # V page [Hkv, D, bs]: token innermost
            else:
                cache[phys, :, slot, :] = vals          # K page [Hkv, bs, D]
        return dgen.get_state()

    if kv_format == "bf16":
        state_v = fill(kc, False, None, state_k)
        fill(vc, True, None, state_v)
    else:
        state_v = dgen.get_state()               # after the K amax pass
        v_scale = _fp8_scale_pass(dgen, kv_lens, num_kv_heads, head_dim, device, chunk_tokens)
        state_after_v_scan = dgen.get_state()
        fill(kc, False, k_scale, state_k)
        fill(vc, True, v_scale, state_v)
        dgen.set_state(state_after_v_scan)

    return PagedCase(q=q, k_cache=kc, v_cache=vc, block_table=table_dev,
                     cu_seqlens_q=_cu(q_lens, device),
                     seq_lens_k=torch.tensor([int(x) for x in kv_lens], dtype=torch.int32, device=device),
                     q_lens=[int(x) for x in q_lens], kv_lens=[int(x) for x in kv_lens], kv_format=kv_format,
                     k_scale=k_scale, v_scale=v_scale, causal=causal,
                     scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
                     num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                     block_size=block_size, used_blocks=used)


# ---------------------------------------------------------------------------------------------
# The five workloads. ``shrink`` > 1 divides the token counts (and caps the request count) so
# the same recipe yields small cases the oracle finishes quickly; shrink = 1 is the full size.
# ---------------------------------------------------------------------------------------------

CONFIGS = {
    "c1_prefill": "Tiny GQA sanity: 1 request, 4 query heads / 1 KV head, D 128, causal prefill over 256 tokens",
    "c1_decode": "Tiny GQA sanity: 1 decode token against 257 cached tokens, block size 16, shuffled pages",
    "c2": "Paged GQA decode: batch 32, 32/8 heads, D 128, bf16 KV in 16-token blocks, lengths U[1024, 8192]",
    "c3": "Causal prefill: 4 x 8192 tokens (varlen), 32/8 heads, D 128, bf16, output + LSE",
    "c4": "Split-KV decode: batch 2 x 131072 tokens, 32/2 heads, D 128, bf16 KV in 64-token blocks",
    "c5": "Mixed step: 8 chunks of 2048 over prefixes U[0, 32768] + 120 decodes U[512, 32768], "
          "16/4 heads, D 256, fp8 e4m3fn KV with per-head scales, block size 16",
}


def config_case(name, shrink=1, device="cpu", poison=POISON_FINITE):
    """Build one of the named workloads (seed c1 = 1 ... c5 = 5)."""
    s = max(1, int(shrink))
    if name == "c1_prefill":
        return make_prefill(1, [256 // s if s > 1 else 256], 4, 1, 128, causal=True, device=device)
    if name == "c1_decode":
        gen = torch.Generator(device="cpu").manual_seed(1)
        return make_paged(1, [257], [1], 4, 1, 128, 16, device=device, poison=poison, lengths_drawn=gen)
    if name == "c2":
        gen = torch.Generator(device="cpu").manual_seed(2)
        nb = 32 if s == 1 else max(2, 32 // s)
        lens = torch.randint(1024, 8193, (32,), generator=gen)[:nb]
        lens = [max(1, int(x) // s) for x in lens]
        return make_paged(2, lens, [1] * nb, 32, 8, 128, 16, device=device, poison=poison, lengths_drawn=gen)
    if name == "c3":
        length = 8192 // s
        return make_prefill(3, [length] * 4, 32, 8, 128, causal=True, device=device)
    if name == "c4":
        gen = torch.Generator(device="cpu").manual_seed(4)
        length = 131072 // s
        return make_paged(4, [length] * 2, [1, 1], 32, 2, 128, 64, device=device, poison=poison,
                          lengths_drawn=gen)
    if name == "c5":
        gen = torch.Generator(device="cpu").manual_seed(5)
        n_chunks, n_dec = (8, 120) if s == 1 else (max(1, 8 // s), max(2, 120 // s))
        prefix = torch.randint(0, 32769, (8,), generator=gen)[:n_chunks]
        ctx = torch.randint(512, 32769, (120,), generator=gen)[:n_dec]
        chunk = 2048 // s
        q_lens = [chunk] * n_chunks + [1] * n_dec
        kv_lens = [int(p) // s + chunk for p in prefix] + [max(1, int(c) // s) for c in ctx]
        return make_paged(5, kv_lens, q_lens, 16, 4, 256, 16, kv_format="e4m3fn", device=device,
                          poison=poison, lengths_drawn=gen)
    raise KeyError(name)


@dataclass
class AppendCase:
    """New tokens to write into a paged cache that already holds each request's prior tokens."""
    k_new: torch.Tensor            # [T_new, Hkv, D] bf16
    v_new: torch.Tensor            # [T_new, Hkv, D] bf16
    k_cache: torch.Tensor          # [N, Hkv, bs, D] bf16 or uint8 codes (random prior content)
    v_cache: torch.Tensor          # [N, Hkv, D, bs]
    k_scale: torch.Tensor          # [Hkv] fp32 or None
    v_scale: torch.Tensor
    block_table: torch.Tensor      # [B, max_blocks] int32
    cu_seqlens_new: torch.Tensor   # [B + 1] int32
    seq_lens_k: torch.Tensor       # [B] int32, prior + new
    prior_lens: list
    new_lens: list
    block_size: int
    kv_format: str


def mixed_step_append_lengths():
    """Cached and new token counts of the KV-cache append of one mixed step: 8 prefill chunks of
    2048 new tokens over prefixes U[0, 32768] and 120 decode tokens over contexts U[512, 32768]
    (seed 5). Returns (prior_lens, new_lens)."""
    g = torch.Generator().manual_seed(5)
    prior = [int(x) for x in torch.randint(0, 32769, (8,), generator=g)] + \
            [int(x) - 1 for x in torch.randint(512, 32769, (120,), generator=g)]
    return prior, [2048] * 8 + [1] * 120


def make_append(seed, prior_lens, new_lens, num_kv_heads, head_dim, block_size, kv_format="bf16",
                value_std=1.0, scales=None, cache_content=True, shared_prior_page=False):
    """Seeded append case. Draw order: page permutation -> prior cache content -> K_new -> V_new.

    The cache pool holds every request's blocks (prior + new tokens) plus spare blocks, in
    randperm order; its prior content is random bf16 bits / fp8 codes (any byte the append must
    not touch). New values are N(0, value_std) rounded to bf16. fp8 scales default to per-head
    values spread over [0.002, 0.05] (so that some quotients saturate and some are subnormal).
    With cache_content=False the caches are left as None (the pool size is
    block_table.max() + 1 or more) and no prior content is drawn.
    With shared_prior_page=True only the blocks that receive new tokens get pages of their own
    (pages 1 .. in randperm order); every other logical block maps to page 0, which the append must
    leave unchanged. This keeps the pool small for long cached prefixes.
    """
    g = torch.Generator().manual_seed(seed)
    lens = [p + n for p, n in zip(prior_lens, new_lens)]
    nblocks = [max(1, -(-L // block_size)) for L in lens]
    max_blocks = max(nblocks)
    table = torch.zeros((len(lens), max_blocks), dtype=torch.int32)
    if shared_prior_page:
        touched = [range(p // block_size, (p + n - 1) // block_size + 1) if n > 0 else range(0)
                   for p, n in zip(prior_lens, new_lens)]
        count = sum(len(r) for r in touched)
        spare = max(2, count // 20)
        pool = 1 + count + spare
        perm = 1 + torch.randperm(pool - 1, generator=g)
        used = 0
        for b, r in enumerate(touched):
            for lb in r:
                table[b, lb] = int(perm[used])
                used += 1
    else:
        spare = max(2, sum(nblocks) // 20)
        pool = sum(nblocks) + spare
        perm = torch.randperm(pool, generator=g)
        used = 0
        for b, nb in enumerate(nblocks):
            table[b, :nb] = perm[used:used + nb].to(torch.int32)
            used += nb
    fp8 = kv_format != "bf16"
    if not cache_content:                    # timing only: the caller allocates the pool
        k_cache = v_cache = None
        kshape = (pool, num_kv_heads, block_size, head_dim)
    elif fp8:
        k_cache = torch.randint(0, 0x7F, (pool, num_kv_heads, block_size, head_dim), generator=g, dtype=torch.uint8)
        v_cache = torch.randint(0, 0x7F, (pool, num_kv_heads, head_dim, block_size), generator=g, dtype=torch.uint8)
    else:
        k_cache = (torch.randn((pool, num_kv_heads, block_size, head_dim), generator=g)).to(torch.bfloat16)
        v_cache = (torch.randn((pool, num_kv_heads, head_dim, block_size), generator=g)).to(torch.bfloat16)
    t_new = sum(new_lens)
    k_new = (torch.randn((t_new, num_kv_heads, head_dim), generator=g) * value_std).to(torch.bfloat16)
    v_new = (torch.randn((t_new, num_kv_heads, head_dim), generator=g) * value_std).to(torch.bfloat16)
    k_scale = v_scale = None
    if fp8:
        if scales is None:
            scales = torch.linspace(0.002, 0.05, 2 * num_kv_heads, dtype=torch.float32)
        scales = torch.as_tensor(scales, dtype=torch.float32)
        k_scale, v_scale = scales[:num_kv_heads].clone(), scales[num_kv_heads:2 * num_kv_heads].clone()
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.tensor(new_lens, dtype=torch.int32).cumsum(0)
    return AppendCase(k_new, v_new, k_cache, v_cache, k_scale, v_scale, table, cu,
                      torch.tensor(lens, dtype=torch.int32), list(prior_lens), list(new_lens), block_size, kv_format)
