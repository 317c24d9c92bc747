"""Seeded synthetic inputs shaped like the pages' attention workloads.

This module serves both the oracle checks and the GPU path and holds none of
the attention arithmetic: it only draws numbers, lays them out in the storage
formats the library reads, and records the shapes. Nothing here imports the
oracle or the library.

Recipe (fixed draw order per case: lengths -> page permutation -> Q -> K -> V):
  * floats are drawn N(0, 1) in float32 by ``torch.randn`` and rounded to
    bfloat16 (round-to-nearest-even);
  * "uniform in [a, b]" integer lengths are inclusive: ``randint(a, b + 1)``;
  * a paged cache holds sum(ceil(len_b / block_size)) blocks plus about 5 %
    spare blocks; the physical order of all blocks is ``randperm`` of the pool;
    logical blocks of request 0, 1, ... take the permuted physical ids in turn;
  * spare blocks and unused tail slots are filled with a poison value (finite
    1e4 by default, NaN for the strict variant) that a correct kernel never
    reads; unused block-table entries are 0;
  * K pages are [num_blocks, Hkv, block_size, D]; V pages are
    [num_blocks, Hkv, D, block_size] (tokens innermost);
  * fp8 caches (OCP e4m3fn codes, ``torch.float8_e4m3fn``) use one fp32 scale
    per KV head and per tensor (k_scale[h], v_scale[h] = amax_h / 448): the
    values are drawn once to find each head's amax, drawn again from the same
    generator state, divided by the scale and cast (round-to-nearest-even).

Generation runs on the device the caller names (a CPU or a GPU torch
generator); the same seed on different devices gives different numbers.
"""

from .cases import (
    PrefillCase,
    PagedCase,
    Fp8PrefillCase,
    make_prefill,
    make_prefill_fp8,
    make_paged,
    AppendCase,
    make_append,
    mixed_step_append_lengths,
    CONFIGS,
    config_case,
)

__all__ = [
    "PrefillCase",
    "PagedCase",
    "Fp8PrefillCase",
    "make_prefill_fp8",
    "AppendCase",
    "make_append",
    "mixed_step_append_lengths",
    "make_prefill",
    "make_paged",
    "CONFIGS",
    "config_case",
]
