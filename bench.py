"""Benchmark of the attention hot path on one MI355X.

A step is one call of the paged GQA decode on the batch-32 workload (32 query /
8 KV heads, head dim 128, bf16 KV in 16-token blocks with shuffled pages,
lengths uniform in [1024, 8192]): the partition kernel (balanced split-KV
shares) plus the LSE merge kernel. `value` is KV bytes read per second over the
timed steps (inputs resident in HBM; the KV cache is rotated over copies so
that no step finds it in the 256 MB last-level cache). The same run also times
the causal varlen prefill (4 x 8192 tokens, 32/8 heads, D 128), the
long-context split-KV decode (2 x 131072 tokens, 32/2 heads, 64-token blocks)
and the mixed fp8 batch (8 prefill chunks of 2048 over cached prefixes + 120
decodes, 16/4 heads, D 256) and the KV-cache append of that step, reports each against its
roofline, checks sampled
outputs against the fp64 oracle, and times the oracle itself on the host cores
(cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only c1|c2|c3|c3w|c3fp8|c4|c5|append]
                       [--no-cpu-baseline] [--quick]
Prints one JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2516.6    # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)
MFMA_FP8_PEAK_TFS = 5033.2     # MI355X dense fp8 MFMA, TFLOP/s (twice the bf16 rate)
CSRC = os.path.join(ROOT, "attention_gqa_flash_02_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Untimed calls before each section's timed ones; whatever this says, every section also warms
    # up for at least WARM_MS of GPU time (the clocks rise over the first 20-40 ms of load).
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--splits", type=int, default=0, help="decode partitions (0 = library choice)")
    ap.add_argument("--only", choices=["c1", "c2", "c3", "c3w", "c3fp8", "c4", "c5", "append"], default=None,
                    help="time one workload only (for profiling); the JSON line still names c2's metric")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the parity samples")
    return ap.parse_args()


def sources_digest(names):
    """sha256 over the named kernel sources: traffic figures are only valid for the code they were
    measured on."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Per traffic case: the kernel-name fragments of one library call, and the sources they are built from.
TRAFFIC_CASES = {
    "decode_paged_c2": (["decode_share_kernel", "decode_merge_kernel"], ["common.h", "decode_core.h", "decode.hip"]),
    "decode_c4": (["decode_share_kernel", "decode_merge_kernel"], ["common.h", "decode_core.h", "decode.hip"]),
    "prefill_c3": (["prefill_pingpong_kernel"], ["common.h", "prefill_core.h", "prefill_pp.h", "prefill.hip"]),
    "prefill_c3_fp8": (["prefill_fp8_kernel"], ["common.h", "prefill_core.h", "prefill_pp.h", "prefill_fp8.h",
                                                 "prefill_fp8.hip"]),
    "append_c5": (["kv_append_kernel"], ["common.h", "append.hip"]),
    "mixed_c5": (["varlen_mixed256_kernel", "decode_merge_kernel"],
                 ["common.h", "decode_core.h", "decode.hip", "prefill_core.h", "prefill_pp.h", "prefill_pp256.h",
                  "prefill.hip"]),
}


def measured_traffic(key):
    """HBM bytes per call from profiles/traffic.json (FETCH_SIZE + WRITE_SIZE of the kernels of one
    call, scaled by a copy-kernel calibration), or None when absent or measured on other sources."""
    sources = TRAFFIC_CASES[key][1]
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("sources_sha256_16") != sources_digest(sources):
        return None
    return entry.get("hbm_bytes_per_call")


# The GPU raises its clocks over the first 20-40 ms of sustained load, so every section runs its
# workload for at least this long (and at least --warmup calls) before the timed calls.
WARM_MS = 50.0


def time_steps(fns, steps, warmup):
    """Run fns round-robin: at least `warmup` calls and at least WARM_MS of GPU time untimed (the host
    synchronises every few calls, so the elapsed time is GPU time), then `steps` timed calls between
    synchronisations. Returns (wall ms per step, per-call event durations in ms, timing summary) --
    events on the current stream, which is the stream the library launches on."""
    import torch
    n = len(fns)
    torch.cuda.synchronize()
    calls = 0
    t0 = time.perf_counter()
    while True:
        fns[calls % n]()
        calls += 1
        if calls % 4 == 0 or calls >= warmup:
            torch.cuda.synchronize()
            elapsed = (time.perf_counter() - t0) * 1e3
            if calls >= warmup and elapsed >= WARM_MS:
                break
    warm_ms = (time.perf_counter() - t0) * 1e3
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fns[i % n]()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t1) * 1e3 / steps
    durs = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    info = {"timed_calls": steps, "mean_ms": statistics.mean(durs), "median_ms": statistics.median(durs),
            "min_ms": min(durs), "max_ms": max(durs), "wall_ms_per_call": wall,
            "warmup_calls": calls, "warmup_ms": round(warm_ms, 2)}
    return wall, durs, info


def to_device(case, dev):
    import torch
    for k, v in list(vars(case).items()):
        if isinstance(v, torch.Tensor):
            setattr(case, k, v.to(dev))
    return case


def decode_section(lib, case, splits, steps, warmup, label, rotate=True):
    import torch
    from attention_gqa_flash_02_amd import workmodel
    kv_bytes = workmodel.kv_bytes(case.kv_lens, case.num_kv_heads, case.head_dim,
                                  2 if case.kv_format == "bf16" else 1)
    copies = max(2, math.ceil(3 * 256e6 / kv_bytes) + 1) if rotate else 1
    caches = [(case.k_cache, case.v_cache)] + [(case.k_cache.clone(), case.v_cache.clone())
                                               for _ in range(copies - 1)]
    b, hq, d = case.q.shape
    hkv, bs = case.num_kv_heads, case.block_size
    maxblk = case.block_table.shape[1]
    s = lib.attn_decode_num_splits(b, hkv, d, 0 if case.kv_format == "bf16" else 1, bs, maxblk, splits)
    ws = torch.empty(max(1, lib.attn_decode_workspace_bytes(b, hq, d, s)), dtype=torch.uint8, device=case.q.device)
    out = torch.empty_like(case.q)
    lse = torch.empty((b, hq), dtype=torch.float32, device=case.q.device)

    def make(kc, vc):
        return lambda: lib.attn_decode_paged(case.q, kc, vc, case.block_table, case.seq_lens_k, case.scale,
                                             k_scale=case.k_scale, v_scale=case.v_scale, out=out, lse=lse,
                                             num_splits=s, workspace=ws)
    wall, durs, info = time_steps([make(kc, vc) for kc, vc in caches], steps, warmup)
    kern = statistics.mean(durs)
    log(f"[bench] {label}: partitions={s} copies={copies} wall/step={wall:.4f} ms call mean={kern:.4f} "
        f"median={statistics.median(durs):.4f} min={min(durs):.4f} ms -> {kv_bytes / kern / 1e6:.1f} GB/s")
    return {"kv_bytes": kv_bytes, "splits": s, "wall_ms": wall, "kernel_ms_mean": kern,
            "kernel_ms_median": statistics.median(durs), "kernel_ms_min": min(durs), "out": out, "lse": lse,
            "timing": info}


def prefill_section(lib, case, steps, warmup, window=0):
    from attention_gqa_flash_02_amd import workmodel
    flops = workmodel.prefill_flops(case.seqlens, case.seqlens, case.num_q_heads, case.head_dim, case.causal, window)
    out, lse = lib.attn_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens, case.causal, case.scale,
                                       max_seqlen=case.max_seqlen, window=window)

    def call():
        lib.attn_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens, case.causal, case.scale, out=out,
                                lse=lse, max_seqlen=case.max_seqlen, window=window)
    wall, durs, info = time_steps([call], steps, warmup)
    kern = statistics.mean(durs)
    log(f"[bench] prefill{f' window={window}' if window else ''}: wall/step={wall:.4f} ms kernel mean={kern:.4f} "
        f"min={min(durs):.4f} ms -> {flops / kern / 1e9:.1f} TFLOP/s")
    return {"flops": flops, "wall_ms": wall, "kernel_ms_mean": kern, "kernel_ms_min": min(durs), "out": out,
            "lse": lse, "timing": info}


def prefill_fp8_section(lib, case, steps, warmup):
    from attention_gqa_flash_02_amd import workmodel
    flops = workmodel.prefill_flops(case.seqlens, case.seqlens, case.num_q_heads, case.head_dim, case.causal)
    mx = max(case.seqlens)
    out, lse = lib.attn_prefill_varlen_fp8(case.q, case.k, case.v, case.q_scale, case.k_scale, case.v_scale,
                                           case.cu_seqlens, case.causal, case.scale, max_seqlen=mx)

    def call():
        lib.attn_prefill_varlen_fp8(case.q, case.k, case.v, case.q_scale, case.k_scale, case.v_scale,
                                    case.cu_seqlens, case.causal, case.scale, out=out, lse=lse, max_seqlen=mx)
    wall, durs, info = time_steps([call], steps, warmup)
    kern = statistics.mean(durs)
    log(f"[bench] prefill fp8: wall/step={wall:.4f} ms kernel mean={kern:.4f} min={min(durs):.4f} ms -> "
        f"{flops / kern / 1e9:.1f} TFLOP/s")
    return {"flops": flops, "wall_ms": wall, "kernel_ms_mean": kern, "kernel_ms_min": min(durs), "out": out,
            "lse": lse, "timing": info}


def mixed_section(lib, case, steps, warmup):
    import torch
    from attention_gqa_flash_02_amd import workmodel
    pre = [(ql, kl) for ql, kl in zip(case.q_lens, case.kv_lens) if ql * (case.num_q_heads // case.num_kv_heads) > 16]
    dec = [kl for ql, kl in zip(case.q_lens, case.kv_lens) if 0 < ql * (case.num_q_heads // case.num_kv_heads) <= 16]
    flops = workmodel.prefill_flops([a for a, _ in pre], [b for _, b in pre], case.num_q_heads, case.head_dim, True)
    dec_bytes = workmodel.kv_bytes(dec, case.num_kv_heads, case.head_dim, 1)
    pre_kv_bytes = workmodel.kv_bytes([b for _, b in pre], case.num_kv_heads, case.head_dim, 1)
    b = case.seq_lens_k.numel()
    s = lib.attn_decode_num_splits(b, case.num_kv_heads, case.head_dim, 1, case.block_size,
                                   case.block_table.shape[1], 0)
    ws = torch.empty(lib.attn_varlen_workspace_bytes(b, case.num_q_heads, case.head_dim, s), dtype=torch.uint8,
                     device=case.q.device)
    out = torch.empty_like(case.q)
    lse = torch.empty((case.q.shape[0], case.q.shape[1]), dtype=torch.float32, device=case.q.device)
    max_q = max(case.q_lens)

    def call():
        lib.attn_varlen_paged(case.q, case.k_cache, case.v_cache, case.block_table, case.cu_seqlens_q,
                              case.seq_lens_k, True, case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                              out=out, lse=lse, max_q_len=max_q, num_splits=s, workspace=ws)
    wall, durs, info = time_steps([call], steps, warmup)
    kern = statistics.mean(durs)
    t_star = max(flops / (MFMA_BF16_PEAK_TFS * 1e9), (dec_bytes + pre_kv_bytes) / (HBM_PEAK_GBS * 1e6))
    log(f"[bench] mixed c5: call mean={kern:.4f} ms -> prefill part {flops / kern / 1e9:.1f} TFLOP/s, decode part "
        f"{dec_bytes / kern / 1e6:.1f} GB/s; roofline lower bound {t_star:.4f} ms ({t_star / kern:.3f})")
    return {"flops": flops, "decode_kv_bytes": dec_bytes, "prefill_kv_bytes": pre_kv_bytes, "ms": kern,
            "wall_ms": wall, "t_star_ms": t_star, "out": out, "lse": lse, "timing": info}


def multi_token_section(lib, case, steps, warmup, q_len=4):
    """Speculative-verification decode on the batch-32 cache: each request's last q_len cached
    tokens are new query rows, through the mixed varlen call (at head_dim 128 up to 32 rows per KV
    head, g * q_len, take the split-KV decode path, in one or two 16-row blocks; more take the
    prefill tiles). Algorithmic bytes: the K/V bytes, as for the decode."""
    import torch
    from attention_gqa_flash_02_amd import workmodel
    dev = case.q.device
    b, hq, d = case.q.shape
    g = torch.Generator().manual_seed(21)
    q = torch.randn((b * q_len, hq, d), generator=g).to(torch.bfloat16).to(dev)
    cu = torch.arange(0, b * q_len + 1, q_len, dtype=torch.int32, device=dev)
    kv_bytes = workmodel.kv_bytes(case.kv_lens, case.num_kv_heads, d, 2)
    s = lib.attn_decode_num_splits(b, case.num_kv_heads, d, 0, case.block_size, case.block_table.shape[1], 0)
    ws = torch.empty(lib.attn_varlen_workspace_bytes(b, hq, d, s), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def call():
        lib.attn_varlen_paged(q, case.k_cache, case.v_cache, case.block_table, cu, case.seq_lens_k, True, case.scale,
                              out=out, max_q_len=q_len, num_splits=s, workspace=ws)
    wall, durs, info = time_steps([call], steps, warmup)
    kern = statistics.mean(durs)
    gbs = kv_bytes / kern / 1e6
    log(f"[bench] multi-token decode q_len={q_len}: call mean={kern * 1e3:.1f} us -> {gbs:.0f} GB/s")
    rows = hq // case.num_kv_heads * q_len
    path = ("split-KV decode path" if rows <= 16 else
            "split-KV decode path, two 16-row blocks" if rows <= 32 and d == 128 else "prefill tiles")
    return {"workload": f"batch-32 paged decode cache (32/8 heads, D 128, bf16, 16-token pages), {q_len} new "
                        f"query rows per request ({rows} rows per KV head: {path})",
            "q_len": q_len, "kv_bytes": kv_bytes, "ms": kern, "wall_ms": wall, "gbs": gbs, "timing": info,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None}}


def append_section(lib, steps, warmup):
    """The KV-cache append of one mixed step at the c5 geometry: 8 prefill chunks of 2048 new
    tokens over prefixes U[0, 32768] and 120 decode tokens over contexts U[512, 32768]; 4 KV heads,
    head_dim 256, bs 16, written as fp8 e4m3fn with per-head scales. Algorithmic bytes: the new
    bf16 K and V read once, their fp8 codes written once."""
    import torch
    import synth
    prior, new = synth.mixed_step_append_lengths()
    case = synth.make_append(5, prior, new, 4, 256, 16, "e4m3fn", cache_content=False)
    dev = torch.device("cuda:0")
    pool = int(case.block_table.max()) + 1
    kc = torch.empty((pool, 4, 16, 256), dtype=torch.uint8, device=dev)
    vc = torch.empty((pool, 4, 256, 16), dtype=torch.uint8, device=dev)
    t = {k: v.to(dev) for k, v in vars(case).items() if isinstance(v, torch.Tensor)}

    def call():
        lib.attn_kv_append_paged(t["k_new"], t["v_new"], kc, vc, t["block_table"], t["cu_seqlens_new"],
                                 t["seq_lens_k"], k_scale=t["k_scale"], v_scale=t["v_scale"])
    wall, durs, info = time_steps([call], steps, warmup)
    kern = statistics.mean(durs)
    tn = sum(new)
    nbytes = tn * 4 * 256 * 2 * 2 + tn * 4 * 256 * 1 * 2
    gbs = nbytes / kern / 1e6
    log(f"[bench] append c5 geometry: {tn} tokens, call mean={kern * 1e3:.1f} us -> {gbs:.0f} GB/s")
    return {"workload": "KV-cache append of a mixed step: 8 x 2048 + 120 x 1 new tokens, 4 KV heads, D 256, "
                        "bf16 in, fp8 e4m3fn out (per-head scales), 16-token pages",
            "tokens": tn, "bytes": nbytes, "ms": kern, "wall_ms": wall, "gbs": gbs, "timing": info,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("append_c5")}}


def parity_stats(out, lse, ref_o, ref_l):
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import bf16_np
    o = bf16_np(out)
    m = ~np.isnan(ref_o)
    err = np.abs(o[m] - ref_o[m])
    l = lse.cpu().numpy().astype(np.float64)
    lm = ~np.isnan(ref_l)
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "lse_max_abs": float(np.abs(l[lm] - ref_l[lm]).max()), "max_ref": float(np.abs(ref_o[m]).max())}


def sampled_parity_paged(case, out, lse, units):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import oracle_paged
    ref_o, ref_l = oracle_paged(case, units=units)
    r = parity_stats(out, lse, ref_o, ref_l)
    r["units"] = len(units)
    return r


def sampled_parity_prefill_fp8(case, out, lse, units):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import oracle_prefill_fp8
    ref_o, ref_l = oracle_prefill_fp8(case, units=units)
    r = parity_stats(out, lse, ref_o, ref_l)
    r["units"] = len(units)
    return r


def sampled_parity_prefill(case, out, lse, units):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import oracle_prefill
    ref_o, ref_l = oracle_prefill(case, units=units)
    r = parity_stats(out, lse, ref_o, ref_l)
    r["units"] = len(units)
    return r


def cpu_baseline_decode(case):
    """The fp64 oracle over the whole batch-32 decode workload on the host cores."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import bf16_np, cache_np
    from oracle import parallel
    from attention_gqa_flash_02_amd import workmodel
    args = (bf16_np(case.q), cache_np(case.k_cache), cache_np(case.v_cache), case.block_table.cpu().numpy(),
            case.cu_seqlens_q.cpu().numpy(), case.seq_lens_k.cpu().numpy(), True, case.scale)
    b, hq, d = case.q.shape
    units = [(i, h) for i in range(b) for h in range(hq)]
    workers = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    _, _, wall, used = parallel.run_units("paged", args, {"kv_format": "bf16"}, units,
                                          case.cu_seqlens_q.cpu().numpy(), (b, hq, d), (b, hq), workers=workers)
    kv = workmodel.kv_bytes(case.kv_lens, case.num_kv_heads, case.head_dim, 2)
    return {"value": kv / wall / 1e9, "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"the whole decode batch ({b} requests x {hq} heads, {kv / 1e6:.0f} MB of KV), "
                      f"fp64 numpy, one worker process with one BLAS thread per host core the process may run "
                      f"on ({workers} of os.cpu_count() = {os.cpu_count()}); wall {wall:.2f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); this library has no multi-GPU "
              f"path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import attention_gqa_flash_02_amd as lib
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] device: {torch.cuda.get_device_name(dev)}; library {lib.library_path()}")
    run = (lambda name: a.only is None or a.only == name)
    extra = {}

    # ---- headline: paged GQA decode, batch 32 (generated on the host, copied to the GPU)
    dec = None
    c2_host = None
    if run("c2"):
        t = time.perf_counter()
        c2_host = synth.config_case("c2")
        c2 = to_device(synth.config_case("c2"), dev)
        log(f"[bench] decode workload ready in {time.perf_counter() - t:.1f} s: sum(len)={sum(c2.kv_lens)}")
        dec = decode_section(lib, c2, a.splits, a.steps, a.warmup, "decode c2")
        if not a.quick:
            rng = np.random.default_rng(0)
            units = [(int(b), int(h)) for b, h in zip(rng.integers(0, 32, 64), rng.integers(0, 32, 64))]
            par = sampled_parity_paged(c2_host, dec["out"], dec["lse"], units)
            log(f"[bench] decode c2 parity on {par['units']} sampled (request, head) units: {par}")
            extra["decode_parity_sample"] = par
        extra["decode_c2_timing"] = dec["timing"]
        extra["multi_token_decode"] = multi_token_section(lib, c2, a.steps, a.warmup)
        extra["multi_token_decode_q8"] = multi_token_section(lib, c2, a.steps, a.warmup, q_len=8)
        del c2
        torch.cuda.empty_cache()

    if run("c1"):
        # the tiny sanity case: latency only (a few microseconds of work, far from any roofline)
        p1 = synth.config_case("c1_prefill", device=dev)
        pre1 = prefill_section(lib, p1, a.steps, a.warmup)
        d1 = synth.config_case("c1_decode", device=dev)
        dec1 = decode_section(lib, d1, 0, a.steps, a.warmup, "decode c1", rotate=False)
        extra["c1_latency"] = {
            "workload": "tiny GQA sanity: causal prefill of 256 tokens (4/1 heads, D 128), then one decode token "
                        "over 257 cached tokens in 16-token pages",
            "prefill_us": pre1["kernel_ms_mean"] * 1e3, "decode_us": dec1["kernel_ms_mean"] * 1e3}
        del p1, d1, pre1, dec1

    if run("c3") or run("c3w"):
        c3 = synth.config_case("c3", device=dev)
    if run("c3"):
        pre = prefill_section(lib, c3, max(10, a.steps // 2), a.warmup)
        tf = pre["flops"] / pre["kernel_ms_mean"] / 1e9
        extra["prefill_c3"] = {
            "workload": "causal varlen prefill, 4 x 8192 tokens, 32/8 heads, D 128, bf16, out + LSE",
            "tflops": tf, "ms": pre["kernel_ms_mean"], "wall_ms": pre["wall_ms"], "timing": pre["timing"],
            "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tf / MFMA_BF16_PEAK_TFS,
                         "traffic": measured_traffic("prefill_c3")},
            "algorithmic_flops": pre["flops"]}
        if not a.quick:
            units = [(0, 0), (1, 7), (2, 19), (3, 31)]
            par = sampled_parity_prefill(c3, pre["out"], pre["lse"], units)
            log(f"[bench] prefill parity on {units}: {par}")
            extra["prefill_c3"]["parity_sample"] = par
        del pre
    if run("c3w"):
        pw = prefill_section(lib, c3, max(10, a.steps // 2), a.warmup, window=4096)
        tfw = pw["flops"] / pw["kernel_ms_mean"] / 1e9
        extra["prefill_c3_window4096"] = {
            "workload": "the same causal prefill with a 4096-key sliding window (algorithmic FLOPs over the "
                        "windowed visible pairs)",
            "tflops": tfw, "ms": pw["kernel_ms_mean"], "algorithmic_flops": pw["flops"], "timing": pw["timing"],
            "roofline": {"bound": "mfma", "achieved": tfw, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tfw / MFMA_BF16_PEAK_TFS, "traffic": None}}
        del pw
    if run("c3") or run("c3w"):
        del c3
        torch.cuda.empty_cache()

    if run("c3fp8"):
        c3f = synth.make_prefill_fp8(3, [8192] * 4, 32, 8, 128, device=dev)
        pf = prefill_fp8_section(lib, c3f, max(10, a.steps // 2), a.warmup)
        tf8 = pf["flops"] / pf["kernel_ms_mean"] / 1e9
        extra["prefill_c3_fp8"] = {
            "workload": "the same causal prefill with e4m3fn Q/K/V and per-head scales (N(0,1) draws, scale = "
                        "amax/448 per head), fp8 MFMA, P rounded to e4m3, out bf16 + LSE",
            "tflops": tf8, "ms": pf["kernel_ms_mean"], "wall_ms": pf["wall_ms"], "algorithmic_flops": pf["flops"],
            "timing": pf["timing"],
            "roofline": {"bound": "mfma", "achieved": tf8, "peak": MFMA_FP8_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tf8 / MFMA_FP8_PEAK_TFS,
                         "traffic": measured_traffic("prefill_c3_fp8")}}
        if not a.quick:
            units = [(0, 0), (1, 7), (2, 19), (3, 31)]
            par = sampled_parity_prefill_fp8(c3f, pf["out"], pf["lse"], units)
            log(f"[bench] prefill fp8 parity on {units}: {par}")
            extra["prefill_c3_fp8"]["parity_sample"] = par
        del c3f, pf
        torch.cuda.empty_cache()

    if run("c4"):
        c4 = synth.config_case("c4", device=dev)
        best = None
        for s in ((a.splits,) if a.splits else (0, 512)):
            r = decode_section(lib, c4, s, a.steps, a.warmup, f"decode c4 partitions={s or 'auto'}")
            if best is None or r["kernel_ms_mean"] < best["kernel_ms_mean"]:
                best = r
        gbs = best["kv_bytes"] / best["kernel_ms_mean"] / 1e6
        extra["decode_c4"] = {
            "workload": "split-KV decode, 2 x 131072 tokens, 32/2 heads, D 128, bf16 KV, 64-token blocks",
            "gbs": gbs, "partitions": best["splits"], "ms": best["kernel_ms_mean"], "timing": best["timing"],
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_c4")}}
        if not a.quick:
            units = [(0, 0), (1, 17), (0, 31)]
            par = sampled_parity_paged(c4, best["out"], best["lse"], units)
            log(f"[bench] decode c4 parity on {units}: {par}")
            extra["decode_c4"]["parity_sample"] = par
        del c4
        torch.cuda.empty_cache()

    if run("c5"):
        t = time.perf_counter()
        c5 = synth.config_case("c5", device=dev)
        log(f"[bench] mixed workload ready in {time.perf_counter() - t:.1f} s: q rows {c5.q.shape[0]}, "
            f"keys {sum(c5.kv_lens)}")
        mx = mixed_section(lib, c5, max(5, a.steps // 5), a.warmup)
        extra["mixed_c5"] = {
            "workload": "one call: 8 prefill chunks of 2048 over cached prefixes U[0, 32768] + 120 decodes with "
                        "contexts U[512, 32768], 16/4 heads, D 256, fp8 e4m3fn KV with per-head scales",
            "ms": mx["ms"], "timing": mx["timing"], "prefill_tflops": mx["flops"] / mx["ms"] / 1e9,
            "decode_gbs": mx["decode_kv_bytes"] / mx["ms"] / 1e6,
            "algorithmic_flops": mx["flops"], "decode_kv_bytes": mx["decode_kv_bytes"],
            "prefill_kv_bytes": mx["prefill_kv_bytes"],
            "roofline": {"bound": "mfma", "lower_bound_ms": mx["t_star_ms"], "frac": mx["t_star_ms"] / mx["ms"],
                         "traffic": measured_traffic("mixed_c5")}}
        if not a.quick:
            n_pre = sum(1 for ql in c5.q_lens if ql > 1)
            units = [(0, 0), (n_pre - 1, 15), (n_pre, 3), (n_pre + 50, 9), (len(c5.q_lens) - 1, 12)]
            par = sampled_parity_paged(c5, mx["out"], mx["lse"], units)
            log(f"[bench] mixed c5 parity on {units}: {par}")
            extra["mixed_c5"]["parity_sample"] = par
        del c5, mx
        torch.cuda.empty_cache()

    if run("append"):
        extra["append_c5"] = append_section(lib, a.steps, a.warmup)

    cpu = None
    if not a.no_cpu_baseline and run("c2"):
        cpu = cpu_baseline_decode(c2_host)
        log(f"[bench] cpu baseline: {cpu}")

    line = {
        "metric": "decode attn KV GB/s (% HBM peak)",
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled pages)",
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if dec is not None:
        achieved = dec["kv_bytes"] / dec["kernel_ms_mean"] / 1e6
        line.update({
            "value": round(dec["kv_bytes"] / dec["wall_ms"] / 1e6, 2),
            "ms_per_step": round(dec["wall_ms"], 5),
            "config": {"workload": "paged GQA decode: batch 32, 32 q / 8 kv heads, head_dim 128, bf16 KV in "
                                   "16-token blocks, lengths U[1024, 8192]",
                       "global_batch": 32, "seq_len": "U[1024, 8192]", "num_partitions": dec["splits"],
                       "kv_bytes": dec["kv_bytes"], "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_paged_c2")},
        })
    else:
        line.update({"value": None, "ms_per_step": None,
                     "config": {"workload": f"only {a.only} timed (see extra)"}, "roofline": None})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
