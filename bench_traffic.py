"""HBM traffic and matrix-core use per call of the attention kernels, from hardware counters,
and the board's power and clocks while a workload runs.

Five sub-commands:

  python bench_traffic.py copy
      Launches a plain elementwise copy (fp32, 1 GiB read + 1 GiB written, 8 times) and nothing
      else on the GPU. Profiled with `rocprofv3 --pmc FETCH_SIZE` and then `--pmc WRITE_SIZE`, it
      gives what each counter reads for a known number of bytes.

  python bench_traffic.py assemble --calib FETCH_CSV WRITE_CSV --case KEY FETCH_CSV WRITE_CSV [...]
      Reads the rocprofv3 counter_collection.csv files of those runs and writes profiles/traffic.json:
      for each case, the counters of every kernel of one library call (the partition kernel and the
      merge kernel of a decode call, the prefill kernel, the mixed kernel and its merge), each
      scaled by the copy's bytes-per-counter factor, summed per call. Each entry records a digest of
      the kernel sources it was measured on; bench.py reports it only while the sources match.

  python bench_traffic.py counters CSV [--kernel FRAGMENT]
      Prints, for every library kernel in a rocprofv3 counter_collection.csv (or those whose name
      holds FRAGMENT), the median over its dispatches of each counter collected, and the matrix-core
      figures derived from them where the counters are present:
        * MFMA FLOP per dispatch = 512 x (SQ_INSTS_VALU_MFMA_MOPS_BF16 + ..._F8) (each MOPS unit is
          512 multiply or add operations);
        * busy cycles = GRBM_GUI_ACTIVE / 8: rocprofv3 sums the counter over the 8 XCDs, each of
          which counts the dispatch's busy cycles at the graphics clock;
        * effective clock = busy cycles / the dispatch's duration (its start and end timestamps);
        * MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (busy cycles x 1024 SIMDs), the figure
          rocprofv3 derives as MfmaUtil;
        * achieved MFMA FLOP per busy cycle against the chip's dense peak per cycle (256 compute
          units x 4096 bf16 FLOP, x 8192 for fp8).

  python bench_traffic.py power [--seconds S]
      Runs the 4 x 8192 causal prefill (bf16, then fp8 e4m3fn) back to back for S seconds each,
      with an idle second before each, while a thread reads the GPU's metrics table through amdsmi
      every 20 ms. Prints, per phase (the first half second of each left out), the calls per second,
      the median board power and graphics clock (the mean over the 8 XCDs), the power cap, and the
      fraction of the phase's time that the firmware spent holding power under the cap (the change
      of ppt_residency_acc over the change of accumulation_counter).

  python bench_traffic.py stream
      Times plain streaming reductions and a copy through torch over 2 GiB tensors (sum, max and
      a copy of bf16 and fp32 data, 4 rotating copies so nothing is served from the 256 MB
      last-level cache), as a practical reference for what one MI355X reads per second outside
      this library; prints the bytes moved per second of each, from HIP events (median of 30
      calls after 20 warm-up calls).
"""

import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

COPY_ELEMS = 1 << 28          # fp32 elements: 1 GiB each way
COPY_REPS = 8

def run_copy():
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(COPY_REPS):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "elementwise add (copy)", "bytes_read": 4 * COPY_ELEMS,
                      "bytes_written": 4 * COPY_ELEMS, "dispatches": COPY_REPS}))


def run_power(seconds):
    import threading
    import time

    import amdsmi
    import torch

    sys.path.insert(0, ROOT)
    import attention_gqa_flash_02_amd as lib
    import synth

    amdsmi.amdsmi_init()
    handle = amdsmi.amdsmi_get_processor_handles()[0]
    cap_w = amdsmi.amdsmi_get_power_cap_info(handle).get("power_cap", 0) / 1e6
    samples, done = [], threading.Event()

    def sample():
        while not done.is_set():
            samples.append((time.time(), amdsmi.amdsmi_get_gpu_metrics_info(handle)))
            time.sleep(0.02)

    dev = torch.device("cuda:0")
    bf = synth.config_case("c3", device=dev)
    f8 = synth.make_prefill_fp8(3, [8192] * 4, 32, 8, 128, device=dev)
    out, lse = lib.attn_prefill_varlen(bf.q, bf.k, bf.v, bf.cu_seqlens, True, bf.scale, max_seqlen=8192)
    out8, lse8 = lib.attn_prefill_varlen_fp8(f8.q, f8.k, f8.v, f8.q_scale, f8.k_scale, f8.v_scale, f8.cu_seqlens,
                                             True, f8.scale, max_seqlen=8192)
    torch.cuda.synchronize()
    calls = {
        "prefill bf16 4x8192": lambda: lib.attn_prefill_varlen(bf.q, bf.k, bf.v, bf.cu_seqlens, True, bf.scale,
                                                               out=out, lse=lse, max_seqlen=8192),
        "prefill fp8 4x8192": lambda: lib.attn_prefill_varlen_fp8(f8.q, f8.k, f8.v, f8.q_scale, f8.k_scale,
                                                                  f8.v_scale, f8.cu_seqlens, True, f8.scale,
                                                                  out=out8, lse=lse8, max_seqlen=8192),
    }
    thread = threading.Thread(target=sample, daemon=True)
    thread.start()
    phases = []
    for name, call in calls.items():
        t0 = time.time()
        time.sleep(1.0)
        phases.append(("idle", t0, time.time(), 0))
        t0, n = time.time(), 0
        while time.time() - t0 < seconds:
            for _ in range(10):
                call()
            n += 10
            torch.cuda.synchronize()
        phases.append((name, t0, time.time(), n))
    done.set()
    thread.join()

    def num(x):
        return isinstance(x, (int, float)) and not isinstance(x, bool)

    for name, t0, t1, n in phases:
        ms = [m for t, m in samples if t0 + 0.5 <= t <= t1]
        if len(ms) < 2:
            continue
        clocks = [statistics.mean(c for c in m["current_gfxclks"] if num(c) and c < 65535) for m in ms]
        power = [m["current_socket_power"] for m in ms if num(m.get("current_socket_power"))]
        acc = ms[-1]["accumulation_counter"] - ms[0]["accumulation_counter"]
        ppt = (ms[-1]["ppt_residency_acc"] - ms[0]["ppt_residency_acc"]) / acc if acc > 0 else None
        print(json.dumps({"phase": name, "calls_per_s": round(n / (t1 - t0), 1) if n else 0,
                          "samples": len(ms), "power_w": statistics.median(power) if power else None,
                          "power_cap_w": cap_w, "gfxclk_mhz": round(statistics.median(clocks), 1),
                          "ppt_limit_frac": round(ppt, 3) if ppt is not None else None}))


def run_stream():
    import torch

    dev = torch.device("cuda:0")
    nbytes = 2 << 30
    results = []
    for dtype in (torch.bfloat16, torch.float32):
        n = nbytes // torch.tensor([], dtype=dtype).element_size()
        xs = [torch.ones(n, dtype=dtype, device=dev) for _ in range(4)]
        out = torch.empty_like(xs[0])
        ops = {"sum": (lambda x: x.sum(), nbytes), "max": (lambda x: x.max(), nbytes),
               "copy": (lambda x: out.copy_(x), 2 * nbytes)}
        for name, (op, moved) in ops.items():
            for i in range(20):
                op(xs[i % 4])
            torch.cuda.synchronize()
            ms = []
            for i in range(30):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                op(xs[i % 4])
                e1.record()
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
            med = statistics.median(ms)
            results.append({"op": f"{name} {str(dtype).replace('torch.', '')}", "bytes_per_call": moved,
                            "ms_median": round(med, 4), "ms_min": round(min(ms), 4),
                            "gb_per_s_median": round(moved / med / 1e6, 1),
                            "gb_per_s_best": round(moved / min(ms) / 1e6, 1)})
            print(json.dumps(results[-1]), flush=True)
        del xs, out


def read_counter(path, counter):
    """{kernel name: [value per dispatch]} for one counter of a counter_collection.csv."""
    per = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return per


def pick(per, fragment):
    vals = [v for name, vs in per.items() if fragment in name for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel named like {fragment!r}")
    return vals


def assemble(a):
    sys.path.insert(0, ROOT)
    from bench import sources_digest, TRAFFIC_CASES as CASES
    f_fetch = pick(read_counter(a.calib[0], "FETCH_SIZE"), "elementwise")
    f_write = pick(read_counter(a.calib[1], "WRITE_SIZE"), "elementwise")
    nbytes = 4 * COPY_ELEMS
    # bytes per KiB that the counter reports (1024 if it counted every byte)
    k_fetch = nbytes / statistics.median(f_fetch)
    k_write = nbytes / statistics.median(f_write)
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table["_calibration"] = {
        "copy": f"elementwise fp32 add, {nbytes} bytes read and {nbytes} written per dispatch",
        "fetch_kib_per_dispatch": statistics.median(f_fetch), "write_kib_per_dispatch": statistics.median(f_write),
        "bytes_per_fetch_kib": k_fetch, "bytes_per_write_kib": k_write}
    for key, fcsv, wcsv in a.case:
        kernels, sources = CASES[key]
        fetch, write = read_counter(fcsv, "FETCH_SIZE"), read_counter(wcsv, "WRITE_SIZE")
        per_kernel = {}
        for frag in kernels:
            fk, wk = pick(fetch, frag), pick(write, frag)
            per_kernel[frag] = {"dispatches": len(fk), "fetch_kib_median": statistics.median(fk),
                                "write_kib_median": statistics.median(wk),
                                "read_bytes": statistics.median(fk) * k_fetch,
                                "written_bytes": statistics.median(wk) * k_write}
        table[key] = {"sources_sha256_16": sources_digest(sources), "kernels": per_kernel,
                      "hbm_bytes_per_call": sum(v["read_bytes"] + v["written_bytes"] for v in per_kernel.values())}
        print(f"{key}: {table[key]['hbm_bytes_per_call'] / 1e6:.1f} MB per call")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


LIBRARY_KERNELS = ("attn::",)
XCDS = 8                      # MI355X: GRBM counters are summed over its 8 XCDs
PEAK_FLOP_PER_CYCLE = {"bf16": 256 * 4096, "fp8": 256 * 8192}


def counters(a):
    """Median per dispatch of each counter, per library kernel, and the derived matrix-core figures."""
    per = {}
    with open(a.csv) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if not any(k in name for k in LIBRARY_KERNELS) or (a.kernel and a.kernel not in name):
                continue
            key = name.split("(")[0]
            disp = row.get("Dispatch_Id") or row.get("Correlation_Id") or ""
            c = per.setdefault(key, {}).setdefault(row["Counter_Name"], {})
            c[disp] = c.get(disp, 0.0) + float(row["Counter_Value"])
            if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                per[key].setdefault("_duration_ns", {})[disp] = \
                    float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    out = {}
    for key, cs in per.items():
        med = {n: statistics.median(d.values()) for n, d in cs.items()}
        rec = {"dispatches": max(len(d) for d in cs.values()), "median": med}
        mops = med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + med.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        busy = med["GRBM_GUI_ACTIVE"] / XCDS if "GRBM_GUI_ACTIVE" in med else None
        if busy:
            rec["busy_cycles_per_xcd"] = busy
            if med.get("_duration_ns"):
                rec["effective_clock_mhz"] = busy / med["_duration_ns"] * 1e3
        if mops:
            rec["mfma_flop"] = 512 * mops
        if busy and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            rec["mfma_busy_fraction"] = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (busy * 1024)
        if busy and mops:
            kind = "fp8" if med.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) > med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) \
                else "bf16"
            rec["mfma_flop_per_busy_cycle"] = 512 * mops / busy
            rec["fraction_of_dense_peak_per_cycle"] = 512 * mops / busy / PEAK_FLOP_PER_CYCLE[kind]
            rec["peak_kind"] = kind
        if "SQ_LDS_BANK_CONFLICT" in med and med.get("SQ_LDS_IDX_ACTIVE"):
            rec["lds_bank_conflict_per_active_cycle"] = med["SQ_LDS_BANK_CONFLICT"] / med["SQ_LDS_IDX_ACTIVE"]
        out[key] = rec
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("copy")
    sub.add_parser("stream")
    pw = sub.add_parser("power")
    pw.add_argument("--seconds", type=float, default=4.0)
    cnt = sub.add_parser("counters")
    cnt.add_argument("csv")
    cnt.add_argument("--kernel", default=None)
    asm = sub.add_parser("assemble")
    asm.add_argument("--calib", nargs=2, required=True, metavar=("FETCH_CSV", "WRITE_CSV"))
    asm.add_argument("--case", nargs=3, action="append", default=[], metavar=("KEY", "FETCH_CSV", "WRITE_CSV"))
    a = ap.parse_args()
    if a.cmd == "copy":
        run_copy()
    elif a.cmd == "power":
        run_power(a.seconds)
    elif a.cmd == "stream":
        run_stream()
    elif a.cmd == "counters":
        counters(a)
    else:
        assemble(a)


if __name__ == "__main__":
    main()
