#!/usr/bin/env python3
"""Benchmark of absorbed-MLA decode on one MI355X.

One step = one whole decode call (plan + attend) of one layer over the
DP-attention-rank workload: 124 requests x 4,096 cached tokens, 128 heads,
576-wide bf16 latent in 64-token pages with a shuffled block table.  Inputs
are resident in HBM before the timed region; three independent caches are
rotated so that no timed call finds its cache in the 256 MB Infinity Cache.
Before the warm-up steps, untimed steps run for --prewarm-ms (250 ms): from
idle the GPU's clock needs ~35 ms of load to settle, and steps in that
window take up to twice as long.

Prints one JSON line with the metric (cached-token reads/s, from the timed
steps between two events), a roofline record for the attend kernel (from a
second run of as many steps with HIP events around every attend launch on
the stream it runs on), and the CPU oracle timed on a bounded sample of the
same workload on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload dp_rank]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MLA decode: cached-token reads/s, achieved HBM TB/s, % of roofline"
PROFILES = os.path.join(ROOT, "profiles")
SRC = os.path.join(ROOT, "mla_latent_cache_absorbed_amd", "csrc", "mla_decode.hip")


def src_hash() -> str:
    return hashlib.sha256(open(SRC, "rb").read()).hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dp_rank",
                   choices=["dp_rank", "tp_slice", "ragged", "step61", "dp_rank_fp8"])
    p.add_argument("--copies", type=int, default=3, help="independent caches rotated")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--prewarm-ms", type=float, default=250.0,
                   help="untimed decode steps for this long before the warm-up steps: "
                        "from idle the GPU clock takes ~35 ms of load to settle")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the fp8, append, absorption and attainable-peak records")
    p.add_argument("--trace-summary", default=None,
                   help="write profiles/bench_default_run_kernel_trace.md from the rocprofv3 "
                        "--kernel-trace --stats output under this directory (the default run), "
                        "then exit (no GPU needed)")
    p.add_argument("--copy-probe", action="store_true",
                   help="run only a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--profile-dir", default=None,
                   help="write the profiles/ summaries of --workload from the rocprofv3 output "
                        "directories under this one (kt, fetch, write, mfma, copy_fetch, "
                        "copy_write), then exit (no GPU needed)")
    return p.parse_args()


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def counter_record_path(name: str) -> str:
    return os.path.join(PROFILES, f"attend_{name}_hbm_counters.json")


def hbm_traffic_record(name: str):
    """Counter-measured HBM bytes per attend launch on this workload, if the
    record was taken on this source (else None)."""
    try:
        rec = json.load(open(counter_record_path(name)))
    except (OSError, ValueError):
        return None
    if rec.get("src_sha256_16") != src_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def _rocprof_rows(d: str, suffix: str):
    """Rows of every rocprofv3 CSV under directory d whose name ends with suffix."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def counter_means(d: str, kernel_prefix: str) -> dict:
    """Per-dispatch means of every counter rocprofv3 --pmc collected under d
    for kernels whose name starts with kernel_prefix: {counter: (mean, n)}.
    A counter's value for one dispatch is the sum over the rows rocprofv3
    writes for it."""
    per = {}
    for r in _rocprof_rows(d, "counter_collection.csv"):
        if not r.get("Kernel_Name", "").startswith(kernel_prefix):
            continue
        key = (r["Counter_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (c, _), v in per.items():
        s, n = out.get(c, (0.0, 0))
        out[c] = (s + v, n + 1)
    return {c: (s / n, n) for c, (s, n) in out.items()}


def write_counter_record(name: str, fetch_dir: str, write_dir: str, cfetch_dir: str,
                         cwrite_dir: str, kernel_prefix: str, commands: list) -> dict:
    """The traffic record bench.py reports as roofline.traffic for a workload:
    FETCH_SIZE and WRITE_SIZE (KiB per attend dispatch) scaled by what the
    same counters read for a plain 1 GiB device copy, per attend launch."""
    from mla_latent_cache_absorbed_amd import accounting as acc
    from mla_latent_cache_absorbed_amd import workloads as wl
    f = counter_means(fetch_dir, kernel_prefix)["FETCH_SIZE"]
    w = counter_means(write_dir, kernel_prefix)["WRITE_SIZE"]
    cf = counter_means(cfetch_dir, "__amd_rocclr_copyBuffer")["FETCH_SIZE"][0]
    cw = counter_means(cwrite_dir, "__amd_rocclr_copyBuffer")["WRITE_SIZE"][0]
    n = 1 << 30
    fetch_scale = n / (cf * 1024.0)
    write_scale = n / (cw * 1024.0)
    sp = wl.spec("dp_rank" if name == "dp_rank_fp8" else name)
    rec = {"kernel": kernel_prefix, "workload": name, "src_sha256_16": src_hash(),
           "commands": commands, "R": "the repository root",
           "attend_dispatches": {"fetch": f[1], "write": w[1]},
           "attend_FETCH_SIZE_KiB_per_dispatch": f[0], "attend_WRITE_SIZE_KiB_per_dispatch": w[0],
           "copy_probe": {"bytes_read": n, "bytes_written": n, "kernel": "__amd_rocclr_copyBuffer",
                          "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw},
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "read_bytes_per_launch": f[0] * 1024.0 * fetch_scale,
           "write_bytes_per_launch": w[0] * 1024.0 * write_scale}
    rec["traffic_bytes_per_launch"] = rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    rec["algorithmic_bytes_per_launch"] = acc.algorithmic_bytes(
        list(sp.seq_lens), sp.H, sp.BS, row_bytes=576 if name == "dp_rank_fp8" else 1152)
    with open(counter_record_path(name), "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def cpu_baseline(w, budget_s: float):
    """The oracle, as it stands, on whole requests of the workload until the budget."""
    import numpy as np
    from mla_latent_cache_absorbed_amd import workloads as wl
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    lens = w.seq_lens_list()
    # host copies of each request's pages, fetched once outside the timed calls
    host = []
    for b in range(w.B):
        nblk = -(-lens[b] // w.BS)
        host.append((wl.bf16_bits(w.q[b:b + 1]), wl.bf16_bits(w.cache[w.block_table[b, :nblk].long()]),
                     np.arange(nblk, dtype=np.int32)[None], np.array([lens[b]], dtype=np.int32)))
    done_tokens = 0
    done_req = 0
    elapsed = 0.0
    while elapsed < budget_s:
        qb, sub, tab, ln = host[done_req % w.B]
        t0 = time.perf_counter()
        orc.oracle_decode(qb, sub, tab, ln, w.scale)
        elapsed += time.perf_counter() - t0
        done_tokens += int(ln[0])
        done_req += 1
    passes = done_req / w.B
    return {"value": done_tokens / elapsed, "unit": "cached-token reads/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"{done_req} request decodes ({passes:.1f} passes over the {w.B} requests, "
                      f"{done_tokens} tokens x {w.H} heads), float64 NumPy, {elapsed:.1f} s"}


def _cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stream_read_record(gib: int = 4, reps: int = 5) -> dict:
    """Read-only streaming bandwidth this GPU attains: the probe library's
    plain 16-byte global loads and direct-to-LDS loads (the path the decode
    kernel stages rows with) over a 4 GiB buffer, 16x the Infinity Cache,
    with 1, 2 and 4 workgroups of 256 threads per CU; HIP events around `reps`
    launches of each.  Two access patterns: the whole GPU sweeping the buffer
    front to back, and every workgroup streaming its own contiguous region
    (the pattern of the decode's work items, each walking its own blocks).
    Reports every setting and the best per mode, in decimal GB/s."""
    import ctypes
    import torch
    from mla_latent_cache_absorbed_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.mla_probe_stream_read.restype = ctypes.c_size_t
    lib.mla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_probe_sink_bytes.restype = ctypes.c_size_t
    lib.mla_probe_sink_bytes.argtypes = [ctypes.c_int32]
    dev = torch.device("cuda")
    x = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(lib.mla_probe_sink_bytes(4), dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()
    runs = {}
    for mode, name in ((0, "global_load_to_registers"), (1, "direct_to_lds"),
                       (2, "own_region_global_load_to_registers"), (3, "own_region_direct_to_lds")):
        for wpc in (1, 2, 4):
            n = lib.mla_probe_stream_read(x.data_ptr(), x.numel(), mode, wpc, sink.data_ptr(),
                                          st.cuda_stream)
            if n == 0:
                raise RuntimeError("stream-read probe failed to launch")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                lib.mla_probe_stream_read(x.data_ptr(), x.numel(), mode, wpc, sink.data_ptr(),
                                          st.cuda_stream)
            e1.record(st)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps * 1e-3
            runs[f"{name}_wg{wpc}"] = n / t / 1e9
    del x, sink
    best = {m: max(v for k, v in runs.items() if k.startswith(m))
            for m in ("global_load_to_registers", "direct_to_lds",
                      "own_region_global_load_to_registers", "own_region_direct_to_lds")}
    return {"bytes_per_launch": int(n), "gb_s": runs, "best_gb_s": best,
            "frac_of_peak": {m: v / HBM_PEAK_GBS for m, v in best.items()}}


def mfma_loop_record(iters: int = 20000, reps: int = 5) -> dict:
    """bf16 MFMA rate this GPU attains: the probe library's loop of
    independent v_mfma_f32_32x32x16_bf16 on random operands, with 1 and 2
    workgroups of 4 waves per CU (one or two waves per SIMD), and the same
    loop on v_mfma_f32_16x16x32_bf16 at one wave per SIMD; HIP events around
    `reps` launches of each; TFLOP/s and the fraction of the 2.5 PFLOP/s
    dense bf16 peak (best of the 32x32x16 runs)."""
    import ctypes
    import torch
    from mla_latent_cache_absorbed_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.mla_probe_mfma.restype = ctypes.c_double
    lib.mla_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_probe_sink_bytes.restype = ctypes.c_size_t
    lib.mla_probe_sink_bytes.argtypes = [ctypes.c_int32]
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    # 4 operand fragments of 64 lanes x 8 bf16, as the kernel indexes them
    ab = torch.randn(4 * 64 * 8, generator=g, device=dev).to(torch.bfloat16).contiguous()
    sink = torch.empty(lib.mla_probe_sink_bytes(2), dtype=torch.uint8, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    st = torch.cuda.current_stream()
    runs, ghz, busy = {}, {}, {}
    for shape, wpc in ((32, 1), (32, 2), (16, 1)):
        key = f"wg{wpc}" if shape == 32 else f"16x16x32_wg{wpc}"
        fl = lib.mla_probe_mfma(ab.data_ptr(), iters, wpc, shape, sink.data_ptr(), None, st.cuda_stream)
        if fl <= 0:
            raise RuntimeError("MFMA probe failed to launch")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for r in range(reps):
            lib.mla_probe_mfma(ab.data_ptr(), iters, wpc, shape, sink.data_ptr(),
                               clk.data_ptr() if r == reps - 1 else None, st.cuda_stream)
        e1.record(st)
        torch.cuda.synchronize()
        runs[key] = fl / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
        cyc, ticks = (int(v) for v in clk.tolist())
        # core clock of the first wave's loop, and the share of its cycles
        # its MFMA pipe was busy if each 32,768 flop take 32 cycles (the
        # 32x32x16 rate; 2 x 4 of them per round)
        ghz[key] = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else None
        busy[key] = wpc * iters * 8 * 32 / cyc if cyc > 0 else None
    del ab, sink, clk
    best = max(v for k, v in runs.items() if not k.startswith("16x16x32"))
    return {"tflops": runs, "best_tflops": best, "frac_of_peak": best / MFMA_BF16_PEAK_TFS,
            "core_clock_ghz": ghz, "simd_mfma_busy": busy}


def attainable_peaks(achieved_gbs: float, tflops: float) -> dict:
    """Peaks this box attains, timed with events: the read-only streaming
    probes (see stream_read_record), the MFMA loop (see mfma_loop_record), a
    device-to-device copy of 2 GiB (reads and writes counted) and a bf16 GEMM
    (8192^3 on hipBLASLt).  The attend kernel's rates are also given as
    fractions of them."""
    import torch
    sr = stream_read_record()
    mf = mfma_loop_record()
    dev = torch.device("cuda")
    x = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16).contiguous()
    bm = torch.randn(8192, 8192, device=dev).to(torch.bfloat16).contiguous()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_cp = timed(lambda: y.copy_(x), 10)
    t_mm = timed(lambda: torch.mm(a, bm), 10)
    cp_gbs = 2 * x.numel() / t_cp / 1e9
    mm_tfs = 2 * 8192 ** 3 / t_mm / 1e12
    del x, y, a, bm
    read_best = max(sr["best_gb_s"][m] for m in ("global_load_to_registers", "direct_to_lds"))
    return {"stream_read": sr, "mfma_loop": mf, "copy_read_write_gbs": cp_gbs, "bf16_gemm_tflops": mm_tfs,
            "attend_frac_of_stream_read": achieved_gbs / read_best,
            "attend_frac_of_copy": achieved_gbs / cp_gbs,
            "attend_frac_of_mfma_loop": tflops / mf["best_tflops"],
            "attend_frac_of_gemm": tflops / mm_tfs}


def prewarm(fn, ms: float) -> int:
    """Untimed calls of fn for about ms milliseconds (in batches of 10, each
    synchronised), so that the timed calls after it run at the loaded clock;
    returns the number of calls."""
    import torch
    n = 0
    t_end = time.time() + ms * 1e-3
    while time.time() < t_end:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def append_record(w, reps: int = 200, prewarm_ms: float = 0.0) -> dict:
    """The paged latent append (the step before decode) on the same cache: one
    new token per request, written over each request's last cached row after
    the timed decode steps.  HIP events around `reps` launches."""
    import torch
    import mla_latent_cache_absorbed_amd as mla
    dev = w.q.device
    g = torch.Generator(device=dev).manual_seed(7)
    new = torch.randn((w.B, 576), generator=g, device=dev).to(torch.bfloat16)
    pos = (w.seq_lens - 1).clamp(min=0).to(torch.int32)
    mla.append_latent(new[:, :512], new[:, 512:], pos, w.block_table, w.cache)
    prewarm(lambda i: mla.append_latent(new[:, :512], new[:, 512:], pos, w.block_table, w.cache),
            prewarm_ms)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mla.append_latent(new[:, :512], new[:, 512:], pos, w.block_table, w.cache)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    moved = w.B * 576 * 2 * 2  # each row read once and written once
    # the fp8 form into an fp8 cache of the same shape (bf16 row read, e4m3 row written)
    c8 = torch.empty(w.cache.shape, dtype=torch.uint8, device=dev)
    kvs = 0.0625

    def app8(i=0):
        mla.append_latent_fp8(new[:, :512], new[:, 512:], pos, w.block_table, c8, kvs)
    app8()
    prewarm(app8, prewarm_ms)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        app8()
    e1.record()
    torch.cuda.synchronize()
    t8 = e0.elapsed_time(e1) / reps * 1e-3
    del c8
    return {"kernel": "mla_append_kernel", "rows": w.B, "launch_us": t * 1e6,
            "gb_s": moved / t / 1e9,
            "fp8": {"kernel": "mla_append_fp8_kernel", "launch_us": t8 * 1e6,
                    "gb_s": w.B * 576 * 3 / t8 / 1e9}}


def absorb_record(B: int, H: int, reps: int = 96, prewarm_ms: float = 0.0, copies: int = 12) -> dict:
    """Query absorption and value up-projection at the decode's batch shape,
    with random weights of the layer's shape (W_UK, W_UV: [H, 128, 512] bf16).
    HIP events around `reps` launches of each, rotating over `copies`
    independent sets of weights and activations (~80 MB each, together well
    past the 256 MB Infinity Cache), as the layers of a model do; bytes are
    the weights plus the activations read and written once.  Reported beside
    it: the time with only the weights rotating (the activations fixed, as
    they are when the kernel before has just written them) and with the same
    inputs every launch (then served from the Infinity Cache)."""
    import torch
    import mla_latent_cache_absorbed_amd as mla
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(11)
    sets = []
    for _ in range(copies):
        q_in = torch.randn((B, H, 192), generator=g, device=dev).to(torch.bfloat16)
        w_uk = (torch.randn((H, 128, 512), generator=g, device=dev) / 128 ** 0.5).to(torch.bfloat16)
        w_uv = (torch.randn((H, 128, 512), generator=g, device=dev) / 512 ** 0.5).to(torch.bfloat16)
        out = torch.randn((B, H, 512), generator=g, device=dev).to(torch.bfloat16)
        w_uk_t = mla.absorb_prepare(w_uk)
        del w_uk
        sets.append((q_in, w_uk_t, w_uv, out, torch.empty((B, H, 576), dtype=torch.bfloat16, device=dev),
                     torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)))

    # which set's activations and which set's weights launch i uses
    modes = {"all": lambda i: (i % copies, i % copies), "weights": lambda i: (0, i % copies),
             "none": lambda i: (0, 0)}

    def timed(fn, mode):
        pick = modes[mode]
        fn(0, 0)
        prewarm(lambda i: fn(*pick(i)), prewarm_ms)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(*pick(i))
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    def absorb(i, j):
        mla.absorb_query(sets[i][0], sets[j][1], sets[i][4])

    def up(i, j):
        mla.up_project(sets[i][3], sets[j][2], sets[i][5])

    flops = 2.0 * B * H * 128 * 512
    res = {}
    for name, fn, nbytes in [
            ("absorb_query", absorb, H * 512 * 128 * 2 + B * H * 192 * 2 + B * H * 576 * 2),
            ("up_project", up, H * 128 * 512 * 2 + B * H * 512 * 2 + B * H * 128 * 2)]:
        t = timed(fn, "all")
        t_w = timed(fn, "weights")
        t_same = timed(fn, "none")
        gbs = nbytes / t / 1e9
        res[name] = {"kernel": "mla_head_gemm_kernel", "launch_us": t * 1e6,
                     "algorithmic_bytes": nbytes, "gb_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                     "tflops": flops / t / 1e12, "copies_rotated": copies,
                     "launch_us_weights_rotating": t_w * 1e6,
                     "hbm_frac_weights_rotating": nbytes / t_w / 1e9 / HBM_PEAK_GBS,
                     "launch_us_same_inputs": t_same * 1e6}
    del sets
    return res


def fp8_record(w, layers_copies: int, steps: int, warmup: int, prewarm_ms: float = 0.0) -> dict:
    """The same decode step over an FP8 (e4m3) copy of the workload's cache:
    fresh fp8 caches rotated like the bf16 ones, plan + attend per step, after
    the same pre-warm as the bf16 steps (building the fp8 caches leaves the
    GPU idle for a while); the steps are timed between two events, then a
    second run brackets every attend launch with HIP events."""
    import torch
    import mla_latent_cache_absorbed_amd as mla
    from mla_latent_cache_absorbed_amd import accounting as acc
    from mla_latent_cache_absorbed_amd import workloads as wl
    dev = w.q.device
    kv = wl.DEFAULT_KV_SCALE
    caches = [wl.fp8_cache(w.cache, kv)]
    for i in range(1, layers_copies):
        g = torch.Generator(device=dev).manual_seed(2000 + i)
        c = torch.randn(w.cache.shape, generator=g, device=dev).to(torch.bfloat16)
        caches.append(wl.fp8_cache(c, kv))
        del c
    B, H, M, BS = w.B, w.H, w.M, w.BS
    ws = mla.Workspace(B, H, M, BS, dev)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    def step(i, ev=None):
        mla.plan(w.seq_lens, H, M, BS, ws)
        if ev is not None:
            ev[0].record()
        mla.attend_fp8(w.q, caches[i % len(caches)], w.block_table, w.scale, kv, out, lse, ws)
        if ev is not None:
            ev[1].record()

    n_pre = prewarm(step, prewarm_ms)
    for i in range(warmup):
        step(n_pre + i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    n0 = n_pre + warmup
    start.record()
    for i in range(steps):
        step(n0 + i)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    # the attend launches on their own, in a second run (each event record
    # adds a few microseconds between launches)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for i in range(steps):
        step(n0 + steps + i, pairs[i])
    torch.cuda.synchronize()
    att = sorted(a.elapsed_time(b) for a, b in pairs)
    att_avg = sum(att) / len(att)
    seq = w.seq_lens_list()
    alg_bytes = acc.algorithmic_bytes(seq, H, BS, row_bytes=576)
    alg_flops = acc.algorithmic_flops(seq, H)
    gbs = alg_bytes / (att_avg * 1e-3) / 1e9
    tfs = alg_flops / (att_avg * 1e-3) / 1e12
    del caches
    return {"kernel": ("mla_attend_narrow_kernel<fp8>" if H <= 32 else "mla_attend_kernel<fp8>"),
            "kv_scale": kv, "ms_per_step": ms_step,
            "value": acc.token_reads(seq) / (ms_step * 1e-3), "unit": "cached-token reads/s",
            "launch_ms": att_avg, "launch_ms_median": att[len(att) // 2], "launch_ms_min": att[0],
            "algorithmic_bytes_per_launch": alg_bytes, "achieved_gb_s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "mfma_tflops": tfs, "mfma_frac": tfs / MFMA_BF16_PEAK_TFS}


def make_copies(name: str, copies: int, dev):
    """The workload's inputs on the device: `copies` independent caches (and
    queries) over one table and length vector, rotated by the timed steps so
    that no call finds its cache in the 256 MB Infinity Cache; step61 holds
    its 61 layers instead."""
    import torch
    from mla_latent_cache_absorbed_amd import workloads as wl
    fp8 = name == "dp_rank_fp8"   # the DP-rank workload over FP8 copies of its caches
    if fp8:
        name = "dp_rank"
    spec = wl.spec(name)
    ncopies = spec.layers if name == "step61" else max(1, copies)
    print(f"[bench] generating {ncopies} x {name} on {torch.cuda.get_device_name(0)}",
          file=sys.stderr, flush=True)
    wls = []
    for i in range(ncopies):
        if name == "step61":
            w = wl.make(name, device=dev, seed=0, layer=i)
        elif i == 0:
            w = wl.make(name, device=dev, seed=0)
        else:  # extra copies: same table and lengths, fresh q and cache
            base = wls[0]
            g = torch.Generator(device=dev).manual_seed(1000 + i)
            q = torch.randn(base.q.shape, generator=g, device=dev).to(torch.bfloat16)
            c = torch.randn(base.cache.shape, generator=g, device=dev).to(torch.bfloat16)
            w = wl.Workload(name, q, c, base.block_table, base.seq_lens, base.scale)
        if fp8:
            w = wl.Workload(w.name, w.q, wl.fp8_cache(w.cache, wl.DEFAULT_KV_SCALE), w.block_table,
                            w.seq_lens, w.scale)
        wls.append(w)
    torch.cuda.synchronize()
    return wls


def measure(wls, steps: int, warmup: int, prewarm_ms: float) -> dict:
    """Timed decode steps over the workload: one step is one plan and one
    attend per layer (step61: 61 layers, each on its own cache), all on the
    current stream.  Untimed steps for prewarm_ms, then `warmup` steps, then
    `steps` steps between two events: the step time.  A second run of `steps`
    steps brackets every attend launch with HIP events (on the stream the
    kernel runs on) for the kernel's own duration; it is kept out of the
    first, since each event record adds a few microseconds between launches."""
    import torch
    import mla_latent_cache_absorbed_amd as mla
    from mla_latent_cache_absorbed_amd import workloads as wl
    w0 = wls[0]
    layers = wl.spec(w0.name).layers if w0.name in wl.NAMES else 1
    B, H, M, BS = w0.B, w0.H, w0.M, w0.BS
    dev = w0.q.device
    ws = mla.Workspace(B, H, M, BS, dev)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    fp8 = w0.cache.dtype == torch.uint8

    def step(i, ev=None):
        mla.plan(w0.seq_lens, H, M, BS, ws)
        for l in range(layers):
            w = wls[(i * layers + l) % len(wls)]
            if ev is not None:
                ev[0].record()
            if fp8:
                mla.attend_fp8(w.q, w.cache, w.block_table, w.scale, wl.DEFAULT_KV_SCALE, out, lse, ws)
            else:
                mla.attend(w.q, w.cache, w.block_table, w.scale, out, lse, ws)
            if ev is not None:
                ev[1].record()
                ev.pop(0)
                ev.pop(0)

    # bring the GPU from idle to its loaded clock (steps take ~2x longer for
    # the first ~10 ms), then the warm-up steps
    n_pre = prewarm(step, prewarm_ms) if prewarm_ms > 0 else 0
    for i in range(warmup):
        step(n_pre + i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    n0 = n_pre + warmup
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(n0 + i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    # the attend launches on their own
    n_attend = steps * layers
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_attend)]
    pairs = [(evs[2 * j], evs[2 * j + 1]) for j in range(n_attend)]
    queue = [e for p in pairs for e in p]
    for i in range(steps):
        step(n0 + steps + i, queue)
    torch.cuda.synchronize()
    attend_ms = sorted(a.elapsed_time(b) for a, b in pairs)
    return {"layers": layers, "ms_step": ms_step, "fp8": fp8,
            "attend_avg_ms": sum(attend_ms) / len(attend_ms),
            "attend_median_ms": attend_ms[len(attend_ms) // 2], "attend_min_ms": attend_ms[0],
            "hdr": ws.header(), "prewarm_steps": n_pre}


def workload_config(name: str, w0, layers: int, copies: int, prewarm_steps: int) -> dict:
    seq = w0.seq_lens_list()
    return {"workload": name, "batch": w0.B,
            "seq_lens": "4096 each" if name in ("dp_rank", "tp_slice", "step61") else f"sum {sum(seq)}",
            "heads": w0.H, "block_size": w0.BS, "blocks": w0.NB, "layers": layers,
            "cache_copies": copies, "prewarm_steps": prewarm_steps}


def workload_record(name: str, w0, m: dict) -> dict:
    """Roofline record of the attend kernel on the workload: algorithmic
    bytes and flops of one launch (one layer) over the mean launch time."""
    from mla_latent_cache_absorbed_amd import accounting as acc
    seq = w0.seq_lens_list()
    H, BS, layers = w0.H, w0.BS, m["layers"]
    alg_bytes = acc.algorithmic_bytes(seq, H, BS, row_bytes=576 if m["fp8"] else 1152)
    alg_flops = acc.algorithmic_flops(seq, H)
    t = m["attend_avg_ms"] * 1e-3
    achieved_gbs = alg_bytes / t / 1e9
    tflops = alg_flops / t / 1e12
    intensity = alg_flops / alg_bytes
    bound = "hbm" if intensity < MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    roof_t = max(alg_bytes / (HBM_PEAK_GBS * 1e9), alg_flops / (MFMA_BF16_PEAK_TFS * 1e12))
    ms_step = m["ms_step"]
    return {
        "achieved_hbm_tb_s": layers * alg_bytes / (ms_step * 1e-3) / 1e12,
        "roofline_frac_step": roof_t * layers / (ms_step * 1e-3),
        "roofline": {
            "bound": bound,
            "kernel": ("mla_attend_narrow_kernel" if H <= 32 else "mla_attend_kernel")
            + ("<fp8>" if m["fp8"] else ""),
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": hbm_traffic_record(name),
            "launch_ms": m["attend_avg_ms"],
            "launch_ms_median": m["attend_median_ms"],
            "launch_ms_min": m["attend_min_ms"],
            "algorithmic_bytes_per_launch": alg_bytes,
            "mfma_tflops": tflops,
            "mfma_frac": tflops / MFMA_BF16_PEAK_TFS,
            "intensity_flop_per_byte": intensity,
        },
        "plan": {"items": m["hdr"][0], "chunk_tokens": m["hdr"][1]},
    }


ATTEND_KERNELS = {  # name prefix (as rocprofv3 reports it) of the attend kernel each workload runs
    "dp_rank": "void (anonymous namespace)::mla_attend_kernel<4, 4, true, false>",
    "ragged": "void (anonymous namespace)::mla_attend_kernel<4, 4, true, false>",
    "step61": "void (anonymous namespace)::mla_attend_kernel<4, 4, true, false>",
    "tp_slice": "void (anonymous namespace)::mla_attend_narrow_kernel<true, false>",
    "dp_rank_fp8": "void (anonymous namespace)::mla_attend_kernel<4, 8, true, true>",
}


def profile_commands(name: str) -> dict:
    """The rocprofv3 commands whose output --profile-dir summarises, with R
    the repository root and O the output directory."""
    run = f"python -u $R/bench.py --workload {name} --no-cpu --no-extras"
    pre = "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3"
    return {
        "kt": f"{pre} --kernel-trace --stats -d $O/kt -o kt --output-format csv -- {run} --steps 20 --warmup 5",
        "fetch": f"{pre} --pmc FETCH_SIZE -d $O/fetch -o p --output-format csv -- {run} --steps 3 --warmup 1 --prewarm-ms 0",
        "write": f"{pre} --pmc WRITE_SIZE -d $O/write -o p --output-format csv -- {run} --steps 3 --warmup 1 --prewarm-ms 0",
        "mfma": f"{pre} --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 -d $O/mfma -o p --output-format csv -- {run} --steps 3 --warmup 1 --prewarm-ms 0",
        "copy_fetch": f"{pre} --pmc FETCH_SIZE -d $O/copy_fetch -o p --output-format csv -- python -u $R/bench.py --copy-probe",
        "copy_write": f"{pre} --pmc WRITE_SIZE -d $O/copy_write -o p --output-format csv -- python -u $R/bench.py --copy-probe",
    }


def write_profiles(name: str, d: str) -> None:
    """profiles/ summaries of one workload from rocprofv3 output under d: the
    HBM-traffic record bench.py reads, a kernel-trace table and the MFMA
    counters of the attend kernel."""
    from mla_latent_cache_absorbed_amd import accounting as acc
    from mla_latent_cache_absorbed_amd import workloads as wl
    cmds = profile_commands(name)
    kp = ATTEND_KERNELS[name]
    sub = lambda k: os.path.join(d, k)  # noqa: E731
    rec = write_counter_record(name, sub("fetch"), sub("write"), sub("copy_fetch"), sub("copy_write"),
                               kp, [cmds[k] for k in ("fetch", "write", "copy_fetch", "copy_write")])
    sp = wl.spec("dp_rank" if name == "dp_rank_fp8" else name)
    seq = list(sp.seq_lens)
    alg_bytes = acc.algorithmic_bytes(seq, sp.H, sp.BS, row_bytes=576 if name == "dp_rank_fp8" else 1152)
    alg_flops = acc.algorithmic_flops(seq, sp.H)
    stats = _rocprof_rows(sub("kt"), "kernel_stats.csv")
    lines = [f"# Attend kernel, {name} workload ({sp.B} requests, {sp.H} heads, BS {sp.BS}, "
             f"{sp.layers} layer(s)): kernel trace and counters", "",
             "Commands, on one MI355X, with `R` the repository root and `O` an output directory:", "",
             "```"] + [cmds[k] for k in ("kt", "fetch", "write", "mfma", "copy_fetch", "copy_write")] + \
            ["```", "", f"Source hash (sha256, first 16 hex of mla_decode.hip): `{src_hash()}`", "",
             "| kernel | calls | average ns | min ns | max ns | % of GPU time |", "|---|---|---|---|---|---|"]
    att = None
    for r in stats:
        nm = r.get("Name", r.get("KernelName", ""))
        short = nm if len(nm) < 70 else nm[:67] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} | "
                     f"{float(r['MaxNs']):.0f} | {float(r['Percentage']):.2f} |")
        if nm.startswith(kp):
            att = float(r["AverageNs"])
    lines += ["", f"Algorithmic bytes per attend launch: {alg_bytes:,} B; flops {alg_flops:.4e}."]
    if att:
        lines.append(f"At the trace's average attend duration ({att / 1e3:.1f} us): "
                     f"{alg_bytes / att:.0f} GB/s ({alg_bytes / att / HBM_PEAK_GBS * 100:.1f} % of 8 TB/s), "
                     f"{alg_flops / att / 1e3:.0f} TFLOP/s.")
    lines += ["", "HBM traffic of one attend launch (counters, scaled by a 1 GiB copy's reading):", "",
              f"* FETCH_SIZE {rec['attend_FETCH_SIZE_KiB_per_dispatch']:.1f} KiB per dispatch x "
              f"{rec['fetch_scale']:.4f} = {rec['read_bytes_per_launch']:,.0f} B read",
              f"* WRITE_SIZE {rec['attend_WRITE_SIZE_KiB_per_dispatch']:.1f} KiB per dispatch x "
              f"{rec['write_scale']:.4f} = {rec['write_bytes_per_launch']:,.0f} B written",
              f"* total {rec['traffic_bytes_per_launch']:,.0f} B = "
              f"{rec['traffic_bytes_per_launch'] / alg_bytes:.3f} x the algorithmic bytes"]
    mf = counter_means(sub("mfma"), kp)
    if mf:
        busy, n = mf["SQ_VALU_MFMA_BUSY_CYCLES"]
        gui = mf["GRBM_GUI_ACTIVE"][0]
        mops = mf["SQ_INSTS_VALU_MFMA_MOPS_BF16"][0]
        lines += ["", f"MFMA counters (means over {n} attend dispatches, summed over the 8 XCDs):", "",
                  f"* SQ_INSTS_VALU_MFMA_MOPS_BF16 {mops:.4e} (x 512 = {mops * 512:.4e} flop; "
                  f"algorithmic {alg_flops:.4e})",
                  f"* SQ_VALU_MFMA_BUSY_CYCLES {busy:.4e}; GRBM_GUI_ACTIVE {gui:.4e} "
                  f"({gui / 8:.4e} per XCD)",
                  f"* MFMA busy = busy / (GUI per XCD x 1,024 SIMDs) = {busy / (gui / 8 * 1024) * 100:.1f} %"]
    with open(os.path.join(PROFILES, f"mla_attend_{name}_profile.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


TRACE_ALL_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 400 rocprofv3 --kernel-trace --stats "
                 "-d $O/kt_all -o kt --output-format csv -- python -u $R/bench.py --no-cpu")


def write_trace_summary(d: str) -> str:
    """profiles/bench_default_run_kernel_trace.md: every kernel of the default
    bench run (all workloads and the fp8, append, absorption and probe
    records), from rocprofv3's kernel statistics under d."""
    stats = _rocprof_rows(d, "kernel_stats.csv")
    lines = ["# Kernel trace of the default benchmark run", "",
             "Command, on one MI355X, with `R` the repository root and `O` an output directory:", "",
             "```", TRACE_ALL_CMD, "```", "",
             f"Source hash (sha256, first 16 hex of mla_decode.hip): `{src_hash()}`", "",
             "Every kernel the run launches: the timed steps of each workload and the records after "
             "them (plan, attend, fp8 attend, append, absorption GEMMs, probes) and the input "
             "generation (torch kernels).", "",
             "| kernel | calls | average ns | min ns | max ns | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats:
        nm = r.get("Name", r.get("KernelName", ""))
        short = nm if len(nm) < 90 else nm[:87] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} | "
                     f"{float(r['MaxNs']):.0f} | {float(r['Percentage']):.2f} |")
    out = os.path.join(PROFILES, "bench_default_run_kernel_trace.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


def main():
    args = parse()
    if args.trace_summary:
        print(write_trace_summary(args.trace_summary))
        return
    if args.profile_dir:
        write_profiles(args.workload, args.profile_dir)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode "
              "path has no multi-GPU code", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe()
        return
    import mla_latent_cache_absorbed_amd as mla
    from mla_latent_cache_absorbed_amd import accounting as acc
    from mla_latent_cache_absorbed_amd import workloads as wl

    dev = torch.device("cuda:0")
    name = args.workload
    wls = make_copies(name, args.copies, dev)
    m = measure(wls, args.steps, args.warmup, args.prewarm_ms)
    w0 = wls[0]
    B, H, M, BS, NB = w0.B, w0.H, w0.M, w0.BS, w0.NB
    seq = w0.seq_lens_list()
    layers = m["layers"]
    ms_step = m["ms_step"]
    rec = {
        "metric": METRIC,
        "value": acc.token_reads(seq, layers) / (ms_step * 1e-3),
        "unit": "cached-token reads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": workload_config(name, w0, layers, len(wls), m["prewarm_steps"]),
    }
    rec.update(workload_record(name, w0, m))
    if not args.no_extras and name == "dp_rank":
        # the other workloads of the path, each measured the same way: one
        # JSON object per workload with its own roofline record
        rec["workloads"] = {}
        for other in ("tp_slice", "ragged", "step61"):
            print(f"[bench] {other}", file=sys.stderr, flush=True)
            ow = make_copies(other, args.copies, dev)
            om = measure(ow, args.steps, args.warmup, args.prewarm_ms)
            o0 = ow[0]
            orec = {"config": workload_config(other, o0, om["layers"], len(ow), om["prewarm_steps"]),
                    "ms_per_step": om["ms_step"],
                    "value": acc.token_reads(o0.seq_lens_list(), om["layers"]) / (om["ms_step"] * 1e-3),
                    "unit": "cached-token reads/s"}
            orec.update(workload_record(other, o0, om))
            rec["workloads"][other] = orec
            del ow, om, o0
            torch.cuda.empty_cache()
    if not args.no_extras:
        if BS >= 32 and name != "step61":
            rec["fp8"] = fp8_record(w0, len(wls), args.steps, args.warmup, args.prewarm_ms)
        rec["append"] = append_record(w0, prewarm_ms=args.prewarm_ms)
        rec["absorb"] = absorb_record(B, H, prewarm_ms=args.prewarm_ms)
        rec["attainable"] = attainable_peaks(rec["roofline"]["achieved"], rec["roofline"]["mfma_tflops"])
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
