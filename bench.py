#!/usr/bin/env python3
"""Attention-forward bench on one MI355X (gfx950).

A step is one call of the hot path -- the HIP attention forward (``attn_fwd``, or
``attn_fwd_varlen`` for the packed workload) -- over one batch of seeded synthetic BF16
inputs that are already resident in HBM. W untimed warm-up steps (by default as many as
take about half a second, at least 3), then exactly K timed steps between device
synchronisations. Throughput counts 4*B*H*N^2*d flops per step
(packed: sum over segments of 4*H*n^2*d) and is reported in TFLOP/s against the MI355X
dense BF16 MFMA peak; the kernel's own duration is measured with HIP events recorded on
the stream it is launched on.

Beside it: the FP64 CPU oracle timed on a bounded seeded sample of query rows of the same
workload (host cores), and a parity check of those rows against the GPU output.

One JSON line is printed (rank 0). Run several GPUs? This bench is single-GPU only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X published dense BF16 MFMA peak
METRIC = "attention TFLOP/s (4·B·H·N²·d) and % of BF16 MFMA peak, 720p-like N"
PEAK_HBM_GBS = 8000.0              # MI355X published HBM3E bandwidth
CSRC = os.path.join(ROOT, "video_diffusion_dit_amd", "csrc")
# sources whose hash a traffic record must match, per kind of call
KERNEL_SOURCES = {
    "dense": ("attn_fwd_gfx950.hip", "key_loop_gfx950.inc"),
    "varlen": ("attn_fwd_gfx950.hip", "key_loop_gfx950.inc"),
    "prologue": ("prologue_gfx950.hip",),
    "packed_prologue": ("prologue_gfx950.hip",),
    "linear": ("linear_gfx950.hip",),
    "block_sparse": ("attn_fwd_gfx950.hip", "key_loop_idx_gfx950.inc", "block_route_gfx950.hip"),
    "block_sparse_varlen": ("attn_fwd_gfx950.hip", "key_loop_idx_gfx950.inc", "block_route_gfx950.hip"),
}
PROFILES = os.path.join(ROOT, "profiles")
WARMUP_S = 0.5   # default warm-up length in seconds


def default_warmup(one_call_s: float) -> int:
    """Warm-up calls for a call of one_call_s seconds: about WARMUP_S seconds of them, at
    least 3 (the two calls that measured the duration included)."""
    import math
    return max(3, math.ceil(WARMUP_S / max(one_call_s, 1e-6)))


def kernel_source_hash(kind: str = "dense") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# Kernels one call dispatches (the first is the dominant one).
CALL_KERNELS = {
    "dense": ("attn_fwd_dense_kernel", "attn_fwd_dense_split_kernel", "merge_kernel"),
    "varlen": ("attn_fwd_varlen_kernel", "build_varlen_schedule", "varlen_split_plan", "attn_fwd_varlen_split_kernel",
               "varlen_merge_kernel"),
    "prologue": ("qk_prologue_kernel",),
    "packed_prologue": ("qk_norm_packed_kernel",),
    "linear": ("linear_out_kernel", "linear_kv_partial_kernel", "linear_kv_reduce_kernel"),
    "block_sparse": ("attn_fwd_block_sparse_kernel", "route_kernel", "pool_kernel", "lpt_order_kernel"),
    "block_sparse_varlen": ("attn_fwd_block_sparse_varlen_kernel", "route_varlen_kernel", "pool_varlen_kernel",
                            "tile_offsets_kernel", "lpt_order_kernel", "scale_count_kernel", "build_varlen_schedule"),
}


def prologue_bytes(B: int, N: int, H: int, d: int = 128) -> float:
    """Algorithmic HBM bytes of one prologue call: Q, K, V rows read once and written once."""
    return float(B) * N * H * d * 2 * 6


def linear_bytes(B: int, N: int, H: int, d: int = 128) -> float:
    """Algorithmic HBM bytes of one linear-attention call: q, k, q_rot, k_rot, v read once, out
    written once (the d x d state and the chunk partials are not counted)."""
    return float(B) * N * H * d * 2 * 6


def measured_traffic(workload: str, kernel: str, split_kv: bool, kind: str = "dense"):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources with the same split-KV setting; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash(kind):
        return None
    if fields.get("split_kv", "false") != ("true" if split_kv else "false"):
        return None
    try:
        return float(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _base_name(name: str) -> str:
    """"void (anonymous namespace)::pool_kernel<64>(...)" -> "pool_kernel"; a name the profiler
    left mangled ("_ZN12_GLOBAL__N_118pool_varlen_kernelILi64EE...") -> "pool_varlen_kernel"."""
    import re
    m = re.match(r"_ZN(?:\d+_GLOBAL__N_1)?(\d+)", name)
    if m:
        return name[m.end():m.end() + int(m.group(1))]
    name = name.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0]
    return name.split("::")[-1].split()[-1]


def _of_call(order, names) -> set:
    """Dispatch ids (of `order`, [(dispatch id, base name)] in dispatch order) that belong to
    one call of the kernels `names`. A kernel that calls of several kinds share (the varlen
    schedule builder, the longest-first sort) belongs to the call whose next own kernel
    follows it."""
    shared = {n for n in names if sum(n in v for v in CALL_KERNELS.values()) > 1}
    known = {n for v in CALL_KERNELS.values() for n in v}
    keep = set()
    for i, (d, n) in enumerate(order):
        if n not in names:
            continue
        if n in shared:
            nxt = next((m for _, m in order[i + 1:] if m in known and m not in shared), None)
            if nxt is not None and nxt not in names:
                continue
        keep.add(d)
    return keep


def _pmc_dispatches(csv_path: str, counter: str):
    """[(dispatch id, kernel name, value in KiB)] for one counter of a rocprofv3 CSV, in order."""
    import csv
    acc = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
            acc[key] = acc.get(key, 0.0) + float(row["Counter_Value"])
    return [(d, name, v) for (d, name), v in sorted(acc.items())]


def write_traffic_profile(args) -> int:
    """Scale FETCH_SIZE/WRITE_SIZE of one call's kernels by what the same counters read for a
    copy of known size, and record the result with the kernel-source hash."""
    fetch_csv, write_csv = args.write_traffic_profile
    kind = args.traffic_kind or ("varlen" if "varlen" in args.workload else "dense")
    names = CALL_KERNELS[kind]
    kernel = names[0]
    copy_bytes = float(args.calibrate_copy_mib << 20)
    if copy_bytes <= 0:
        raise SystemExit("--calibrate-copy-mib (the copy size of the profiled run) is required")

    base = _base_name

    def split(rows):
        mine = _of_call([(d, base(name)) for d, name, _ in rows], names)
        att = [(name, v) for d, name, v in rows if d in mine]
        others = [(d, name, v) for d, name, v in rows if base(name) not in names]
        calls = sum(1 for name, _ in att if base(name) == names[0])
        return att, calls, others[-1]    # the calibration copy is the last dispatch of the run

    f_att, f_calls, (_, copy_key, f_copy_kib) = split(_pmc_dispatches(fetch_csv, "FETCH_SIZE"))
    w_att, w_calls, (_, _, w_copy_kib) = split(_pmc_dispatches(write_csv, "WRITE_SIZE"))
    split_kv = any(k in name for name, _ in f_att for k in ("attn_fwd_dense_split_kernel", "varlen_split_plan"))
    f_copy, w_copy = f_copy_kib * 1024.0, w_copy_kib * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    fetch_b = sum(v for _, v in f_att) / f_calls * 1024.0 * f_scale
    write_b = sum(v for _, v in w_att) / w_calls * 1024.0 * w_scale
    from workloads import WORKLOADS
    w = WORKLOADS[args.workload]
    tokens = w.B * w.N if w.kind == "dense" else w.total_tokens
    if kind == "prologue":
        algorithmic = prologue_bytes(w.B, w.N, w.H, w.d)
    elif kind == "packed_prologue":
        algorithmic = float(w.total_tokens) * w.H * w.d * 2 * 4
    elif kind == "linear":
        algorithmic = linear_bytes(w.B, w.N, w.H, w.d)
    else:
        algorithmic = tokens * w.H * (8.0 * w.d + 4.0)
    path = os.path.join(PROFILES, f"{kernel}_{args.workload}_hbm_traffic.txt")
    with open(path, "w") as f:
        f.write(f"# HBM traffic of one call ({', '.join(n for n in names)} as dispatched) on the "
                f"{args.workload} workload ({w.description})\n")
        f.write("# from two rocprofv3 --pmc runs of bench.py, each also copying a buffer of known size\n")
        for line in (args.profile_command or "").split(";"):
            if line.strip():
                f.write(f"# command: {line.strip()}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash(kind)}\n")
        f.write(f"copy_kernel: {copy_key}\n")
        f.write(f"copy_bytes: {copy_bytes:.0f}\n")
        f.write(f"copy_fetch_kib_per_dispatch: {f_copy / 1024.0:.1f}\n")
        f.write(f"copy_write_kib_per_dispatch: {w_copy / 1024.0:.1f}\n")
        f.write(f"fetch_scale: {f_scale:.4f}\n")
        f.write(f"write_scale: {w_scale:.4f}\n")
        f.write(f"split_kv: {'true' if split_kv else 'false'}\n")
        for name in names:
            fk = sum(v for n, v in f_att if base(n) == name) / f_calls
            wk = sum(v for n, v in w_att if base(n) == name) / w_calls
            if fk or wk:
                f.write(f"raw_kib_per_call {name}: fetch {fk:.1f} write {wk:.1f}\n")
        f.write(f"fetch_bytes_per_call: {fetch_b:.0f}\n")
        f.write(f"write_bytes_per_call: {write_b:.0f}\n")
        f.write(f"traffic_bytes_per_call: {fetch_b + write_b:.0f}\n")
        f.write(f"algorithmic_bytes_per_call: {algorithmic:.0f}\n")
        f.write(f"traffic_over_algorithmic: {(fetch_b + write_b) / algorithmic:.3f}\n")
    print(open(path).read())
    return 0


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
FLOP_PER_MFMA = 32 * 32 * 16 * 2      # v_mfma_f32_32x32x16_bf16, the only MFMA the attention kernels issue


def write_mfma_profile(args) -> int:
    """Turn one rocprofv3 --pmc run of SQ_INSTS_MFMA, SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE into the profiles/ record of one call's matrix-core use: counter FLOP per
    call (MFMA instructions x 32768) against the algorithmic 4*B*H*N^2*d, that FLOP over the
    kernels' own durations in the same run against the published peak, the fraction of clocked
    cycles the matrix cores were busy, and the average shader clock."""
    import csv
    counter_csv, agent_csv = args.write_mfma_profile
    kind = args.traffic_kind or ("varlen" if "varlen" in args.workload else "dense")
    names = CALL_KERNELS[kind]
    kernel = names[0]

    base = _base_name
    with open(counter_csv) as f:
        seen = {int(row["Dispatch_Id"]): base(row["Kernel_Name"]) for row in csv.DictReader(f)}
    mine = _of_call(sorted(seen.items()), names)

    vals, spans, kname = {}, {}, {}
    with open(counter_csv) as f:
        for row in csv.DictReader(f):
            d = int(row["Dispatch_Id"])
            if d not in mine:
                continue
            kname[d] = base(row["Kernel_Name"])
            key = (d, row["Counter_Name"])
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
            spans[d] = (int(row["Start_Timestamp"]), int(row["End_Timestamp"]))
    simds, xcc = 1024, 8
    with open(agent_csv) as f:
        for row in csv.DictReader(f):
            if row.get("Name", "").startswith("gfx"):
                simds, xcc = int(row["Simd_Count"]), int(row["Num_Xcc"])
    calls = sum(1 for d in kname if kname[d] == kernel)
    if calls == 0:
        raise SystemExit(f"no {kernel} dispatch in {counter_csv}")

    def per_call(counter):
        return sum(v for (d, c), v in vals.items() if c == counter) / calls
    mfma = per_call("SQ_INSTS_MFMA")
    busy = per_call("SQ_VALU_MFMA_BUSY_CYCLES")
    grbm = per_call("GRBM_GUI_ACTIVE")
    ns = sum(e - s for s, e in spans.values()) / calls
    from workloads import WORKLOADS
    w = WORKLOADS[args.workload]
    counter_flops = mfma * FLOP_PER_MFMA
    algorithmic = w.flops()
    split_kv = any(kname[d] in ("attn_fwd_dense_split_kernel", "varlen_split_plan") for d in kname)
    path = os.path.join(PROFILES, f"{kernel}_{args.workload}_mfma_counters.txt")
    with open(path, "w") as f:
        f.write(f"# Matrix-core counters of one call ({', '.join(names)} as dispatched) on the "
                f"{args.workload} workload ({w.description})\n")
        f.write("# from one rocprofv3 --pmc run of bench.py; durations are the same run's dispatch timestamps\n")
        for line in (args.profile_command or "").split(";"):
            if line.strip():
                f.write(f"# command: {line.strip()}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash(kind)}\n")
        f.write(f"split_kv: {'true' if split_kv else 'false'}\n")
        f.write(f"calls: {calls}\n")
        for name in names:
            ds = [d for d in kname if kname[d] == name]
            if ds:
                m = sum(vals.get((d, "SQ_INSTS_MFMA"), 0.0) for d in ds) / calls
                ms = sum(spans[d][1] - spans[d][0] for d in ds) / calls / 1e6
                f.write(f"per_call {name}: SQ_INSTS_MFMA {m:.0f} duration_ms {ms:.3f}\n")
        f.write(f"simd_count: {simds}\n")
        f.write(f"xcc_count: {xcc}\n")
        f.write(f"sq_insts_mfma_per_call: {mfma:.0f}\n")
        f.write(f"sq_valu_mfma_busy_cycles_per_call: {busy:.0f}\n")
        f.write(f"grbm_gui_active_per_call: {grbm:.0f}\n")
        f.write(f"kernel_ms_per_call: {ns / 1e6:.4f}\n")
        f.write(f"counter_flops_per_call: {counter_flops:.6e}\n")
        if kind.startswith("block_sparse"):   # kept pairs only: the ratio to the dense FLOP is the density
            f.write(f"dense_flops_per_call: {algorithmic:.6e}\n")
            f.write(f"counter_over_dense_flops: {counter_flops / algorithmic:.4f}\n")
        else:
            f.write(f"algorithmic_flops_per_call: {algorithmic:.6e}\n")
            f.write(f"counter_over_algorithmic_flops: {counter_flops / algorithmic:.4f}\n")
        f.write(f"counter_tflops: {counter_flops / (ns * 1e-9) / 1e12:.1f}\n")
        f.write(f"mfma_util_of_peak: {counter_flops / (ns * 1e-9) / 1e12 / PEAK_BF16_TFLOPS:.4f}\n")
        f.write(f"mfma_busy_of_clocked_cycles: {(busy / simds) / (grbm / xcc):.4f}\n")
        f.write(f"avg_shader_clock_ghz: {(grbm / xcc) / ns:.3f}\n")
    print(open(path).read())
    return 0


def measured_mfma(workload: str, kernel: str, split_kv: bool, kind: str = "dense"):
    """Matrix-core figures of one call from the committed rocprofv3 counter record, if it was
    taken on the current kernel sources with the same split-KV setting; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_mfma_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash(kind):
        return None
    if fields.get("split_kv", "false") != ("true" if split_kv else "false"):
        return None
    keys = {"util_of_peak": "mfma_util_of_peak", "counter_tflops": "counter_tflops",
            "counter_over_algorithmic_flops": "counter_over_algorithmic_flops",
            "counter_over_dense_flops": "counter_over_dense_flops",
            "busy_of_clocked_cycles": "mfma_busy_of_clocked_cycles",
            "avg_shader_clock_ghz": "avg_shader_clock_ghz", "kernel_ms": "kernel_ms_per_call"}
    try:
        out = {k: float(fields[f]) for k, f in keys.items() if f in fields}
    except ValueError:
        return None
    if "util_of_peak" not in out:
        return None
    out["source"] = os.path.relpath(path, ROOT)
    return out


def time_prologue(args, w, vd, dev) -> dict:
    """Time the Q/K RMSNorm + 3-D RoPE prologue (with V re-laid) at the workload's token grid,
    on seeded projected inputs resident in HBM; check seeded tokens against the oracle."""
    import numpy as np
    import torch

    from workloads import make_projected
    t0 = time.time()
    xb = make_projected(w.B, w.grid, w.H, seed=0)
    xs = [dev(b) for b in xb]
    outs = tuple(torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda:0") for _ in range(3))
    print(f"[bench] prologue inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def call():
        vd.qk_prologue(xs[0], xs[1], xs[2], grid=w.grid, out=outs)

    stream = torch.cuda.current_stream()
    for _ in range(2):
        call()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.prologue_steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.prologue_steps)]
    torch.cuda.synchronize()
    for i in range(args.prologue_steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg = float(np.mean(ms))
    nbytes = prologue_bytes(w.B, w.N, w.H, w.d)
    gbs = nbytes / (avg * 1e-3) / 1e9
    rec = {
        "kernel": "qk_prologue_kernel",
        "what": "per-head RMSNorm + interleaved 3-D RoPE of Q and K, V re-laid, [B,N,H,128] -> [B,H,N,128] BF16",
        "bound": "hbm",
        "achieved": round(gbs, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(gbs / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(w.name, "qk_prologue_kernel", False, "prologue"),
        "algorithmic_bytes": nbytes,
        "ms": {"avg": round(avg, 4), "min": round(min(ms), 4), "max": round(max(ms), 4)},
        "steps": args.prologue_steps,
    }
    print(f"[bench] prologue {args.prologue_steps} calls: {avg:.4f} ms -> {gbs:.0f} GB/s "
          f"({100 * gbs / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:.0f})", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        from oracle import bf16_bits_to_f64, bf16_faithful, qk_norm_rope
        toks = np.random.default_rng(1).choice(w.N, 4096, replace=False)
        got = outs[0].view(torch.int16).cpu().numpy().view(np.uint16)[:, :, toks]
        t1 = time.perf_counter()
        exact = qk_norm_rope(xb[0], w.grid, tokens=toks)
        cpu_s = time.perf_counter() - t1
        m = bf16_faithful(bf16_bits_to_f64(got), exact)
        rec["parity"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in m.items()}
        sample_bytes = float(len(toks)) * w.B * w.H * w.d * 2 * 2      # Q rows read and written
        rec["cpu_baseline"] = {"value": round(sample_bytes / cpu_s / 1e9, 4), "unit": "GB/s",
                               "cores": oracle_cores(), "kind": "oracle",
                               "sample": f"Q of {len(toks)} seeded tokens x {w.H} heads (the GPU call also does K and V), "
                                         f"FP64 NumPy, {cpu_s:.2f} s"}
    # a practical ceiling for this byte mix: plain device-to-device copies of the same three
    # tensors (the same bytes read and written), timed the same way
    def copies():
        for x, o in zip(xs, outs):
            o.view(torch.int16).copy_(x.view(torch.int16).view(o.shape[0], o.shape[2], o.shape[1], o.shape[3])
                                      .reshape(o.shape))
    copies()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(5):
        copies()
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 5
    rec["copy_reference"] = {"what": "device-to-device copies of the same three tensors (same bytes read and written)",
                             "achieved": round(nbytes / (copy_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                             "ms": round(copy_ms, 4)}
    print(f"[bench] plain copy of the same bytes: {copy_ms:.4f} ms -> {nbytes / (copy_ms * 1e-3) / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)
    del xs, outs
    torch.cuda.empty_cache()
    return rec


def time_packed_norm(args, w, vd, dev) -> dict:
    """Time the packed prologue (per-head RMSNorm of THD Q and K, in their own layout) at the
    packed workload's tokens and heads, on seeded projected rows resident in HBM; check seeded
    tokens against the oracle."""
    import numpy as np
    import torch

    T = w.total_tokens
    g = torch.Generator(device="cuda:0").manual_seed(20261202)
    xs = [torch.randn((T, w.H, w.d), generator=g, device="cuda:0").to(torch.bfloat16) for _ in range(2)]
    outs = [torch.empty_like(x) for x in xs]
    lib = vd.load_library()

    def call():
        st = lib.attn_qk_norm_packed(xs[0].data_ptr(), xs[1].data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                                     None, None, T, w.H, w.d, 1e-6, torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    stream = torch.cuda.current_stream()
    for _ in range(3):
        call()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.prologue_steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.prologue_steps)]
    torch.cuda.synchronize()
    for i in range(args.prologue_steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg = float(np.mean(ms))
    nbytes = float(T) * w.H * w.d * 2 * 4          # Q and K rows read once and written once
    gbs = nbytes / (avg * 1e-3) / 1e9
    rec = {
        "kernel": "qk_norm_packed_kernel",
        "what": "per-head RMSNorm of packed Q and K, THD [T,H,128] BF16 in and out (V untouched)",
        "bound": "hbm",
        "achieved": round(gbs, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(gbs / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(w.name, "qk_norm_packed_kernel", False, "packed_prologue"),
        "algorithmic_bytes": nbytes,
        "ms": {"avg": round(avg, 4), "min": round(min(ms), 4), "max": round(max(ms), 4)},
        "steps": args.prologue_steps,
    }
    print(f"[bench] packed prologue {args.prologue_steps} calls: {avg:.4f} ms -> {gbs:.0f} GB/s "
          f"({100 * gbs / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:.0f})", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        from oracle import bf16_bits_to_f64, bf16_faithful, qk_norm
        toks = np.random.default_rng(1).choice(T, 4096, replace=False)
        xq = xs[0].view(torch.int16).cpu().numpy().view(np.uint16)
        got = outs[0].view(torch.int16).cpu().numpy().view(np.uint16)[toks]
        t1 = time.perf_counter()
        exact = qk_norm(xq, tokens=toks)
        cpu_s = time.perf_counter() - t1
        m = bf16_faithful(bf16_bits_to_f64(got), exact)
        rec["parity"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in m.items()}
        sample_bytes = float(len(toks)) * w.H * w.d * 2 * 2             # Q rows read and written
        rec["cpu_baseline"] = {"value": round(sample_bytes / cpu_s / 1e9, 4), "unit": "GB/s",
                               "cores": oracle_cores(), "kind": "oracle",
                               "sample": f"Q of {len(toks)} seeded tokens x {w.H} heads (the GPU call also does K), "
                                         f"FP64 NumPy, {cpu_s:.2f} s"}
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(5):
        for x, o in zip(xs, outs):
            o.copy_(x)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 5
    rec["copy_reference"] = {"what": "device-to-device copies of Q and K (same bytes read and written)",
                             "achieved": round(nbytes / (copy_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                             "ms": round(copy_ms, 4)}
    del xs, outs
    torch.cuda.empty_cache()
    return rec


def time_linear(args, w, vd, dev) -> dict:
    """Time the SANA-Video linear attention at the workload's token grid and heads, on seeded
    ReLU'd/rotated inputs resident in HBM; check seeded tokens against the oracle."""
    import numpy as np
    import torch

    from workloads import make_linear_inputs
    t0 = time.time()
    xb = make_linear_inputs(w.B, w.grid, w.H, seed=0)
    xs = [dev(b) for b in xb]
    out = torch.empty_like(xs[0])
    print(f"[bench] linear-attention inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def call():
        vd.linear_attention(*xs, out=out)

    stream = torch.cuda.current_stream()
    for _ in range(2):
        call()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.linear_steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.linear_steps)]
    torch.cuda.synchronize()
    for i in range(args.linear_steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg = float(np.mean(ms))
    nbytes = linear_bytes(w.B, w.N, w.H, w.d)
    gbs = nbytes / (avg * 1e-3) / 1e9
    flops = 2 * 2.0 * w.B * w.H * w.N * w.d * w.d          # the two d x d products per token
    rec = {
        "kernel": "linear_out_kernel",
        "what": "SANA-Video linear attention (V K_rot^T) Q_rot / (K.sum Q + 1e-15), BF16 [B,N,H,128]",
        "timed": "whole call: linear_kv_partial_kernel, linear_kv_reduce_kernel, linear_out_kernel",
        "bound": "hbm",
        "achieved": round(gbs, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(gbs / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(w.name, "linear_out_kernel", False, "linear"),
        "algorithmic_bytes": nbytes,
        "tflops": round(flops / (avg * 1e-3) / 1e12, 2),
        "ms": {"avg": round(avg, 4), "min": round(min(ms), 4), "max": round(max(ms), 4)},
        "steps": args.linear_steps,
    }
    print(f"[bench] linear attention {args.linear_steps} calls: {avg:.4f} ms -> {gbs:.0f} GB/s "
          f"({100 * gbs / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:.0f})", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        from oracle import bf16_bits_to_f64
        from oracle.linear import linear_attention
        toks = np.random.default_rng(2).choice(w.N, 256, replace=False)
        heads = [0, w.H - 1]                         # the key-side sums run over every token
        got = bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)[:, toks][:, :, heads])
        t1 = time.perf_counter()
        ref = linear_attention(*[x[:, :, heads] for x in xb], tokens=toks)
        cpu_s = time.perf_counter() - t1
        # what the sample reads and writes: k, k_rot, v of every token and q, q_rot, out of
        # the 256 tokens, for the two heads
        sample_bytes = float(w.B) * len(heads) * w.d * 2 * (3.0 * w.N + 3.0 * len(toks))
        rec["cpu_baseline"] = {"value": round(sample_bytes / cpu_s / 1e9, 4), "unit": "GB/s",
                               "cores": oracle_cores(), "kind": "oracle",
                               "sample": f"heads {heads} over all {w.N} tokens, outputs of 256 seeded tokens, "
                                         f"FP64 NumPy, {cpu_s:.2f} s"}
        rec["parity"] = {"rel_l2": round(float(np.linalg.norm(got - ref) / np.linalg.norm(ref)), 8),
                         "n_elems": int(got.size), "ok": bool(np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref))}
    del xs, out
    torch.cuda.empty_cache()
    return rec


def time_block_sparse(args, w, vd, q, k, v, qb, kb, vb, dense_ms: float) -> dict:
    """Time block-skip attention (routing, then the block-sparse pass) on the workload's
    resident Q/K/V at threshold --block-skip-tau; FLOP counts only the (query, key) pairs the
    kept tiles cover. Checks seeded rows against the oracle over the kept tiles."""
    import numpy as np
    import torch

    tau = args.block_skip_tau
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(2):
            fn()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        res = None
        for i in range(n):
            starts[i].record(stream)
            res = fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in zip(starts, ends)], res

    order_name = "longest-first per head" if args.block_skip_order == "auto" else args.block_skip_order
    lpt = order_name != "item"
    route_ms, routed = timed(lambda: vd.block_route(q, k, tau=tau, scale=w.scale, with_order=lpt),
                             args.block_skip_steps)
    kv_idx, kv_cnt, order = routed if lpt else (*routed, None)
    sparse_ms, _ = timed(lambda: vd.attn_fwd_block_sparse(q, k, v, kv_idx, kv_cnt, scale=w.scale, out=out,
                                                          order=order), args.block_skip_steps)
    ntq, ntk = -(-w.N // 256), -(-w.N // 64)
    cnt = kv_cnt.cpu().numpy().astype(np.int64)
    idx = kv_idx.cpu().numpy()
    last_kept = np.take_along_axis(idx, np.maximum(cnt - 1, 0)[..., None], -1)[..., 0] == ntk - 1
    keys = cnt * 64 - last_kept * (64 * ntk - w.N)
    rows = np.minimum(256, w.N - 256 * np.arange(ntq))
    pairs = float((keys * rows).sum())
    density = pairs / (float(w.B) * w.H * w.N * w.N)
    avg_s, avg_r = float(np.mean(sparse_ms)), float(np.mean(route_ms))
    flops = 4.0 * w.d * pairs
    tf = flops / (avg_s * 1e-3) / 1e12
    rec = {
        "kernel": "attn_fwd_block_sparse_kernel",
        "what": "block-skip attention: pooled-proxy routing of 64-key tiles per 256-row query tile "
                "(keep z >= max z - tau), then exact softmax attention over the kept tiles",
        "tau": tau,
        "order": order_name,
        "density": round(density, 4),
        "bound": "mfma",
        "achieved": round(tf, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tf / PEAK_BF16_TFLOPS, 4),
        "flops_per_call": flops,
        "traffic": measured_traffic(w.name, "attn_fwd_block_sparse_kernel", False, "block_sparse"),
        "mfma_counters": measured_mfma(w.name, "attn_fwd_block_sparse_kernel", False, "block_sparse"),
        "ms": {"sparse": round(avg_s, 4), "sparse_min": round(min(sparse_ms), 4),
               "sparse_max": round(max(sparse_ms), 4), "route": round(avg_r, 4)},
        "speedup_vs_dense_call": round(dense_ms / (avg_s + avg_r), 3),
        "steps": args.block_skip_steps,
    }
    print(f"[bench] block-skip tau={tau}: density {density:.4f}, route {avg_r:.3f} ms, sparse {avg_s:.3f} ms "
          f"-> {tf:.1f} TFLOP/s on kept pairs ({100 * tf / PEAK_BF16_TFLOPS:.1f} % of peak), "
          f"{dense_ms / (avg_s + avg_r):.2f}x the dense call", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        from oracle import compare
        from oracle.block_sparse import attention_kept
        keep = np.zeros((w.B, w.H, ntq, ntk), bool)
        b_, h_, i_ = np.nonzero(cnt > 0)
        for b, h, i in zip(b_, h_, i_):
            keep[b, h, i, idx[b, h, i, :cnt[b, h, i]]] = True
        rows_s = np.random.default_rng(3).choice(w.B * w.H * w.N, 128, replace=False)
        t1 = time.perf_counter()
        o_ref, _ = attention_kept(qb, kb, vb, w.scale, keep, rows=rows_s)
        cpu_s = time.perf_counter() - t1
        tile_keys = np.minimum(64, w.N - 64 * np.arange(ntk))
        bh_r, n_r = rows_s // w.N, rows_s % w.N
        kept_keys = (keep.reshape(-1, ntq, ntk)[bh_r, n_r // 256] * tile_keys).sum(axis=1)
        cpu_flops = 4.0 * w.d * float(kept_keys.sum())
        rec["cpu_baseline"] = {"value": round(cpu_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle_cores(), "kind": "oracle",
                               "sample": f"128 seeded query rows over their kept keys, FP64 NumPy, {cpu_s:.2f} s"}
        vd.attn_fwd_block_sparse(q, k, v, kv_idx, kv_cnt, scale=w.scale, out=out, order=order)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, w.d)[rows_s]
        from oracle import bf16_bits_to_f64
        m = compare(bf16_bits_to_f64(got), o_ref)
        rec["parity"] = {"rel_l2": round(float(m["rel_l2"]), 8), "n_elems": int(m["n_elems"]), "ok": bool(m["ok"])}
    del out, lse, kv_idx, kv_cnt, order
    torch.cuda.empty_cache()
    return rec


def time_block_sparse_varlen(args, w, vd, q, k, v, qb, kb, vb, cu, dense_ms: float) -> dict:
    """Block-skip attention on the packed workload (routing per segment, then the block-sparse
    varlen pass) at --block-skip-tau; FLOP counts the (query, key) pairs of the kept tiles."""
    import numpy as np
    import torch

    tau = args.block_skip_tau
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(q.device)
    cu_h = [int(x) for x in cu]
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(2):
            fn()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        res = None
        for i in range(n):
            starts[i].record(stream)
            res = fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        return [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)], res

    order_name = "longest-first" if args.block_skip_order == "auto" else args.block_skip_order
    lpt = order_name == "longest-first"
    route_ms, routed = timed(lambda: vd.block_route_varlen(q, k, cu_d, tau=tau, scale=w.scale, cu_seqlens_host=cu_h,
                                                           with_order=lpt), args.block_skip_steps)
    kv_idx, kv_cnt, order = routed if lpt else (*routed, None)
    sparse_ms, _ = timed(lambda: vd.attn_fwd_block_sparse_varlen(q, k, v, cu_d, kv_idx, kv_cnt, scale=w.scale,
                                                                 out=out, cu_seqlens_host=cu_h, order=order),
                         args.block_skip_steps)
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    offs = vd.varlen_tile_offsets(cu_h)
    pairs, full, keeps = 0.0, 0.0, []
    for s_, (a, e) in enumerate(zip(cu_h[:-1], cu_h[1:])):
        n = e - a
        if n == 0:
            keeps.append(None)
            continue
        ntq, ntk = -(-n // 256), -(-n // 64)
        rows = np.minimum(256, n - 256 * np.arange(ntq))
        tkeys = np.minimum(64, n - 64 * np.arange(ntk))
        keep = np.zeros((w.H, ntq, ntk), bool)
        for i in range(ntq):
            for h in range(w.H):
                keep[h, i, idx[offs[s_] + i, h, :cnt[offs[s_] + i, h]]] = True
        keeps.append(keep)
        pairs += float((keep * rows[None, :, None] * tkeys[None, None, :]).sum())
        full += float(w.H) * n * n
    avg_s, avg_r = float(np.mean(sparse_ms)), float(np.mean(route_ms))
    flops = 4.0 * w.d * pairs
    tf = flops / (avg_s * 1e-3) / 1e12
    rec = {
        "kernel": "attn_fwd_block_sparse_varlen_kernel",
        "what": "block-skip attention on the packed batch: per-segment pooled-proxy routing of 64-key tiles per "
                "256-row query tile (keep z >= max z - tau), then exact softmax over the kept tiles",
        "tau": tau, "order": order_name, "density": round(pairs / full, 4), "bound": "mfma",
        "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
        "flops_per_call": flops,
        "traffic": measured_traffic(w.name, "attn_fwd_block_sparse_varlen_kernel", False, "block_sparse_varlen"),
        "mfma_counters": measured_mfma(w.name, "attn_fwd_block_sparse_varlen_kernel", False, "block_sparse_varlen"),
        "ms": {"sparse": round(avg_s, 4), "sparse_min": round(min(sparse_ms), 4),
               "sparse_max": round(max(sparse_ms), 4), "route": round(avg_r, 4)},
        "speedup_vs_dense_call": round(dense_ms / (avg_s + avg_r), 3),
        "steps": args.block_skip_steps,
    }
    print(f"[bench] block-skip varlen tau={tau}: density {pairs / full:.4f}, route {avg_r:.3f} ms, sparse "
          f"{avg_s:.3f} ms -> {tf:.1f} TFLOP/s on kept pairs ({100 * tf / PEAK_BF16_TFLOPS:.1f} % of peak), "
          f"{dense_ms / (avg_s + avg_r):.2f}x the dense call", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        from oracle import bf16_bits_to_f64, compare
        from oracle.block_sparse import attention_kept_varlen
        T = int(cu_h[-1])
        rows_s = np.random.default_rng(3).choice(w.H * T, 128, replace=False)
        t1 = time.perf_counter()
        o_ref, _ = attention_kept_varlen(qb, kb, vb, cu_h, w.scale, keeps, rows=rows_s)
        cpu_s = time.perf_counter() - t1
        got = out.view(torch.int16).cpu().numpy().view(np.uint16).transpose(1, 0, 2).reshape(-1, w.d)[rows_s]
        m = compare(bf16_bits_to_f64(got), o_ref)
        rec["parity"] = {"rel_l2": round(float(m["rel_l2"]), 8), "n_elems": int(m["n_elems"]), "ok": bool(m["ok"])}
        h_r, t_r = rows_s // T, rows_s % T
        seg = np.searchsorted(np.asarray(cu_h), t_r, side="right") - 1
        kept_keys = 0.0
        for hh, tt, ss in zip(h_r, t_r, seg):
            n = cu_h[ss + 1] - cu_h[ss]
            tkeys = np.minimum(64, n - 64 * np.arange(-(-n // 64)))
            kept_keys += float((keeps[ss][hh, (tt - cu_h[ss]) // 256] * tkeys).sum())
        rec["cpu_baseline"] = {"value": round(4.0 * w.d * kept_keys / cpu_s / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle_cores(), "kind": "oracle",
                               "sample": f"128 seeded query rows over their kept keys, FP64 NumPy, {cpu_s:.2f} s"}
    del out, kv_idx, kv_cnt
    torch.cuda.empty_cache()
    return rec


def head_share(w, heads: int):
    """The workload restricted to its first `heads` heads: one GPU's share when the heads are
    split over GPUs (each head's values are the full workload's, since the seeded streams are
    spawned head by head)."""
    import dataclasses
    if w.kind != "dense" or not 1 <= heads <= w.H:
        raise SystemExit(f"--heads needs a dense workload and 1 <= heads <= {w.H}")
    if heads == w.H:
        return w
    desc = w.description.replace(f"H={w.H}", f"H={heads}")
    if w.H % heads == 0:
        desc += f", one GPU's share of a {w.H // heads}-way head split"
    return dataclasses.replace(w, name=f"{w.name}_h{heads}", H=heads, description=desc)


def oracle_cores() -> int:
    """Threads the FP64 oracle's BLAS calls use on this host."""
    from threadpoolctl import threadpool_info
    blas_threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    return min(blas_threads, host_cores())


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed calls before the timed ones (default: enough for about half a second, at "
                         "least 3; short calls timed from a cold GPU run before the shader clock has settled)")
    ap.add_argument("--workload", default="video_720p")
    ap.add_argument("--heads", type=int, default=0,
                    help="dense workloads: run the first HEADS heads only (the same values), i.e. one "
                         "GPU's share of a head-sharded call at full N (0: all heads)")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="query rows of the seeded sample the FP64 oracle is timed and checked on (8192: 7-20 s of "
                         "FP64 work on 16 host cores at 720p, depending on the box)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-split-kv", action="store_true",
                    help="plain attn_fwd / attn_fwd_varlen, without cutting the last tiles over keys")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many MiB "
                         "(the known-size reference for the HBM byte counters)")
    ap.add_argument("--write-traffic-profile", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                         "WRITE_SIZE) of a run with --calibrate-copy-mib into the profiles/ record; no GPU")
    ap.add_argument("--write-mfma-profile", nargs=2, metavar=("COUNTER_CSV", "AGENT_CSV"),
                    help="turn a rocprofv3 --pmc run of " + " ".join(MFMA_COUNTERS) + " (its "
                         "counter_collection.csv and agent_info.csv) into the profiles/ record; no GPU")
    ap.add_argument("--traffic-kind", choices=sorted(CALL_KERNELS), default=None,
                    help="with --write-traffic-profile / --write-mfma-profile: which call's kernels to "
                         "record (default: the workload's)")
    ap.add_argument("--prologue-steps", type=int, default=20,
                    help="timed calls of the Q/K RMSNorm+RoPE prologue at the workload's grid (0: skip)")
    ap.add_argument("--linear-steps", type=int, default=10,
                    help="timed calls of the SANA-Video linear attention at the workload's grid (0: skip)")
    ap.add_argument("--block-skip-steps", type=int, default=5,
                    help="dense workloads: timed calls of block-skip attention on the same inputs (0: skip)")
    ap.add_argument("--block-skip-tau", type=float, default=0.02,
                    help="routing threshold of the timed block-skip calls")
    ap.add_argument("--block-skip-order", choices=("auto", "longest-first", "item"), default="auto",
                    help="dispatch order of the block-sparse pass: the routing's longest-first order (per "
                         "head on dense batches, over all items on packed ones), or item order; auto: the "
                         "routing's order")
    ap.add_argument("--profile-command", default="",
                    help="the command lines that produced the counter files (recorded in the profile)")
    args = ap.parse_args()

    if args.write_traffic_profile:
        return write_traffic_profile(args)
    if args.write_mfma_profile:
        return write_mfma_profile(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the attention kernel is sharded over heads by the caller, not here.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import video_diffusion_dit_amd as vd
    from workloads import WORKLOADS, make_dense, make_varlen, sample_rows

    w = WORKLOADS[args.workload]
    if args.heads > 0:
        w = head_share(w, args.heads)
    t0 = time.time()
    if w.kind == "dense":
        qb, kb, vb = make_dense(w)
        cu = None
    else:
        qb, kb, vb, cu = make_varlen(w)
    print(f"[bench] generated {w.description} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)

    q, k, v = dev(qb), dev(kb), dev(vb)
    out = torch.empty_like(q)
    if w.kind == "dense":
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    else:
        lse = torch.empty((w.H, w.total_tokens), dtype=torch.float32, device="cuda:0")
    cu_d = None if cu is None else torch.from_numpy(cu).to("cuda:0")
    cu_host = None if cu is None else [int(x) for x in cu]
    vd.load_library()
    if w.kind == "dense":
        split = not args.no_split_kv and vd.splitkv_workspace_bytes(w.B, w.H, w.N) > 0
    else:   # the packed call plans its split on the device; it may split nothing
        split = not args.no_split_kv
    kernel = CALL_KERNELS[w.kind][0]

    def step():
        if w.kind == "dense" and split:
            vd.attention._launch_dense_splitkv(q, k, v, out, lse, w.scale, 0)
        elif w.kind == "dense":
            vd.attention._launch_dense(q, k, v, out, lse, w.scale)
        elif split:
            vd.attention._launch_varlen_splitkv(q, k, v, cu_d, out, lse, w.scale, 0)
        else:
            vd.attention._launch_varlen(q, k, v, cu_d, out, lse, w.scale, cu_host)

    stream = torch.cuda.current_stream()
    done = 0
    if args.warmup is None:   # size the warm-up from the second call's duration
        step()
        torch.cuda.synchronize()
        t_one = time.perf_counter()
        step()
        torch.cuda.synchronize()
        args.warmup = default_warmup(time.perf_counter() - t_one)
        done = 2
    for _ in range(args.warmup - done):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warm-up done ({args.warmup} steps)", file=sys.stderr, flush=True)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall_ms / args.steps
    avg_kernel_ms = float(np.mean(kernel_ms))
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_kernel_ms * 1e-3) / 1e12
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step wall, kernel avg {avg_kernel_ms:.3f} ms "
          f"(min {min(kernel_ms):.3f}, max {max(kernel_ms):.3f}) -> {achieved:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.description,
            "B": w.B, "H": w.H, "N": w.N if w.kind == "dense" else w.total_tokens, "d": w.d,
            "segments": list(w.seqlens) if w.seqlens else None,
            "flops_per_step": flops,
            "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
            "split_kv": bool(split),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "timed": ("whole call on its stream: " + kernel +
                      ((" for whole query tiles, then attn_fwd_dense_split_kernel and merge_kernel"
                        " for the last round's tiles") if split and w.kind == "dense" else
                       (" after build_varlen_schedule and varlen_split_plan, then attn_fwd_varlen_split_kernel"
                        " and varlen_merge_kernel for the planned tail") if split else
                       " after build_varlen_schedule" if w.kind == "varlen" else "")),
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name, kernel, split, w.kind),
            "mfma_counters": measured_mfma(w.name, kernel, split, w.kind),
            "kernel_ms": {"avg": round(avg_kernel_ms, 4), "median": round(float(np.median(kernel_ms)), 4),
                          "min": round(min(kernel_ms), 4), "max": round(max(kernel_ms), 4)},
        },
        "cpu_baseline": None,
    }

    if w.kind == "dense" and args.block_skip_steps > 0:
        result["block_skip"] = time_block_sparse(args, w, vd, q, k, v, qb, kb, vb, avg_kernel_ms)
    elif args.block_skip_steps > 0:
        result["block_skip"] = time_block_sparse_varlen(args, w, vd, q, k, v, qb, kb, vb, cu, avg_kernel_ms)
    if w.grid is not None and args.prologue_steps > 0:
        result["prologue"] = time_prologue(args, w, vd, dev)
    elif w.kind == "varlen" and args.prologue_steps > 0:
        result["prologue"] = time_packed_norm(args, w, vd, dev)
    if w.grid is not None and args.linear_steps > 0:
        result["linear_attention"] = time_linear(args, w, vd, dev)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")   # contents irrelevant: bytes are counted
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        from oracle import attention_dense, attention_varlen, compare
        from threadpoolctl import threadpool_info
        rows = sample_rows(w, args.cpu_rows)
        t1 = time.perf_counter()
        if w.kind == "dense":
            o_ref, lse_ref = attention_dense(qb, kb, vb, w.scale, rows=rows)
        else:
            o_ref, lse_ref = attention_varlen(qb, kb, vb, cu, w.scale, rows=rows)
        cpu_s = time.perf_counter() - t1
        if w.kind == "dense":
            keys_per_row = np.full(rows.size, w.N, dtype=np.float64)
        else:
            T = w.total_tokens
            seg = np.searchsorted(cu, rows % T, side="right") - 1
            keys_per_row = (cu[seg + 1] - cu[seg]).astype(np.float64)
        cpu_flops = float(np.sum(4.0 * w.d * keys_per_row))
        blas_threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
        result["cpu_baseline"] = {
            "value": round(cpu_flops / cpu_s / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": min(blas_threads, host_cores()),
            "kind": "oracle",
            "sample": f"{rows.size} seeded query rows of {w.name} (each over its full key range), "
                      f"FP64 NumPy/OpenBLAS, {cpu_s:.1f} s",
        }
        # the same oracle on one core (BLAS limited to one thread), on the first eighth of the rows
        from threadpoolctl import threadpool_limits
        rows1 = rows[:max(1, rows.size // 8)]
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            if w.kind == "dense":
                attention_dense(qb, kb, vb, w.scale, rows=rows1)
            else:
                attention_varlen(qb, kb, vb, cu, w.scale, rows=rows1)
            cpu1_s = time.perf_counter() - t1
        flops1 = float(np.sum(4.0 * w.d * keys_per_row[:rows1.size]))
        result["cpu_baseline"]["one_core"] = {
            "value": round(flops1 / cpu1_s / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "sample": f"the first {rows1.size} of those rows, BLAS on one thread, {cpu1_s:.2f} s"}
        # parity of the same rows on the GPU output of the last timed step
        og = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        og = (og.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        lg = lse.cpu().numpy().astype(np.float64)
        if w.kind == "dense":
            og, lg = og.reshape(-1, w.d)[rows], lg.reshape(-1)[rows]
        else:
            T = w.total_tokens
            og, lg = og[rows % T, rows // T], lg[rows // T, rows % T]
        m = compare(og, o_ref, lg, lse_ref)
        result["parity"] = {k: (round(v, 8) if isinstance(v, float) else v) for k, v in m.items()}
        print(f"[bench] oracle {rows.size} rows in {cpu_s:.1f}s; parity {result['parity']}",
              file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
