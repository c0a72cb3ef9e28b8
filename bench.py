"""Benchmark of the layout-aware bf16->fp32 reduce-scatter + all-gather placement on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--launch FORM] [--rs-launch FORM]
                    [--ag-launch FORM] [--ag-mode kernel|sdma|copy2d] [--graph]

FORM is a launch form of include/tide.h: default, bounded:B, cu_exclusive:N or per_cu_cap:N (RS only).

One step = one pass of the whole hot path over one parameter group already resident in HBM: the
in-place reduce-scatter (C bf16 contributors -> R fp32 shards) followed by the all-gather placement
(rank-major bf16 stage -> per-parameter storage).  The default group is the Llama-3.1-70B decoder
layer (R = 8, C = 8, 17.1 GB of RS traffic per call), the largest of the layer groups.  The JSON line
reports:

  value       the RS's effective HBM GB/s: its algorithmic bytes / the mean duration of its launches,
              measured with HIP events on the launch stream (the metric's own quantity);
  step_gbps   the whole step's algorithmic bytes (RS + AG) / the step time; ag_gbps the placement's;
  roofline    the RS kernel (the dominant one): the same achieved rate against the 8 TB/s HBM peak;
  calibration a runtime device-to-device copy moving the RS's bytes, timed in the same run (the
              rate a plain stream reaches on this device), and the RS's ratio to it;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload (same byte formula).

Algorithmic bytes: RS = 2*C*numel (bf16 reads) + 4*R*S (fp32 writes, padding included);
AG = 2*numel (reads) + 2*numel (writes).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "RS effective HBM GB/s (bf16 in + fp32 out) and % of 8 TB/s peak, 1 GPU"
HBM_PEAK_GBPS = 8000.0


def parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_1_70b_layer")
    ap.add_argument("--launch", default="default",
                    help="launch form of both collectives: default, bounded:B, cu_exclusive:N, per_cu_cap:N (RS only)")
    ap.add_argument("--rs-launch", default=None, help="launch form of the RS (overrides --launch)")
    ap.add_argument("--ag-launch", default=None, help="launch form of the placement kernel (overrides --launch)")
    ap.add_argument("--ag-mode", choices=["kernel", "sdma", "copy2d"], default="kernel")
    ap.add_argument("--contributors", type=int, default=0,
                    help="override the workload's contributor count C (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain torch device copy of this many MiB per step (counter calibration)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the step (prepared RS + AG calls) in a HIP graph and time its replays")
    ap.add_argument("--interference", action="store_true",
                    help="instead of the step benchmark: slowdown of a concurrent one-wave bf16 GEMM per launch form")
    ap.add_argument("--launches", default=",".join(
        ["default", "per_cu_cap:1", "per_cu_cap:2", "per_cu_cap:4"] + [f"cu_exclusive:{n}" for n in (1, 2, 4, 6, 8)]
        + [f"bounded:{b}" for b in (8, 16, 32, 64, 128, 256, 512, 768, 1024, 1536, 2048)]),
        help="--interference / --overlap: the launch forms to measure (comma list)")
    ap.add_argument("--ag-launches", default="default,bounded:512,bounded:768,cu_exclusive:2,cu_exclusive:4,cu_exclusive:6",
                    help="--interference: the launch forms of the placement kernel's rows (comma list)")
    ap.add_argument("--gemm", default="4096,4096,4096", help="victim GEMM M,N,K (bf16)")
    ap.add_argument("--probe-launches",
                    default="none,default,bounded:16,bounded:64,bounded:256,bounded:512,bounded:768,bounded:1024,"
                            "bounded:2048,cu_exclusive:1,cu_exclusive:4,cu_exclusive:8,per_cu_cap:2",
                    help="--probes: RS launch forms of the occupancy-probe rows (none = no RS)")
    ap.add_argument("--cu-masks", default="16,32,64,128",
                    help="--interference: also the RS confined to K CUs by a CU-masked stream, and the GEMM on "
                         "the other CUs (comma list of K; empty: none)")
    ap.add_argument("--reps", type=int, default=31,
                    help="repetitions per row of the interference measurements (medians)")
    ap.add_argument("--probes", action="store_true",
                    help="instead of the step benchmark: occupancy probe, spin-kernel curve and more victims")
    ap.add_argument("--engines", action="store_true",
                    help="instead of the step benchmark: AG placement on CUs vs copy engines, served GB/s and victim slowdown")
    ap.add_argument("--overlap", action="store_true",
                    help="communication on one stream beside back-to-back GEMMs on another, per --launches")
    ap.add_argument("--overlap-comm", choices=["rs", "ag_kernel", "ag_sdma", "ag_copy2d"], default="rs")
    ap.add_argument("--mix-bound", action="store_true",
                    help="the RS's access shape with reads or writes left out, beside the library RS (C = 1-8)")
    ap.add_argument("--group-sizes", action="store_true",
                    help="RS and placement on Llama-shaped layer groups of hidden size 256-8192 (17 MB to 17 GB)")
    ap.add_argument("--copy-sizes", action="store_true",
                    help="placement of one flat parameter of 1-256 MiB over R = 1 and 8 ranks on each engine")
    ap.add_argument("--dma-rect", action="store_true",
                    help="placement on the four layer groups: kernel, DMA engines per segment, and one DMA-engine "
                         "rectangular copy per parameter (the copy-engine form of a strided copy per parameter)")
    ap.add_argument("--slot-reuse", action="store_true",
                    help="instead of the step benchmark: Slot-Reuse (pack into slots + RS from slots) vs in-place RS")
    return ap


def parse():
    return parser().parse_args()


def parse_launch(text: str):
    """A launch form from the command line: default, bounded:B, cu_exclusive:N or per_cu_cap:N."""
    from all_gather_placement_amd import Launch

    t = text.strip()
    if t == "default":
        return Launch.default()
    name, _, n = t.partition(":")
    make = {"bounded": Launch.bounded, "cu_exclusive": Launch.cu_exclusive, "per_cu_cap": Launch.per_cu_cap}.get(name)
    if make is None or not n.isdigit():
        raise SystemExit(f"unknown launch form {text!r}: use default, bounded:B, cu_exclusive:N or per_cu_cap:N")
    return make(int(n))


def launch_mode(launch, C: int = 8, kind: str = "rs") -> str:
    """How an RS (or, kind "ag", a placement-kernel) call in `launch` runs (include/tide.h)."""
    from all_gather_placement_amd import TIDE_LAUNCH_BOUNDED, TIDE_LAUNCH_CU_EXCLUSIVE, TIDE_LAUNCH_DEFAULT

    if launch.form == TIDE_LAUNCH_DEFAULT:
        if kind != "rs":
            return "one launch, one workgroup per item"
        n = 16 if C <= 3 else 8
        return f"one launch, CU-exclusive workgroups of {n} items (the default for C = {C})"
    if launch.form == TIDE_LAUNCH_BOUNDED:
        return f"bounded launches, {256 * launch.count} threads"
    if launch.form == TIDE_LAUNCH_CU_EXCLUSIVE:
        return f"one launch, CU-exclusive workgroups of {launch.count} items"
    return f"one launch, single-item workgroups, at most {launch.count} per CU"


def rs_kernel_name(C: int, launch) -> str:
    """The RS kernel a launch runs for C contributors (aligned buffers, in-place source)."""
    from all_gather_placement_amd import TIDE_LAUNCH_CU_EXCLUSIVE, TIDE_LAUNCH_DEFAULT

    ct = C if C <= 16 else 0
    if launch.form in (TIDE_LAUNCH_DEFAULT, TIDE_LAUNCH_CU_EXCLUSIVE):
        n = launch.count if launch.form == TIDE_LAUNCH_CU_EXCLUSIVE else (16 if C <= 3 else 8)
        return f"rs_cu_kernel<{ct}, {n // 8 if n > 8 else 1}, true, false>"
    return f"rs_kernel<{ct}, true, false>"


def shard_numel(shapes, R: int) -> int:
    """S, the elements of one rank's flat shard, from the library's own layout (host only)."""
    from all_gather_placement_amd import Layout

    with Layout(shapes, R) as L:
        return L.S


def kernel_source_hash() -> str:
    """Build id of libtide.so for the sources in the tree: kernels, launch plan (entry points and
    layout code), headers and compile flags.  Profiles record it, so any change to what runs on the
    device, or how it is launched, marks them stale."""
    from all_gather_placement_amd.build import LIB, source_hash

    return source_hash(LIB)


def read_traffic(workload: str, kernel: str):
    """HBM bytes per RS launch from the committed counter summary, if it was taken on this kernel
    (same kernel source and the same kernel, as the launch form depends on host code too)."""
    path = os.path.join(ROOT, "profiles", f"rs_kernel_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_k = re.search(r"rs_kernel_name:\s*(.+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_k and m_b) or m_src.group(1) != kernel_source_hash() or m_k.group(1).strip() != kernel:
        return None
    return float(m_b.group(1))


def cpu_baseline(cfg, log, min_seconds: float = 10.0):
    """Time the oracle on a bounded sample of the workload (about 10-30 s of CPU work).

    The sample is the group's leading parameters (storage order) up to ~45M elements (at least the
    first parameter), with the workload's R, C and value scale; the oracle's RS and AG run over it
    repeatedly until at least `min_seconds` have passed.  `value` is the oracle RS's rate by the
    metric's byte formula (the quantity the GPU line reports); `ag_gbps` the copy-out's.  Threads
    used = process CPU time / wall time over the timed passes.
    """
    import resource

    import numpy as np

    import oracle
    from oracle.geometry import group_geometry
    from workloads import normal_bf16_bits

    shapes, total = [], 0
    for s in cfg.shapes:
        n = int(np.prod(s))
        if total and total + n > 45_000_000:
            break
        shapes.append(s)
        total += n
    grads = [[normal_bf16_bits(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(shapes)] for c in range(cfg.C)]
    _, S = group_geometry(shapes, cfg.R)
    stage = normal_bf16_bits((cfg.R * S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
    rs_bytes = 2 * cfg.C * total + 4 * cfg.R * S
    ag_bytes = 4 * total
    passes, t_rs, t_ag = 0, 0.0, 0.0
    cpu0 = resource.getrusage(resource.RUSAGE_SELF)
    wall0 = time.perf_counter()
    while t_rs + t_ag < min_seconds:
        t0 = time.perf_counter()
        oracle.reduce_scatter(grads, shapes, cfg.R)
        t1 = time.perf_counter()
        oracle.all_gather_place(stage, shapes, cfg.R)
        t2 = time.perf_counter()
        t_rs += t1 - t0
        t_ag += t2 - t1
        passes += 1
    wall = time.perf_counter() - wall0
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    threads = max(1, round(cpu / wall))
    log(f"cpu oracle sample: {len(shapes)} params, {total} elems, {passes} passes: RS {t_rs:.2f} s, "
        f"AG {t_ag:.2f} s, cpu/wall {cpu / wall:.2f}")
    return {
        "value": round(passes * rs_bytes / t_rs / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{cfg.name}: parameters {[n for n, _ in cfg.params[:len(shapes)]]} "
                   f"({total} elements, R={cfg.R}, C={cfg.C}); numpy pack-then-sum RS + copy-out AG, "
                   f"{passes} passes in {t_rs + t_ag:.1f} s; host has {os.cpu_count()} logical CPUs"),
        "ag_gbps": round(passes * ag_bytes / t_ag / 1e9, 3),
        "cpu_over_wall": round(cpu / wall, 3),
    }


def cu_placement(stream, n_wgs: int) -> dict:
    """Where `stream`'s workgroups run: n_wgs small probe workgroups (~50 us each) record their
    CU; returns the number of distinct CUs and the distinct CUs per XCD."""
    import numpy as np
    import torch

    from all_gather_placement_amd import probe as pr

    rec = torch.zeros(n_wgs * pr.RECORD_BYTES, dtype=torch.uint8, device="cuda")
    ticks = max(1, pr.wall_clock_khz() // 20)  # 50 us
    pr.probe_launch(n_wgs, pr.TIDE_PROBE_SMALL, ticks, rec, stream)
    torch.cuda.synchronize()
    d = pr.decode(rec.cpu().numpy().view(np.uint64))
    keys = np.unique(d["cu_key"])
    per_xcc = [int(len(np.unique(d["cu_key"][d["xcc"] == x]))) for x in range(8)]
    return {"cus": int(len(keys)), "cus_per_xcd": per_xcc}


def cu_mask_rows(masks, comm_alone, gemm_once, gemm_alone, rs_bytes, reps, log):
    """Interference rows for the RS confined by CU masks (see interference())."""
    import statistics

    import torch

    from all_gather_placement_amd import Launch
    from all_gather_placement_amd import probe as pr

    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for k in masks:
        if not 0 < k < n_cus:
            raise SystemExit(f"--cu-masks: K must be in 1..{n_cus - 1}, got {k}")
        rs_stream, rs_h = pr.cu_mask_stream(0, k)
        gemm_stream, gemm_h = pr.cu_mask_stream(k, n_cus - k)
        try:
            where_rs = cu_placement(rs_stream, 8 * k)
            where_gemm = cu_placement(gemm_stream, 8 * (n_cus - k))
            t_comm = comm_alone("rs", Launch.default(), rs_stream)
            g_masked = statistics.median(gemm_once(gemm_stream=gemm_stream)[0] for _ in range(reps))
            for kind, gs in (("rs_cumask", None), ("rs_cumask_partition", gemm_stream)):
                conc, outlast = [], 0
                for _ in range(reps):
                    t, started_first, outlasted = gemm_once("rs", Launch.default(), gemm_stream=gs, comm_stream=rs_stream)
                    if started_first:
                        conc.append(t)
                        outlast += int(outlasted)
                med = statistics.median(conc) if conc else None
                row = {
                    "comm": kind, "launch": "default", "cu_mask_cus": k,
                    "comm_ms": round(t_comm, 4),
                    "comm_gbps": round(rs_bytes / (t_comm * 1e-3) / 1e9, 1),
                    "gemm_alone_us": round(gemm_alone * 1e3, 2),
                    "gemm_concurrent_us": round(med * 1e3, 2) if med else None,
                    "gemm_concurrent_min_max_us": [round(min(conc) * 1e3, 2), round(max(conc) * 1e3, 2)] if conc else None,
                    "slowdown_pct": round((med / gemm_alone - 1) * 100, 2) if med else None,
                    "reps": len(conc),
                    "comm_outlasts_gemm": round(outlast / len(conc), 2) if conc else None,
                    "rs_stream_placement": where_rs,
                }
                if gs is not None:
                    row["gemm_masked_alone_us"] = round(g_masked * 1e3, 2)
                    row["gemm_stream_placement"] = where_gemm
                log(json.dumps(row))
                rows.append(row)
        finally:
            torch.cuda.synchronize()
            pr.destroy_stream(rs_h)
            pr.destroy_stream(gemm_h)
    return rows


def interference(args, log):
    """Slowdown of a concurrent one-wave bf16 GEMM while the RS runs in each launch form.

    The victim is a torch bf16 matmul (hipBLASLt) whose kernel is one wave on the device: at
    4096^3 it runs 256 workgroups of 256x256 tiles, one per CU.  For each repetition the GEMM's
    stream first runs a short spin kernel (so the RS is already resident when the GEMM starts), then
    the GEMM between two events; the RS is enqueued on a second stream right after.  A repetition
    counts when the RS started before the GEMM; `rs_outlasts_gemm` is the fraction of those where
    it was still running when the GEMM finished (when it is not, the GEMM waited for the RS to
    drain).  slowdown = median(GEMM with RS) / median(GEMM alone) - 1, the pages' statistic
    (medians of launches).  The same is measured for the AG placement on each engine.

    CU masks (--cu-masks K,...) are the other way to keep communication off compute units: the RS
    (one unbounded launch) on a stream whose CU mask allows K CUs, (a) beside the GEMM on all CUs
    ("rs_cumask") and (b) with the GEMM's own stream masked to the other CUs ("rs_cumask_partition";
    its slowdown is against the unmasked GEMM alone, and `gemm_masked_alone_us` is the GEMM alone on
    its share).  A CU-id probe on each masked stream records how many CUs, on which XCDs, its
    workgroups ran on.
    """
    import statistics

    import torch

    from all_gather_placement_amd import Launch, Layout
    from workloads import CONFIGS, normal_bf16_cuda

    cfg = CONFIGS[args.workload]
    if args.contributors:
        import dataclasses

        cfg = dataclasses.replace(cfg, C=args.contributors)
    dev = torch.device("cuda:0")
    M, N, K = (int(x) for x in args.gemm.split(","))
    a = torch.randn(M, K, dtype=torch.bfloat16, device=dev)
    b = torch.randn(K, N, dtype=torch.bfloat16, device=dev)
    grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
             for c in range(cfg.C)]
    S = shard_numel(cfg.shapes, cfg.R)
    shards = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(cfg.R)]
    rs_bytes = 2 * cfg.C * cfg.numel() + 4 * cfg.R * S
    L = Layout(cfg.shapes, cfg.R)
    L.prepare()
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    spin_cycles = 400_000  # ~0.2 ms at 2.4 GHz: the RS is resident before the GEMM starts

    from all_gather_placement_amd import TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA

    stage = normal_bf16_cuda((cfg.R * S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
    params = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in cfg.shapes]
    ag_bytes = 4 * cfg.numel()

    bound = {}

    def comm(kind, launch, stream=None):
        stream = sB if stream is None else stream
        if (kind, launch) not in bound:
            if kind == "rs":
                bound[kind, launch] = L.bind_rs(grads, shards, launch=launch)
            else:
                mode = {"ag_sdma": TIDE_AG_SDMA, "ag_copy2d": TIDE_AG_COPY2D}.get(kind, TIDE_AG_KERNEL)
                bound[kind, launch] = L.bind_ag(stage, params, mode=mode, launch=launch)
        reps = 1 if kind in ("rs", "ag_sdma") else 4  # long enough to cover the GEMM
        for _ in range(reps):
            bound[kind, launch].launch(stream)

    def gemm_once(kind=None, launch=None, gemm_stream=None, comm_stream=None):
        gs = sA if gemm_stream is None else gemm_stream
        cs = sB if comm_stream is None else comm_stream
        torch.cuda.synchronize()
        e0, e1, r0, r1 = ev(), ev(), ev(), ev()
        with torch.cuda.stream(gs):
            torch.cuda._sleep(spin_cycles)
            e0.record(gs)
            torch.matmul(a, b)
            e1.record(gs)
        if kind is not None:
            r0.record(cs)
            comm(kind, launch, cs)
            r1.record(cs)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        if kind is None:
            return t, True, True
        return t, r0.elapsed_time(e0) > 0, e1.elapsed_time(r1) > 0

    def comm_alone(kind, launch, stream=None):
        cs = sB if stream is None else stream
        ts = []
        for _ in range(3):
            torch.cuda.synchronize()
            r0, r1 = ev(), ev()
            r0.record(cs)
            comm(kind, launch, cs)
            r1.record(cs)
            torch.cuda.synchronize()
            ts.append(r0.elapsed_time(r1))
        return statistics.median(ts)

    for _ in range(3):
        gemm_once()
    alone_all = [gemm_once()[0] for _ in range(max(args.reps, 15))]
    alone = statistics.median(alone_all)
    log(f"victim GEMM {M}x{N}x{K} bf16 alone: {alone * 1e3:.1f} us (median of {len(alone_all)})")
    rows = []
    cases = [("rs", parse_launch(x)) for x in args.launches.split(",") if x.strip()]
    cases += [("ag_kernel", parse_launch(x)) for x in args.ag_launches.split(",") if x.strip()]
    cases += [("ag_copy2d", Launch.default()), ("ag_sdma", Launch.default())]
    for kind, launch in cases:
        t_alone = comm_alone(kind, launch)
        conc, outlast = [], 0
        for _ in range(args.reps):
            t, started_first, outlasted = gemm_once(kind, launch)
            if started_first:
                conc.append(t)
                outlast += int(outlasted)
        nbytes = rs_bytes if kind == "rs" else (1 if kind == "ag_sdma" else 4) * ag_bytes
        med = statistics.median(conc) if conc else None
        row = {
            "comm": kind, "launch": str(launch),
            "mode": launch_mode(launch, cfg.C, "rs" if kind == "rs" else "ag") if kind in ("rs", "ag_kernel") else None,
            "comm_ms": round(t_alone, 4),
            "comm_gbps": round(nbytes / (t_alone * 1e-3) / 1e9, 1),
            "gemm_alone_us": round(alone * 1e3, 2),
            "gemm_concurrent_us": round(med * 1e3, 2) if med else None,
            "gemm_concurrent_min_max_us": [round(min(conc) * 1e3, 2), round(max(conc) * 1e3, 2)] if conc else None,
            "slowdown_pct": round((med / alone - 1) * 100, 2) if med else None,
            "reps": len(conc),
            "comm_outlasts_gemm": round(outlast / len(conc), 2) if conc else None,
        }
        log(json.dumps(row))
        rows.append(row)
    masks = [int(x) for x in args.cu_masks.split(",") if x.strip()]
    if masks:
        rows += cu_mask_rows(masks, comm_alone, gemm_once, alone, rs_bytes, args.reps, log)
    L.close()
    out = {"experiment": "concurrent one-wave GEMM slowdown vs communication launch form", "workload": cfg.name,
           "C": cfg.C, "R": cfg.R,
           "gemm": [M, N, K], "gemm_alone_us_min_max": [round(min(alone_all) * 1e3, 2), round(max(alone_all) * 1e3, 2)],
           "rows": rows}
    print(json.dumps(out), flush=True)


def slot_reuse(args, log):
    """Slot-Reuse against In-Place on one workload: times, GB/s and the bytes live during the RS.

    Slot-Reuse packs each contributor's gradients into an all-gather slot that is free again (R*S bf16, the
    stage layout) and reduces from the slots; the per-parameter gradients can be released after
    their pack.  In-Place reads the gradients where they are.  Bytes: pack = 2*numel read +
    2*R*S written per contributor; RS from slots = 2*C*R*S read + 4*R*S written.
    """
    import statistics

    import torch

    from all_gather_placement_amd import Layout
    from workloads import CONFIGS, normal_bf16_cuda

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    S = shard_numel(cfg.shapes, cfg.R)
    numel = cfg.numel()
    grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
             for c in range(cfg.C)]
    slots = [torch.empty(cfg.R * S, dtype=torch.bfloat16, device=dev) for _ in range(cfg.C)]
    shards = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(cfg.R)]
    L = Layout(cfg.shapes, cfg.R)
    L.prepare()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(calls, n):
        """Median GPU time of one round of `calls`, rounds enqueued back to back (pipelined)."""
        for _ in range(3):
            for c in calls:
                c.launch()
        torch.cuda.synchronize()
        evs = [(ev(), ev()) for _ in range(n)]
        for a, b in evs:
            a.record()
            for c in calls:
                c.launch()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in evs)

    rs_launch = parse_launch(args.rs_launch or args.launch)
    ag_launch = parse_launch(args.ag_launch or args.launch)
    t_inplace = timed([L.bind_rs(grads, shards, launch=rs_launch)], args.steps)
    t_pack = timed([L.bind_slot_pack(grads[c], slots[c], launch=ag_launch) for c in range(cfg.C)], args.steps)
    t_rs_slots = timed([L.bind_rs_slots(slots, shards, launch=rs_launch)], args.steps)
    L.close()
    rs_bytes = 2 * cfg.C * numel + 4 * cfg.R * S
    pack_bytes = cfg.C * (2 * numel + 2 * cfg.R * S)
    rs_slot_bytes = 2 * cfg.C * cfg.R * S + 4 * cfg.R * S
    out = {
        "experiment": "Slot-Reuse vs In-Place reduce-scatter", "workload": cfg.name, "R": cfg.R, "C": cfg.C,
        "rs_launch": str(rs_launch), "pack_launch": str(ag_launch),
        "in_place_rs_ms": round(t_inplace, 4), "in_place_rs_gbps": round(rs_bytes / t_inplace / 1e6, 1),
        "pack_all_contributors_ms": round(t_pack, 4), "pack_gbps": round(pack_bytes / t_pack / 1e6, 1),
        "rs_from_slots_ms": round(t_rs_slots, 4), "rs_from_slots_gbps": round(rs_slot_bytes / t_rs_slots / 1e6, 1),
        "slot_reuse_total_ms": round(t_pack + t_rs_slots, 4),
        "bytes_live_during_rs_in_place": 2 * cfg.C * numel + 4 * cfg.R * S,
        "bytes_live_during_rs_slot_reuse": 2 * cfg.C * cfg.R * S + 4 * cfg.R * S,
        "note": "Slot-Reuse's slots are all-gather buffers that are free again (already allocated); the gradients can be "
                "released once packed, so their 2*C*numel bytes are not live during its RS.",
    }
    log(json.dumps(out))
    print(json.dumps(out), flush=True)


def probes(args, log):
    """Interference instruments: the pages' SM-id probe, spin-kernel curve and extra victims.

    (1) Occupancy probe (Table 5 analogue): 256 GEMM-shaped probe workgroups (256 threads, 64 KiB
        LDS, 256 VGPRs per wave: the one-wave GEMM's footprint, one per CU) spin ~100 us and record
        their CU and start/end; launched while the RS runs in a given launch form.  A probe workgroup
        that starts more than 5 us after the first one was displaced into a second wave.
    (2) Spin-kernel curve (Figure 4 lines): k small workgroups resident for ~2 ms, the one-wave GEMM
        launched meanwhile; GEMM slowdown against k.
    (3) Victims of Table 4's other columns: a ~28-wave GEMM and a memory-bound elementwise add,
        with the RS in its default launch, bounded and CU-exclusive (the training setting, 4 items).
    """
    import statistics

    import numpy as np
    import torch

    from all_gather_placement_amd import Launch, Layout
    from all_gather_placement_amd import probe as pr
    from workloads import CONFIGS, normal_bf16_cuda

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    khz = pr.wall_clock_khz()
    tpu = khz / 1000.0  # wall-clock ticks per microsecond
    grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
             for c in range(cfg.C)]
    S = shard_numel(cfg.shapes, cfg.R)
    shards = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(cfg.R)]
    L = Layout(cfg.shapes, cfg.R)
    L.prepare()
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    spin_cycles = 400_000
    rs_calls = {}

    def rs_call(launch):
        if launch not in rs_calls:
            rs_calls[launch] = L.bind_rs(grads, shards, launch=launch)
        return rs_calls[launch]

    # (1) occupancy probe.  A one-wave marker workgroup (one wave, 8 VGPRs: it fits beside
    # anything but a full SIMD) runs on the probe's stream just before it and records when the
    # stream reached the probe; start delay = first probe start - marker end.
    recs = torch.zeros(256 * 4, dtype=torch.int64, device=dev)
    marker = torch.zeros(4, dtype=torch.int64, device=dev)
    probe_ticks = int(100 * tpu)

    def probe_once(launch):
        torch.cuda.synchronize()
        with torch.cuda.stream(sA):
            torch.cuda._sleep(spin_cycles)
            pr.probe_launch(1, pr.TIDE_PROBE_SMALL, 0, marker, sA)
            pr.probe_launch(256, pr.TIDE_PROBE_GEMM_SHAPED, probe_ticks, recs, sA)
        if launch is not None:
            rs_call(launch).launch(sB)
        torch.cuda.synchronize()
        d = pr.decode(recs.cpu().numpy().view(np.uint64))
        m = pr.decode(marker.cpu().numpy().view(np.uint64))
        t0 = d["start"].min()
        displaced = int((d["start"] > t0 + 5 * tpu).sum())
        span_us = (d["end"].max() - t0) / tpu
        delay_us = (t0 - m["end"][0]) / tpu
        return displaced, span_us, len(np.unique(d["cu_key"])), d, delay_us

    for _ in range(2):
        probe_once(None)
    table5 = []
    probe_launches = [None if x.strip() == "none" else parse_launch(x) for x in args.probe_launches.split(",")
                      if x.strip()]
    for launch in probe_launches:
        res = [probe_once(launch) for _ in range(max(args.reps, 15))]
        disp = [r[0] for r in res]
        row = {"launch": None if launch is None else str(launch), "displaced_median": statistics.median(disp), "displaced_max": max(disp),
               "reps_with_displacement_pct": round(100 * sum(1 for x in disp if x) / len(disp), 1),
               "start_delay_us_median": round(statistics.median(r[4] for r in res), 1),
               "start_delay_us_max": round(max(r[4] for r in res), 1),
               "probe_span_us_median": round(statistics.median(r[1] for r in res), 1),
               "distinct_cus": statistics.median(r[2] for r in res)}
        log("probe " + json.dumps(row))
        table5.append(row)
    d_alone = probe_once(None)[3]
    per_xcc = np.bincount(d_alone["xcc"], minlength=8).tolist()

    # (2) spin-kernel curve against the one-wave GEMM
    a = torch.randn(4096, 4096, dtype=torch.bfloat16, device=dev)
    b = torch.randn(4096, 4096, dtype=torch.bfloat16, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def victim_once(victim, comm):
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(sA):
            torch.cuda._sleep(spin_cycles)
            e0.record(sA)
            victim()
            e1.record(sA)
        if comm is not None:
            comm()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    gemm1 = lambda: torch.matmul(a, b)
    for _ in range(3):
        victim_once(gemm1, None)
    alone = statistics.median(victim_once(gemm1, None) for _ in range(args.reps))
    spin = []
    for k in [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048]:
        t = statistics.median(victim_once(gemm1, lambda: pr.probe_launch(k, pr.TIDE_PROBE_SMALL, int(2000 * tpu),
                                                                           None, sB)) for _ in range(args.reps))
        row = {"spin_wgs": k, "gemm_us": round(t * 1e3, 2), "slowdown_pct": round((t / alone - 1) * 100, 2)}
        log("spin " + json.dumps(row))
        spin.append(row)

    # (3) more victims
    big_a = torch.randn(21504, 2048, dtype=torch.bfloat16, device=dev)
    big_b = torch.randn(2048, 21504, dtype=torch.bfloat16, device=dev)
    ea = torch.randn(256 << 20, dtype=torch.bfloat16, device=dev)
    eb = torch.randn(256 << 20, dtype=torch.bfloat16, device=dev)
    ec = torch.empty_like(ea)
    victims = {"gemm_one_wave_4096^3": gemm1,
               "gemm_28_wave_21504x21504x2048": lambda: torch.matmul(big_a, big_b),
               "elementwise_add_256M_bf16": lambda: torch.add(ea, eb, out=ec)}
    table4 = []
    for name, fn in victims.items():
        for _ in range(2):
            victim_once(fn, None)
        t_alone = statistics.median(victim_once(fn, None) for _ in range(args.reps))
        row = {"victim": name, "alone_us": round(t_alone * 1e3, 1)}
        for launch in (Launch.default(), Launch.bounded(512), Launch.cu_exclusive(4)):
            t = statistics.median(victim_once(fn, lambda: rs_call(launch).launch(sB)) for _ in range(args.reps))
            row[f"slowdown_pct_rs_{launch}"] = round((t / t_alone - 1) * 100, 2)
        log("victim " + json.dumps(row))
        table4.append(row)
    L.close()
    out = {"experiment": "interference instruments", "workload": cfg.name, "wall_clock_khz": khz,
           "probe_cus_per_xcc_alone": per_xcc, "occupancy_probe": table5, "spin_curve": spin,
           "gemm_one_wave_alone_us": round(alone * 1e3, 2), "victims": table4}
    print(json.dumps(out), flush=True)


def engines(args, log):
    """CU-initiated vs copy-engine placement (analogue of [Endgame] Table 3 on one GPU).

    The same placement bytes (the workload's AG, repeated so it covers the victim) are moved by the
    placement kernel (compute units), by the DMA engines (1-D no-compute-unit copies) and by the
    runtime's 2-D copy; for each, the traffic it serves alone and the slowdown of two victims: the
    one-wave bf16 GEMM (compute-bound) and a 256M-element bf16 add (HBM-bound).  Peer pull/push
    directions of the pages' table need a second GPU and are not measured.
    """
    import statistics

    import torch

    from all_gather_placement_amd import Launch, Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA
    from workloads import CONFIGS, normal_bf16_cuda

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    S = shard_numel(cfg.shapes, cfg.R)
    stage = normal_bf16_cuda((cfg.R * S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
    params = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in cfg.shapes]
    ag_bytes = 4 * cfg.numel()
    L = Layout(cfg.shapes, cfg.R)
    L.prepare()
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a = torch.randn(4096, 4096, dtype=torch.bfloat16, device=dev)
    b = torch.randn(4096, 4096, dtype=torch.bfloat16, device=dev)
    ea = torch.randn(256 << 20, dtype=torch.bfloat16, device=dev)
    eb = torch.randn(256 << 20, dtype=torch.bfloat16, device=dev)
    ec = torch.empty_like(ea)
    victims = {"gemm_one_wave_4096^3": lambda: torch.matmul(a, b),
               "elementwise_add_256M_bf16": lambda: torch.add(ea, eb, out=ec)}
    engines_ = {"cu_kernel": (TIDE_AG_KERNEL, Launch.default()), "cu_kernel_bounded_512": (TIDE_AG_KERNEL, Launch.bounded(512)),
                "cu_kernel_cu_exclusive_4": (TIDE_AG_KERNEL, Launch.cu_exclusive(4)),
                "copy_engine_sdma": (TIDE_AG_SDMA, Launch.default()), "runtime_copy2d": (TIDE_AG_COPY2D, Launch.default())}
    calls = {k: L.bind_ag(stage, params, mode=m, launch=lc) for k, (m, lc) in engines_.items()}

    def alone_ms(call, reps):
        for _ in range(2):  # first calls on a stream stage the pointer table
            call.launch(sB)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(sB)
        for _ in range(reps):
            call.launch(sB)
        e1.record(sB)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def victim_once(fn, comm):
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(sA):
            torch.cuda._sleep(400_000)
            e0.record(sA)
            fn()
            e1.record(sA)
        if comm is not None:
            comm()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    rows = []
    for name, call in calls.items():
        t1 = alone_ms(call, 3)
        reps = max(1, int(2.0 / t1) + 1)  # cover >= 2 ms
        row = {"engine": name, "served_gbps_alone": round(ag_bytes / (t1 * 1e-3) / 1e9, 1), "placements": reps}
        for vname, fn in victims.items():
            for _ in range(2):
                victim_once(fn, None)
            t_alone = statistics.median(victim_once(fn, None) for _ in range(args.reps))

            def comm():
                for _ in range(reps):
                    call.launch(sB)
            t_conc = statistics.median(victim_once(fn, comm) for _ in range(args.reps))
            row[f"{vname}_slowdown_pct"] = round((t_conc / t_alone - 1) * 100, 2)
        log("engine " + json.dumps(row))
        rows.append(row)
    L.close()
    print(json.dumps({"experiment": "placement engines vs victims", "workload": cfg.name, "rows": rows}), flush=True)


def group_sizes(args, log):
    """RS and placement across group sizes: Llama-shaped layer groups (q, o h x h; k, v h/4 x h; gate,
    up 3.5h x h; down h x 3.5h; two norms; R = 8, C = 8) for h = 256 .. 8192, i.e. 17 MB to 17 GB of RS
    traffic per call, each collective in its default launch through a prepared call; mean of 20
    HIP-event timings after 3 warm-up launches.  Shows where launch overhead stops mattering."""
    import statistics

    import torch

    from all_gather_placement_amd import Layout, TIDE_AG_KERNEL

    def mean_ms(call, n=20):
        for _ in range(3):
            call.launch()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record()
            call.launch()
            b.record()
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) for a, b in evs)

    R, C = 8, 8
    rows = []
    for h in (256, 512, 1024, 2048, 4096, 8192):
        f = h * 7 // 2
        shapes = [(h, h), (h // 4, h), (h // 4, h), (h, h), (f, h), (f, h), (h, f), (h,), (h,)]
        numel = sum(int(torch.tensor(s).prod()) for s in shapes)
        with Layout(shapes, R) as L:
            grads = [[torch.randn(s, device="cuda").to(torch.bfloat16) for s in shapes] for _ in range(C)]
            shards = [torch.empty(L.S, dtype=torch.float32, device="cuda") for _ in range(R)]
            stage = torch.randn(R * L.S, device="cuda").to(torch.bfloat16)
            params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
            rs_b, ag_b = 2 * C * numel + 4 * R * L.S, 4 * numel
            rs = L.bind_rs(grads, shards)
            ag = L.bind_ag(stage, params, mode=TIDE_AG_KERNEL)
            t_rs, t_ag = mean_ms(rs), mean_ms(ag)
            rs.close()
            ag.close()
            row = {"h": h, "numel": numel, "rs_bytes": rs_b, "rs_us": round(t_rs * 1e3, 1),
                   "rs_gbps": round(rs_b / t_rs / 1e6, 1), "rs_frac": round(rs_b / t_rs / 1e6 / 8000, 4),
                   "ag_bytes": ag_b, "ag_us": round(t_ag * 1e3, 1), "ag_gbps": round(ag_b / t_ag / 1e6, 1)}
            log(json.dumps(row))
            rows.append(row)
            del grads, shards, stage, params
        torch.cuda.empty_cache()
    print(json.dumps({"experiment": "RS and placement vs group size", "R": R, "C": C, "rows": rows}), flush=True)


def copy_sizes(args, log):
    """Per-copy cost of the placement engines: one flat bf16 parameter of 1, 8, 64 and 256 MiB placed
    from a stage over R = 1 (one copy) and R = 8 (eight copies), on the DMA engines, the runtime 2-D
    copy and the kernel; median of 7 HIP-event timings each."""
    import statistics

    import torch

    from all_gather_placement_amd import Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA

    def med(call, n=7):
        call.launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call.launch()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    rows = []
    for mib in (1, 8, 64, 256):
        for R in (1, 8):
            n = mib << 19
            with Layout([(n,)], R) as L:
                stage = torch.randn(R * L.S, device="cuda").to(torch.bfloat16)
                param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
                row = {"param_mib": mib, "R": R, "copies": R}
                for mode, name in ((TIDE_AG_SDMA, "sdma"), (TIDE_AG_COPY2D, "copy2d"), (TIDE_AG_KERNEL, "kernel")):
                    call = L.bind_ag(stage, [param], mode=mode)
                    t = med(call)
                    call.close()
                    row[f"{name}_ms"] = round(t, 4)
                    row[f"{name}_gbps_copied"] = round(mib * 2**20 / (t * 1e-3) / 1e9, 1)
                log(json.dumps(row))
                rows.append(row)
    print(json.dumps({"experiment": "placement engines vs copy size", "rows": rows}), flush=True)


def overlap(args, log):
    """Communication hidden behind compute, as FSDP overlaps it with forward and backward: n
    back-to-back bf16 GEMMs on one stream, the communication (--overlap-comm: the RS, or the AG
    placement on the compute units or the DMA engines; one call in each launch form) on another,
    both enqueued at once.
    Reports each part alone, the overlapped makespan (first start to last end), the GEMM stream's
    own time while overlapped, and how much of the shorter part was hidden:
    hidden = (alone_gemms + alone_rs - makespan) / min(alone_gemms, alone_rs).  Medians of reps."""
    import statistics

    import torch

    from all_gather_placement_amd import TIDE_LAUNCH_CU_EXCLUSIVE, TIDE_LAUNCH_PER_CU_CAP, Launch, Layout
    from workloads import CONFIGS, normal_bf16_cuda

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    M, N, K = (int(x) for x in args.gemm.split(","))
    a = torch.randn(M, K, dtype=torch.bfloat16, device=dev)
    b = torch.randn(K, N, dtype=torch.bfloat16, device=dev)
    from all_gather_placement_amd import TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA

    kind = args.overlap_comm
    S = shard_numel(cfg.shapes, cfg.R)
    L = Layout(cfg.shapes, cfg.R)
    L.prepare()
    if kind == "rs":
        grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
                 for c in range(cfg.C)]
        shards = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(cfg.R)]
        bind = lambda launch: L.bind_rs(grads, shards, launch=launch)
    else:
        stage = normal_bf16_cuda((cfg.R * S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
        params = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in cfg.shapes]
        mode = {"ag_kernel": TIDE_AG_KERNEL, "ag_sdma": TIDE_AG_SDMA, "ag_copy2d": TIDE_AG_COPY2D}[kind]
        bind = lambda launch: L.bind_ag(stage, params, mode=mode, launch=launch if kind == "ag_kernel" else Launch())
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def gemms(n):
        for _ in range(n):
            torch.matmul(a, b)

    def timed(fn, stream):
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(stream):
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    t_one = statistics.median(timed(lambda: gemms(1), sA) for _ in range(args.reps))
    rows = []
    launches = [parse_launch(x) for x in args.launches.split(",") if x.strip()] if kind in ("rs", "ag_kernel") \
        else [Launch()]
    if kind == "ag_kernel":  # per-CU caps and more than 8 items per workgroup are the RS's only
        launches = [lc for lc in launches if lc.form != TIDE_LAUNCH_PER_CU_CAP and not
                    (lc.form == TIDE_LAUNCH_CU_EXCLUSIVE and lc.count > 8)]
    for launch in launches:
        call = bind(launch)
        t_rs = statistics.median(timed(lambda: call.launch(sB), sB) for _ in range(args.reps))  # the comm alone
        n = max(1, round(t_rs / t_one))  # GEMM work about as long as the RS
        t_g = statistics.median(timed(lambda: gemms(n), sA) for _ in range(args.reps))
        spans, gemm_spans = [], []
        for _ in range(args.reps):
            torch.cuda.synchronize()
            g0, g1, r0, r1 = ev(), ev(), ev(), ev()
            with torch.cuda.stream(sA):
                g0.record(sA)
                gemms(n)
                g1.record(sA)
            r0.record(sB)
            call.launch(sB)
            r1.record(sB)
            torch.cuda.synchronize()
            first = g0 if g0.elapsed_time(r0) >= 0 else r0  # whichever stream started first
            last = g1 if r1.elapsed_time(g1) >= 0 else r1   # whichever ended last
            spans.append(first.elapsed_time(last))
            gemm_spans.append(g0.elapsed_time(g1))
        call.close()
        span, t_gc = statistics.median(spans), statistics.median(gemm_spans)
        row = {"launch": str(launch), "gemms": n, "gemms_alone_ms": round(t_g, 4), "comm_alone_ms": round(t_rs, 4),
               "overlapped_makespan_ms": round(span, 4), "gemms_while_overlapped_ms": round(t_gc, 4),
               "gemm_slowdown_pct": round((t_gc / t_g - 1) * 100, 2),
               "serial_ms": round(t_g + t_rs, 4),
               "hidden_fraction": round((t_g + t_rs - span) / min(t_g, t_rs), 3)}
        log(json.dumps(row))
        rows.append(row)
    L.close()
    print(json.dumps({"experiment": "communication overlapped with back-to-back GEMMs", "comm": kind,
                      "workload": cfg.name, "gemm": [M, N, K], "gemm_alone_ms": round(t_one, 4), "rows": rows}),
          flush=True)


def rect_plan(L, stage, params):
    """One rectangular copy per parameter of the placement (rows = the ranks whose slice is full,
    source pitch = one stage slot, destination contiguous) plus one single-row copy for the rank whose
    slice is part padding, from the library's layout.  (dst, src, dst_pitch, src_pitch, width, rows)."""
    S = L.S
    base = stage.data_ptr()
    rects = []
    for p, q in enumerate(params):
        rows, Lp, m, o = L.param(p)
        if rows * Lp == 0:
            continue
        e = m * Lp
        full = rows // m
        if full:
            rects.append((q.data_ptr(), base + 2 * o, 2 * e, 2 * S, 2 * e, full))
        v = rows - full * m
        if v:
            rects.append((q.data_ptr() + 2 * full * e, base + 2 * (full * S + o), 2 * v * Lp, 2 * v * Lp, 2 * v * Lp, 1))
    return rects


def dma_rect(args, log):
    """AG placement of each layer group three ways, timed on the same stage and parameters: the
    placement kernel (default launch), the DMA engines with one 1-D copy per (parameter, rank) segment
    (TIDE_AG_SDMA), and the DMA engines with one rectangular copy per parameter (libtide_probe's
    tide_probe_dma_rect_copies, all issued before waiting; host-synchronous, not stream-ordered).
    The rectangular placement is checked bit for bit against the kernel's.  GB/s = 4 * numel / t."""
    import statistics

    import torch

    from all_gather_placement_amd import Layout, TIDE_AG_KERNEL, TIDE_AG_SDMA
    from all_gather_placement_amd import probe as pr
    from workloads import CONFIGS, normal_bf16_cuda

    dev = torch.device("cuda:0")
    rows = []
    for name in ("llama3_1_8b_layer", "llama3_1_70b_layer", "qwen3_30b_a3b", "wan2_2_block"):
        cfg = CONFIGS[name]
        L = Layout(cfg.shapes, cfg.R)
        L.prepare()
        stage = normal_bf16_cuda((cfg.R * L.S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
        ref = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in cfg.shapes]
        out = [torch.full(s, float("nan"), dtype=torch.bfloat16, device=dev) for s in cfg.shapes]
        nbytes = 4 * cfg.numel()

        def timed(fn, n):
            ts = []
            for _ in range(n):
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return statistics.median(ts)

        L.ag_place(stage, ref, mode=TIDE_AG_KERNEL)
        t_kernel = timed(lambda: L.ag_place(stage, ref, mode=TIDE_AG_KERNEL), 9)
        L.ag_place(stage, out, mode=TIDE_AG_SDMA)
        t_sdma = timed(lambda: L.ag_place(stage, out, mode=TIDE_AG_SDMA), 3)
        segments = sum(1 for p in range(L.P) for r in range(L.R) if L.segment(p, r)[1] > 0)
        rects = rect_plan(L, stage, out)
        for q in out:
            q.view(torch.int16).fill_(0x7FC1)
        torch.cuda.synchronize()
        t_rect = [pr.dma_rect_copies(rects) / 1e3 for _ in range(3)]
        exact = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(out, ref))
        row = {"workload": name, "P": cfg.P, "R": cfg.R, "bytes": nbytes,
               "kernel_ms": round(t_kernel, 4), "kernel_gbps": round(nbytes / t_kernel / 1e6, 1),
               "sdma_segments": segments, "sdma_ms": round(t_sdma, 3), "sdma_gbps": round(nbytes / t_sdma / 1e6, 1),
               "rect_copies": len(rects), "rect_ms_median": round(statistics.median(t_rect), 3),
               "rect_gbps": round(nbytes / statistics.median(t_rect) / 1e6, 1), "rect_bit_exact": exact}
        log(json.dumps(row))
        rows.append(row)
        L.close()
        del stage, ref, out
        torch.cuda.empty_cache()
    print(json.dumps({"experiment": "AG placement: kernel vs DMA engines per segment vs one DMA rectangular copy "
                                    "per parameter", "rows": rows}), flush=True)


def mix_bound(args, log):
    """The RS's access shape with its writes or its reads left out (the mix probe of libtide_probe.so),
    beside the library RS on the same buffers: one flat parameter of 2^27 elements, R = 1, C = 1, 2,
    4 and 8 separate contributor buffers.  The probe runs one item per workgroup, so it is launched
    with as many items resident per CU as the library's default RS launch keeps (its items per
    CU-exclusive workgroup); the library RS is timed in its default launch and in the per-CU cap of
    the same item count, which is the probe's own launch shape.  The HBM bus carries reads and
    writes in turn, so reads-only + writes-only time bounds the RS from below.  Medians of 21
    HIP-event timings per row, three interleaved rounds; the row keeps the round medians' median."""
    import statistics

    import torch

    from all_gather_placement_amd import Launch, Layout, tide_rs_launch_shape
    from all_gather_placement_amd import probe as pr

    items = 1 << 17
    n = items * 1024
    grads = [torch.full((n,), 0.01, dtype=torch.bfloat16, device="cuda") for _ in range(8)]
    dst = torch.empty(n, dtype=torch.float32, device="cuda")
    src = torch.tensor([g.data_ptr() for g in grads], dtype=torch.int64, device="cuda")
    L = Layout([(n,)], 1)
    modes = (("reads_only", pr.TIDE_PROBE_MIX_READS), ("writes_only", pr.TIDE_PROBE_MIX_WRITES),
             ("both", pr.TIDE_PROBE_MIX_BOTH))

    def med(fn, reps=21):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    kinds = ("reads_only", "writes_only", "both", "library_rs", "library_rs_per_cu_cap")
    per_cu = {C: tide_rs_launch_shape(C)["items_per_workgroup"] for C in (1, 2, 4, 8)}
    cap = {C: Launch.per_cu_cap(per_cu[C]) for C in per_cu}
    times = {}
    for rnd in range(3):
        for C in (1, 2, 4, 8):
            lds = tide_rs_launch_shape(C, cap[C])["lds_bytes"]
            for name, mode in modes:
                t = med(lambda: pr.mix_launch(C, mode, src, dst, items, lds))
                times.setdefault((C, name), []).append(t)
            for name, launch in (("library_rs", Launch.default()), ("library_rs_per_cu_cap", cap[C])):
                call = L.bind_rs([[g] for g in grads[:C]], [dst], launch=launch)
                times.setdefault((C, name), []).append(med(call.launch))
                call.close()
            log(f"round {rnd} C={C}: " + ", ".join(f"{k} {times[(C, k)][-1]:.4f} ms" for k in kinds))
    rows = []
    for C in (1, 2, 4, 8):
        t = {k: statistics.median(times[(C, k)]) for k in kinds}
        rb, wb = 2 * C * n, 4 * n
        row = {"C": C, "items_resident_per_cu": per_cu[C],
               "probe_lds_bytes": tide_rs_launch_shape(C, cap[C])["lds_bytes"]}
        for k, v in t.items():
            row[f"{k}_ms"] = round(v, 4)
        row["reads_only_gbps"] = round(rb / (t["reads_only"] * 1e-3) / 1e9, 1)
        row["writes_only_gbps"] = round(wb / (t["writes_only"] * 1e-3) / 1e9, 1)
        for k in ("both", "library_rs", "library_rs_per_cu_cap"):
            row[f"{k}_gbps"] = round((rb + wb) / (t[k] * 1e-3) / 1e9, 1)
        bound = t["reads_only"] + t["writes_only"]
        row["sum_bound_ms"] = round(bound, 4)
        row["sum_bound_gbps"] = round((rb + wb) / (bound * 1e-3) / 1e9, 1)
        row["library_rs_over_sum_bound"] = round(bound / t["library_rs"], 4)
        rows.append(row)
    L.close()
    print(json.dumps({"experiment": "RS read/write mix bound", "outputs": n, "rows": rows}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the node-local level on one GPU only; runs on more than one GPU "
              "(--gpus > 1) are not supported.", file=sys.stderr, flush=True)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import torch

    from all_gather_placement_amd import Launch, Layout, TIDE_AG_COPY2D, TIDE_AG_KERNEL, TIDE_AG_SDMA, tide_rs_launch_shape
    from workloads import CONFIGS, normal_bf16_cuda

    from all_gather_placement_amd.build import ensure_built

    ensure_built()  # load what is built; build only when nothing is
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.interference:
        torch.cuda.set_device(0)
        interference(args, log)
        return
    if args.slot_reuse:
        torch.cuda.set_device(0)
        slot_reuse(args, log)
        return
    if args.dma_rect:
        torch.cuda.set_device(0)
        dma_rect(args, log)
        return
    if args.probes:
        torch.cuda.set_device(0)
        probes(args, log)
        return
    if args.engines:
        torch.cuda.set_device(0)
        engines(args, log)
        return
    if args.copy_sizes:
        torch.cuda.set_device(0)
        copy_sizes(args, log)
        return
    if args.group_sizes:
        torch.cuda.set_device(0)
        group_sizes(args, log)
        return
    if args.mix_bound:
        torch.cuda.set_device(0)
        mix_bound(args, log)
        return
    if args.overlap:
        torch.cuda.set_device(0)
        overlap(args, log)
        return
    cfg = CONFIGS[args.workload]
    if args.contributors:
        import dataclasses

        cfg = dataclasses.replace(cfg, C=args.contributors)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {cfg.name}: P={cfg.P} R={cfg.R} C={cfg.C}")

    numel = cfg.numel()
    S = shard_numel(cfg.shapes, cfg.R)
    rs_bytes = 2 * cfg.C * numel + 4 * cfg.R * S
    ag_bytes = 4 * numel

    grads = [[normal_bf16_cuda(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
             for c in range(cfg.C)]
    shards = [torch.empty(S, dtype=torch.float32, device=dev) for _ in range(cfg.R)]
    stage = normal_bf16_cuda((cfg.R * S,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)
    params = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in cfg.shapes]
    calib_src = calib_dst = None
    if args.calib_copy_mib:
        calib_src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        calib_dst = torch.empty_like(calib_src)
    ag_mode = {"kernel": TIDE_AG_KERNEL, "sdma": TIDE_AG_SDMA, "copy2d": TIDE_AG_COPY2D}[args.ag_mode]

    L = Layout(cfg.shapes, cfg.R)
    L.prepare()
    stream = torch.cuda.current_stream()
    # Arguments are validated and marshalled once; each call below is one C-ABI call.
    rs_launch = parse_launch(args.rs_launch or args.launch)
    ag_launch = parse_launch(args.ag_launch or args.launch) if args.ag_mode == "kernel" else Launch()
    rs_call = L.bind_rs(grads, shards, launch=rs_launch)
    ag_call = L.bind_ag(stage, params, mode=ag_mode, launch=ag_launch)

    def step(ev_rs=None, ev_ag=None):
        if ev_rs:
            ev_rs[0].record(stream)
        rs_call.launch(stream)
        if ev_rs:
            ev_rs[1].record(stream)
        if ev_ag:
            ev_ag[0].record(stream)
        ag_call.launch(stream)
        if ev_ag:
            ev_ag[1].record(stream)
        if calib_src is not None:
            calib_dst.copy_(calib_src)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rs_ev = [(ev(), ev()) for _ in range(K)]
    ag_ev = [(ev(), ev()) for _ in range(K)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(rs_ev[i], ag_ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    rs_ms = [a.elapsed_time(b) for a, b in rs_ev]
    ag_ms = [a.elapsed_time(b) for a, b in ag_ev]
    ms_per_step = total_ms / K
    rs_mean = sum(rs_ms) / K
    ag_mean = sum(ag_ms) / K
    rs_sorted, ag_sorted = sorted(rs_ms), sorted(ag_ms)
    log(f"{K} steps: {total_ms:.3f} ms GPU ({t_wall * 1e3:.1f} ms wall); RS mean {rs_mean:.4f} ms "
        f"min {rs_sorted[0]:.4f} med {rs_sorted[K // 2]:.4f}; AG mean {ag_mean:.4f} ms min {ag_sorted[0]:.4f}")

    # Host cost per call (enqueue only; the GPU is kept busy by a long queue of earlier calls):
    # the bound C-ABI call, and the unbound binding call that validates and marshals every time.
    def host_us(fn, n=20):
        t = time.perf_counter()
        for _ in range(n):
            fn()
        return (time.perf_counter() - t) / n * 1e6
    host_bound = host_us(lambda: rs_call.launch(stream))
    host_unbound = host_us(lambda: L.rs_bf16_to_fp32(grads, shards, launch=rs_launch, stream=stream))
    torch.cuda.synchronize()

    graph_info = None
    if args.graph and args.ag_mode != "kernel":
        log("--graph: only the kernel placement is captured; skipped for --ag-mode " + args.ag_mode)
    elif args.graph:
        # The same two prepared calls captured once on a side stream; K replays timed between events.
        side = torch.cuda.Stream()
        rs_call.launch(side)
        ag_call.launch(side)
        side.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            rs_call.launch(side)
            ag_call.launch(side)
        with torch.cuda.stream(side):
            for _ in range(args.warmup):
                graph.replay()
            g0, g1 = ev(), ev()
            side.synchronize()
            g0.record(side)
            for _ in range(K):
                graph.replay()
            g1.record(side)
        g1.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        graph_info = {"ms_per_step": round(graph_ms, 5),
                      "step_gbps": round((rs_bytes + ag_bytes) / (graph_ms * 1e-3) / 1e9, 2)}
        log(f"graph replay: {graph_ms:.4f} ms per step ({graph_info['step_gbps']:.0f} GB/s)")
        del graph
        torch.cuda.synchronize()

    # Same-run calibration: a runtime device-to-device copy moving the RS's bytes (half read, half
    # written), the practical ceiling a plain stream reaches on this device; median of 10.
    cal_src = torch.empty(rs_bytes // 2, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_ms = []
    for i in range(13):
        a, b = ev(), ev()
        a.record(stream)
        cal_dst.copy_(cal_src)
        b.record(stream)
        b.synchronize()
        if i >= 3:
            cal_ms.append(a.elapsed_time(b))
    cal_med = sorted(cal_ms)[len(cal_ms) // 2]
    cal_gbps = 2 * cal_src.numel() / (cal_med * 1e-3) / 1e9
    del cal_src, cal_dst
    log(f"device-to-device copy of the same bytes: {cal_gbps:.0f} GB/s (median {cal_med:.4f} ms)")

    # Shader clock (clocks are not fixed on these devices, so they are recorded): one sleeping probe
    # wave on a side stream reads the shader cycle counter against the wall clock for 2 ms, once with
    # the device idle and once while RS calls run back to back beside it (outside the timed region).
    clock_info = None
    try:
        from all_gather_placement_amd import probe as pr

        khz = pr.wall_clock_khz()
        ticks = 2 * khz  # 2 ms
        out = torch.zeros(4, dtype=torch.int64, device=dev)
        side = torch.cuda.Stream(device=dev)
        pr.clock_probe(ticks, out, side)
        side.synchronize()
        idle = pr.clock_mhz(out.cpu().tolist(), khz)
        torch.cuda.synchronize()
        pr.clock_probe(ticks, out, side)
        for _ in range(int(2.5 / max(rs_mean, 1e-3)) + 2):  # > 2.5 ms of RS, covering the probe
            rs_call.launch(stream)
        torch.cuda.synchronize()
        clock_info = {"idle_mhz": round(idle, 1), "during_rs_mhz": round(pr.clock_mhz(out.cpu().tolist(), khz), 1),
                      "method": "s_memtime cycles / wall clock over 2 ms, one probe wave on a side stream"}
        log(f"shader clock: idle {clock_info['idle_mhz']} MHz, during the RS {clock_info['during_rs_mhz']} MHz")
    except (RuntimeError, OSError) as e:  # a measurement aid only: the line is still printed
        clock_info = {"error": str(e)}

    step_gbps = (rs_bytes + ag_bytes) / (ms_per_step * 1e-3) / 1e9
    rs_gbps = rs_bytes / (rs_mean * 1e-3) / 1e9
    ag_gbps = ag_bytes / (ag_mean * 1e-3) / 1e9
    # counters were taken for the workload's own contributor count and its default launch
    rs_kernel = rs_kernel_name(cfg.C, rs_launch)
    traffic = read_traffic(cfg.name, rs_kernel) if rs_launch == Launch() and not args.contributors else None

    out = {
        "metric": METRIC,
        "value": round(rs_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name} RS+AG step (R={cfg.R}, C={cfg.C}, P={cfg.P})",
            "R": cfg.R, "C": cfg.C, "P": cfg.P, "numel": numel, "S": S,
            "rs_launch": str(rs_launch), "rs_mode": launch_mode(rs_launch, cfg.C),
            "ag_mode": args.ag_mode, "ag_launch": str(ag_launch),
            "rs_bytes": rs_bytes, "ag_bytes": ag_bytes, "parallelism": "none (1 GPU, node-local level)",
        },
        "rs_gbps": round(rs_gbps, 2),
        "rs_frac_of_peak": round(rs_gbps / HBM_PEAK_GBPS, 4),
        "step_gbps": round(step_gbps, 2),
        "rs_ms_mean": round(rs_mean, 5),
        "rs_ms_min_median": [round(rs_sorted[0], 5), round(rs_sorted[K // 2], 5)],
        "ag_gbps": round(ag_gbps, 2),
        "ag_frac_of_peak": round(ag_gbps / HBM_PEAK_GBPS, 4),
        "ag_ms_mean": round(ag_mean, 5),
        "rs_host_us_per_call": {"bound": round(host_bound, 1), "validate_and_marshal": round(host_unbound, 1)},
        "rs_launch_shape": tide_rs_launch_shape(cfg.C, rs_launch),
        "graph_replay": graph_info,
        "calibration": {"d2d_copy_gbps": round(cal_gbps, 2), "bytes_moved": 2 * (rs_bytes // 2),
                        "rs_over_d2d_copy": round(rs_gbps / cal_gbps, 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": rs_kernel,
            "achieved": round(rs_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(rs_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "kernel_source_sha256_16": kernel_source_hash(),
        "software": {"torch": torch.__version__, "hip": torch.version.hip},
        "shader_clock": clock_info,
        "device": {"name": torch.cuda.get_device_name(dev),
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count},
    }
    L.close()
    del grads, shards, stage, params
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, log)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
