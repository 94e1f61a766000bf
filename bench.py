"""Benchmark of PISA pyramid Top-K block selection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick [--workload p64k|p16k]] [--no-cpu]
    python bench.py --traffic FETCH_DIR WRITE_DIR   (no GPU: counters -> profiles/traffic.json)

One step = one pass of the selection path over the 262,144-token workload
(batch 1, 16 query heads sharing 4 KV heads, d=128, C=64, g=4, K_top=8,
causal, bf16 N(0,1) Q/K with 32 planted key blocks per KV head): the pyramid
build followed by prefill routing of every position ("Block Sparse Attention
with Log-Linear Complexity", appendix B: selection timings include the
summary construction and every selection stage, not the attention).
`value` is routed queries per second (positions x batch / step time) with
inputs resident in HBM.

Also reported (field "extra"): route-only time of the routers, the
exhaustive BSA-style selector on the same inputs, the 16K and 64K prefill
workloads, block-sparse attention at 64K, decode (32 sequences, 262,144
cached tokens, 256 appended tokens: append + route microseconds per step),
and a sweep of N = 4K .. 1M at the appendix's own selection-benchmark
shape (32 query / 2 KV heads, d=64, g=2).

Prints ONE JSON line. Only one GPU is used; --gpus above 1 exits with an error.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np
import torch

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

from hierarchical_top_amd import pisa, synth, workcount  # noqa: E402

METRIC = "routed queries/sec at 64K and 256K tokens (GQA prefill); decode route µs/step"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# v_exp_f32 lane results per second from the unit counts: 256 CUs x 4 SIMDs x 16 lanes per
# clock at 2.4 GHz, issued at half rate (the rate the in-run exp loop measures on gfx950)
PEAK_EXP_GPS = 256 * 4 * 16 * 2.4 / 2
MODES = {"levels": pisa.LEVELS, "two_stage": pisa.TWO_STAGE, "fused": pisa.FUSED}
STAGES_TWO = ["build", "upper", "cluster", "leaf", "final"]
STAGES_FUSED = ["build", "route_fused"]
ARMED = {"build": 1, "route_fused": 1, "leaf": 1, "upper": 8, "cluster": 8, "final": 8}
# kernel (name fragment in a rocprofv3 trace) of each single-kernel stage
STAGE_KERNEL = {"leaf": "leaf_kernel", "build": "build_block_kernel", "route_fused": "route_query_kernel"}
# kernel-name patterns (re.search) of the counter records: the fused router and the first stage of
# the two-stage router are two instantiations of route_query_kernel (mode 0 and mode 1)
KERNEL_PATTERN = {"leaf": "leaf_kernel", "build": "build_block_kernel",
                  "route_fused": r"route_query_kernel\w*Li0ELi\d+EEEvNS_9RouteArgsE",
                  "route_stage1": r"route_query_kernel\w*Li1ELi\d+EEEvNS_9RouteArgsE",
                  "route_stage2": "stage2_kernel", "upper_sparse": "upper_ring_kernel",
                  "upper_dense": "dense_kernel", "select": "select_kernel", "bsa": "bsa_tile_kernel"}
# kernels of the 64K attention workload whose HBM traffic the counters measure (bench.py --only attn_bwd)
ATTN_KERNEL = {"attn_fwd": "attn_cl_kernel", "attn_bwd": "attn_bwd_kernel", "dq_combine": "dq_combine_kernel"}
# kernels of a decode step (bench.py --only decode): append the new token's pyramid path, route it,
# attend over the selected blocks
DECODE_KERNEL = {"decode_append": "append_kernel", "decode_route": "route_decode_kernel",
                 "decode_attn": r"11attn_kernelI|^attn_kernel$"}
COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read and 1 GiB written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def events():
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    return a, b


class Prefill:
    """Inputs, pyramid, workspace and outputs of one prefill workload on the GPU."""

    def __init__(self, w: synth.Workload, with_v=False):
        self.w = w
        Q, K, V, _ = synth.make_prefill(w)
        self.Q_cpu, self.K_cpu = Q, K
        self.Q, self.K = Q.cuda(), K.cuda()
        self.V = V.cuda() if (with_v and V is not None) else None
        self.pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
        need = max(pisa.route_workspace_bytes(self.pyr, w.N, w.H_q, w.K_top, m) for m in (pisa.TWO_STAGE, pisa.LEVELS))
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.idx = torch.empty(w.B, w.H_kv, w.N, w.K_top, dtype=torch.int32, device="cuda")
        self.bidx = torch.empty_like(self.idx)

    def step(self, mode, stage_events=None, score_kind="lse"):
        """Pyramid build + routing of every position. stage_events: {stage: [(start, stop), ...]}
        armed for this step; returns {stage: number of pairs the step consumed}."""
        w = self.w
        if stage_events:
            for name, pairs in stage_events.items():
                for a, b in pairs:
                    pisa.time_stage(name, a, b)
        self.pyr.build(self.K, w.N)
        pisa.route_prefill(self.pyr, self.Q, self.K, w.N, w.K_top, mode=mode, workspace=self.ws, out=self.idx,
                           score_kind=score_kind)
        fired = {}
        if stage_events:
            for name, pairs in stage_events.items():
                fired[name] = len(pairs) - pisa.time_stage_pending(name)
                pisa.time_stage_clear(name)
        return fired

    def route_only(self, mode):
        w = self.w
        pisa.route_prefill(self.pyr, self.Q, self.K, w.N, w.K_top, mode=mode, workspace=self.ws, out=self.idx)

    def bsa(self):
        w = self.w
        pisa.bsa_select(self.pyr, self.Q, w.N, w.K_top, out=self.bidx)


def graph_ms(fn, reps):
    """ms per replay of fn captured in a HIP graph (torch.cuda.CUDAGraph on its stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    ms = time_fn(g.replay, reps)
    del g
    return ms


def time_fn(fn, reps, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = events()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


# the sources each counted kernel is compiled from (its file, the headers it includes and
# the host code that launches it): a counter record stays valid while these are unchanged
_COMMON_SRC = ("pisa_device.hpp", "pisa_internal.hpp")
STAGE_SOURCES = {
    "build": ("pyramid.hip",),
    "leaf": ("levels.hip", "levels_impl.hpp", "levels_bf16.hip", "stream.hpp"),
    "route_fused": ("route.hip", "route_impl.hpp", "route_bf16.hip"),
    "route_stage1": ("route.hip", "route_impl.hpp", "route_bf16.hip"),
    "route_stage2": ("route.hip", "route_impl.hpp", "route_bf16.hip"),
    "upper_sparse": ("levels.hip", "levels_impl.hpp", "levels_bf16.hip", "stream.hpp"),
    "upper_dense": ("levels.hip", "levels_impl.hpp", "levels_bf16.hip"),
    "select": ("levels.hip",),
    "bsa": ("bsa.hip",),
    "decode_append": ("pyramid.hip",),
    "decode_route": ("route.hip", "route_impl.hpp", "route_bf16.hip"),
    "decode_attn": ("attn.hip",),
    "attn_fwd": ("attn_cl.hip", "attn_bwd.hpp", "stream.hpp"),
    "attn_bwd": ("attn_bwd.hip", "attn_bwd.hpp", "attn_cl.hip"),
    "dq_combine": ("attn_bwd.hip", "attn_bwd.hpp"),
}


def source_hash(stage: str) -> str:
    h = hashlib.sha256()
    for name in sorted(_COMMON_SRC + STAGE_SOURCES[stage]):
        p = ROOT / "hierarchical_top_amd" / "csrc" / name
        h.update(name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch of stage `kernel` from the committed rocprofv3 counter
    summary, if it was taken on that kernel's current sources (else None)."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text()).get("%s/%s" % (workload, kernel))
    except (ValueError, OSError):
        return None
    if not rec or kernel not in STAGE_SOURCES or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def roofline(stage, ms, w, traffic):
    """Roofline entry of one stage from its average duration (ms per launch)."""
    G = w.H_q // w.H_kv
    rw = workcount.route_work(w.B, w.N, w.H_kv, G, w.d, w.C, w.g, w.K_top)
    if stage in ("build",):
        byts = workcount.build_bytes(w.B, w.N, w.H_kv, w.d, w.C, w.g)
        ach = byts / (ms * 1e-3) / 1e9
        return dict(kernel=stage, bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS,
                    traffic=traffic, algorithmic=byts, ms_per_launch=ms)
    flops = {"leaf": 2 * rw["leaf_mac"], "upper": 2 * rw["upper_mac"],
             "route_fused": 2 * (rw["leaf_mac"] + rw["upper_mac"])}.get(stage)
    if flops is None:  # clustering / final select: integer passes over the per-query lists
        items = w.B * w.H_kv * w.N
        byts = items * (w.K_top * 4 * 3 + 8) if stage == "cluster" else items * (w.K_top * 4 * 2 + 8 + w.g * w.K_top * 4)
        ach = byts / (ms * 1e-3) / 1e9
        return dict(kernel=stage, bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS,
                    traffic=traffic, algorithmic=byts, ms_per_launch=ms)
    ach = flops / (ms * 1e-3) / 1e12
    return dict(kernel=stage, bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=ach / PEAK_BF16_TFLOPS, traffic=traffic, algorithmic=flops, ms_per_launch=ms)


def leaf_roofs(roof, w, peaks):
    """The leaf scoring against the roofs measured in the same run: its MFMA work against the
    MFMA loop and against the MFMA rate of the 1:1 MFMA + exp mix (the leaf's own mix: per 16 x 64
    logit tile 16 MFMAs and 16 wave-wide exponentials), and its exponentials (one per raw-key
    logit of a scored leaf and head, section 3.2 eq 21) against the exp loop; when the kernel's
    HBM traffic per launch is known from counters (roof["traffic"]), also those bytes against
    the gather loop (almost all of them are gathered 1 KiB query rows) and, for reference, the
    copy loop. The binding roof is the slowest of these floors."""
    G = w.H_q // w.H_kv
    rw = workcount.route_work(w.B, w.N, w.H_kv, G, w.d, w.C, w.g, w.K_top)
    s = roof["ms_per_launch"] * 1e-3
    flops, exps = 2 * rw["leaf_mac"], rw["leaf_exp"]
    floors = {"mfma": flops / (peaks["mfma_bf16_tflops"] * 1e12),
              "exp": exps / (peaks["exp_gps"] * 1e9),
              "mfma+exp": flops / (peaks["mix_mfma_tflops"] * 1e12)}
    moved = roof.get("traffic")
    if moved:
        floors["traffic"] = moved / (peaks["gather_gbs"] * 1e9)
    bind = max(floors, key=floors.get)
    return dict(algorithmic_exp=exps, achieved_exp_gps=exps / s / 1e9,
                traffic_bytes=moved, traffic_gbs=moved / s / 1e9 if moved else None,
                traffic_frac_of_measured_copy=moved / s / 1e9 / peaks["copy_gbs"] if moved else None,
                traffic_frac_of_measured_gather=moved / s / 1e9 / peaks["gather_gbs"] if moved else None,
                exp_frac_of_derived_peak=exps / s / 1e9 / PEAK_EXP_GPS, derived_exp_peak_gps=PEAK_EXP_GPS,
                measured_mfma_tflops=peaks["mfma_bf16_tflops"], frac_of_measured_mfma=roof["achieved"] / peaks["mfma_bf16_tflops"],
                measured_mix_mfma_tflops=peaks["mix_mfma_tflops"],
                frac_of_measured_mix=roof["achieved"] / peaks["mix_mfma_tflops"],
                measured_exp_gps=peaks["exp_gps"], frac_of_measured_exp=exps / s / 1e9 / peaks["exp_gps"],
                floors_ms={k: v * 1e3 for k, v in floors.items()}, binding_roof=bind,
                time_over_binding_floor=s / floors[bind])


PEAKS_LIB = ROOT / "hierarchical_top_amd" / "libpisa_peaks.so"


def unit_peaks(reps: int = 5):
    """The units the selection kernels are bound by, timed in this run (include/pisa_peaks.h):
    v_exp_f32 throughput, bf16 MFMA 16x16x32 throughput, the two issued 1:1 from the same waves
    (the mix of the leaf scoring: per 16 x 64 logit tile, 16 MFMAs and 16 wave-wide exponentials
    per wave), and an HBM copy."""
    import ctypes
    L = ctypes.CDLL(str(PEAKS_LIB))
    for f in ("pisa_peak_exp", "pisa_peak_mfma", "pisa_peak_mix"):
        getattr(L, f).argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.pisa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.pisa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.pisa_peak_gather.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_uint32, ctypes.c_void_p]
    blocks, iters = 2048, 4096                      # 8 waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def run(f):
        rc = f()
        if rc != 0:
            raise RuntimeError("peak kernel launch failed (%d)" % rc)

    ms_exp = time_fn(lambda: run(lambda: L.pisa_peak_exp(out.data_ptr(), blocks, iters, st)), reps)
    ms_mfma = time_fn(lambda: run(lambda: L.pisa_peak_mfma(out.data_ptr(), blocks, iters, st)), reps)
    ms_mix = time_fn(lambda: run(lambda: L.pisa_peak_mix(out.data_ptr(), blocks, iters, st)), reps)
    exps = blocks * 256 * iters * 8
    mfmas = blocks * 4 * iters * 8
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ms_copy = time_fn(lambda: run(lambda: L.pisa_peak_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, st)), reps)
    ok = bool(torch.equal(src, dst))
    def read4():  # four back-to-back passes over the 1 GiB buffer (larger than the 256 MB MALL)
        for _ in range(4):
            run(lambda: L.pisa_peak_read(src.data_ptr(), COPY_BYTES, out.data_ptr(), st))
    ms_read = time_fn(read4, reps)
    rows_per_wave = 512                             # 2048 x 4 waves x 512 rows of 1 KiB = 4 GiB
    ms_gather = time_fn(lambda: run(lambda: L.pisa_peak_gather(src.data_ptr(), COPY_BYTES, out.data_ptr(), blocks,
                                                               rows_per_wave, 12345, st)), reps)
    gathered = blocks * 4 * rows_per_wave * 1024
    del src, dst, out
    torch.cuda.empty_cache()
    return dict(exp_gps=exps / (ms_exp * 1e-3) / 1e9,
                mfma_bf16_tflops=mfmas * 16384 / (ms_mfma * 1e-3) / 1e12,
                mix_mfma_tflops=mfmas * 16384 / (ms_mix * 1e-3) / 1e12,
                mix_exp_gps=mfmas * 64 / (ms_mix * 1e-3) / 1e9,
                mix_over_mfma_time=ms_mix / ms_mfma,
                copy_gbs=2 * COPY_BYTES / (ms_copy * 1e-3) / 1e9, copy_verified=ok,
                read_gbs=4 * COPY_BYTES / (ms_read * 1e-3) / 1e9,
                gather_gbs=gathered / (ms_gather * 1e-3) / 1e9,
                how="exp: 8 independent chains x <- 2^-x per thread; mfma: 8 independent accumulators per wave; "
                    "mix: the two interleaved 1:1 in every wave; copy: 1 GiB read + 1 GiB written, 16-byte "
                    "accesses; read: the same 1 GiB read four times over; gather: 4 GiB of 1 KiB rows at hashed positions "
                    "of that 1 GiB (one row per wave and load: the routers' per-entry query gathers); "
                    "%d workgroups of 256 threads" % blocks)


def copy_calibration():
    """A plain 1 GiB device-to-device copy, so that a counter run over this program
    also holds the counters of a transfer of known size."""
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def _counter_rows(d):
    import csv
    files = sorted(Path(d).rglob("*counter_collection.csv"))
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (str(f), r["Dispatch_Id"])
            e = per.setdefault(key, {"name": r["Kernel_Name"], "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return list(per.values())


def traffic_from_counters(fetch_dir, write_dir, workload="p256k", kernels=None):
    """HBM bytes per launch of the stage kernels from two rocprofv3 --pmc runs of
    `bench.py --quick --no-cpu --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, in
    KiB per dispatch), each scaled so that the calibration copy reads / writes
    exactly COPY_BYTES. Writes profiles/traffic.json; returns the records."""
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)

    def avg(rows, pat, counter):
        v = [r["c"][counter] for r in rows if re.search(pat, r["name"]) and counter in r["c"]]
        return (float(np.mean(v)) * 1024.0, len(v)) if v else (None, 0)

    def largest(rows, counter):  # the calibration copy: the largest copy dispatch (a decode run has small ones)
        v = [r["c"][counter] for r in rows if "copyBuffer" in r["name"] and counter in r["c"]]
        return max(v) * 1024.0 if v else None

    f_copy, w_copy = largest(fetch, "FETCH_SIZE"), largest(write, "WRITE_SIZE")
    if not f_copy or not w_copy:
        raise SystemExit("the calibration copy is missing from the counter runs")
    kf, kw = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    out_file = ROOT / "profiles" / "traffic.json"
    recs = json.loads(out_file.read_text()) if out_file.exists() else {}
    for stage, pat in (kernels or KERNEL_PATTERN).items():
        fb, nf = avg(fetch, pat, "FETCH_SIZE")
        wb, nw = avg(write, pat, "WRITE_SIZE")
        if fb is None or wb is None:
            continue
        recs["%s/%s" % (workload, stage)] = dict(
            kernel=pat, bytes_per_launch=fb * kf + wb * kw, fetch_bytes=fb * kf, write_bytes=wb * kw,
            dispatches=[nf, nw], scale=dict(fetch=kf, write=kw), source_hash=source_hash(stage))
    out_file.write_text(json.dumps(recs, indent=1, sort_keys=True) + "\n")
    return recs


def sample_positions(N, C, n):
    t = np.linspace(0, N - 1, n).astype(np.int64)
    return np.unique(np.concatenate([t, np.arange(3 * C), np.arange(N - C, N)]))


def cpu_baseline(P: Prefill, budget_s: float):
    """The oracle on the host cores: full pyramid build, then routing of a growing
    evenly spaced sample of positions until one sample takes at least 0.8 * budget_s seconds."""
    import oracle  # test infrastructure: only this leg of the benchmark calls it
    w = P.w
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    Kf = P.K_cpu.float().numpy()
    t0 = time.perf_counter()
    opyr = oracle.Pyramid(Kf, w.N, w.C, w.g)
    t_build = time.perf_counter() - t0
    n = 256
    gpu_idx = P.idx.cpu().numpy()
    while True:
        t = sample_positions(w.N, w.C, n)
        Qs = P.Q_cpu[0, t].float().numpy()
        t0 = time.perf_counter()
        orc = oracle.route(opyr, Qs, [0] * len(t), t, w.K_top, causal=True, threads=threads)
        dt = time.perf_counter() - t0
        if dt >= 0.8 * budget_s or n >= w.N:
            break
        n = min(w.N, int(n * min(8.0, max(1.25, budget_s / max(dt, 1e-3)))))
    # routing cost per query position, weighted to the full sequence by the scored work
    full = workcount.route_work(w.B, w.N, w.H_kv, w.H_q // w.H_kv, w.d, w.C, w.g, w.K_top)
    samp = workcount.route_work(w.B, w.N, w.H_kv, w.H_q // w.H_kv, w.d, w.C, w.g, w.K_top, positions=t)
    scale = (full["upper_mac"] + full["leaf_mac"]) / max(1, samp["upper_mac"] + samp["leaf_mac"])
    t_route_full = dt * scale
    qps = w.B * w.N / (t_build + t_route_full)
    # parity of the GPU selection on the sampled positions
    parity = selection_parity(opyr, Qs, t, gpu_idx[0][:, t].transpose(1, 0, 2), orc, w.K_top, threads)
    # cores: the threads the oracle ran on; the host's own core count is stated beside it
    res = dict(value=qps, unit="queries/s", cores=threads, threads=threads, host_cores=os.cpu_count(),
               host_cores_available=len(os.sched_getaffinity(0)), kind="oracle",
               sample="full fp64 pyramid build (%.2f s) + routing of %d evenly spaced positions x %d KV heads "
                      "(%.2f s), extrapolated to all %d positions by the scored work (x%.1f)"
                      % (t_build, len(t), w.H_kv, dt, w.N, scale),
               build_s=t_build, route_sample_s=dt)
    return res, parity


def selection_parity(opyr, Qs, t, gi, orc, K_top, threads, band=1e-3, strict=1e-5):
    """Parity of GPU selections gi [n][H][K_top] with the oracle's on positions t: exact
    wherever every ranked level's margin is at least `strict`; elsewhere a differing selection
    must be a tie resolution of the oracle's route within `band` (the oracle's search)."""
    import oracle  # test infrastructure: parity of the timed selection
    same = (gi == orc["idx"]).all(-1)
    mism = np.argwhere(~same)
    eps = np.zeros(0)
    if len(mism):
        eps = oracle.route_reach(opyr, Qs[mism[:, 0]], [0] * len(mism), np.asarray(t)[mism[:, 0]], mism[:, 1],
                                 gi[mism[:, 0], mism[:, 1]], K_top, cap=band, threads=threads)
    return dict(sampled_positions=int(len(t)), items=int(same.size), identical=int(same.sum()),
                near_tie_items=int((orc["gap"] < band).sum()), band=band, strict_band=strict,
                mismatches_outside_strict=int((~same & (orc["gap"] >= strict)).sum()),
                invalid_tie_resolutions=int((~(eps <= band)).sum()),
                max_tie_resolution_cost=float(eps.max()) if len(eps) else 0.0)


def decode_bench(reps_steps: int):
    w = synth.workload("decode", steps=reps_steps)
    Kc, Vc, q, k, v = synth.make_decode(w, "cuda")
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N + w.steps)
    pyr.build(Kc, w.N)
    idx = torch.empty(w.B, w.H_kv, w.K_top, dtype=torch.int32, device="cuda")
    O = torch.empty(w.B, 1, w.H_q, w.d, dtype=torch.bfloat16, device="cuda")
    seqlens = [torch.full((w.B,), w.N + s + 1, dtype=torch.int64, device="cuda") for s in range(w.steps)]
    # one untimed step on the built cache (appending its last token again rewrites the same
    # path bit for bit), so that no timed step pays a kernel's first launch
    built = torch.full((w.B,), w.N, dtype=torch.int64, device="cuda")
    pyr.append(Kc, built)
    pisa.route_decode(pyr, q[0], Kc, built, w.K_top, out=idx)
    pisa.sparse_attn(q[0].unsqueeze(1), Kc, Vc, idx.unsqueeze(2), w.C, w.N, kv_len=built, out=O)
    torch.cuda.synchronize()
    ev = [(events(), events(), events()) for _ in range(w.steps)]
    for s in range(w.steps):
        n = w.N + s + 1
        Kc[:, n - 1] = k[s]
        Vc[:, n - 1] = v[s]
        (a0, a1), (r0, r1), (t0, t1) = ev[s]
        pisa.time_stage("append", a0, a1)
        pisa.time_stage("route_decode", r0, r1)
        pisa.time_stage("attn", t0, t1)
        pyr.append(Kc, seqlens[s])
        pisa.route_decode(pyr, q[s], Kc, seqlens[s], w.K_top, out=idx)
        pisa.sparse_attn(q[s].unsqueeze(1), Kc, Vc, idx.unsqueeze(2), w.C, n, kv_len=seqlens[s], out=O)
    torch.cuda.synchronize()
    app = np.array([a.elapsed_time(b) for (a, b), _, _ in ev]) * 1e3
    rt = np.array([a.elapsed_time(b) for _, (a, b), _ in ev]) * 1e3
    at = np.array([a.elapsed_time(b) for _, _, (a, b) in ev]) * 1e3
    both = app + rt
    dw = workcount.decode_work([w.N + w.steps // 2] * w.B, w.H_kv, w.H_q // w.H_kv, w.d, w.C, w.g, w.K_top)
    gbs = dw["bytes"] / (np.median(rt) * 1e-6) / 1e9
    res = dict(steps=w.steps, B=w.B, cache_tokens=w.N, route_us_median=float(np.median(rt)),
               route_us_p99=float(np.percentile(rt, 99)), append_us_median=float(np.median(app)),
               append_plus_route_us_median=float(np.median(both)),
               append_plus_route_us_p99=float(np.percentile(both, 99)),
               attn_us_median=float(np.median(at)),
               route_gathered_bytes=dw["bytes"], route_hbm_gbs=gbs, route_hbm_frac=gbs / PEAK_HBM_GBS)
    del Kc, Vc
    torch.cuda.empty_cache()
    return res


def prefill_extra(name, reps, with_attn=False):
    w = synth.workload(name)
    P = Prefill(w, with_v=with_attn)
    G = w.H_q // w.H_kv
    out = {}
    for mname, mode in MODES.items():
        out["build_route_ms_" + mname] = time_fn(lambda: P.step(mode), reps)
        out["route_ms_" + mname] = time_fn(lambda: P.route_only(mode), reps)
    best = min(out["build_route_ms_" + m] for m in MODES)
    out["routed_queries_per_s"] = w.B * w.N / (best * 1e-3)
    # the same build + level route captured once in a HIP graph and replayed: at short
    # lengths the route is a chain of small launches whose gaps a graph removes
    out["build_route_ms_levels_graph"] = graph_ms(lambda: P.step(pisa.LEVELS), reps)
    out["routed_queries_per_s_graph"] = w.B * w.N / (out["build_route_ms_levels_graph"] * 1e-3)
    out["bsa_ms"] = time_fn(P.bsa, max(2, reps // 2))
    bw = workcount.bsa_work(w.B, w.N, w.H_kv, G, w.d, w.C, w.K_top)
    out["bsa_alg_tflops_one_pass"] = 2 * bw["mac"] / (out["bsa_ms"] * 1e-3) / 1e12
    # the pages' comparison: selection with summary construction vs the exhaustive selector
    # (whose level-1 means come from the same build)
    bms = time_fn(lambda: P.pyr.build(P.K, w.N), reps)
    out["build_ms"] = bms
    if name == "p16k":
        out["selection_quality"] = selection_quality_table(P)
    out["speedup_vs_bsa"] = (out["bsa_ms"] + bms) / best
    if with_attn:
        P.step(pisa.LEVELS)
        O = torch.empty_like(P.Q)
        aw = workcount.attn_work(w.B, w.N, w.H_q, w.d, w.C, w.K_top)
        ws = torch.empty(pisa.sparse_attn_workspace_bytes(w.B, w.N, w.N, w.H_q, w.H_kv, w.d, w.C, w.K_top),
                         dtype=torch.uint8, device="cuda")
        ms_rows = time_fn(lambda: pisa.sparse_attn(P.Q, P.K, P.V, P.idx, w.C, w.N, out=O), max(2, reps // 2))
        ms_cl = time_fn(lambda: pisa.sparse_attn_clustered(P.Q, P.K, P.V, P.idx, w.C, w.N, workspace=ws, out=O),
                        reps)
        del ws
        ms = min(ms_rows, ms_cl)
        out["attn_ms_per_row"] = ms_rows
        out["attn_ms_clustered"] = ms_cl
        out["attn_ms"] = ms
        out["attn_tflops"] = 2 * aw["mac"] / (ms * 1e-3) / 1e12
        out["attn_mfma_frac"] = out["attn_tflops"] / PEAK_BF16_TFLOPS
        # backward with the routed blocks fixed (dQ, dK, dV in fp32 from the forward's O and lse)
        O, lse = pisa.sparse_attn_clustered(P.Q, P.K, P.V, P.idx, w.C, w.N, with_lse=True)
        dO = synth.make_grad_out(P.Q.shape, 303).cuda()
        bws = torch.empty(pisa.sparse_attn_bwd_workspace_bytes(w.B, w.N, w.N, w.H_q, w.H_kv, w.d, w.C, w.K_top),
                          dtype=torch.uint8, device="cuda")
        grads = tuple(torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (P.Q, P.K, P.V))
        bw = workcount.attn_bwd_work(w.B, w.N, w.H_q, w.d, w.C, w.K_top)
        ms_b = time_fn(lambda: pisa.sparse_attn_bwd(P.Q, P.K, P.V, O, dO, lse, P.idx, w.C, w.N, workspace=bws,
                                                    out=grads), reps)
        out["attn_bwd_ms"] = ms_b
        for st, ms_st in (("attn_fwd", None), ("attn_bwd", None)):
            tr = load_traffic(st, "p64k")
            if tr is not None:
                out[st + "_traffic_bytes"] = tr
        out["attn_bwd_tflops"] = 2 * bw["mac"] / (ms_b * 1e-3) / 1e12
        out["attn_bwd_mfma_frac"] = out["attn_bwd_tflops"] / PEAK_BF16_TFLOPS
        del O, lse, dO, bws, grads
    del P
    torch.cuda.empty_cache()
    return out


def selection_quality_table(P):
    """Recall@K, captured mass and mass ratio against full attention (section 4.4, appendix
    D.2) of PISA and its score ablations (level router) and of the exhaustive BSA-style
    selector, averaged over the rows with more than K_top eligible blocks, as the appendix
    does. Synthetic planted inputs: not comparable with the appendix's model activations."""
    w = P.w
    rows = torch.arange(w.N, device="cuda") // w.C + 1 > w.K_top
    res = {}
    sels = {}
    for kind in ("lse", "mean", "mean_var"):
        P.pyr.build(P.K, w.N)
        pisa.route_prefill(P.pyr, P.Q, P.K, w.N, w.K_top, mode=pisa.LEVELS, workspace=P.ws, out=P.idx,
                           score_kind=kind)
        sels[{"lse": "pisa", "mean": "pisa1", "mean_var": "pisa2"}[kind]] = P.idx.clone()
    P.bsa()
    sels["bsa"] = P.bidx.clone()
    for name, sel in sels.items():
        q = pisa.selection_quality(P.Q, P.K, sel, w.C)
        res[name] = {k: float(q[k][:, :, rows].double().mean()) for k in ("recall", "captured", "ratio")}
    res["rows"] = int(rows.sum()) * w.B * w.H_kv
    return res


def attn_bwd_alone(reps: int = 10):
    """The 64K attention backward alone (random causal selection of the routing shape)."""
    w = synth.workload("p64k")
    Q, K, V, _ = synth.make_prefill(w)
    Q, K, V = Q.cuda(), K.cuda(), V.cuda()
    idx = torch.from_numpy(synth.random_selection(8, w.B, w.H_kv, w.N, w.K_top, w.C, [w.N], causal=True)).cuda()
    O, lse = pisa.sparse_attn_clustered(Q, K, V, idx, w.C, w.N, with_lse=True)
    dO = synth.make_grad_out(Q.shape, 303).cuda()
    ws = torch.empty(pisa.sparse_attn_bwd_workspace_bytes(w.B, w.N, w.N, w.H_q, w.H_kv, w.d, w.C, w.K_top),
                     dtype=torch.uint8, device="cuda")
    g = tuple(torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (Q, K, V))
    ms = time_fn(lambda: pisa.sparse_attn_bwd(Q, K, V, O, dO, lse, idx, w.C, w.N, workspace=ws, out=g), reps)
    bw = workcount.attn_bwd_work(w.B, w.N, w.H_q, w.d, w.C, w.K_top)
    return dict(attn_bwd_ms=ms, attn_bwd_tflops=2 * bw["mac"] / (ms * 1e-3) / 1e12)


PAPER_SWEEP_N = (4096, 8192, 16384, 32768, 65536, 131072, 262144, 1048576)


def paper_sweep(check: bool, sizes=PAPER_SWEEP_N):
    """Build + route at the appendix's selection-benchmark shape (32 query / 2 KV heads,
    d=64, C=64, g=2, K_top=8, random bf16 Q and K) for N = 4K .. 256K and 1M: every router, the
    exhaustive BSA-style selector and the build alone, in ms. With check, the longest
    sequence's level-router selection is compared with the oracle on sampled positions."""
    out = {}
    for N in sizes:
        w = synth.paper_shape(N)
        log("paper sweep", N)
        P = Prefill(w)
        r = {}
        for mname, mode in MODES.items():
            r["build_route_ms_" + mname] = time_fn(lambda: P.step(mode), 10 if mname == "levels" else 3,
                                                   warm=2 if N < (1 << 20) else 1)
        r["build_ms"] = time_fn(lambda: P.pyr.build(P.K, N), 10)
        r["bsa_ms"] = time_fn(P.bsa, 3, warm=2 if N < (1 << 20) else 1)
        best = min(r["build_route_ms_" + m] for m in MODES)
        r["routed_queries_per_s"] = N / (best * 1e-3)
        r["speedup_vs_bsa"] = (r["bsa_ms"] + r["build_ms"]) / best
        rw = workcount.route_work(w.B, N, w.H_kv, w.G_Q, w.d, w.C, w.g, w.K_top)
        r["levels_tflops"] = 2 * (rw["upper_mac"] + rw["leaf_mac"]) / (r["build_route_ms_levels"] * 1e-3) / 1e12
        if check and N == sizes[-1]:
            import oracle  # test infrastructure: sampled parity of the sweep's longest run
            P.step(pisa.LEVELS)
            torch.cuda.synchronize()
            t = sample_positions(N, w.C, 256)
            opyr = oracle.Pyramid(P.K_cpu.float().numpy(), N, w.C, w.g)
            orc = oracle.route(opyr, P.Q_cpu[0, t].float().numpy(), [0] * len(t), t, w.K_top, causal=True,
                               threads=max(1, min(len(os.sched_getaffinity(0)), 16)))
            gi = P.idx.cpu().numpy()[0][:, t].transpose(1, 0, 2)
            r["parity"] = selection_parity(opyr, P.Q_cpu[0, t].float().numpy(), t, gi, orc, w.K_top,
                                           max(1, min(len(os.sched_getaffinity(0)), 16)))
        out[str(N)] = r
        del P
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=["auto", "levels", "fused", "two_stage"], default="auto")
    ap.add_argument("--quick", action="store_true", help="headline workload only (no extra workloads)")
    ap.add_argument("--workload", choices=["p256k", "p64k", "p16k"], default="p256k",
                    help="with --quick: the prefill workload timed (for kernel traces of the smaller ones)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle routing to time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a 1 GiB device copy (counter calibration for --traffic)")
    ap.add_argument("--only", choices=["attn_bwd", "decode"],
                    help="time one part alone (for kernel traces): the 64K attention backward, or 32 decode steps")
    ap.add_argument("--traffic-workload", choices=["p256k", "p64k", "decode"], default="p256k",
                    help="with --traffic: the counter runs were of the headline (p256k), of --only attn_bwd "
                         "(p64k) or of --only decode (decode)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json")
    args = ap.parse_args()
    if args.traffic:
        kern = {"p64k": ATTN_KERNEL, "decode": DECODE_KERNEL}.get(args.traffic_workload, KERNEL_PATTERN)
        print(json.dumps(traffic_from_counters(*args.traffic, workload=args.traffic_workload, kernels=kern), indent=1,
                         sort_keys=True))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the selection path is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pisa.lib()  # fail loudly when the library is missing
    if args.only:
        print(json.dumps({"only": args.only, **(attn_bwd_alone() if args.only == "attn_bwd" else decode_bench(32))}),
              flush=True)
        if args.copy_calibration:
            copy_calibration()
        return

    if args.workload != "p256k" and not args.quick:
        raise SystemExit("--workload other than p256k is for --quick runs (kernel traces)")
    w = synth.workload(args.workload)
    log("generating", w)
    P = Prefill(w)
    torch.cuda.synchronize()

    # pick the router: both are timed once after warm-up
    pre = {m: time_fn(lambda: P.step(v), 3, warm=1) for m, v in MODES.items()}
    mname = min(pre, key=pre.get) if args.mode == "auto" else args.mode
    mode = MODES[mname]
    stage_names = STAGES_FUSED if mode == pisa.FUSED else STAGES_TWO
    log("pre-measure ms/step", pre, "->", mname)

    for _ in range(args.warmup):
        P.step(mode)
    stage_ev = [{s: [events() for _ in range(ARMED[s])] for s in stage_names} for _ in range(args.steps)]
    fired = []
    torch.cuda.synchronize()
    t0, t1 = events()
    t0.record()
    for k in range(args.steps):
        fired.append(P.step(mode, stage_ev[k]))
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    # per stage: summed over its launches in one step, averaged over the steps
    stages_ms = {s: float(np.mean([sum(a.elapsed_time(b) for a, b in e[s][:f[s]]) for e, f in zip(stage_ev, fired)]))
                 for s in stage_names}
    launches = {s: fired[0][s] for s in stage_names}
    # the dominant kernel: the single-kernel stage with the longest launch
    dom = max((s for s in stage_names if s in STAGE_KERNEL), key=lambda s: stages_ms[s] / max(1, launches[s]))
    log("ms/step", ms, "stages", stages_ms)
    traffic = load_traffic(dom, w.name)
    roof = roofline(dom, stages_ms[dom], w, traffic)
    roof["kernel"] = STAGE_KERNEL[dom]
    roof["launches_per_step"] = launches[dom]
    roof_all = {s: {k: roofline(s, stages_ms[s], w, load_traffic(s, w.name))[k]
                    for k in ("bound", "achieved", "unit", "frac")} for s in stage_names}

    # the units the leaf kernel is bound by, measured on this GPU in this run
    peaks = unit_peaks()
    log("unit peaks", peaks)
    if dom == "leaf":
        roof["measured_roofs"] = leaf_roofs(roof, w, peaks)
    extra = dict(headline_mode=mname, premeasure_ms=pre, stage_ms=stages_ms, stage_launches=launches,
                 stage_roofline=roof_all, unit_peaks=peaks)
    for m, v in MODES.items():
        extra["route_ms_" + m] = time_fn(lambda: P.route_only(v), 5)
    if not args.quick:
        # the same build + route step replayed from a HIP graph (no per-launch host gaps); the
        # headline value above stays the eager step
        extra["build_route_ms_levels_graph"] = graph_ms(lambda: P.step(mode), 10)
        extra["routed_queries_per_s_graph"] = w.B * w.N / (extra["build_route_ms_levels_graph"] * 1e-3)
    extra["bsa_ms"] = time_fn(P.bsa, 3)
    extra["build_ms"] = stages_ms["build"]
    extra["speedup_vs_bsa"] = (extra["bsa_ms"] + stages_ms["build"]) / ms
    G = w.H_q // w.H_kv
    bw = workcount.bsa_work(w.B, w.N, w.H_kv, G, w.d, w.C, w.K_top)
    extra["bsa_alg_tflops_one_pass"] = 2 * bw["mac"] / (extra["bsa_ms"] * 1e-3) / 1e12

    # the section 4.4 ablations on the same inputs: PISA-1 (mean) and PISA-2 (mean + var / 2)
    # block scores in the level router, build + route (not under --quick, whose kernel trace and
    # counters must hold the headline's kernels only)
    if not args.quick:
        extra["score_kinds_build_route_ms"] = {k: time_fn(lambda: P.step(pisa.LEVELS, score_kind=k), 10)
                                               for k in ("lse", "mean", "mean_var")}

    # the headline selection is left in P.idx for the parity check below
    P.step(mode)
    torch.cuda.synchronize()
    cpu, parity = (None, None)
    if not args.no_cpu:
        log("cpu oracle baseline")
        cpu, parity = cpu_baseline(P, args.cpu_budget)
        log("cpu", cpu, parity)
    del P
    torch.cuda.empty_cache()

    if args.copy_calibration:
        copy_calibration()

    if not args.quick:
        for name, reps, attn in (("p16k", 10, False), ("p64k", 5, True)):
            log("extra", name)
            extra[name] = prefill_extra(name, reps, with_attn=attn)
        log("extra decode")
        extra["decode"] = decode_bench(256)
        # the decode router only reads: its gathered bytes against this run's read loop
        extra["decode"]["route_frac_of_measured_read"] = extra["decode"]["route_hbm_gbs"] / peaks["read_gbs"]
        extra["paper_shape_sweep"] = dict(
            shape="B=1, H_q=32, H_kv=2, d=64, C=64, g=2, K_top=8, causal, random bf16 Q/K (seed 40)",
            by_N=paper_sweep(check=not args.no_cpu))

    line = {
        "metric": METRIC,
        "value": w.B * w.N / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill routing %dK: pyramid build + routing of every position" % (w.N // 1024),
                   "B": w.B, "N": w.N, "H_q": w.H_q, "H_kv": w.H_kv, "d": w.d, "C": w.C, "g": w.g,
                   "K_top": w.K_top, "causal": True, "planted_blocks_per_head": w.planted, "seed": w.seed,
                   "router": mname},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
