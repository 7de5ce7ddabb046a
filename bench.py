#!/usr/bin/env python3
"""Benchmark of the TwELL sparse gated-FFN forward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
tokens: ``tw_pack_gate`` (gate GEMM + ReLU + TwELL packing, overflow list)
then ``tw_sparse_ffn_fwd`` (fused sparse up+down, dense fallback for the
overflow rows).  Inputs are resident in HBM before the timed region.  The
dense gated FFN ``tw_ffn_fwd`` is timed the same way at the same shape for
the speedup.  Per-kernel durations come from HIP events recorded on the
launch stream between the library's kernels.

Prints one JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-FFN fwd tokens/s + %HBM/%MFMA roofline; speedup vs dense FFN @99% sparse"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# What the matrix cores sustain on pseudo-random bf16 operands with no memory
# traffic at all (peak_probe's register-only loop; profiles/achievable_peaks.md):
# the part lowers its clock under the power that toggling multiplier inputs
# draw, so on real data this, not the published rate, is the attainable ceiling.
ACHIEVABLE_BF16_RANDOM_TFLOPS = 1771.9
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded.

    The events are created with hipEventDisableSystemFence: they only time
    work, so recording one needs no system-scope release, whose cache
    write-back and invalidation would otherwise fall between every bracketed
    kernel and the next and add to the measured durations."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            out.append(e.value)
        return out

    def ms(self, a, b) -> float:
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(f.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# headers every kernel source includes: a change there changes the kernels too
_SHARED_HEADERS = ("tw_device.hpp", "tw_gemm.hpp", "tw_internal.hpp", "tw_split.hpp")


def _src_sha(name: str) -> str:
    """Hash of a kernel source together with the shared device headers."""
    h = hashlib.sha256()
    for part in (name, *_SHARED_HEADERS):
        with open(os.path.join(ROOT, "activation_sparse_feed_gate_amd", "csrc", part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, src: str, w, registered: dict, r_max_override=None):
    """HBM bytes per launch from committed rocprofv3 counter summaries, only
    when they were taken on the current kernel source and this workload:
    the profiles cover the registered workloads at the default backup
    capacity, so a density, batch-size or capacity override gives None."""
    if r_max_override is not None or registered.get(w.name) != w:
        return None
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)[w.name][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("src_sha") != _src_sha(src):
        return None
    return float(rec["bytes_per_launch"])


def _cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, w, budget_s: float):
    """The oracle's own TwELL forward (gate, packing, sparse evaluation with
    the dense recompute of overflow rows) on an evenly strided row sample."""
    import numpy as np

    import oracle

    orc = oracle.default()
    wg, wu, wd = (oracle.widen_bf16(d[k]) for k in ("wg_t", "wu_t", "wd"))

    def run(rows):
        xs = oracle.widen_bf16(d["x"][rows])
        t = time.perf_counter()
        z = orc.gate(xs, wg)
        p = orc.pack(z, w.T, w.C, len(rows))
        orc.sparse_ffn(xs, wg, wu, wd, w.T, w.C, p)
        return time.perf_counter() - t

    pilot = np.linspace(0, w.M - 1, min(w.M, 64)).astype(np.int64)
    per_row = run(pilot) / len(pilot)
    n = int(min(w.M, max(64, budget_s / max(per_row, 1e-9))))
    rows = np.linspace(0, w.M - 1, n).astype(np.int64)
    # whole passes over the sample until about half the budget has been spent
    # (at least one), so that a sample that is the whole batch is still timed
    # over seconds rather than a fraction of one
    secs, passes = 0.0, 0
    while passes == 0 or secs < 0.5 * budget_s:
        secs += run(rows)
        passes += 1
    # the oracle's plain dense FFN on the same rows, for the CPU's own
    # sparse-over-dense ratio (one pass, a quarter of the budget at most)
    xs = oracle.widen_bf16(d["x"][rows])
    nd = max(1, min(len(rows), int(0.25 * budget_s / max(secs / passes / len(rows) * 4, 1e-9))))
    t = time.perf_counter()
    orc.dense_ffn(xs[:nd], wg, wu, wd)
    dsecs = time.perf_counter() - t
    return {"value": passes * len(rows) / secs, "unit": "tokens/s", "cores": orc.threads(),
            "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"{len(rows)} of {w.M} token rows, evenly strided, {passes} pass(es); "
                      f"float64 gate, TwELL packing, sparse up+down with dense recompute of "
                      f"overflow rows; {secs:.1f} s",
            "dense_value": nd / dsecs,
            "dense_sample": f"oracle dense gated FFN (float64) on {nd} of those rows; "
                            f"{dsecs:.1f} s"}


def hybrid_forward_bench(args, tw, torch, w, x, wg, wu, wdn, bufs, ws, R_max, stream, hev,
                         t_dense, step):
    """The training forward over hybrid storage: gate + TwELL, TwELL ->
    hybrid (P = 128 entries per sparse row, backup room M / 8), up at the
    stored entries (keeping g and u for the backward), down to dense.
    Timed the same way as the inference step; per-kernel durations from
    eager launches with HIP events between kernels."""
    import numpy as np

    M, K, N, T, C = w.M, w.K, w.N, w.T, w.C
    P, Rh = 128, max(M // 8, 1)
    hy = tw.alloc_hybrid(M, N, P, Rh, keep=True)
    wsh = torch.empty((max(tw.tw_hybrid_down_workspace_bytes(Rh), 1),), dtype=torch.uint8,
                      device="cuda")
    yh = torch.empty((M, K), dtype=torch.float32, device="cuda")

    def hstep(ev=None, st=stream):
        # st=None: the current stream (the capture stream inside a graph capture)
        e = ev or (None, None, None, None)
        # no overflow list: the hybrid packing routes rows from the counts
        tw.tw_pack_gate(x, wg, T, C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"],
                        None, None, R_max, ws, stream=st, events=e[0])
        tw.tw_hybrid_pack(T, C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"], P, hy["hy_g"],
                          hy["hy_idx"], hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"],
                          Rh, stream=st, events=e[1])
        tw.tw_hybrid_up(x, wg, wu, P, hy["hy_g"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                        hy["bk_rows"], hy["bk_count"], Rh, hy["hy_u"], hy["hy_h"], hy["bk_g"],
                        hy["bk_u"], hy["bk_h"], stream=st, events=e[2])
        tw.tw_hybrid_down(wdn, M, P, hy["hy_h"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                          hy["bk_rows"], hy["bk_count"], Rh, hy["bk_h"], yh, wsh, stream=st,
                          events=e[3])

    for _ in range(max(args.warmup, 1)):
        hstep()
    torch.cuda.synchronize()
    bk_count = int(hy["bk_count"].cpu()[0])
    if bk_count > Rh:
        return {"skipped": f"{bk_count} backup rows exceed the room of {Rh} (M / 8): the "
                           f"caller would retry with more storage"}
    hy_cnt = hy["hy_cnt"].cpu().numpy().astype(np.int64)
    route = hy["route"].cpu().numpy().astype(bool)
    nnz_sp = int(hy_cnt[~route].sum())
    rows_sp = int((~route).sum())
    rows_sp_act = int(((hy_cnt > 0) & ~route).sum())

    Ks = args.steps
    evl = [(hev.create(3), hev.create(3), hev.create(3), hev.create(4)) for _ in range(Ks)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(Ks):
        hstep(evl[i])
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / Ks
    G = max(1, min(args.graph_steps, Ks))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for _ in range(G):
                hstep(st=None)
    torch.cuda.current_stream().wait_stream(cap)
    g.replay()
    n_rep = max(1, Ks // G)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_rep):
        g.replay()
    torch.cuda.synchronize()
    t_h = (time.perf_counter() - t0) / (n_rep * G)
    del g

    def avg(j, i):
        return sum(hev.ms(e[j][i], e[j][i + 1]) for e in evl) / len(evl) * 1e-3

    kern = {"gate_twell": avg(0, 0), "hybrid_pack": avg(1, 0),
            "route_compact": avg(1, 1), "hybrid_up": avg(2, 0), "backup_gateup": avg(2, 1),
            "backup_down": avg(3, 0), "hybrid_down": avg(3, 1)}
    for e in evl:
        for q in e:
            hev.destroy(q)
    NT = N // T
    # algorithmic bytes per launch: what each kernel must read and write
    bytes_ = {
        "hybrid_pack": M * (4 * NT + 4 + 1) + nnz_sp * 16,
        "hybrid_up": nnz_sp * (2 * K + 4 + 4 + 8) + rows_sp_act * 2 * K + M * 5,
        # (+ the backup rows of y it finishes; the split partials it reads
        # are not counted)
        "hybrid_down": nnz_sp * (2 * K + 8) + rows_sp * 4 * K + M * 5 + bk_count * 4 * K,
    }
    roof = {k: {"bound": "hbm", "achieved": b / kern[k] / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": b / kern[k] / 1e9 / PEAK_HBM_GBS, "bytes": b,
                "avg_us": kern[k] * 1e6}
            for k, b in bytes_.items() if kern[k] > 0}
    for k, f in (("backup_gateup", 4.0), ("backup_down", 2.0)):
        if kern[k] > 0:
            a = f * bk_count * K * N / kern[k] / 1e12
            roof[k] = {"bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": a / PEAK_BF16_TFLOPS, "avg_us": kern[k] * 1e6}
    storage = M * P * (4 * 4) + M * (4 + 1) + Rh * N * 2 * 3 + Rh * 4
    bwd = hybrid_backward_bench(args, tw, torch, w, x, wg, wu, wdn, hy, Rh, P, hev)
    return {
        "ms_per_step": t_h * 1e3, "value": M / t_h, "unit": "tokens/s",
        "speedup_vs_dense": t_dense / t_h, "eager_ms_per_step": t_eager * 1e3,
        "P": P, "R_max": Rh, "backup_rows": bk_count,
        "nnz_per_sparse_row": nnz_sp / max(1, rows_sp),
        "kernels_us": {k: v * 1e6 for k, v in kern.items()},
        "stages": roof,
        "storage_bytes": storage,
        "dense_activation_bytes": 3 * M * N * 2,
        "backward": bwd,
        "note": "tw_pack_gate + tw_hybrid_pack + tw_hybrid_up (g and u kept) + tw_hybrid_down; "
                "speedup against tw_ffn_fwd; storage = hybrid g, u, h (sparse rows fp32 with "
                "indices, backup rows bf16) against dense bf16 g, u, h",
    }


def hybrid_backward_bench(args, tw, torch, w, x, wg, wu, wdn, hy, Rh, P, hev):
    """Backward over the stored hybrid activations (dh with L1 injection,
    dx, transpose + weight gradients) for a seeded dy, against the same
    backward on torch.matmul (hipBLASLt) from dense bf16 g and u."""
    import numpy as np

    M, K, N = w.M, w.K, w.N
    l1 = 2e-5  # the L1 gradient on a positive activation (any value: same work)
    gen = torch.Generator(device="cuda").manual_seed(11)
    dy = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    R1 = max(Rh, 1)
    o = {"hy_du": torch.empty((M, P), dtype=torch.float32, device="cuda"),
         "hy_dz": torch.empty((M, P), dtype=torch.float32, device="cuda"),
         "bk_du": torch.empty((R1, N), dtype=torch.bfloat16, device="cuda"),
         "bk_dz": torch.empty((R1, N), dtype=torch.bfloat16, device="cuda"),
         "dx": torch.empty((M, K), dtype=torch.float32, device="cuda"),
         "dwg": torch.empty((N, K), dtype=torch.float32, device="cuda"),
         "dwu": torch.empty((N, K), dtype=torch.float32, device="cuda"),
         "dwd": torch.empty((N, K), dtype=torch.float32, device="cuda")}
    wsx = torch.empty((max(tw.tw_hybrid_bwd_dx_workspace_bytes(Rh), 1),), dtype=torch.uint8,
                      device="cuda")
    wsw = torch.empty((tw.tw_hybrid_bwd_dw_workspace_bytes(M, K, N, P, Rh),), dtype=torch.uint8,
                      device="cuda")

    def bstep(ev=None, st=torch.cuda.current_stream()):
        e = ev or (None, None, None)
        tw.tw_hybrid_bwd_dh(dy, wdn, P, l1, hy["hy_g"], hy["hy_u"], hy["hy_idx"], hy["hy_cnt"],
                            hy["route"], hy["bk_rows"], hy["bk_count"], Rh, hy["bk_g"],
                            hy["bk_u"], o["hy_du"], o["hy_dz"], o["bk_du"], o["bk_dz"], stream=st,
                            events=e[0])
        tw.tw_hybrid_bwd_dx(wg, wu, M, P, o["hy_du"], o["hy_dz"], hy["hy_idx"], hy["hy_cnt"],
                            hy["route"], hy["bk_rows"], hy["bk_count"], Rh, o["bk_du"],
                            o["bk_dz"], o["dx"], wsx, stream=st, events=e[1])
        tw.tw_hybrid_bwd_dw(x, dy, P, hy["hy_h"], o["hy_du"], o["hy_dz"], hy["hy_idx"],
                            hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"], Rh,
                            hy["bk_h"], o["bk_du"], o["bk_dz"], o["dwg"], o["dwu"],
                            o["dwd"], wsw, stream=st, events=e[2])

    # dense reference backward on hipBLASLt from dense bf16 g, u (as a dense
    # training step would keep them)
    gd = torch.relu(x @ wg.t()).to(torch.bfloat16)
    ud = (x @ wu.t()).to(torch.bfloat16)
    hd = gd * ud
    wgu_k = torch.cat([wu, wg], dim=0)  # [2N, K]: dx = [du dz] @ [W_u^T; W_g^T]

    def dense_bwd():
        dh = dy @ wdn.t()
        du = dh * gd
        dz = torch.where(gd > 0, dh * ud + l1, torch.zeros_like(dh))
        dx = torch.cat([du, dz], dim=1) @ wgu_k
        dwd = hd.t() @ dy
        dwu = du.t() @ x
        dwg = dz.t() @ x
        return dx, dwd, dwu, dwg

    for _ in range(max(args.warmup, 1)):
        bstep()
        dense_bwd()
    torch.cuda.synchronize()
    Ks = args.steps
    evl = [(hev.create(3), hev.create(3), hev.create(4)) for _ in range(Ks)]
    t0 = time.perf_counter()
    for i in range(Ks):
        bstep(evl[i])
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / Ks
    G = max(1, min(args.graph_steps, Ks))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for _ in range(G):
                bstep(st=None)
    torch.cuda.current_stream().wait_stream(cap)
    g.replay()
    n_rep = max(1, Ks // G)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_rep):
        g.replay()
    torch.cuda.synchronize()
    t_b = (time.perf_counter() - t0) / (n_rep * G)
    del g
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(Ks):
        dense_bwd()
    torch.cuda.synchronize()
    t_dense = (time.perf_counter() - t0) / Ks

    def avg(j, i):
        return sum(hev.ms(e[j][i], e[j][i + 1]) for e in evl) / len(evl) * 1e-3

    kern = {"hybrid_dh": avg(0, 0), "backup_dh": avg(0, 1), "backup_dx": avg(1, 0),
            "hybrid_dx": avg(1, 1), "transpose": avg(2, 0), "weight_grads": avg(2, 1),
            "backup_weight_grads": avg(2, 2)}
    for e in evl:
        for q in e:
            hev.destroy(q)
    return {"ms_per_step": t_b * 1e3, "eager_ms_per_step": t_eager * 1e3,
            "hipblaslt_dense_ms": t_dense * 1e3, "speedup_vs_hipblaslt_dense": t_dense / t_b,
            "kernels_us": {k: v * 1e6 for k, v in kern.items()},
            "note": "tw_hybrid_bwd_dh + tw_hybrid_bwd_dx + tw_hybrid_bwd_dw; the reference is "
                    "the same backward on torch.matmul from dense bf16 g and u"}


# Workloads measured besides the headline: every other block at >= 99%
# sparsity, the 2B shape at 0% and 5% density (the crossover), and the pages'
# own block width.
SIDE_CONFIGS = [("ffn-1b", None), ("ffn-2b", None), ("ffn-ovf", None), ("ffn-2b", 0.0),
                ("ffn-2b", 0.05), ("ffn-paper", None)]


class ClockSampler:
    """Current shader (sclk) and memory (mclk) clocks of the GPU, sampled
    from the amdgpu driver's sysfs DPM tables (the level marked '*') on a
    background thread while the timed loops run."""

    def __init__(self, torch):
        import glob
        import threading

        self.card = None
        self.why = "no amdgpu DPM clock table under /sys/class/drm"
        bus = None
        try:
            p = torch.cuda.get_device_properties(0)
            bus = "%04x:%02x:%02x" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
        except Exception:
            pass
        cards = [c for c in sorted(glob.glob("/sys/class/drm/card*/device"))
                 if os.path.exists(os.path.join(c, "pp_dpm_sclk"))]
        for c in cards:
            try:
                slot = open(os.path.join(c, "uevent")).read()
            except OSError:
                continue
            if bus and bus in slot.lower():
                self.card = c
        if self.card is None and len(cards) == 1:
            self.card = cards[0]
        if self.card is None and cards:
            self.why = f"{len(cards)} cards, none matching PCI {bus}"
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self._threading = threading

    @staticmethod
    def _level(path):
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    v = line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                    return float(v.replace("mhz", "").strip())
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append((self._level(os.path.join(self.card, "pp_dpm_sclk")),
                                     self._level(os.path.join(self.card, "pp_dpm_mclk"))))
            except (OSError, ValueError, IndexError):
                pass
            self._stop.wait(0.005)

    def __enter__(self):
        if self.card:
            self._stop.clear()
            self._thread = self._threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self):
        import numpy as np

        s = [v for v in self.samples if v[0] is not None]
        if not s:
            return {"unavailable": self.why if not self.card else "no readable samples"}
        sc = np.array([v[0] for v in s])
        mc = np.array([v[1] for v in s if v[1] is not None])
        return {"sclk_mhz_min_median_max": [float(sc.min()), float(np.median(sc)), float(sc.max())],
                "mclk_mhz_min_median_max": ([float(mc.min()), float(np.median(mc)), float(mc.max())]
                                            if len(mc) else None),
                "samples": len(s), "source": os.path.join(self.card, "pp_dpm_{sclk,mclk}"),
                "note": "DPM level marked current, sampled every ~5 ms during the timed loops; "
                        "fractions are against the published peaks, not these clocks"}


def eager_record(args, w, M, K, N, T, C, R_max, retries, t_sparse, t_dense, hev, evp, evs, evd,
                 nnz, ovf, R, sparse_nnz):
    """The record of an --eager-only run: eager step times and per-kernel
    durations (what a profiler run's averages are compared with)."""
    def avg(evl, i):
        return sum(hev.ms(e[i], e[i + 1]) for e in evl) / len(evl) * 1e-3

    def span(evl, i, j):
        return sum(hev.ms(e[i], e[j]) for e in evl) / len(evl) * 1e-3

    kern = {"gate_twell": avg(evp, 0), "ovf_compact": avg(evp, 1),
            "fallback_gateup": span(evs, 0, 1), "fallback_down": span(evs, 1, 2),
            "sparse_updown": span(evs, 2, 3), "dense_gateup": avg(evd, 0),
            "dense_down": avg(evd, 1)}
    for l in (evp, evs, evd):
        for e in l:
            hev.destroy(e)
    return {"value": M / t_sparse, "ms_per_step": t_sparse * 1e3,
            "speedup_vs_dense": t_dense / t_sparse,
            "config": {"workload": w.name, "M": M, "K": K, "N": N, "T": T, "C": C,
                       "density": w.density, "sigma_s": w.sigma_s, "seed": w.seed,
                       "R_max": R_max, "capacity_retries": retries},
            "timing": "eager launches with HIP events between kernels (--eager-only)",
            "dense": {"ms_per_step": t_dense * 1e3},
            "kernels_us": {k: v * 1e6 for k, v in kern.items()},
            "realized": {"density": float(nnz.sum()) / (M * N), "overflow_rows": R,
                         "nnz_per_sparse_row": sparse_nnz / max(1, int((~ovf).sum()))}}


def measure(args, w, torch, tw, hev, clocks, full: bool):
    """Everything measured on one workload: the step (Infinity-Cache-cold as
    the headline figure, warm graph replays beside it), the dense
    comparators, per-kernel durations and rooflines, the realized sparsity;
    with ``full`` also the fusion ablation and the hybrid training forward
    and backward.  Returns (record, inputs)."""
    import numpy as np

    from activation_sparse_feed_gate_amd import synth

    M, K, N, T, C = w.M, w.K, w.N, w.T, w.C
    # overflow capacity: the static backup capacity of the review §4-3 (an
    # eighth of the batch, rounded down: none below 8 tokens, so a decode
    # step launches no backup kernels unless it overflows); if the batch
    # overflows it, the retry rule there (read the true count on the host,
    # allocate more) runs before timing
    R_max = min(M, args.r_max) if args.r_max is not None else M // 8
    d = synth.make_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    x, wg, wu, wdn = dev(d["x"]), dev(d["wg_t"]), dev(d["wu_t"]), dev(d["wd"])
    bufs = tw.alloc_pack(M, N, T, C, R_max)
    ws = tw.workspace(M, K, N, T, C, R_max)
    y = torch.empty((M, K), dtype=torch.float32, device="cuda")
    yd = torch.empty((M, K), dtype=torch.float32, device="cuda")
    wsd = torch.empty((tw.tw_ffn_workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(evp=None, evs=None):
        tw.tw_pack_gate(x, wg, T, C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"],
                        bufs["ovf_rows"], bufs["ovf_count"], R_max, ws, stream=stream,
                        events=evp)
        tw.tw_sparse_ffn_fwd(x, wg, wu, wdn, T, C, bufs["tw_val"], bufs["tw_idx"],
                             bufs["tw_cnt"], bufs["ovf_rows"], bufs["ovf_count"], R_max, y, ws,
                             stream=stream, events=evs)

    def dense(ev=None):
        tw.tw_ffn_fwd(x, wg, wu, wdn, yd, wsd, stream=stream, events=ev)

    retries = 0
    while True:
        tw.tw_pack_gate(x, wg, T, C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"],
                        bufs["ovf_rows"], bufs["ovf_count"], R_max, ws, stream=stream)
        n_ovf = int(bufs["ovf_count"].cpu()[0])
        if n_ovf <= R_max:
            break
        R_max = min(M, max(2 * R_max, n_ovf))
        bufs = tw.alloc_pack(M, N, T, C, R_max)
        ws = tw.workspace(M, K, N, T, C, R_max)
        retries += 1

    if full and args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
        dense()
    torch.cuda.synchronize()

    # realized sparsity of this batch (deterministic; outside the timed region)
    cnt = bufs["tw_cnt"].cpu().numpy().astype(np.int64)
    ovf = (cnt > C).any(axis=1)
    nnz = cnt.sum(axis=1)
    R = int(ovf.sum())
    sparse_nnz = int(nnz[~ovf].sum())

    Ks = args.steps

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(Ks):
            fn(s_)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / Ks

    # ---- per-kernel durations: eager launches with HIP events between kernels ----
    evp = [hev.create(3) for _ in range(Ks)]
    evs = [hev.create(5) for _ in range(Ks)]
    evd = [hev.create(3) for _ in range(Ks)]
    t_sparse_eager = timed(lambda i: step(evp[i], evs[i]))
    t_dense_eager = timed(lambda i: dense(evd[i]))

    if args.eager_only:
        return eager_record(args, w, M, K, N, T, C, R_max, retries, t_sparse_eager,
                            t_dense_eager, hev, evp, evs, evd, nnz, ovf, R, sparse_nnz), d

    # ---- G consecutive steps of each path captured in one HIP graph (as a
    # model forward would chain its layers) ----
    G = max(1, min(args.graph_steps, Ks))
    sizes = [G] * (Ks // G) + ([Ks % G] if Ks % G else [])
    step_cap = lambda: (tw.tw_pack_gate(x, wg, T, C, bufs["tw_val"], bufs["tw_idx"],
                                        bufs["tw_cnt"], bufs["ovf_rows"],
                                        bufs["ovf_count"], R_max, ws),
                        tw.tw_sparse_ffn_fwd(x, wg, wu, wdn, T, C, bufs["tw_val"],
                                             bufs["tw_idx"], bufs["tw_cnt"],
                                             bufs["ovf_rows"], bufs["ovf_count"], R_max,
                                             y, ws))
    dense_cap = lambda: tw.tw_ffn_fwd(x, wg, wu, wdn, yd, wsd)
    graphs = {}
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for n in set(sizes):
            gs, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs, stream=cap):
                for _ in range(n):
                    step_cap()
            with torch.cuda.graph(gd, stream=cap):
                for _ in range(n):
                    dense_cap()
            graphs[n] = (gs, gd)
    torch.cuda.current_stream().wait_stream(cap)
    for n in graphs:
        graphs[n][0].replay()
        graphs[n][1].replay()

    def timed_graphs(which):
        """Warm steps: mean step time over the Ks steps (host clock around the
        whole loop), and per-replay step times from events between replays."""
        evs_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in sizes]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for (a, b), n in zip(evs_, sizes):
            a.record()
            graphs[n][which].replay()
            b.record()
        torch.cuda.synchronize()
        mean = (time.perf_counter() - t0) / Ks
        per = [a.elapsed_time(b) * 1e-3 / n for (a, b), n in zip(evs_, sizes)]
        return mean, per

    # ---- Infinity-Cache-cold steps (the headline): an in-place pass over
    # 512 MB (twice the 256 MB cache) before each step evicts the weights, as
    # in a deep model where the other layers' weights pass through the cache
    # between two uses of this one.  Exactly Ks steps of each path run, one
    # per graph replay; step time = (pass + step) - pass, each the median of
    # Ks replays. ----
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    gf, gfs, gfd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gf, stream=cap):
            flush.add_(1)
        with torch.cuda.graph(gfs, stream=cap):
            flush.add_(1)
            step_cap()
        with torch.cuda.graph(gfd, stream=cap):
            flush.add_(1)
            dense_cap()
    torch.cuda.current_stream().wait_stream(cap)

    def replays(g):
        ts = []
        for _ in range(Ks):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return np.array(ts)

    for g in (gf, gfs, gfd):
        g.replay()
    torch.cuda.synchronize()
    with clocks:
        t_sparse, per_sparse = timed_graphs(0)
        t_dense, per_dense = timed_graphs(1)
        f_ts = replays(gf)
        cs_ts = replays(gfs)
        cd_ts = replays(gfd)
    t_f = float(np.median(f_ts))
    per_cold = cs_ts - t_f
    t_cs = float(np.median(cs_ts)) - t_f
    t_cd = float(np.median(cd_ts)) - t_f
    del flush, gf, gfs, gfd

    # ---- the fusion the method turns on: packing in the gate's epilogue
    # (tw_pack_gate) against the unfused path that writes the dense gate and
    # packs it in a separate pass (tw_gate_dense + tw_pack_dense) ----
    fusion = None
    if full and args.fusion_ablation:
        zbuf = torch.empty((M, N), dtype=torch.float32, device="cuda")
        wsp = torch.empty((tw.tw_pack_dense_workspace_bytes(M, N),), dtype=torch.uint8,
                          device="cuda")
        bu = tw.alloc_pack(M, N, T, C, R_max)
        fused_cap = lambda: tw.tw_pack_gate(x, wg, T, C, bufs["tw_val"], bufs["tw_idx"],
                                            bufs["tw_cnt"], bufs["ovf_rows"],
                                            bufs["ovf_count"], R_max, ws)
        unfused_cap = lambda: (tw.tw_gate_dense(x, wg, zbuf),
                               tw.tw_pack_dense(zbuf, T, C, bu["tw_val"], bu["tw_idx"],
                                                bu["tw_cnt"], bu["ovf_rows"],
                                                bu["ovf_count"], R_max, wsp))
        ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(ga, stream=cap):
                for _ in range(G):
                    fused_cap()
            with torch.cuda.graph(gb, stream=cap):
                for _ in range(G):
                    unfused_cap()
        torch.cuda.current_stream().wait_stream(cap)

        def per_call(g):
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(max(1, Ks // G)):
                g.replay()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) / (max(1, Ks // G) * G)

        t_fu, t_un = per_call(ga), per_call(gb)
        fusion = {"fused_pack_us": t_fu * 1e6, "unfused_pack_us": t_un * 1e6,
                  "unfused_over_fused": t_un / t_fu,
                  "dense_gate_bytes": M * N * 4,
                  "note": "tw_pack_gate vs tw_gate_dense + tw_pack_dense (dense fp32 gate "
                          "written, read back and packed), HIP graphs, same outputs"}
        del zbuf, ga, gb
    del graphs

    hybrid = hybrid_forward_bench(args, tw, torch, w, x, wg, wu, wdn, bufs, ws, R_max, stream,
                                  hev, t_dense, step) if (full and args.hybrid) else None

    # ---- the same dense FFN on torch.matmul (hipBLASLt) ----
    wgu = torch.cat([wg, wu], dim=0)
    wd_row = wdn  # [N, K]: y = h @ W_d

    def blas_ffn():
        gu = x @ wgu.t()
        h = (torch.relu(gu[:, :N]) * gu[:, N:]).to(torch.bfloat16)
        return h @ wd_row

    for _ in range(3):
        blas_ffn()
    t_blas = timed(lambda i: blas_ffn())
    # the two bare hipBLASLt products alone (no ReLU product, no bf16
    # rounding of h in between): a lower bound for any dense FFN built on
    # them; the down product reads this batch's own h (as sparse as ours)
    h_bl = (torch.relu(x @ wg.t()) * (x @ wu.t())).to(torch.bfloat16)

    def blas_gemms():
        x @ wgu.t()
        h_bl @ wd_row

    for _ in range(3):
        blas_gemms()
    t_blas_bare = timed(lambda i: blas_gemms())
    del wgu, h_bl

    def avg(evl, i):
        return sum(hev.ms(e[i], e[i + 1]) for e in evl) / len(evl) * 1e-3  # seconds

    def span(evl, i, j):
        return sum(hev.ms(e[i], e[j]) for e in evl) / len(evl) * 1e-3

    # the overflow path runs first; the sparse kernel follows on the same
    # stream and also sums the overflow rows' split partials
    kern = {
        "gate_twell": avg(evp, 0),
        "ovf_compact": avg(evp, 1),
        "fallback_gateup": span(evs, 0, 1),
        "fallback_down": span(evs, 1, 2),
        "sparse_updown": span(evs, 2, 3),
    }
    kern_dense = {"dense_gateup": avg(evd, 0), "dense_down": avg(evd, 1)}
    for l in (evp, evs, evd):
        for e in l:
            hev.destroy(e)

    NT = N // T
    # per non-overflow row: its entries (two weight rows, index and value),
    # x, the y row and the counts; per overflow row: the counts and the y row
    # it finishes (the split partials it reads are not counted)
    sparse_bytes = (sparse_nnz * (4 * K + 8) + int((~ovf).sum()) * (2 * K + 4 * K + 4 * NT)
                    + R * (4 * NT + 4 * K))
    work = {  # algorithmic work per launch: (amount, bound)
        "gate_twell": (2.0 * M * K * N, "mfma"),
        "sparse_updown": (float(sparse_bytes), "hbm"),
        "fallback_gateup": (4.0 * R * K * N, "mfma"),
        "fallback_down": (2.0 * R * K * N, "mfma"),
        "dense_gateup": (4.0 * M * K * N, "mfma"),
        "dense_down": (2.0 * M * K * N, "mfma"),
    }
    srcs = {"gate_twell": "gate_twell.hip", "sparse_updown": "sparse_updown.hip",
            "fallback_gateup": "dense_ffn.hip", "fallback_down": "dense_ffn.hip",
            "dense_gateup": "dense_ffn.hip", "dense_down": "dense_ffn.hip"}

    def roof(name, secs):
        amount, bound = work[name]
        if bound == "mfma":
            a = amount / secs / 1e12
            r = {"bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": a / PEAK_BF16_TFLOPS,
                 "frac_of_random_operand_peak": a / ACHIEVABLE_BF16_RANDOM_TFLOPS}
        else:
            a = amount / secs / 1e9
            r = {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": a / PEAK_HBM_GBS}
        r["kernel"] = name
        r["avg_us"] = secs * 1e6
        r["traffic"] = _traffic(name, srcs[name], w, synth.WORKLOADS, args.r_max)
        if r["traffic"] is not None:
            # the bytes the counters saw leave or enter HBM, per launch, over
            # the same duration: measured DRAM throughput beside the
            # algorithmic figure
            r["counter_GBs"] = r["traffic"] / secs / 1e9
            r["counter_frac"] = r["counter_GBs"] / PEAK_HBM_GBS
        return r

    path_kernels = ["gate_twell", "sparse_updown", "fallback_gateup", "fallback_down"]
    dominant = max(path_kernels, key=lambda k: kern[k])
    stages = {k: roof(k, kern[k]) for k in path_kernels if kern[k] > 0}
    stages.update({k: roof(k, v) for k, v in kern_dense.items()})
    pct = lambda a: [float(np.percentile(a, q)) * 1e3 for q in (10, 50, 90)]
    best_dense = min(t_cd, t_blas)
    rec = {
        "value": M / t_cs,
        "ms_per_step": t_cs * 1e3,
        "ms_per_step_p10_p50_p90": pct(per_cold),
        "speedup_vs_dense": t_cd / t_cs,
        "speedup_vs_best_dense": best_dense / t_cs,
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "T": T, "C": C,
                   "density": w.density, "sigma_s": w.sigma_s, "seed": w.seed, "R_max": R_max,
                   "capacity_retries": retries},
        "roofline": roof(dominant, kern[dominant]),
        "cache": ("Infinity-Cache-cold: each step follows a 512 MB in-place pass; step time = "
                  f"median of {Ks} replays of (pass + step) minus the median pass "
                  f"({t_f * 1e3:.3f} ms)"),
        "dense": {"ms_per_step": t_cd * 1e3, "value": M / t_cd, "cache": "cold",
                  "kernel": "tw_ffn_fwd (our MFMA dense gated FFN)"},
        "warm": {"ms_per_step": t_sparse * 1e3, "value": M / t_sparse,
                 "ms_per_step_p10_p50_p90": pct(per_sparse),
                 "dense_ms_per_step": t_dense * 1e3,
                 "dense_ms_per_step_p10_p50_p90": pct(per_dense),
                 "speedup_vs_dense": t_dense / t_sparse,
                 "timing": f"HIP graphs of {G} consecutive steps, replayed to run {Ks} steps, "
                           f"back to back (weights stay in the Infinity Cache)"},
        "eager": {"sparse_ms_per_step": t_sparse_eager * 1e3,
                  "dense_ms_per_step": t_dense_eager * 1e3},
        "hipblaslt_dense": {"ms_per_step": t_blas * 1e3,
                            "speedup_vs": t_blas / t_cs,
                            "note": "torch.matmul gate+up GEMM, ReLU*u in torch, bf16 h, "
                                    "torch.matmul down, back to back (warm)"},
        "hipblaslt_bare_gemms": {"ms_per_step": t_blas_bare * 1e3,
                                 "speedup_vs_cold_step": t_blas_bare / t_cs,
                                 "speedup_vs_warm_step": t_blas_bare / t_sparse,
                                 "note": "the gate+up and down torch.matmul products alone, "
                                         "back to back (warm): a lower bound for a dense FFN "
                                         "on hipBLASLt, not a complete FFN"},
        "kernels_us": {k: v * 1e6 for k, v in {**kern, **kern_dense}.items()},
        "stages": stages,
        "realized": {"density": float(nnz.sum()) / (M * N), "overflow_rows": R,
                     "nnz_per_sparse_row": sparse_nnz / max(1, int((~ovf).sum())),
                     "max_nnz_sparse_row": int(nnz[~ovf].max(initial=0)),
                     # active neurons per token over all rows (the true counts,
                     # overflow rows included): the tail the capacities face
                     "nnz_per_row_mean_p50_p95_p99_max": [
                         float(nnz.mean()) if M else 0.0,
                         *[float(np.percentile(nnz, q)) if M else 0.0 for q in (50, 95, 99)],
                         int(nnz.max(initial=0))]},
    }
    if full:
        rec["fusion"] = fusion
        rec["hybrid_training_forward"] = hybrid
    del x, wg, wu, wdn, bufs, ws, y, yd, wsd
    return rec, d


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ffn-0.5b")
    ap.add_argument("--density", type=float, default=None, help="override the target density")
    ap.add_argument("--M", type=int, default=None,
                    help="override the token count (decode-like batches)")
    ap.add_argument("--r-max", type=int, default=None,
                    help="overflow-row capacity (default: an eighth of the batch, grown by "
                         "the retry rule before timing)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run a plain elementwise copy of MB megabytes (fp32, read + "
                         "write) so that a counter profile can scale FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--no-fusion-ablation", dest="fusion_ablation", action="store_false",
                    help="skip timing the unfused gate + pack path")
    ap.add_argument("--no-hybrid", dest="hybrid", action="store_false",
                    help="skip the hybrid training-forward measurement")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="measure the headline workload only (not the other blocks)")
    ap.add_argument("--eager-only", action="store_true",
                    help="time only the eager launches whose per-kernel durations the roofline "
                         "uses (for profiler runs: no graph replays, cache-cold steps or "
                         "comparison lines); implies --no-configs")
    ap.add_argument("--graph-steps", type=int, default=5,
                    help="consecutive steps captured in one HIP graph for the warm line "
                         "(1: a graph launch per step)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the path is data-parallel over tokens with no exchange, so N GPUs "
              f"run N independent copies; no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import torch

    from activation_sparse_feed_gate_amd import synth, tw

    w = synth.WORKLOADS[args.workload]
    if args.density is not None:
        w = w.with_(density=args.density)
    if args.M is not None:
        w = w.with_(M=args.M)
    hev = HipEvents()
    clocks = ClockSampler(torch)
    rec, d = measure(args, w, torch, tw, hev, clocks, full=True)
    head = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    out = {**head, **rec}
    configs = {}
    if (args.configs and not args.eager_only and args.M is None and args.density is None
            and args.workload == "ffn-0.5b"):
        for name, dens in SIDE_CONFIGS:
            wc = synth.WORKLOADS[name] if dens is None else \
                synth.WORKLOADS[name].with_(density=dens)
            key = name if dens is None else f"{name}@{dens:g}"
            rc, _ = measure(args, wc, torch, tw, hev, clocks, full=False)
            configs[key] = rc
            torch.cuda.empty_cache()
    out["configs"] = configs or None
    out["clocks"] = clocks.summary()
    out["device"] = torch.cuda.get_device_properties(0).name
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, w, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
