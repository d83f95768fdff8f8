#!/usr/bin/env python3
"""Benchmark: potrf + logdet + potrs throughput on one MI355X.

One step = the whole solve path on one synthetic input: Cholesky
factorization of A (in place), log det from the factor, and the blocked
forward/back substitution of B (in place), by default as one spd_posv call
(which overlaps the forward substitution with the factorization; --separate
times spd_potrf, spd_logdet and spd_potrs instead).  Inputs are generated once, with
a pristine copy kept in HBM; before every step A and B are restored from it
by a device-to-device copy that is outside the step's timed events.

Default workload: fp64 SPD solve, N = 32768, N_RHS = 128, T_A = 512,
A = G G^T / N + 0.05 I (G iid N(0,1), seeded), B iid N(0,1).

TFLOP/s = (N^3/3 + 2 N^2 N_RHS) / step time (x4 for complex: real-equivalent).

With --workload gp a step is instead the factorization plus the Gaussian-
process marginal log-likelihood of the N_RHS columns of B taken as residuals
(forward substitution and a per-column reduction);
TFLOP/s = (N^3/3 + N^2 N_RHS) / step time.

With --workload sygst a step is the factorization B = L L^H (B the
config's SPD matrix) plus the reduction of the generalized eigenproblem
A v = w B v (--itype 1; 2 and 3 for A B v = w v, B A v = w v) to standard
form, A symmetric indefinite (G + G^T)/sqrt(2N); TFLOP/s = (N^3/3 + N^3) /
step time, N^3 being the reduction's conventional flop count; the roofline is
that of the trailing-update kernel in its rank-2k form, which carries the
bulk of the reduction's flops.

Printed: one JSON line with the metric, the roofline of the dominant kernel
(the trailing update A22 -= L21 L21^H, timed live with HIP events around each
launch on its stream) and the CPU oracle timed on a bounded sample of the same
workload (its leading principal block).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {  # MI355X published dense peaks, TFLOP/s
    "f64": 78.6,
    "c128": 78.6,
    "f32": 157.3,
    "c64": 157.3,
}
HBM_PEAK_GBS = 8000.0
# HBM bytes per trailing-update launch on the caller's stream at the default
# workload (fp64 N=32768, T_A=512), from FETCH_SIZE and WRITE_SIZE counter
# passes scaled by a plain copy's reading
# (profiles/counters_syrk_f64_n32768_t512.md).  Valid for the trailing-update
# kernels and schedule as they were when the counters were taken; emptied when
# they change.
SYRK_TRAFFIC_BYTES = {("f64", 32768, 512, "posv"): 9.214e9}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", type=int, default=5, help="workload 1..5 (default 5: fp64 N=32768)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the backward-error check of the last step")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only copy 1 GiB device to device (twice), for scaling HBM byte counters")
    p.add_argument("--workload", choices=("solve", "gp", "sygst"), default="solve",
                   help="solve (default): potrf + logdet + potrs; gp: potrf + the Gaussian-process marginal "
                        "log-likelihood of the N_RHS residual columns (forward substitution + reduction); "
                        "sygst: potrf of B + reduction of the generalized eigenproblem (A, B) to standard form")
    p.add_argument("--itype", type=int, choices=(1, 2, 3), default=1, help="problem type of --workload sygst")
    p.add_argument("--no-phases", action="store_true",
                   help="skip the three-call loop that gives potrf's own rate and the phase times")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other workloads (1-4 and complex64 N=8192) reported beside workload 5")
    p.add_argument("--separate", action="store_true",
                   help="solve workload: time spd_potrf, spd_logdet and spd_potrs as three calls instead of the "
                        "one-call spd_posv")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "requested_gpus": args.gpus}), flush=True)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read and 1 GiB written per copy
        nbytes = 1 << 30
        src = torch.ones(nbytes // 8, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        print(json.dumps({"copy_bytes": nbytes, "ms": ms, "read_plus_write_GBs": 2 * nbytes / ms / 1e6}), flush=True)
        return 0

    import cholesky_spd_solve_amd as spd
    import spdgen

    spd.load()
    cfg = dict(spdgen.CONFIGS[args.config])
    dt, n, nrhs, T = cfg["dtype"], cfg["n"], cfg["nrhs"], cfg["T_A"]
    cplx = dt in ("c64", "c128")
    fmul = 4.0 if cplx else 1.0
    gp = args.workload == "gp"
    if gp and cplx:
        print(json.dumps({"error": "the Gaussian-process likelihood is defined for real types"}), flush=True)
        return 2
    if args.workload == "sygst":
        return bench_sygst(args, cfg)
    flops_potrf = fmul * n**3 / 3.0
    flops_potrs = fmul * (1.0 if gp else 2.0) * n * n * nrhs  # gp: forward substitution only
    flops = flops_potrf + flops_potrs

    t0 = time.time()
    log(f"[bench] generating config {args.config}: {dt} N={n} N_RHS={nrhs} T_A={T} seed={args.seed}")
    A0, B0, _ = spdgen.make_config(args.config, args.seed, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    bufs = SolveBuffers(spd, A0, B0, T)
    peak = PEAK[dt]

    mode = "gp" if gp else "three" if args.separate else "posv"
    three = None
    if mode == "posv" and not args.no_phases:
        # the three calls on the same inputs, for the factorization's own rate
        # and the per-phase times (timed before the headline loop, whose
        # output the check below reads)
        three = solve_loop(spd, bufs, cfg, "three", args.steps, min(args.warmup, 2), False, "three calls")
    r = solve_loop(spd, bufs, cfg, mode, args.steps, args.warmup, True, mode)
    ms = float(np.mean(r["step_ms"]))
    status = r["info"]
    A, B = bufs.A, bufs.B

    check = None
    if not args.no_check and gp:
        # normwise backward error of the forward substitution L Y = R, with the
        # computed factor, in double on the GPU
        Lw = torch.tril(A).to(torch.float64)
        Yw, Rw = B.to(torch.float64), B0.to(torch.float64)
        rr = Rw - Lw @ Yw
        eta = (rr.abs().amax(dim=0) / (Lw.abs().sum(dim=1).max() * Yw.abs().amax(dim=0) + Rw.abs().amax(dim=0))).max()
        eps = 2.0**-52 if dt == "f64" else 2.0**-23
        gpout = bufs.gpout
        finite = bool(torch.isfinite(gpout).all().item())
        check = {"forward_backward_error": float(eta.item()), "bound_64_n_eps": 64 * n * eps,
                 "loglik_first": float(gpout[0].item()), "ok": bool(eta.item() <= 64 * n * eps and status == 0
                                                                   and finite)}
        del Lw, Yw, Rw, rr
        log(f"[bench] forward-substitution backward error {check['forward_backward_error']:.3e} "
            f"(bound {check['bound_64_n_eps']:.3e}); loglik[0] = {check['loglik_first']:.6f}")
    elif not args.no_check:
        check = backward_check(A0, B, B0, dt, n, status)
        log(f"[bench] backward error {check['backward_error']:.3e} (bound {check['bound_64_n_eps']:.3e})")

    value = flops / (ms * 1e-3) / 1e12
    phases = three if three is not None else r if mode != "posv" else None
    potrf_tf = None
    phase_ms = {"posv": ms} if mode == "posv" else {}
    if phases is not None:
        potrf_ms = float(np.mean(phases["potrf_ms"]))
        potrf_tf = flops_potrf / (potrf_ms * 1e-3) / 1e12
        phase_ms.update({"potrf": potrf_ms, "logdet": float(np.mean(phases["logdet_ms"])),
                         ("gp_loglik" if gp else "potrs"): float(np.mean(phases["potrs_ms"])),
                         "three_calls": float(np.mean(phases["step_ms"]))})
    syrk_ms, syrk_launches, syrk_flops = r["syrk"]
    aux_ms, aux_launches, aux_flops = r["aux"]
    syrk_avg_ms = syrk_ms / max(syrk_launches, 1)
    syrk_achieved = (syrk_flops / syrk_launches) / (syrk_avg_ms * 1e-3) / 1e12 if syrk_launches else None
    aux_avg_ms = aux_ms / max(aux_launches, 1)
    roofline = {
        "kernel": "syrk_kernel (trailing update A22 -= L21 L21^H, lower tiles; launches on the caller's stream)",
        "bound": "mfma",
        "achieved": syrk_achieved,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": (syrk_achieved / peak) if syrk_achieved else None,
        "traffic": SYRK_TRAFFIC_BYTES.get((dt, n, T, mode)) if not gp else None,
        "launches": syrk_launches,
        "avg_launch_ms": syrk_avg_ms,
        "flops_per_launch": syrk_flops / max(syrk_launches, 1),
        # the same kernel's launches on the factorization's auxiliary stream
        # (the next tile columns), timed while they share the GPU
        "aux_stream": {"launches": aux_launches, "avg_launch_ms": aux_avg_ms,
                       "flops_per_launch": aux_flops / max(aux_launches, 1),
                       "achieved": (aux_flops / aux_launches) / (aux_avg_ms * 1e-3) / 1e12 if aux_launches else None,
                       "flop_share": aux_flops / max(aux_flops + syrk_flops, 1.0)},
    }

    if mode == "posv" and not args.no_phases:
        # the same trailing-update kernel with nothing beside it: the
        # sequential schedule (every launch in order on the caller's stream),
        # its launches timed by the same events
        with spd.options({spd.OPT_LOOKAHEAD: 0}):
            seq = solve_loop(spd, bufs, cfg, "three", 2, 1, True, "sequential schedule")
        s_ms, s_launches, s_flops = seq["syrk"]
        s_avg = s_ms / max(s_launches, 1)
        s_ach = (s_flops / s_launches) / (s_avg * 1e-3) / 1e12 if s_launches else None
        roofline["alone"] = {"schedule": "sequential (SPD_OPT_LOOKAHEAD = 0): no launch shares the GPU",
                             "achieved": s_ach, "frac": (s_ach / peak) if s_ach else None, "launches": s_launches,
                             "avg_launch_ms": s_avg, "potrf_ms": float(np.mean(seq["potrf_ms"]))}

    others = None
    if not gp and args.config == 5 and not args.no_configs:
        del bufs, A, B
        torch.cuda.empty_cache()
        others = other_configs(spd, args, cpu=not args.no_cpu_baseline)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A0, B0, n, nrhs, fmul, args.cpu_seconds, gp)

    dname = {"f64": "fp64", "f32": "fp32", "c128": "complex128", "c64": "complex64"}[dt]
    metric = (f"GP marginal log-likelihood (potrf + forward substitution) TFLOP/s, {dname} N={n}, 1 MI355X" if gp
              else f"potrf+potrs TFLOP/s and % of MFMA peak, {dname} N={n}, 1 MI355X")
    workload = (f"{dt} Gaussian-process log-likelihood N={n}, {nrhs} residual columns, T_A={T}, "
                f"A = G G^H/N + {cfg['delta']} I, seed {args.seed}" if gp else
                f"{dt} SPD solve N={n} N_RHS={nrhs} T_A={T}, A = G G^H/N + {cfg['delta']} I, seed {args.seed}")
    out = {
        "metric": metric,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": workload, "n": n, "n_rhs": nrhs, "T_A": T, "logdet": cfg["logdet"] or gp},
        "pct_of_peak": 100.0 * value / peak,
        "potrf_tflops": potrf_tf,
        "potrf_pct_of_peak": None if potrf_tf is None else 100.0 * potrf_tf / peak,
        "entry_points": ("spd_posv (potrf + logdet + potrs in one call); phases from spd_potrf, spd_logdet, "
                         "spd_potrs timed on the same inputs" if mode == "posv" else
                         "spd_potrf, spd_gp_loglik" if gp else "spd_potrf, spd_logdet, spd_potrs"),
        "phase_ms": phase_ms,
        "wall_ms_per_step_incl_restore": r["wall_ms"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "configs": others,
        "check": check,
    }
    print(json.dumps(out), flush=True)
    ok = check is None or check["ok"]
    if others is not None:
        ok = ok and all(v.get("check_ok", True) for v in others.values())
    return 0 if ok else 1


class SolveBuffers:
    """Working copies of A and B (restored from the pristine A0, B0 before
    every step, outside the timed events), the workspace and small outputs."""

    def __init__(self, spd, A0, B0, T):
        import torch
        import spdgen
        n, nrhs = B0.shape
        self.A0, self.B0 = A0, B0
        self.A = spdgen.to_colmajor(A0)
        self.B = spdgen.to_colmajor(B0)
        self.work = spd.workspace(self.A.dtype, n, nrhs, T)
        self.info = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ldbuf = torch.zeros(1, dtype=torch.float64, device="cuda")
        self.gpout = torch.zeros(nrhs, dtype=torch.float64, device="cuda")

    def restore(self):
        self.A.copy_(self.A0)
        self.B.copy_(self.B0)


def solve_loop(spd, bufs, cfg, mode, steps, warmup, profile, tag):
    """Warm up, then time ``steps`` steps of ``mode``: "posv" (one call),
    "three" (spd_potrf, spd_logdet, spd_potrs) or "gp" (spd_potrf,
    spd_gp_loglik).  Each step is bracketed by HIP events on the caller's
    stream, with the phase boundaries of the multi-call modes; with
    ``profile`` the trailing-update launches are timed by the library's own
    events on the streams they run on."""
    import numpy as np
    import torch

    T = cfg["T_A"]
    stream = torch.cuda.current_stream()
    A, B = bufs.A, bufs.B
    want_ld = cfg["logdet"]

    def step(ev):
        ev[0].record(stream)
        if mode == "posv":
            spd.posv(A, B, T, info=bufs.info, logdet_out=bufs.ldbuf if want_ld else None, work=bufs.work)
            for e in ev[1:]:
                e.record(stream)
            return
        spd.potrf(A, T, info=bufs.info, work=bufs.work)
        ev[1].record(stream)
        if want_ld and mode != "gp":
            spd.logdet(A, bufs.info, out=bufs.ldbuf)
        ev[2].record(stream)
        if mode == "gp":
            spd.gp_loglik(A, B, T, info=bufs.info, work=bufs.work, out=bufs.gpout)
        else:
            spd.potrs(A, B, T, info=bufs.info, work=bufs.work)
        ev[3].record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    for w in range(warmup):
        bufs.restore()
        step(events())
        torch.cuda.synchronize()
        log(f"[bench] {tag}: warmup {w + 1}/{warmup} done")
    if profile:
        spd.profile_enable((1 << spd.PROF_SYRK) | (1 << spd.PROF_SYRK_AUX))
        spd.profile_read(spd.PROF_SYRK)
        spd.profile_read(spd.PROF_SYRK_AUX)
    evs = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(steps):
        bufs.restore()
        ev = events()
        step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    syrk = aux = (0.0, 0, 0.0)
    if profile:
        spd.profile_enable(0)
        syrk = spd.profile_read(spd.PROF_SYRK)
        aux = spd.profile_read(spd.PROF_SYRK_AUX)
    out = {
        "step_ms": [e[0].elapsed_time(e[3]) for e in evs],
        "potrf_ms": [e[0].elapsed_time(e[1]) for e in evs],
        "logdet_ms": [e[1].elapsed_time(e[2]) for e in evs],
        "potrs_ms": [e[2].elapsed_time(e[3]) for e in evs],
        "wall_ms": 1e3 * wall / max(steps, 1),
        "syrk": syrk,
        "aux": aux,
        "info": int(bufs.info.item()),
    }
    log(f"[bench] {tag}: steps {', '.join(f'{x:.2f}' for x in out['step_ms'])} ms; "
        f"mean {np.mean(out['step_ms']):.3f} ms; info={out['info']}")
    return out


def backward_check(A0, X, B0, dt, n, status):
    """Normwise backward error of X (residual in double on the GPU)."""
    import torch
    wd = torch.complex128 if A0.is_complex() else torch.float64
    Aw, Xw, Bw = A0.to(wd), X.to(wd), B0.to(wd)
    rr = Bw - Aw @ Xw
    eta = (rr.abs().amax(dim=0) / (Aw.abs().sum(dim=1).max() * Xw.abs().amax(dim=0) + Bw.abs().amax(dim=0))).max()
    eps = 2.0**-52 if dt in ("f64", "c128") else 2.0**-23
    return {"backward_error": float(eta.item()), "bound_64_n_eps": 64 * n * eps,
            "ok": bool(eta.item() <= 64 * n * eps and status == 0)}


# The other workloads reported beside the headline one: the four smaller
# benchmark configurations, and complex64 at the complex128 workload's shape.
EXTRA_WORKLOADS = {"c64_n8192": dict(dtype="c64", n=8192, nrhs=32, T_A=256, delta=0.5, logdet=True)}


def other_configs(spd, args, cpu):
    """ms per solve (one call and three calls), TFLOP/s and % of the matrix
    peak for workloads 1-4 and complex64 N = 8192, each on its own inputs,
    plus, for the fp32 workload, the single-precision oracle on a bounded
    sample as its own-precision CPU baseline."""
    import numpy as np
    import torch

    import spdgen

    out = {}
    items = [(str(k), dict(spdgen.CONFIGS[k]), k) for k in (1, 2, 3, 4)]
    items += [(name, dict(c), None) for name, c in EXTRA_WORKLOADS.items()]
    for name, c, k in items:
        dt, n, nrhs, T = c["dtype"], c["n"], c["nrhs"], c["T_A"]
        fmul = 4.0 if dt in ("c64", "c128") else 1.0
        t0 = time.time()
        if k is not None:
            A0, B0, _ = spdgen.make_config(k, args.seed, device="cuda")
        else:
            A0 = spdgen.make_A(n, dt, c["delta"], args.seed, device="cuda")
            B0 = spdgen.make_B(n, nrhs, dt, args.seed, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] workload {name}: {dt} N={n} N_RHS={nrhs} T_A={T}, inputs in {time.time() - t0:.1f} s")
        bufs = SolveBuffers(spd, A0, B0, T)
        steps = max(args.steps, 10)
        three = solve_loop(spd, bufs, c, "three", steps, 2, False, f"{name} three calls")
        one = solve_loop(spd, bufs, c, "posv", steps, 2, False, f"{name} posv")
        chk = backward_check(A0, bufs.B, B0, dt, n, one["info"])
        flops_potrf = fmul * n**3 / 3.0
        flops = flops_potrf + fmul * 2.0 * n * n * nrhs
        ms = float(np.mean(one["step_ms"]))
        potrf_ms = float(np.mean(three["potrf_ms"]))
        peak = PEAK[dt]
        rec = {"workload": f"{dt} N={n} N_RHS={nrhs} T_A={T} delta={c['delta']}" + ("" if k else " (extra)"),
               "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "pct_of_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / peak,
               "peak": peak, "three_calls_ms": float(np.mean(three["step_ms"])), "potrf_ms": potrf_ms,
               "potrf_tflops": flops_potrf / (potrf_ms * 1e-3) / 1e12,
               "potrf_pct_of_peak": 100.0 * flops_potrf / (potrf_ms * 1e-3) / 1e12 / peak,
               "logdet_ms": float(np.mean(three["logdet_ms"])), "potrs_ms": float(np.mean(three["potrs_ms"])),
               "backward_error": chk["backward_error"], "check_ok": chk["ok"]}
        if cpu and dt == "f32":
            rec["cpu_baseline"] = cpu_baseline(A0, B0, n, nrhs, fmul, args.cpu_seconds / 2, single=True)
        out[name] = rec
        del bufs, A0, B0
        torch.cuda.empty_cache()
    return out


def bench_sygst(args, cfg):
    """potrf of B, then the reduction of (A, B) to standard form."""
    import numpy as np
    import torch

    import cholesky_spd_solve_amd as spd
    import spdgen

    dt, n, T, itype = cfg["dtype"], cfg["n"], cfg["T_A"], args.itype
    cplx = dt in ("c64", "c128")
    fmul = 4.0 if cplx else 1.0
    flops_potrf = fmul * n**3 / 3.0
    flops_gst = fmul * float(n) ** 3
    t0 = time.time()
    log(f"[bench] generating sygst itype {itype}: {dt} N={n} T_A={T} seed={args.seed}")
    B0 = spdgen.make_A(n, dt, cfg["delta"], args.seed, device="cuda")
    H0 = spdgen.make_herm(n, dt, args.seed + 1, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    Lb = spdgen.to_colmajor(B0)
    H = spdgen.to_colmajor(H0)
    work = spd.workspace(Lb.dtype, n, 0, T)
    gbytes = spd.sygst_workspace_size(H.dtype, itype, n, T)
    gwork = torch.empty(max(gbytes, 1), dtype=torch.uint8, device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def restore():
        Lb.copy_(B0)
        H.copy_(H0)

    def step(ev):
        ev[0].record(stream)
        spd.potrf(Lb, T, info=info, work=work)
        ev[1].record(stream)
        spd.sygst(itype, H, Lb, T, info=info, work=gwork)
        ev[2].record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    for w in range(args.warmup):
        restore()
        step(events())
        torch.cuda.synchronize()
        log(f"[bench] warmup {w + 1}/{args.warmup} done")
    cls = spd.PROF_SYRK  # the rank-2k (and, for itypes 2 and 3, rank-n) products
    spd.profile_enable(1 << cls)
    spd.profile_read(cls)
    evs = []
    torch.cuda.synchronize()
    for k in range(args.steps):
        restore()
        ev = events()
        step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    spd.profile_enable(0)
    k_ms, k_launches, k_flops = spd.profile_read(cls)
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    potrf_ms = [e[0].elapsed_time(e[1]) for e in evs]
    gst_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms = float(np.mean(step_ms))
    status = int(info.item())
    log(f"[bench] steps: {', '.join(f'{x:.2f}' for x in step_ms)} ms; info={status}")

    check = None
    if not args.no_check:
        # L C L^H = A (itype 1) or C = L^H A L (itypes 2, 3), in double on the GPU
        wd = torch.complex128 if cplx else torch.float64
        Lw = torch.tril(Lb).to(wd)
        C = torch.tril(H, -1).to(wd)
        C = C + C.mH + torch.diag_embed(torch.diagonal(H).real.to(wd))
        Aw = H0.to(wd)
        if itype == 1:
            err = ((Lw @ C @ Lw.mH - Aw).abs().max() / Aw.abs().max()).item()
        else:
            err = ((C - Lw.mH @ Aw @ Lw).abs().max() / C.abs().max()).item()
        eps = 2.0**-52 if dt in ("f64", "c128") else 2.0**-23
        check = {"identity_error": float(err), "bound_64_n_eps": 64 * n * eps,
                 "ok": bool(err <= 64 * n * eps and status == 0)}
        del Lw, C, Aw
        log(f"[bench] reduction identity error {err:.3e} (bound {64 * n * eps:.3e})")

    peak = PEAK[dt]
    avg = k_ms / max(k_launches, 1)
    ach = (k_flops / k_launches) / (avg * 1e-3) / 1e12 if k_launches else None
    roofline = {
        "kernel": ("syrk_kernel: potrf's trailing update and the reduction's rank-2k updates "
                   "A22 -= Z L21^H + L21 Z^H" if itype == 1 else
                   "syrk_kernel: potrf's trailing update and the reduction's products "
                   "Wf += A_panel L_panel and C += w_k^H l21 + l21^H w_k"),
        "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
        "frac": (ach / peak) if ach else None, "traffic": None, "launches": k_launches,
        "avg_launch_ms": avg, "flops_per_launch": k_flops / max(k_launches, 1),
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_sygst(B0, H0, n, itype, fmul, args.cpu_seconds)
    value = (flops_potrf + flops_gst) / (ms * 1e-3) / 1e12
    out = {
        "metric": f"generalized-eigenproblem reduction (potrf of B + sygst itype {itype}) TFLOP/s, 1 MI355X",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": f"{dt} reduction of A v = w B v type {itype}, N={n}, T_A={T}, "
                               f"B = G G^H/N + {cfg['delta']} I, A = (G' + G'^H)/sqrt(2N), seed {args.seed}",
                   "n": n, "T_A": T, "itype": itype},
        "pct_of_peak": 100.0 * value / peak,
        "phase_ms": {"potrf": float(np.mean(potrf_ms)), "sygst": float(np.mean(gst_ms))},
        "sygst_tflops": flops_gst / (float(np.mean(gst_ms)) * 1e-3) / 1e12,
        "roofline": roofline, "cpu_baseline": cpu, "check": check,
    }
    print(json.dumps(out), flush=True)
    return 0 if (check is None or check["ok"]) else 1


def sample_size(run, n, target_s):
    """Order of the leading block the CPU oracle takes about ``target_s``
    seconds on: a small block fits the host caches and runs faster per flop
    than a large one, so a first estimate from a 1024 block is refined by a
    run at about a quarter of the target before the cubic scaling is trusted."""
    def scale(m0, t0, goal):
        m = int(m0 * (goal / max(t0, 1e-3)) ** (1.0 / 3.0))
        return max(256, min(n, (m // 256) * 256))

    m0 = min(n, 1024)
    t0 = run(m0)
    m1 = scale(m0, t0, target_s / 4.0)
    t1 = run(m1) if m1 > m0 else t0
    m1 = max(m1, m0)
    m = scale(m1, t1, target_s)
    log(f"[bench] cpu oracle: {m0} took {t0:.2f} s, {m1} took {t1:.2f} s; sample size {m}")
    return m


def cpu_baseline_sygst(B0, H0, n, itype, fmul, target_s):
    """The CPU oracle on the leading principal blocks of B and A: potrf, then
    the reduction by its definition; same flop formula as the GPU value."""
    import oracle

    def run(m):
        b = B0[:m, :m].cpu().numpy()
        a = H0[:m, :m].cpu().numpy()
        t = time.perf_counter()
        l, info = oracle.potrf(b)
        oracle.sygst(itype, a, l)
        return time.perf_counter() - t

    m = sample_size(lambda k: run(k), n, target_s)
    t = run(m)
    fl = fmul * (m**3 / 3.0 + float(m) ** 3)
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"leading {m} x {m} principal blocks of the same B and A (potrf + reduction by its "
                      f"definition), {t:.2f} s", "seconds": t}


def host_cpu():
    """CPU model, socket count and logical CPUs of this host (from
    /proc/cpuinfo), and the CPUs this process may run on."""
    model, sockets, logical = None, set(), 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    sockets.add(val)
                elif key == "processor":
                    logical += 1
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        allowed = os.cpu_count()
    return {"model": model, "sockets": len(sockets) or None, "logical_cpus": logical or None,
            "cpus_allowed": allowed}


def cpu_baseline(A0, B0, n, nrhs, fmul, target_s, gp=False, single=False):
    """The CPU oracle, as it stands, on the leading principal block of the same
    matrix (and the matching rows of B): a bounded sample sized for about
    ``target_s`` seconds, scaled to TFLOP/s with the same flop formula.  For
    the likelihood workload the oracle's own definition (a full solve and
    log det) is what runs; with ``single`` the oracle's single-precision
    routines (the fp32 workload in its own precision)."""
    import oracle

    def run(m):
        a = A0[:m, :m].cpu().numpy()
        b = B0[:m, :].cpu().numpy()
        t = time.perf_counter()
        if gp:
            _, info = oracle.gp_loglik(a, b)
            return time.perf_counter() - t, info
        if single:
            l, info = oracle.potrf_single(a)
            oracle.potrs_single(l, b)
            oracle.logdet_single(l)
            return time.perf_counter() - t, info
        l, info = oracle.potrf(a)
        oracle.potrs(l, b)
        oracle.logdet(l)
        return time.perf_counter() - t, info

    m = sample_size(lambda k: run(k)[0], n, target_s)
    t, info = run(m)
    fl = fmul * (m**3 / 3.0 + (1.0 if gp else 2.0) * m * m * nrhs)
    what = ("GP log-likelihood by its definition" if gp else
            "potrf+potrs+logdet, float32 oracle" if single else "potrf+potrs+logdet, float64 oracle")
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"leading {m}^2 block of A, first {m} rows of B ({what}), {t:.1f} s",
            "seconds": t, "sample_n": m, "cpu": host_cpu()}


if __name__ == "__main__":
    sys.exit(main())
