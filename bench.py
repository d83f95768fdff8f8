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
SYRK_TRAFFIC_BYTES = {("f64", 32768, 512): 8.931e9}


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
    A = spdgen.to_colmajor(A0)
    B = spdgen.to_colmajor(B0)
    work = spd.workspace(A.dtype, n, nrhs, T)
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    ldbuf = torch.zeros(1, dtype=torch.float64, device="cuda")
    gpout = torch.zeros(nrhs, dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()

    def restore():
        A.copy_(A0)
        B.copy_(B0)

    fused = not gp and not args.separate

    def step(ev):
        ev[0].record(stream)
        if fused:  # potrf, logdet and potrs in one call (spd_posv)
            spd.posv(A, B, T, info=info, logdet_out=ldbuf if cfg["logdet"] else None, work=work)
            for e in ev[1:]:
                e.record(stream)
            return
        spd.potrf(A, T, info=info, work=work)
        ev[1].record(stream)
        if cfg["logdet"] and not gp:
            spd.logdet(A, info, out=ldbuf)
        ev[2].record(stream)
        if gp:
            spd.gp_loglik(A, B, T, info=info, work=work, out=gpout)
        else:
            spd.potrs(A, B, T, info=info, work=work)
        ev[3].record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    for w in range(args.warmup):
        restore()
        step(events())
        torch.cuda.synchronize()
        log(f"[bench] warmup {w + 1}/{args.warmup} done")

    # timed region: K steps; restores happen between steps, outside the events
    spd.profile_enable((1 << spd.PROF_SYRK) | (1 << spd.PROF_SYRK_AUX))
    spd.profile_read(spd.PROF_SYRK)
    spd.profile_read(spd.PROF_SYRK_AUX)
    evs = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(args.steps):
        restore()
        ev = events()
        step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    spd.profile_enable(0)
    syrk_ms, syrk_launches, syrk_flops = spd.profile_read(spd.PROF_SYRK)
    aux_ms, aux_launches, aux_flops = spd.profile_read(spd.PROF_SYRK_AUX)

    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    potrf_ms = [e[0].elapsed_time(e[1]) for e in evs]
    logdet_ms = [e[1].elapsed_time(e[2]) for e in evs]
    potrs_ms = [e[2].elapsed_time(e[3]) for e in evs]
    ms = float(np.mean(step_ms))
    status = int(info.item())
    log(f"[bench] steps: {', '.join(f'{x:.2f}' for x in step_ms)} ms; info={status}")

    check = None
    if not args.no_check and gp:
        # normwise backward error of the forward substitution L Y = R, with the
        # computed factor, in double on the GPU
        Lw = torch.tril(A).to(torch.float64)
        Yw, Rw = B.to(torch.float64), B0.to(torch.float64)
        r = Rw - Lw @ Yw
        eta = (r.abs().amax(dim=0) / (Lw.abs().sum(dim=1).max() * Yw.abs().amax(dim=0) + Rw.abs().amax(dim=0))).max()
        eps = 2.0**-52 if dt == "f64" else 2.0**-23
        finite = bool(torch.isfinite(gpout).all().item())
        check = {"forward_backward_error": float(eta.item()), "bound_64_n_eps": 64 * n * eps,
                 "loglik_first": float(gpout[0].item()), "ok": bool(eta.item() <= 64 * n * eps and status == 0
                                                                   and finite)}
        del Lw, Yw, Rw, r
        log(f"[bench] forward-substitution backward error {check['forward_backward_error']:.3e} "
            f"(bound {check['bound_64_n_eps']:.3e}); loglik[0] = {check['loglik_first']:.6f}")
    elif not args.no_check:
        # normwise backward error of the last step's X, residual in double on the GPU
        wd = torch.complex128 if cplx else torch.float64
        Aw, Xw, Bw = A0.to(wd), B.to(wd), B0.to(wd)
        r = Bw - Aw @ Xw
        eta = (r.abs().amax(dim=0) / (Aw.abs().sum(dim=1).max() * Xw.abs().amax(dim=0) + Bw.abs().amax(dim=0))).max()
        eps = 2.0**-52 if dt in ("f64", "c128") else 2.0**-23
        check = {"backward_error": float(eta.item()), "bound_64_n_eps": 64 * n * eps,
                 "ok": bool(eta.item() <= 64 * n * eps and status == 0)}
        del Aw, Xw, Bw, r
        log(f"[bench] backward error {check['backward_error']:.3e} (bound {check['bound_64_n_eps']:.3e})")

    value = flops / (ms * 1e-3) / 1e12
    potrf_tf = None if fused else flops_potrf / (float(np.mean(potrf_ms)) * 1e-3) / 1e12
    syrk_avg_ms = syrk_ms / max(syrk_launches, 1)
    syrk_achieved = (syrk_flops / syrk_launches) / (syrk_avg_ms * 1e-3) / 1e12 if syrk_launches else None
    peak = PEAK[dt]
    aux_avg_ms = aux_ms / max(aux_launches, 1)
    roofline = {
        "kernel": "syrk_kernel (trailing update A22 -= L21 L21^H, lower tiles; launches on the caller's stream)",
        "bound": "mfma",
        "achieved": syrk_achieved,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": (syrk_achieved / peak) if syrk_achieved else None,
        "traffic": SYRK_TRAFFIC_BYTES.get((dt, n, T)) if not gp else None,
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
        "entry_points": ("spd_posv (potrf + logdet + potrs in one call)" if fused else
                         "spd_potrf, spd_gp_loglik" if gp else "spd_potrf, spd_logdet, spd_potrs"),
        "phase_ms": ({"posv": ms} if fused else
                     {"potrf": float(np.mean(potrf_ms)), "gp_loglik": float(np.mean(potrs_ms))} if gp else
                     {"potrf": float(np.mean(potrf_ms)), "logdet": float(np.mean(logdet_ms)),
                      "potrs": float(np.mean(potrs_ms))}),
        "wall_ms_per_step_incl_restore": 1e3 * wall / args.steps,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "check": check,
    }
    print(json.dumps(out), flush=True)
    return 0 if (check is None or check["ok"]) else 1


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


def cpu_baseline(A0, B0, n, nrhs, fmul, target_s, gp=False):
    """The CPU oracle, as it stands, on the leading principal block of the same
    matrix (and the matching rows of B): a bounded sample sized for about
    ``target_s`` seconds, scaled to TFLOP/s with the same flop formula.  For
    the likelihood workload the oracle's own definition (a full solve and
    log det) is what runs."""
    import numpy as np

    import oracle

    def run(m):
        a = A0[:m, :m].cpu().numpy()
        b = B0[:m, :].cpu().numpy()
        t = time.perf_counter()
        if gp:
            _, info = oracle.gp_loglik(a, b)
            return time.perf_counter() - t, info
        l, info = oracle.potrf(a)
        oracle.potrs(l, b)
        oracle.logdet(l)
        return time.perf_counter() - t, info

    m = sample_size(lambda k: run(k)[0], n, target_s)
    t, info = run(m)
    fl = fmul * (m**3 / 3.0 + (1.0 if gp else 2.0) * m * m * nrhs)
    what = "Gaussian-process log-likelihood by its definition" if gp else "potrf + potrs + logdet"
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"leading {m} x {m} principal block of the same A with the first {m} rows of all "
                      f"{nrhs} right-hand sides ({what}), {t:.2f} s",
            "seconds": t}


if __name__ == "__main__":
    sys.exit(main())
