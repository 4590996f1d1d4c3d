"""Benchmark of the Hyena order-N forward (hyena_forward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4] [--also C3]

A step is one hyena_forward over one batch of synthetic inputs already
resident in HBM (v, x_1..x_N and the precomputed filter spectrum).  Inputs
rotate over several independent sets so the working set exceeds the 256 MB
Infinity Cache and every step reads from HBM.  Prints one JSON line with
channel-tokens/s (B*D*L per second), the HBM roofline fraction of the forward
(algorithmic bytes over the event-timed forward), and the float64 CPU oracle
run on a bounded sample of the same rows on the host cores -- its time is the
CPU baseline and its output checks the GPU's on those rows (parity).

The default workload is the 1M-token shape (order 2, B=1, D=256, L=2^20,
fp32), with the 64K shape (order 2, B=1, D=768, L=65536, bf16 I/O) reported
under "also"; --config selects the main shape (C1, C2, C3, C4, C5a, C5b).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12                  # B/s, MI355X HBM3E
# Non-packed FP32 VALU: 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz.
ALU_PEAK = 256 * 4 * 16 * 2 * 2.4e9
ALU_PEAK_PACKED = 157.3e12        # vendor figure, needs packed-FP32 instructions (not used)
MALL_BYTES = 256 << 20


def min_bytes(cfg, circular: bool = False) -> int:
    """Algorithmic HBM bytes of one forward: v, x_1..x_N, y in the I/O dtype
    plus the spectrum read once as complex64 with L+1 bins per (n, d) (L/2+1
    in circular mode, where the FFT length is L)."""
    s = 4 if cfg.io == "fp32" else 2
    bins = cfg.L // 2 + 1 if circular else cfg.L + 1
    return (cfg.N + 2) * cfg.B * cfg.D * cfg.L * s + cfg.N * cfg.D * bins * 8


def algo_flops(cfg, circular: bool = False) -> float:
    """N * (10 log2(2L) + 7) flops per channel-token: forward and inverse real
    FFT of 2L points at 2.5 M log2 M each, one complex product per bin, gate
    (circular mode, M = L: N * (5 log2 L + 4))."""
    if circular:
        return cfg.N * cfg.B * cfg.D * cfg.L * (5.0 * math.log2(cfg.L) + 4.0)
    return cfg.N * cfg.B * cfg.D * cfg.L * (10.0 * math.log2(2 * cfg.L) + 7.0)


# Sources that make up the code of each counted kernel (its translation unit
# and the device headers it includes).
KERNEL_SOURCES = {
    "k_single_forward": ["kernels_single.hip", "fft_engine.hpp", "plan.hpp"],
    "k_nd_forward": ["kernels_nd.hip", "fft_engine.hpp", "plan.hpp"],
    # the four-step forward: its kernels, and the host code that sizes its pass groups
    "fourstep_forward": ["api.cpp", "kernels_fourstep.hip", "fft_engine.hpp", "plan.hpp", "launch.hpp"],
}


def source_hash(files=None) -> str:
    """Hash of the given csrc files (all of csrc when None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hyena_long_conv_amd", "csrc")
    paths = sorted(glob.glob(os.path.join(csrc, "*"))) if files is None else [os.path.join(csrc, f) for f in sorted(files)]
    for f in paths:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def work_point_bytes(cfg) -> int:
    """Bytes per point of the four-step intermediate: bf16 pairs for bf16
    activations up to order 2, else float2."""
    return 4 if bf16_work(cfg) else 8


def bf16_work(cfg) -> bool:
    return cfg.io == "bf16" and cfg.N <= 2


def measured_traffic(cfg_name: str):
    """HBM bytes per forward from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg_name}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash(d.get("sources")):
        return None
    return d.get("hbm_bytes_per_step")


TOL = {"fp32": 1e-4, "fp32_1M": 5e-4, "bf16": 2e-2}


def tolerance(cfg) -> float:
    """Per-row normalised max error bound: 1e-4 (fp32, L <= 64K), 5e-4 (fp32
    beyond), 2e-2 (bf16 I/O against the oracle fed the same bf16 inputs)."""
    if cfg.io == "bf16":
        return TOL["bf16"]
    return TOL["fp32"] if cfg.L <= 65536 else TOL["fp32_1M"]


def sample_rows(cfg, n: int):
    """n flat rows b*D + d: (0, 0), (0, D-1), (B-1, D-1) first, then a seeded
    uniform sample."""
    import numpy as np
    total = cfg.B * cfg.D
    first = [0, cfg.D - 1, total - 1]
    rows = list(dict.fromkeys(r for r in first if r < total))
    rest = [r for r in np.random.default_rng(cfg.seed).permutation(total).tolist() if r not in rows]
    return (rows + rest)[:max(1, min(n, total))]


def _pin_threads():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"


def _oracle_rows(cfg, rows, v_rows, x_rows):
    """Float64 oracle forward for flat rows b*D + d on the given inputs
    (v_rows [n, L], x_rows [N][n, L], float64): filters from the same seeded
    FFN weights, then the recurrence.  Returns y [n, L]."""
    import numpy as np

    import oracle as O
    from workloads import make_filter_params
    p = make_filter_params(cfg)
    ds = sorted({r % cfg.D for r in rows})
    h = O.filter_gen(p, cfg.L, channels=ds)
    col = {d: i for i, d in enumerate(ds)}
    hh = np.stack([h[:, col[r % cfg.D]] for r in rows], axis=1)  # [N, rows, L]
    return O.hyena_forward(np.asarray(v_rows), [np.asarray(x) for x in x_rows], hh)


def cpu_baseline_parity(cfg, v, xs, y, budget_s: float = 12.0):
    """The float64 oracle on a bounded sample of the measured workload's own
    rows, on the host cores (one single-threaded worker per core, at most 16),
    and the GPU output's error on those rows.

    One row ((0, 0): alpha = 1, the longest filter memory) runs first on its
    own and sizes the sample to about ``budget_s`` of wall time on the
    workers; rows (0, D-1) and (B-1, D-1) are always part of it.  Returns
    (cpu_baseline, parity) dicts."""
    import multiprocessing as mp

    import numpy as np

    host_cores = len(os.sched_getaffinity(0))
    total = cfg.B * cfg.D

    def rows_of(rows):
        b = [r // cfg.D for r in rows]
        d = [r % cfg.D for r in rows]
        vr = v[b, d].double().cpu().numpy()
        xr = [x[b, d].double().cpu().numpy() for x in xs]
        yr = y[b, d].double().cpu().numpy()
        return vr, xr, yr

    t0 = time.perf_counter()
    v0, x0, y0 = rows_of([0])
    ref0 = _oracle_rows(cfg, [0], v0, x0)
    one = time.perf_counter() - t0
    workers = max(1, min(16, host_cores))
    n = int(min(total, max(workers + 1, 1 + budget_s * workers / max(one, 1e-3))))
    rows = sample_rows(cfg, n)
    pool_rows = [r for r in rows if r != 0]
    refs, gots, checked = [ref0], [y0], [0]
    wall, used = 0.0, 0
    if pool_rows:
        used = min(workers, len(pool_rows))
        chunks = [pool_rows[i::used] for i in range(used)]
        args = []
        for c in chunks:
            vr, xr, yr = rows_of(c)
            args.append((cfg, c, vr, xr))
            gots.append(yr)
            checked += c
        ctx = mp.get_context("spawn")
        t1 = time.perf_counter()
        with ctx.Pool(used, initializer=_pin_threads) as pool:
            refs += pool.starmap(_oracle_rows, args)
        wall = time.perf_counter() - t1
    ref = np.concatenate(refs, axis=0)
    got = np.concatenate(gots, axis=0)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num <= 1e-30, 0.0, np.inf))
    worst = int(np.argmax(err))
    tol = tolerance(cfg)
    parity = {"max_norm_err": float(err[worst]),
              "worst_channel": {"b": checked[worst] // cfg.D, "d": checked[worst] % cfg.D},
              "channels_checked": len(checked), "tolerance": tol, "pass": bool(err[worst] <= tol),
              "metric": "max over checked (b,d) rows of max_t|y - y_ref| / max_t|y_ref|, y_ref the float64 oracle"}
    if pool_rows:
        base = {"value": len(pool_rows) * cfg.L / wall, "unit": "channel-tokens/s", "cores": used,
                "host_cores": host_cores, "kind": "oracle",
                "sample": f"{len(pool_rows)} of {total} (b,d) rows of {cfg.name} on {used} single-threaded workers "
                          f"(float64 oracle: filter FFN for the rows' channels, then direct conv for L<=8192 else "
                          f"its radix-2 FFT), {wall:.1f} s wall",
                "extrapolated_full_s": wall * total / len(pool_rows), "extrapolated": True}
    else:
        base = {"value": cfg.L / one, "unit": "channel-tokens/s", "cores": 1, "host_cores": host_cores,
                "kind": "oracle", "sample": f"1 of {total} rows of {cfg.name}, {one:.1f} s",
                "extrapolated_full_s": one * total, "extrapolated": True}
    return base, parity


def measure_copy(torch, dev, reps=4, nbytes=1 << 30):
    """Best of `reps` timed 1 GiB device copies, in B/s of read + write."""
    a = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3
        best = t if best is None else min(best, t)
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / best


MFMA_PEAK = {"fp32": 157.3e12, "bf16": 2.5e15}   # dense matrix-core peaks, FLOP/s


def _time_steps(torch, dev, step, steps, warmup):
    """Warm-up (given count, or >= 3 steps and 100 ms), then `steps` timed
    steps (or >= 20 and 200 ms) bracketed by events on the current stream;
    returns (mean ms, steps, warmup)."""
    est = None
    if warmup is not None:
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
    else:
        done, t_w = 0, time.perf_counter()
        while done < 3 or time.perf_counter() - t_w < 0.1:
            step(done)
            done += 1
            if done % 8 == 0 or done < 3:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        warmup = done
        est = (time.perf_counter() - t_w) / done
    if steps is None:
        if est is None:
            t_e = time.perf_counter()
            step(0)
            torch.cuda.synchronize()
            est = time.perf_counter() - t_e
        steps = int(min(5000, max(20, math.ceil(0.2 / max(est, 1e-6)))))
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, steps, warmup


def run_block(args, cfg, torch, H, dev):
    """The block around the operator: u [B, L, D] -> in-projection with the
    short convolutions -> operator -> out-projection.  One step = one
    hyena_block_forward.  The roofline is the in-projection GEMM's (the
    block's dominant kernel), against the dense matrix-core peak of the I/O
    dtype; the pieces are also timed on their own."""
    import numpy as np
    from workloads import make_block_input, make_block_params, make_filter_params

    dt = torch.float32 if cfg.io == "fp32" else torch.bfloat16
    s = 4 if cfg.io == "fp32" else 2
    B, D, L, N = cfg.B, cfg.D, cfg.L, cfg.N
    bp = make_block_params(cfg)
    bpd = {"D": D, "N": N, "T": bp["T"], "b_in": None, "b_out": None,
           "W_in": torch.from_numpy(bp["W_in"]).to(dev).to(dt).contiguous(),
           "W_out": torch.from_numpy(bp["W_out"]).to(dev).to(dt).contiguous(),
           "w_short": torch.from_numpy(bp["w_short"]).to(dev)}
    fp = make_filter_params(cfg)
    h = H.filter_gen({k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v) for k, v in fp.items()}, L)
    spec0 = H.filter_spectrum(h)
    per_set = 2 * B * L * D * s + spec0.numel()
    sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / per_set))
    us, outs, specs = [], [], []
    for k in range(sets):
        us.append(make_block_input(cfg.with_(seed=cfg.seed * 100 + k), dev))
        outs.append(torch.empty_like(us[-1]))
        specs.append(spec0 if k == 0 else spec0.clone())
    ws = torch.empty(H.block_workspace_bytes(B, D, N, L, cfg.io), dtype=torch.uint8, device=dev)
    streams = [torch.empty((B, D, L), dtype=dt, device=dev) for _ in range(N + 1)]
    y = torch.empty((B, D, L), dtype=dt, device=dev)
    blk = [H.prepare_block_forward(us[k], bpd, specs[k], outs[k], ws) for k in range(sets)]
    inp = [H.prepare_in_projection(us[k], bpd, streams) for k in range(sets)]
    fwd = [H.PreparedForward(streams[0], streams[1:], specs[k], out=y,
                             workspace=ws if ws.numel() > 0 else None) for k in range(sets)]
    outp = [H.prepare_out_projection(y, bpd, outs[k]) for k in range(sets)]
    torch.cuda.synchronize()
    ms, steps, warmup = _time_steps(torch, dev, lambda i: blk[i % sets](), args.steps, args.warmup)
    ms_in, _, _ = _time_steps(torch, dev, lambda i: inp[i % sets](), steps, 3)
    ms_fwd, _, _ = _time_steps(torch, dev, lambda i: fwd[i % sets](), steps, 3)
    ms_out, _, _ = _time_steps(torch, dev, lambda i: outp[i % sets](), steps, 3)
    t = ms / 1e3
    C = (N + 1) * D
    fl_in, fl_out = 2.0 * B * L * D * C, 2.0 * B * L * D * D
    peak = MFMA_PEAK[cfg.io]
    roof = {"bound": "mfma", "achieved": fl_in / (ms_in / 1e3) / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
            "frac": fl_in / (ms_in / 1e3) / peak, "traffic": None,
            "kernel": (("k_inproj_wide" if cfg.io == "bf16" and D % 8 == 0 and bp["T"] <= 8 else "k_inproj")
                       + " (in-projection GEMM + bias + short causal FIR + stream split)"),
            "algorithmic_flops_per_launch": fl_in,
            "out_projection": {"TFLOPs": fl_out / (ms_out / 1e3) / 1e12, "frac": fl_out / (ms_out / 1e3) / peak}}
    out = {
        "metric": "Hyena block fwd channel-tokens/sec (B*D*L/s): projections, short convs, order-N operator",
        "value": B * D * L / t, "unit": "channel-tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32" if cfg.io == "fp32" else "bf16 operands, fp32 accumulation",
        "data": "synthetic (seeded N(0,1) input, random-init projections, short filters and filter FFN)",
        "config": {"workload": cfg.desc + ", full block (T=3 short filters)", "name": cfg.name, "N": N, "B": B,
                   "D": D, "L": L, "io": cfg.io, "short_taps": bp["T"], "input_sets": sets},
        "block": {"ms_in_projection": ms_in, "ms_operator": ms_fwd, "ms_out_projection": ms_out},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(cfg, bp, h.cpu().numpy())
    print(json.dumps(out))
    return 0


def backward_bytes(cfg) -> int:
    """Algorithmic bytes of one backward: v, x_1..x_N, gy read and gv,
    gx_1..gx_N written in the I/O dtype, the spectrum (L+1 bins per (n, d),
    complex64) read, gh written (fp32)."""
    s = 4 if cfg.io == "fp32" else 2
    return ((2 * cfg.N + 3) * cfg.B * cfg.D * cfg.L * s + cfg.N * cfg.D * (cfg.L + 1) * 8
            + cfg.N * cfg.D * cfg.L * 4)


def backward_flops(cfg) -> float:
    """N * (25 log2(2L) + 20) per channel-token: five real FFTs of 2L points
    per order (the forward's two, recomputed, plus those of z_n, of the
    gradient and of its adjoint) and the spectral products."""
    return cfg.N * cfg.B * cfg.D * cfg.L * (25.0 * math.log2(2 * cfg.L) + 20.0)


def run_fir(args, cfg, torch, H, dev):
    """The recurrence with explicit short filters (Hyena-SE / Hyena-MR)
    evaluated directly: one launch per step, bound by HBM (v, x_1..x_N in,
    y out, the filters)."""
    import ctypes
    import numpy as np
    from workloads import make_activations

    Lh = args.fir
    s = 4 if cfg.io == "fp32" else 2
    mb = (cfg.N + 2) * cfg.B * cfg.D * cfg.L * s + cfg.N * cfg.D * Lh * 4
    fl = 2.0 * cfg.N * cfg.B * cfg.D * cfg.L * (Lh + 1)
    hs = torch.from_numpy((np.random.default_rng(cfg.seed).standard_normal((cfg.N, cfg.D, Lh)) / np.sqrt(Lh))
                          .astype(np.float32)).to(dev)
    sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / mb))
    lib = H.lib()
    io = 0 if cfg.io == "fp32" else 1
    calls = []
    for k in range(sets):
        v, xs = make_activations(cfg.with_(seed=cfg.seed * 100 + k), dev)
        y = torch.empty_like(v)
        xp = (ctypes.c_void_p * cfg.N)(*[t.data_ptr() for t in xs])
        calls.append(H.PreparedCall(lib.hyena_forward_fir,
                                    (H._ptr(v), xp, H._ptr(hs), Lh, H._ptr(y), cfg.B, cfg.D, cfg.N, cfg.L, io,
                                     H._stream(v)), (v, xs, xp, y, hs), y, "hyena_forward_fir"))
    torch.cuda.synchronize()
    ms, steps, warmup = _time_steps(torch, dev, lambda i: calls[i % sets](), args.steps, args.warmup)
    t = ms / 1e3
    copy_bps = measure_copy(torch, dev)
    roof = {"bound": "hbm", "achieved": mb / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": mb / t / HBM_PEAK,
            "traffic": None, "kernel": "k_fir_forward (one launch per step)", "copy_GBps": copy_bps / 1e9,
            "hbm_frac_vs_copy": mb / t / copy_bps, "alu_frac": fl / t / ALU_PEAK,
            "algorithmic_bytes_per_step": mb, "algorithmic_flops_per_step": fl}
    out = {
        "metric": "Hyena order-N fwd with explicit short filters, channel-tokens/sec (B*D*L/s)",
        "value": cfg.B * cfg.D * cfg.L / t, "unit": "channel-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic (seeded N(0,1) activations and filters)",
        "config": {"workload": cfg.desc + f", explicit {Lh}-tap filters", "name": cfg.name, "N": cfg.N, "B": cfg.B,
                   "D": cfg.D, "L": cfg.L, "io": cfg.io, "taps": Lh, "input_sets": sets},
        "roofline": roof,
    }
    print(json.dumps(out))
    return 0


def run_backward(args, cfg, torch, H, dev):
    """The backward of the operator: one step = one hyena_backward (recomputes
    the forward's convolutions, then gradients of v, every x_n and the
    filters): one launch on single-pass lengths, a pipeline of four-step
    convolutions and elementwise kernels beyond."""
    import numpy as np
    from workloads import make_activations, make_filter_params

    if args.copy_calib:
        measure_copy(torch, dev, reps=1)             # reference dispatch for counter scaling
    fp = make_filter_params(cfg)
    h = H.filter_gen({k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v) for k, v in fp.items()},
                     cfg.L)
    spec0 = H.filter_spectrum(h)
    del h
    sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / backward_bytes(cfg)))
    data = []
    for k in range(sets):
        c = cfg.with_(seed=cfg.seed * 100 + k)
        v, xs = make_activations(c, dev)
        g = torch.Generator(device=dev)
        g.manual_seed(c.seed * 7 + 1)
        gy = torch.randn(v.shape, generator=g, device=dev).to(v.dtype)
        data.append((v, xs, spec0 if k == 0 else spec0.clone(), gy))
    wsb = H.backward_workspace_bytes(cfg.B, cfg.D, cfg.N, cfg.L, cfg.io)
    if wsb < 0:
        print(f"backward not available for L = {cfg.L}", file=sys.stderr)
        return 2
    one_launch = H.plan(cfg.L)["path"] == "single" and cfg.L <= 8192
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    gv = torch.empty_like(data[0][0])
    gxs = [torch.empty_like(gv) for _ in range(cfg.N)]
    gh = torch.empty((cfg.N, cfg.D, cfg.L), dtype=torch.float32, device=dev)
    lib = H.lib()
    import ctypes
    io = 0 if cfg.io == "fp32" else 1
    gp = (ctypes.c_void_p * cfg.N)(*[t.data_ptr() for t in gxs])
    calls = []
    for v, xs, spec, gy in data:
        xp = (ctypes.c_void_p * cfg.N)(*[t.data_ptr() for t in xs])
        calls.append(H.PreparedCall(lib.hyena_backward,
                                    (H._ptr(v), xp, H._ptr(spec), H._ptr(gy), H._ptr(gv), gp, H._ptr(gh), cfg.B,
                                     cfg.D, cfg.N, cfg.L, io, H._ptr(ws), wsb, H._stream(v)),
                                    (v, xs, spec, gy, xp, gp), None, "hyena_backward"))
    torch.cuda.synchronize()
    ms, steps, warmup = _time_steps(torch, dev, lambda i: calls[i % sets](), args.steps, args.warmup)
    t = ms / 1e3
    mb, fl = backward_bytes(cfg), backward_flops(cfg)
    roof = {"bound": "alu", "achieved": fl / t / 1e12, "peak": ALU_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": fl / t / ALU_PEAK, "traffic": None,
            "kernel": ("k_single_backward (one launch per step)" if one_launch else
                       "four-step backward pipeline (forward recompute, per-row spectra, convolutions, "
                       "elementwise kernels; many launches per step)"),
            "hbm_frac": mb / t / HBM_PEAK, "algorithmic_bytes_per_step": mb, "algorithmic_flops_per_step": fl}
    out = {
        "metric": "Hyena order-N backward channel-tokens/sec (B*D*L/s)",
        "value": cfg.B * cfg.D * cfg.L / t, "unit": "channel-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32" if cfg.io == "fp32" else "bf16 I/O, fp32 compute",
        "data": "synthetic (seeded N(0,1) activations and output gradient, random-init filter FFN)",
        "config": {"workload": cfg.desc + ", backward", "name": cfg.name, "N": cfg.N, "B": cfg.B, "D": cfg.D,
                   "L": cfg.L, "io": cfg.io, "input_sets": sets},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        # one more backward on the first input set, outside the timed region:
        # its inputs and outputs are what the oracle checks
        v, xs, spec, gy = data[0]
        calls[0]()
        torch.cuda.synchronize()
        out["cpu_baseline"], out["parity"] = cpu_baseline_backward(cfg, fp, (v, xs, gy), (gv, gxs, gh))
    print(json.dumps(out))
    return 0


def cpu_baseline_backward(cfg, fp, inputs, outputs, budget_s: float = 12.0):
    """The float64 oracle's backward over all B rows of as many channels as
    take about `budget_s` (channels are independent in the backward):
    channels 0 and D - 1 first, then a seeded sample.  `inputs` (v, x_n,
    dloss/dy) and `outputs` (gv, gx_n, gh) are the device tensors of one GPU
    backward; the oracle runs on those inputs and its gradients give the
    parity of that call on the checked channels."""
    import numpy as np
    import oracle as O
    v, xs, gy = inputs
    gv, gxs, gh = outputs
    order = [0] + ([cfg.D - 1] if cfg.D > 1 else [])
    rest = [d for d in np.random.default_rng(11).permutation(cfg.D).tolist() if d not in order]
    order += rest
    host = lambda t, d: t[:, d:d + 1].double().cpu().numpy()
    errs, done, t0, wall = {"gv": 0.0, "gx": 0.0, "gh": 0.0}, 0, time.perf_counter(), 0.0
    worst = {"gv": None, "gx": None, "gh": None}

    def norm_err(a, r):
        num = np.max(np.abs(a - r), axis=-1)
        den = np.max(np.abs(r), axis=-1)
        e = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num <= 1e-30, 0.0, np.inf))
        return float(np.max(e))

    while done < cfg.D and (done < 1 or time.perf_counter() - t0 < budget_s):
        d = order[done]
        vd, xd, gyd = host(v, d), [host(x, d) for x in xs], host(gy, d)
        t1 = time.perf_counter()
        h = O.filter_gen(fp, cfg.L, channels=[d])
        rv, rxs, rgh = O.hyena_backward(vd, xd, h, gyd)
        wall += time.perf_counter() - t1
        for key, e in (("gv", norm_err(host(gv, d), rv)),
                       ("gx", max(norm_err(host(g, d), r) for g, r in zip(gxs, rxs))),
                       ("gh", norm_err(gh[:, d:d + 1].double().cpu().numpy(), rgh))):
            if e >= errs[key]:
                errs[key], worst[key] = e, d
        done += 1
    tol = tolerance(cfg)
    tol_gh = TOL["fp32"] if cfg.L <= 65536 else TOL["fp32_1M"]
    parity = {"max_norm_err": errs, "worst_channel": worst, "channels_checked": done,
              "tolerance": {"gv": tol, "gx": tol, "gh": tol_gh},
              "pass": bool(errs["gv"] <= tol and errs["gx"] <= tol and errs["gh"] <= tol_gh),
              "metric": "max over checked channels (all B rows) of max_t|g - g_ref| / max_t|g_ref| per row, "
                        "g_ref the float64 oracle backward on the same inputs"}
    base = {"value": cfg.B * done * cfg.L / wall, "unit": "channel-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {cfg.D} channels x {cfg.B} rows (channels 0, D-1, then seeded), "
                      f"float64 oracle backward, {wall:.1f} s"}
    return base, parity


def cpu_baseline_block(cfg, bp, h, budget_s: float = 12.0):
    """The float64 oracle's block on batch row 0 over a causal prefix of the
    sequence (the first Lp steps need only the first Lp inputs and taps),
    Lp doubled from 64 while the run stays within the budget."""
    import numpy as np
    import oracle as O
    from workloads import make_block_input
    u = make_block_input(cfg, "cpu", B=1).float().numpy()
    Lp, best = 64, None
    while Lp <= cfg.L:
        t0 = time.perf_counter()
        O.block_forward(u[:, :Lp], bp, h[:, :, :Lp])
        dt_ = time.perf_counter() - t0
        best = (Lp, dt_)
        if dt_ * 4 > budget_s or Lp == cfg.L:
            break
        Lp = min(cfg.L, Lp * 2)
    Lp, dt_ = best
    return {"value": cfg.D * Lp / dt_, "unit": "channel-tokens/s", "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0)),
            "kind": "oracle", "sample": f"block on batch row 0, first {Lp} of {cfg.L} steps (causal prefix), float64, {dt_:.1f} s"}


def grid_bytes(cfg, P: int) -> int:
    """Algorithmic bytes of one grid forward: v, x_1..x_N, y in the I/O dtype
    plus the kernels' spectra read once, complex64 over the Hermitian half
    of the padded grid (P^(k-1) * (P/2 + 1) bins per kernel)."""
    s = 4 if cfg.io == "fp32" else 2
    pts = math.prod(cfg.dims)
    rows = cfg.N * cfg.D * (cfg.B if cfg.per_sample else 1)
    bins = P ** (cfg.ndim - 1) * (P // 2 + 1)
    return (cfg.N + 2) * cfg.B * cfg.D * pts * s + rows * bins * 8


def grid_flops(cfg, P: int) -> float:
    """Per grid and order: forward and inverse real FFT of M = P^k points at
    2.5 M log2 M each, one complex product per Hermitian bin (3M), the gate."""
    M = P ** cfg.ndim
    return cfg.N * cfg.B * cfg.D * (5.0 * M * math.log2(M) + 3.0 * M + math.prod(cfg.dims))


def _oracle_grids(cfg, pairs):
    """Oracle grid forward for (b, d) pairs: seeded kernels of the workload,
    activations drawn from N(0, 1) on the CPU (the cost does not depend on
    the values)."""
    import numpy as np

    import oracle as O
    from workloads import make_grid_kernel
    K = make_grid_kernel(cfg)
    rs = np.random.default_rng([cfg.seed, len(pairs), pairs[0][0], pairs[0][1]])
    for b, d in pairs:
        v = rs.standard_normal((1, 1) + tuple(cfg.dims))
        xs = [rs.standard_normal((1, 1) + tuple(cfg.dims)) for _ in range(cfg.N)]
        Kd = K[b][:, d:d + 1] if cfg.per_sample else K[:, d:d + 1]
        O.nd_forward(v, xs, Kd, cfg.ndim, cfg.circular)
    return len(pairs)


def cpu_baseline_grid(cfg, budget_s: float = 12.0):
    import multiprocessing as mp

    import numpy as np

    cores = min(16, len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    _oracle_grids(cfg, [(0, 0)])
    one = time.perf_counter() - t0
    total = cfg.B * cfg.D
    n = max(1, min(total, int(max(cores, budget_s * cores / max(one, 1e-3)))))
    rng = np.random.default_rng(cfg.seed)
    flat = sorted(rng.choice(total, size=n, replace=False).tolist())
    pairs = [(r // cfg.D, r % cfg.D) for r in flat]
    chunks = [pairs[i::cores] for i in range(cores) if pairs[i::cores]]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(len(chunks), initializer=_pin_threads) as pool:
        pool.starmap(_oracle_grids, [(cfg, c) for c in chunks])
    wall = time.perf_counter() - t0
    pts = math.prod(cfg.dims)
    return {"value": n * pts / wall, "unit": "channel-tokens/s", "cores": len(chunks), "kind": "oracle",
            "sample": f"{n} of {total} (b,d) grids of {cfg.name} (float64 oracle, its N-D FFT path or brute force), "
                      f"{wall:.1f} s wall",
            "extrapolated_full_s": wall * total / n}


def run_grid(args, torch, H, dev):
    """Convolutions on 2-D/3-D grids: one step = one hyena_nd_forward over
    one batch of grids (spectra precomputed), inputs rotating over sets that
    exceed the Infinity Cache."""
    from workloads import GRID_CONFIGS, make_grid_activations, make_grid_kernel

    cfg = GRID_CONFIGS[args.grid]
    P = H.nd_plan(cfg.dims, cfg.circular)
    mb, fl = grid_bytes(cfg, P), grid_flops(cfg, P)
    sets = args.sets or min(64, max(1, math.ceil(2 * MALL_BYTES / mb)))
    K = torch.from_numpy(make_grid_kernel(cfg)).to(dev)
    spec0 = H.nd_filter_spectrum(K, cfg.dims, cfg.circular)
    del K
    calls = []
    for k in range(sets):
        v, xs = make_grid_activations(cfg.with_(seed=cfg.seed * 100 + k), dev)
        spec = spec0 if k == 0 else spec0.clone()
        calls.append(H.prepare_nd_forward(v, xs, spec, cfg.circular, cfg.per_sample))
    torch.cuda.synchronize()
    ms, steps, warmup = _time_steps(torch, dev, lambda i: calls[i % sets](), args.steps, args.warmup)
    t = ms / 1e3
    copy_bps = measure_copy(torch, dev)
    if fl / mb > ALU_PEAK / HBM_PEAK:
        roof = {"bound": "alu", "achieved": fl / t / 1e12, "peak": ALU_PEAK / 1e12, "unit": "TFLOP/s",
                "frac": fl / t / ALU_PEAK}
    else:
        roof = {"bound": "hbm", "achieved": mb / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": mb / t / HBM_PEAK}
    multi = P > (128 if cfg.ndim == 2 else 32)
    passes = "k_grid_row" if cfg.ndim == 2 else "k_grid_plane"
    roof.update({"traffic": measured_traffic(cfg.name),
                 "kernel": (f"grid passes (k_col grid mode + {passes}, 2N+1 passes per pass group)" if multi
                            else "k_nd_forward (one launch per step)"),
                 "launches_per_step": None if multi else 1,
                 "hbm_frac": mb / t / HBM_PEAK, "hbm_GBps": mb / t / 1e9, "copy_GBps": copy_bps / 1e9,
                 "hbm_frac_vs_copy": mb / t / copy_bps, "alu_frac": fl / t / ALU_PEAK,
                 "alu_TFLOPs": fl / t / 1e12, "algorithmic_bytes_per_step": mb, "algorithmic_flops_per_step": fl})
    pts = math.prod(cfg.dims)
    out = {
        "metric": "Hyena order-N fwd on grids (HyenaND), channel-tokens/sec (B*D*grid points/s)",
        "value": cfg.B * cfg.D * pts / t, "unit": "channel-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic (seeded N(0,1) activations, Gaussian-windowed random kernels)",
        "config": {"workload": cfg.desc, "name": cfg.name, "N": cfg.N, "B": cfg.B, "D": cfg.D,
                   "dims": list(cfg.dims), "circular": cfg.circular, "io": cfg.io, "per_sample": cfg.per_sample,
                   "fft_side": P, "input_sets": sets},
        "roofline": roof,
    }
    del calls
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_grid(cfg)
    print(json.dumps(out))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: >= 20 and >= 200 ms of work)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: >= 3 and >= 100 ms of work)")
    ap.add_argument("--config", default="C4",
                    help="forward workload of the main line (default C4: order 2, L = 1M, fp32)")
    ap.add_argument("--also", default="C3",
                    help="comma-separated forward workloads reported under 'also' after the main line "
                         "(default C3, the 64K shape; '' for none)")
    ap.add_argument("--sets", type=int, default=0, help="input sets to rotate (0: enough to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--circular", action="store_true",
                    help="periodic convolution (FFT length L, no zero padding; L a power of two)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the operator (gradients of v, x_n and the filters)")
    ap.add_argument("--fir", type=int, default=0, metavar="LH",
                    help="time the recurrence with explicit short filters of LH taps (hyena_forward_fir)")
    ap.add_argument("--block", action="store_true",
                    help="time the whole block (in-projection + short convolutions, operator, out-projection)")
    ap.add_argument("--grid", default=None, metavar="NAME",
                    help="time the grid convolutions (HyenaND) on workload G1, G2, G3, GP, G4, GP2 or G5")
    ap.add_argument("--work-mb", default=None, metavar="LIST",
                    help="also time the main forward with four-step pass groups sized by each of these work "
                         "budgets (MiB, comma-separated), reported under 'work_mb_sweep'")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run one 1 GiB device copy first (reference dispatch for counter scaling)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the operator shards by channel with no communication); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import hyena_long_conv_amd as H
    from workloads import CONFIGS, make_activations, make_filter_params

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H.lib()
    if args.grid:
        return run_grid(args, torch, H, dev)
    if args.block:
        return run_block(args, cfg, torch, H, dev)
    if args.backward:
        return run_backward(args, cfg, torch, H, dev)
    if args.fir:
        return run_fir(args, cfg, torch, H, dev)

    # Device-to-device copy of 1 GiB: the practical HBM ceiling on this machine,
    # reported beside the datasheet peak (also the reference dispatch for
    # rocprofv3 counter scaling).
    copy_bps = measure_copy(torch, dev, reps=1 if args.copy_calib else 4)
    out, keep = run_forward(args, cfg, torch, H, dev, copy_bps, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline_parity(cfg, *keep)
    del keep
    torch.cuda.empty_cache()
    also = [c for c in (args.also or "").split(",") if c and c != cfg.name]
    if also:
        out["also"] = {}
        for name in also:
            c = CONFIGS[name]
            o, keep = run_forward(args, c, torch, H, dev, copy_bps, None, None)
            line = {"workload": c.desc, "value": o["value"], "unit": o["unit"], "ms_per_step": o["ms_per_step"],
                    "steps": o["steps"], "dtype": o["dtype"], "roofline": o["roofline"], "timing": o["timing"]}
            if not args.no_cpu_baseline:
                line["cpu_baseline"], line["parity"] = cpu_baseline_parity(c, *keep)
            out["also"][name] = line
            del keep
            torch.cuda.empty_cache()
    print(json.dumps(out))
    return 0


def run_forward(args, cfg, torch, H, dev, copy_bps, steps, warmup):
    """Time hyena_forward on one configuration.  Returns the JSON dict and
    (v, xs, y) of input set 0 for the parity check."""
    import numpy as np
    from workloads import make_activations, make_filter_params

    per_set = min_bytes(cfg)
    sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / per_set))
    p = make_filter_params(cfg)
    pd = {k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    h = H.filter_gen(pd, cfg.L)
    spec0 = H.filter_spectrum(h, circular=args.circular)
    # filter generation and spectrum: once per weight set, outside the timed
    # region; timed here on their own (median of 3, HIP events)
    setup = {}
    for name, fn in (("filter_gen_ms", lambda: H.filter_gen(pd, cfg.L, out=h)),
                     ("filter_spectrum_ms", lambda: H.filter_spectrum(h, out=spec0, circular=args.circular))):
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        setup[name] = sorted(ts)[1]
    del h
    data = []
    for s in range(sets):
        c = cfg.with_(seed=cfg.seed * 100 + s)
        v, xs = make_activations(c, dev)
        spec = spec0 if s == 0 else spec0.clone()
        data.append((v, xs, spec, torch.empty_like(v)))
    wsb = H.forward_workspace_bytes(cfg.B, cfg.D, cfg.N, cfg.L, cfg.io, circular=args.circular)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # One prepared C-ABI call per input set: the timed loop pays no Python
    # argument checks (the library still validates every call on the host).
    calls = [H.PreparedForward(v, xs, spec, out=y, workspace=ws, circular=args.circular) for v, xs, spec, y in data]

    def step(i):
        calls[i % sets]()

    # Warm-up: the given count, or at least 3 steps and 100 ms of GPU work (the
    # clocks settle); the timed count likewise defaults to >= 20 steps and
    # >= 200 ms.
    est = None   # seconds per step, from the warm-up
    if warmup is not None:
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
    else:
        done, t_w = 0, time.perf_counter()
        while done < 3 or time.perf_counter() - t_w < 0.1:
            step(done)
            done += 1
            if done % 8 == 0 or done < 3:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        warmup = done
        est = (time.perf_counter() - t_w) / done
    if steps is None:
        if est is None:
            t_e = time.perf_counter()
            step(0)
            torch.cuda.synchronize()
            est = time.perf_counter() - t_e
        steps = int(min(5000, max(20, math.ceil(0.2 / max(est, 1e-6)))))
    # Timed region: K back-to-back steps between two events on the stream the
    # library launches on (torch's current stream), synchronised on both sides.
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # Step-to-step spread, from a second, untimed pass with an event before
    # every step (each event adds a few microseconds between launches, so
    # these per-step figures sit slightly above ms_per_step).
    n_spread = min(steps, 1000)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
    for i in range(n_spread):
        ev[i].record(stream)
        step(i)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n_spread))
    q = lambda f: per_step[min(len(per_step) - 1, int(f * len(per_step)))]
    t = ms / 1e3
    tokens = cfg.B * cfg.D * cfg.L
    value = tokens / t
    mb, fl = min_bytes(cfg, args.circular), algo_flops(cfg, args.circular)
    hbm_frac = mb / t / HBM_PEAK
    alu_frac = fl / t / ALU_PEAK
    plan = H.plan(cfg.L, circular=args.circular)
    traffic = None if args.circular else measured_traffic(cfg.name)
    single = plan["path"] == "single"
    nc = plan["M"] // 2
    rows = cfg.B * cfg.D
    group = max(1, wsb // (nc * work_point_bytes(cfg))) if not single else rows
    groups = -(-rows // group)
    # The metric's roofline is HBM bandwidth: algorithmic bytes (v, x_1..x_N,
    # y in the I/O dtype, the spectrum once) over the event-timed forward.
    # The unit is one forward: one launch on the single path, (2N + 1)
    # launches per pass group on the four-step path.
    roof = {"bound": "hbm", "achieved": mb / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": hbm_frac,
            "traffic": traffic,
            "kernel": ("k_single_forward" if single else
                       f"four-step forward: {groups} pass group(s) x {2 * cfg.N + 1} launches "
                       f"(k_col FIRST, then per order k_row + k_col)"),
            "unit_of_work": "one hyena_forward (all launches of one step)",
            "launches_per_step": 1 if single else groups * (2 * cfg.N + 1),
            "hbm_GBps": mb / t / 1e9, "copy_GBps": copy_bps / 1e9, "hbm_frac_vs_copy": mb / t / copy_bps,
            "alu_frac": alu_frac, "alu_TFLOPs": fl / t / 1e12, "alu_peak_unpacked_TFLOPs": ALU_PEAK / 1e12,
            "alu_frac_vs_packed_peak": fl / t / ALU_PEAK_PACKED,
            "algorithmic_bytes_per_step": mb, "algorithmic_flops_per_step": fl}
    out = {
        "metric": "Hyena order-N fwd channel-tokens/sec (B*D*L/s) + % of HBM roofline",
        "value": value, "unit": "channel-tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp32" if cfg.io == "fp32" else
                  "bf16 I/O, fp32 compute" + (", bf16 four-step intermediate" if bf16_work(cfg) and not single
                                              else "")),
        "data": "synthetic (seeded N(0,1) activations, DNA-token v for the 1M shape, random-init filter FFN)",
        "config": {"workload": cfg.desc, "name": cfg.name, "N": cfg.N, "B": cfg.B, "D": cfg.D, "L": cfg.L,
                   "io": cfg.io, "ffn_hidden": cfg.H, "fft_len": plan["M"], "path": plan["path"],
                   "n1": plan["n1"], "n2": plan["n2"], "rows_per_group": group if not single else None,
                   "conv": "circular" if args.circular else "linear (zero-padded)",
                   "input_sets": sets, "wall_s": wall},
        "timing": {"ms_mean": ms, "ms_median": q(0.5), "ms_p10": q(0.1), "ms_p90": q(0.9),
                   "spread_from": f"untimed pass of {n_spread} steps with an event before each"},
        "setup": setup,
        "roofline": roof,
    }
    if getattr(args, "work_mb", None):
        out["work_mb_sweep"] = work_budget_sweep(args, cfg, torch, H, dev, data, sets, stream)
    v0, xs0, _, y0 = data[0]
    del data, calls, ws
    return out, (v0, xs0, y0)


def work_budget_sweep(args, cfg, torch, H, dev, data, sets, stream):
    """The same forward with the four-step pass groups sized by each work
    budget of --work-mb (MiB; the library reads HYENA_WORK_MB at every call):
    ms per forward from events around max(20, steps) forwards after 3 warm-up
    forwards, and the HBM roofline fraction."""
    budgets = [int(b) for b in str(args.work_mb).split(",") if b]
    nc = H.plan(cfg.L)["M"] // 2
    esz = work_point_bytes(cfg)
    ws = torch.empty(max(max(budgets) << 20, nc * esz), dtype=torch.uint8, device=dev)
    old = os.environ.get("HYENA_WORK_MB")
    res = {}
    try:
        for mb in budgets:
            os.environ["HYENA_WORK_MB"] = str(mb)
            calls = [H.PreparedForward(v, xs, spec, out=y, workspace=ws) for v, xs, spec, y in data]
            for i in range(3):
                calls[i % sets]()
            n = 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n):
                calls[i % sets]()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            rows = max(1, min(cfg.B * cfg.D, (mb << 20) // (nc * esz)))
            res[str(mb)] = {"ms_per_step": ms, "rows_per_group_max": rows,
                            "hbm_frac": min_bytes(cfg) / (ms / 1e3) / HBM_PEAK}
    finally:
        if old is None:
            os.environ.pop("HYENA_WORK_MB", None)
        else:
            os.environ["HYENA_WORK_MB"] = old
    del ws
    return res


if __name__ == "__main__":
    sys.exit(main())
