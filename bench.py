"""Benchmark of the hierarchical locality-preserving attention path on one GPU.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM, raster-order q, k, v in and raster-order o out:
    cube reorder + 3D RoPE of q and of k, fused in one pass (detail rows read
      in raster order, written rotated in cube order; the global proxy
      rotated in place)
    cube reorder of v (raster -> cube order)
    hierarchical attention (detail -> own cube + all global; global -> global)
      with the cube unorder fused into its epilogue (detail output written in
      raster order)
``--unfused`` runs the same path as four separate passes (reorder q, k, v;
RoPE q, k; attention; unorder o).  The global q/k are rotated in place, so
each step first restores them from pristine copies (two device-to-device
copies, 0.67 GB at 4K, counted in the step time).

Prints ONE JSON line.  ``value`` is the useful attention FLOPs of a step
divided by the step time (TFLOP/s); the per-kernel figures come from HIP
events recorded around every launch on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hier-attn TFLOP/s (useful FLOPs) + % bf16 MFMA peak at 4K; reorder GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "windowed_global_local_amd", "csrc", "hier_attn.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def file_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def pmc_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary of
    this workload, or None when there is none or the kernel source changed
    since it was taken."""
    try:
        with open(os.path.join(PROFILES, f"hier_attn_{workload}_pmc.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != file_sha256(ATTN_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model():
    """CPU model name of this host (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_sample(cfg, rng, max_outliers=1024):
    """Query rows the attention oracle is timed on: every row of 4 windows
    (first, last, two random) in each of 4 heads (first, last, two random),
    4,096 random detail rows over all heads, 1,024 random global rows and, on
    workloads with outlier rows, up to max_outliers q outlier rows of the 4
    sampled heads.  Returns (rows, heads, is_global) and its useful FLOPs."""
    from workload import outlier_rows
    N, V, G, H, C = cfg.N, cfg.V, cfg.G, cfg.heads, cfg.C
    hs = np.unique(np.concatenate([[0, H - 1], rng.choice(H, 2, replace=False)]))
    ws = np.unique(np.concatenate([[0, C - 1], rng.choice(C, 2, replace=False)]))
    rows, heads = [], []
    for h in hs:
        for c in ws:
            rows.append(np.arange(c * V, (c + 1) * V))
            heads.append(np.full(V, h))
    rows.append(rng.integers(0, N, 4096))
    heads.append(rng.integers(0, H, 4096))
    if cfg.outliers:
        # the oracle is handed the input tensors as they are, so the q outlier
        # rows of the input are outlier queries of the timed computation
        orows = np.nonzero(outlier_rows(cfg.seed, 0, N))[0]
        pick = rng.choice(orows, size=min(max_outliers, orows.size), replace=False)
        rows.append(pick)
        heads.append(rng.choice(hs, pick.size))
    n_d = sum(r.size for r in rows)
    n_g = min(1024, G)
    rows.append(rng.integers(0, G, n_g))
    heads.append(rng.integers(0, H, n_g))
    glob = np.concatenate([np.zeros(n_d), np.ones(n_g)]).astype(np.int8)
    flops = 4.0 * cfg.head_dim * (n_d * (V + G) + n_g * G)
    return (np.concatenate(rows).astype(np.int64), np.concatenate(heads).astype(np.int32), glob), flops


def cpu_baseline(cfg, ins, full_attention):
    """Time the fp64 oracle, untuned, on this host: the reorder at full size,
    the attention on the sampled rows of oracle_sample (or on every row when
    full_attention), with the full-size attention time extrapolated by the
    useful-FLOP ratio."""
    import oracle
    oracle._load()
    rng = np.random.default_rng(7)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    full_flops = 4.0 * cfg.head_dim * cfg.heads * (cfg.N * (cfg.V + cfg.G) + cfg.G * cfg.G)
    row_bytes = cfg.heads * cfg.head_dim * cfg.esize

    t0 = time.perf_counter()
    y = oracle.cube_reorder(ins["v_d"], cfg.grid, cfg.cube)
    t_reorder = time.perf_counter() - t0
    del y

    if full_attention:
        # head by head (heads are independent), with a progress line per head;
        # only the oracle calls are timed
        t_attn = 0.0
        for h in range(cfg.heads):
            one = {k: (np.ascontiguousarray(v[:, h:h + 1]) if v is not None else None) for k, v in ins.items()}
            t0 = time.perf_counter()
            oracle.hier_attn(one["q_d"], one["k_d"], one["v_d"], one["q_g"], one["k_g"], one["v_g"], cfg.V)
            t_attn += time.perf_counter() - t0
            log(f"cpu baseline: head {h + 1}/{cfg.heads} done, {t_attn:.1f} s of oracle time")
        flops = full_flops
        sample = f"every query row of every head of the {cfg.name} workload (full attention oracle, one head per call)"
    else:
        sel, flops = oracle_sample(cfg, rng)
        t0 = time.perf_counter()
        oracle.hier_attn(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"], ins["v_g"], cfg.V,
                         sel=sel)
        t_attn = time.perf_counter() - t0
        n_g = int(sel[2].sum())
        sample = (f"{sel[0].size - n_g} detail query rows (all rows of 4 windows x 4 heads, 4096 random "
                  f"rows{', up to 1024 q outlier rows of the sampled heads' if cfg.outliers else ''}) + "
                  f"{n_g} global query rows of the {cfg.name} workload (inputs unrotated, as the "
                  f"attention stage consumes them); value = useful FLOPs of the sample / wall time")
    value = flops / t_attn / 1e12
    return {
        "value": value, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": sample,
        "seconds": round(t_attn, 3),
        "attention_full_s": round(full_flops / (value * 1e12), 3),
        "attention_full_s_kind": "measured" if full_attention else "extrapolated (useful-FLOP ratio)",
        "reorder_full_s": round(t_reorder, 3),
        "reorder_GBps": round(2 * cfg.N * row_bytes / t_reorder / 1e9, 2),
    }


def time_backward(A, cfg, x, qc, kc, vc, qg, kg, stream, reps, fwd_flops, subset=None):
    """Forward with log-sum-exp, then the backward, on the step's cube-order
    rotated q/k and reordered v; seeded N(0,1) upstream gradients.  subset =
    (goff, gidx) device lists times the per-window subset mask instead."""
    import numpy as np
    import torch

    from workload import gen_grad_outputs

    g, c, gp = cfg.grid, cfg.cube, cfg.gproxy
    log("backward: generating upstream gradients")
    gos = gen_grad_outputs(cfg)
    dO = {k: torch.from_numpy(v.view(np.int16)).to("cuda").view(torch.bfloat16)
          if v.dtype == np.uint16 else torch.from_numpy(v).to("cuda") for k, v in gos.items()}
    del gos
    o_c, o_g = torch.empty_like(qc), torch.empty_like(qg)
    lse_d = torch.empty(cfg.heads, cfg.N, dtype=torch.float32, device="cuda")
    lse_g = torch.empty(cfg.heads, cfg.G, dtype=torch.float32, device="cuda")
    ws_fn = A.atlas_hier_attn_subset_bwd_workspace_bytes if subset else A.atlas_hier_attn_bwd_workspace_bytes
    ws = torch.empty(ws_fn(g, c, gp, cfg.heads, cfg.head_dim) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(qc) for _ in range(3))
    dqg, dkg, dvg = (torch.empty_like(qg) for _ in range(3))

    if subset:
        goff, gidx = subset

        def fwd():
            A.atlas_hier_attn_subset_fwd(o_c, o_g, lse_d, lse_g, qc, kc, vc, qg, kg, x["v_g"], goff, gidx,
                                         g, c, gp, 0.0, stream)

        def bwd():
            A.atlas_hier_attn_subset_bwd(dq, dk, dv, dqg, dkg, dvg, qc, kc, vc, qg, kg, x["v_g"], o_c, o_g,
                                         dO["do_d"], dO["do_g"], lse_d, lse_g, goff, gidx, ws, g, c, gp,
                                         0.0, stream)
    else:
        def fwd():
            A.atlas_hier_attn_fwd(o_c, o_g, lse_d, lse_g, qc, kc, vc, qg, kg, x["v_g"], g, c, gp, 0.0,
                                  stream)

        def bwd():
            A.atlas_hier_attn_bwd(dq, dk, dv, dqg, dkg, dvg, qc, kc, vc, qg, kg, x["v_g"], o_c, o_g,
                                  dO["do_d"], dO["do_g"], lse_d, lse_g, ws, g, c, gp, 0.0, stream)

    fwd()
    bwd()
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("fwd_lse", fwd), ("bwd", bwd)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    ok = all(bool(torch.isfinite(t.float()).all()) for t in (dq, dk, dv, dqg, dkg, dvg))
    # useful backward FLOPs: 2.5x the forward's (five products of 2*head_dim per
    # allowed pair against the forward's two); the kernels execute S and dP
    # twice (dq pass and dk/dv pass): 14*head_dim per pair
    useful = 2.5 * fwd_flops
    executed = 3.5 * fwd_flops
    tfl = useful / (res["bwd"] * 1e-3) / 1e12
    log(f"backward {res['bwd']:.1f} ms, {tfl:.1f} TFLOP/s useful")
    out = {
        "ms": round(res["bwd"], 3),
        "fwd_lse_ms": round(res["fwd_lse"], 3),
        "useful_flops": useful,
        "useful_tflops": round(tfl, 2),
        "frac_bf16_peak": round(tfl / PEAK_BF16_TFLOPS, 4),
        "executed_tflops": round(executed / (res["bwd"] * 1e-3) / 1e12, 2),
        "reps": reps,
        "finite": ok,
    }
    del dO, o_c, o_g, lse_d, lse_g, ws, dq, dk, dv, dqg, dkg, dvg
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="4k-latent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the attention oracle on every row (tiny and 720P workloads), "
                         "not on the sample")
    ap.add_argument("--mask", choices=("cube", "aligned", "block"), default="cube",
                    help="cube: detail queries see their cube + all global keys (default); "
                         "aligned: their cube + the co-located global keys; "
                         "block: naive block attention on raster order (no reorder)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of the attention backward pass")
    ap.add_argument("--backward-reps", type=int, default=2)
    ap.add_argument("--calib-bytes", type=int, default=0,
                    help="before the warmup, run one plain elementwise copy (torch.neg of an int32 "
                         "tensor) that reads and writes exactly this many bytes: the reference "
                         "dispatch that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters; at "
                         "most 2 GiB, since torch splits a larger one into several dispatches")
    ap.add_argument("--unfused", action="store_true",
                    help="run reorder, RoPE, attention and unorder as separate passes")
    args = ap.parse_args()

    if args.calib_bytes > 2 ** 31:
        ap.error("--calib-bytes above 2 GiB would run as several dispatches")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import windowed_global_local_amd as A
    from workload import by_name, gen_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    A.load()
    cfg = by_name(args.workload)
    g, c, gp = cfg.grid, cfg.cube, cfg.gproxy

    log(f"generating {cfg.name} inputs")
    t0 = time.time()
    ins = gen_inputs(cfg)
    log(f"generated in {time.time() - t0:.1f}s; uploading")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    x = {k: to_dev(v) for k, v in ins.items()}
    qc, kc, vc = (torch.empty_like(x[n]) for n in ("q_d", "k_d", "v_d"))
    qg, kg = torch.empty_like(x["q_g"]), torch.empty_like(x["k_g"])
    oc = torch.empty_like(qc) if args.unfused else None
    og, od = torch.empty_like(qg), torch.empty_like(qc)
    stream = torch.cuda.current_stream()

    flops = A.atlas_hier_attn_useful_flops(g, c, gp, cfg.heads, cfg.head_dim)
    if args.mask == "aligned":
        goff_h, gidx_h = A.atlas_aligned_subset(g, c, gp, cfg.r_t)
        goff_t = torch.as_tensor(goff_h, device="cuda")
        gidx_t = torch.as_tensor(gidx_h, device="cuda")
        oc = torch.empty_like(qc)
        names = ("reorder_rope_q", "reorder_rope_k", "reorder_v", "hier_attn", "unorder_o")
        calls = (
            ("reorder_rope_q", lambda: A.atlas_cube_reorder_rope3d(qc, x["q_d"], qg, g, c, gp, cfg.r_t,
                                                                   cfg.theta, stream)),
            ("reorder_rope_k", lambda: A.atlas_cube_reorder_rope3d(kc, x["k_d"], kg, g, c, gp, cfg.r_t,
                                                                   cfg.theta, stream)),
            ("reorder_v", lambda: A.atlas_cube_reorder(vc, x["v_d"], g, c, stream)),
            ("hier_attn", lambda: A.atlas_hier_attn_subset(oc, og, qc, kc, vc, qg, kg, x["v_g"], goff_t,
                                                           gidx_t, g, c, gp, 0.0, stream)),
            ("unorder_o", lambda: A.atlas_cube_unorder(od, oc, g, c, stream)),
        )
        # allowed pairs: window keys for every detail query, the listed global
        # keys for the queries of their window, all global keys per global query
        V = cfg.V
        pairs = cfg.N * V + V * float(goff_h[-1]) + float(cfg.G) * cfg.G
        flops = 4.0 * cfg.head_dim * cfg.heads * pairs
    elif args.mask == "block":
        # no reorder: RoPE at raster positions (cube = grid), attention on the
        # raster tensors (windows = V consecutive raster tokens), raster output
        qr, kr = torch.empty_like(x["q_d"]), torch.empty_like(x["k_d"])
        names = ("rope_q", "rope_k", "hier_attn")
        calls = (
            ("rope_q", lambda: (qr.copy_(x["q_d"]), A.atlas_rope3d(qr, qg, g, g, gp, cfg.r_t, cfg.theta,
                                                                   stream))),
            ("rope_k", lambda: (kr.copy_(x["k_d"]), A.atlas_rope3d(kr, kg, g, g, gp, cfg.r_t, cfg.theta,
                                                                   stream))),
            ("hier_attn", lambda: A.atlas_hier_attn(od, og, qr, kr, x["v_d"], qg, kg, x["v_g"], g, c, gp,
                                                    0.0, stream)),
        )
    elif args.unfused:
        names = ("reorder_q", "reorder_k", "reorder_v", "rope_q", "rope_k", "hier_attn", "unorder_o")
        calls = (
            ("reorder_q", lambda: A.atlas_cube_reorder(qc, x["q_d"], g, c, stream)),
            ("reorder_k", lambda: A.atlas_cube_reorder(kc, x["k_d"], g, c, stream)),
            ("reorder_v", lambda: A.atlas_cube_reorder(vc, x["v_d"], g, c, stream)),
            ("rope_q", lambda: A.atlas_rope3d(qc, qg, g, c, gp, cfg.r_t, cfg.theta, stream)),
            ("rope_k", lambda: A.atlas_rope3d(kc, kg, g, c, gp, cfg.r_t, cfg.theta, stream)),
            ("hier_attn", lambda: A.atlas_hier_attn(oc, og, qc, kc, vc, qg, kg, x["v_g"], g, c, gp,
                                                    0.0, stream)),
            ("unorder_o", lambda: A.atlas_cube_unorder(od, oc, g, c, stream)),
        )
    else:
        names = ("reorder_rope_q", "reorder_rope_k", "reorder_v", "hier_attn")
        calls = (
            ("reorder_rope_q", lambda: A.atlas_cube_reorder_rope3d(qc, x["q_d"], qg, g, c, gp, cfg.r_t,
                                                                   cfg.theta, stream)),
            ("reorder_rope_k", lambda: A.atlas_cube_reorder_rope3d(kc, x["k_d"], kg, g, c, gp, cfg.r_t,
                                                                   cfg.theta, stream)),
            ("reorder_v", lambda: A.atlas_cube_reorder(vc, x["v_d"], g, c, stream)),
            ("hier_attn", lambda: A.atlas_hier_attn_raster(od, og, qc, kc, vc, qg, kg, x["v_g"], g, c,
                                                           gp, 0.0, stream)),
        )
    times = {n: [] for n in names}

    def step(rec):
        qg.copy_(x["q_g"])
        kg.copy_(x["k_g"])
        evs = []
        for name, fn in calls:
            if rec:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                evs.append((name, e0, e1))
            else:
                fn()
        return evs

    if args.calib_bytes > 0:
        n = args.calib_bytes // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: {4 * n} bytes read and written by one neg kernel")
        del src, dst

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    all_evs = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        all_evs.extend(step(True))
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    for name, e0, e1 in all_evs:
        times[name].append(e0.elapsed_time(e1))
    avg = {n: float(np.mean(times[n])) for n in names}
    med = {n: float(np.median(times[n])) for n in names}
    ms_per_step = total_ms / args.steps

    if not (torch.isfinite(od.float()).all() and torch.isfinite(og.float()).all()):
        log("non-finite outputs")
        sys.exit(1)

    row_bytes = cfg.heads * cfg.head_dim * cfg.esize
    copy_bytes = 2 * cfg.N * row_bytes
    rope_bytes = 2 * (cfg.N + cfg.G) * row_bytes
    attn_tflops = flops / (avg["hier_attn"] * 1e-3) / 1e12
    if args.mask == "block":
        # no reorder; the timed rotation includes a copy of the raster input
        reorder_gbps = rope_gbps = None
    elif args.unfused:
        reorder_gbps = 3 * copy_bytes / ((avg["reorder_q"] + avg["reorder_k"] + avg["reorder_v"]) * 1e-3) / 1e9
        rope_gbps = 2 * rope_bytes / ((avg["rope_q"] + avg["rope_k"]) * 1e-3) / 1e9
    else:
        reorder_gbps = copy_bytes / (avg["reorder_v"] * 1e-3) / 1e9
        # the fused pass moves the bytes of the RoPE pass alone (rows in, rows out)
        rope_gbps = 2 * rope_bytes / ((avg["reorder_rope_q"] + avg["reorder_rope_k"]) * 1e-3) / 1e9
    value = flops / (ms_per_step * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v; 1% q/k outlier rows x8 on the 4K workload)",
        "config": dict(cfg.describe(), parallelism="single GPU"),
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": pmc_traffic(cfg.name),
        },
        "kernels_ms": {n: round(avg[n], 4) for n in names},
        "kernels_ms_median": {n: round(med[n], 4) for n in names},
        "hier_attn_tflops_median": round(flops / (med["hier_attn"] * 1e-3) / 1e12, 2),
        "hier_attn_tflops": round(attn_tflops, 2),
        "hier_attn_frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "reorder_GBps": None if reorder_gbps is None else round(reorder_gbps, 1),
        "reorder_frac_hbm": None if reorder_gbps is None else round(reorder_gbps / PEAK_HBM_GBPS, 4),
        "rope_GBps": None if rope_gbps is None else round(rope_gbps, 1),
        "rope_frac_hbm": None if rope_gbps is None else round(rope_gbps / PEAK_HBM_GBPS, 4),
        "path": {"aligned": "aligned global subset: fused reorder+RoPE, subset attention, unorder",
                 "block": "naive block attention on raster order: RoPE, attention (no reorder)"}.get(
                     args.mask, "unfused" if args.unfused else
                     "fused (reorder+RoPE, attention raster epilogue)"),
        "mask": args.mask,
        "useful_flops_per_step": flops,
        "gpu": torch.cuda.get_device_name(0),
        "cpu_baseline": None,
    }
    if not args.no_backward and args.mask in ("cube", "aligned"):
        out["backward"] = time_backward(A, cfg, x, qc, kc, vc, qg, kg, stream, args.backward_reps,
                                        flops, (goff_t, gidx_t) if args.mask == "aligned" else None)
    del x, qc, kc, vc, qg, kg, oc, og, od
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle (reorder at full size, attention on "
            + ("every row)" if args.cpu_full else "the sample)"))
        out["cpu_baseline"] = cpu_baseline(cfg, ins, args.cpu_full)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
