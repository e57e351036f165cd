"""Benchmark: one step = the whole hot path on one seeded synthetic batch:
build the neighbour map from coordinates (key pack + Morton sort + hash insert
+ tile query), pack the weights and run the fused gather-GEMM-accumulate
forward.

Headline workload: surf256 -- the union of 16 random sphere shells and 8
random planes clipped to a 256^3 grid (1,006,716 surface voxels), K=27 (3x3x3,
dilation 1), Ci=Co=128, bf16 features and weights, fp32 accumulation, bf16
out.

Prints one JSON line.  `value` = effective TFLOP/s of a step,
2 * valid_pairs * Ci * Co / step time (inputs resident in HBM).  The forward
kernel's own rate against the bf16 MFMA peak is in `roofline`; the oracle's
rate on the host cores is in `cpu_baseline`.  `configs` times the forward of
each of the five workloads (uniform32, shell64, surf256, surf1024,
surf512d2) with its peak extra device memory, roofline fraction and an oracle
baseline.  Hardware counters (HBM traffic, matrix-core busy fraction) come
from the summaries rocprof_harness.py writes under profiles/, used while the
kernel source they were taken on is unchanged.

`--profile-run` is the short program the harness runs under rocprofv3: one
workload's map, packed weights and a few forwards (plus, optionally, a copy
of known size for scaling the byte counters).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (2·valid_pairs·Ci·Co) + peak extra HBM, 1 MI355X"
# MI355X published dense peaks (256 CUs at 2.4 GHz) and HBM bandwidth
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
ALL_WORKLOADS = ["uniform32", "shell64", "surf256", "surf1024", "surf512d2"]
FORWARD_SRC = os.path.join(ROOT, "submanifold_sparse_convolution_spconv_amd", "csrc", "forward.hip")
WGRAD_SRC = os.path.join(ROOT, "submanifold_sparse_convolution_spconv_amd", "csrc", "wgrad.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="surf256")
    p.add_argument("--fwd-iters", type=int, default=50, help="extra forward-only launches timed with events")
    p.add_argument("--cpu-seconds", type=float, default=4.0, help="budget of each oracle CPU-baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--configs", default=",".join(ALL_WORKLOADS),
                   help="workloads whose forward is timed in `configs` ('' skips)")
    p.add_argument("--shard-workload", default="surf1024", help="workload of the one-GPU shard run ('' skips it)")
    p.add_argument("--shard-parts", type=int, default=8)
    p.add_argument("--profile-run", action="store_true",
                   help="only build, pack and run --fwd-iters forwards of --workload (for rocprofv3)")
    p.add_argument("--wgrad-iters", type=int, default=0,
                   help="--profile-run: weight-gradient calls after the forwards")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="after the run, copy a buffer of this many MiB a few times (a plain copy kernel "
                        "of known size, for scaling hardware byte counters)")
    return p.parse_args()


def source_hash(path=FORWARD_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def profile_summary(wl, kind="fwd"):
    """Fields of the committed rocprof summary of this workload's forward
    (kind "fwd") or weight gradient ("wgrad"), provided it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{wl.dtype}_{wl.name}_rocprof.txt")
    try:
        fields = {}
        for line in open(path):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
        if fields.get("kernel_source_sha256_16") != source_hash(FORWARD_SRC if kind == "fwd" else WGRAD_SRC):
            return None
        return fields
    except OSError:
        return None


def fwd_flops(wl, vp):
    return 2.0 * vp * wl.Ci * wl.Co


def fwd_alg_bytes(wl, N):
    s = 2 if wl.dtype == "bf16" else 4
    return N * wl.Ci * s + wl.K * wl.Ci * wl.Co * s + 4 * wl.K * N + N * wl.Co * s + 4 * wl.Co


def wgrad_alg_bytes(wl, N):
    """feats and dout read once, the map's K x N neighbour indices, dw written once"""
    s = 2 if wl.dtype == "bf16" else 4
    return N * wl.Ci * s + N * wl.Co * s + 4 * wl.K * N + wl.K * wl.Ci * wl.Co * s


def dtype_code(sp, wl):
    return sp.SPCONV_BF16 if wl.dtype == "bf16" else sp.SPCONV_F32


def device_values(torch, wl, N, dev, seed):
    """Values of the workload's distributions drawn on the device (the timing
    does not depend on them; the seeded host recipe is used where outputs are
    checked)."""
    g = torch.Generator(device=dev).manual_seed(seed)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    f = torch.randn((N, wl.Ci), generator=g, device=dev).to(dt)
    w = (torch.randn((wl.K, wl.Ci, wl.Co), generator=g, device=dev) / (27 * wl.Ci) ** 0.5).to(dt)
    b = torch.randn((wl.Co,), generator=g, device=dev) * 0.1 ** 0.5
    return f, w, b


def oracle_sample(coords, feats, w, bias, K, dilation, budget_s, full_map):
    """One bounded timing of the oracle: (map time, forward time per row, rows
    done, valid pairs).  With full_map the whole neighbour map is built and
    timed; otherwise only the sampled rows' columns are looked up (untimed)."""
    import numpy as np
    import oracle
    N = coords.shape[0]
    t_map = None
    if full_map:
        t0 = time.perf_counter()
        nb = oracle.nmap(coords, K, dilation)
        t_map = time.perf_counter() - t0
    done, t_fwd, chunk = 0, 0.0, 4096
    while done < N and t_fwd < budget_s:
        m = min(chunk, N - done)
        cols = (np.ascontiguousarray(nb[:, done:done + m]) if full_map
                else oracle.nmap_rows(coords, np.arange(done, done + m), K, dilation))
        t0 = time.perf_counter()
        oracle.forward(feats, cols, w, bias, with_abs=False)
        t_fwd += time.perf_counter() - t0
        done += m
        chunk = min(chunk * 2, 1 << 16)
    return t_map, t_fwd / done, done


def cpu_baseline(coords, feats, w, bias, wl, vp, budget_s, runs, full_map):
    """The oracle timed on the host cores on bounded samples of the workload:
    median of `runs` samples on all threads, plus one single-thread sample.
    value = effective TFLOP/s of the oracle's step (map + forward, the forward
    time scaled from the sampled rows to all rows), or of its forward alone
    when full_map is False."""
    import oracle
    N = coords.shape[0]
    flops = fwd_flops(wl, vp)
    cores = oracle.threads()

    def one(budget):
        t_map, per_row, done = oracle_sample(coords, feats, w, bias, wl.K, wl.dilation, budget, full_map)
        return (t_map or 0.0) + per_row * N, t_map, done

    res = sorted((one(budget_s) for _ in range(runs)), key=lambda r: r[0])
    t_step, t_map, done = res[len(res) // 2]
    oracle.set_threads(1)
    try:
        t1, _, done1 = one(budget_s / 2)
    finally:
        oracle.set_threads(cores)
    what = "full neighbour map + " if full_map else ""
    return {"value": flops / t_step / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}fp64 forward of the first {done} of {N} caller rows, forward time scaled to "
                      f"all rows; median of {runs} sample(s)"
                      + (f" (map {t_map:.2f}s)" if t_map is not None else " (map columns looked up, untimed)"),
            "one_thread": {"value": flops / t1 / 1e12, "cores": 1,
                           "sample": f"{what}fp64 forward of {done1} rows on one thread, scaled"}}


def per_launch(torch, fn, stream, dev, runs=20):
    """Median and min of `runs` launches of fn, flushed (a 512 MB write before
    each, beyond the 256 MB Infinity Cache) and warm (back to back).  The
    device is kept busy while the host queues the launches (the flush itself,
    or a spin kernel ahead of the warm ones), so that the events time the
    launches and not the host's call overhead."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for kind in ("flushed", "warm"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        if kind == "warm":
            torch.cuda._sleep(40_000_000)
        for i in range(runs):
            if kind == "flushed":
                flush.fill_(i + 1)
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        t = sorted(s_.elapsed_time(e_) for s_, e_ in evs)
        out[kind] = {"median_ms": (t[runs // 2 - 1] + t[runs // 2]) / 2, "min_ms": t[0]}
    del flush
    return out


def config_run(sp, torch, W, dev, name, cpu_budget, with_cpu):
    """Forward of one workload: peak extra device memory of build + pack +
    forward, flushed and warm per-launch times, roofline fraction against the
    dtype's peak, and an oracle baseline on a bounded sample."""
    wl = W.by_name(name)
    coords = W.geometry(wl)
    N = coords.shape[0]
    c_d = torch.from_numpy(coords).to(dev)
    f_d, w_d, b_d = device_values(torch, wl, N, dev, 1000 + wl.index)
    out = torch.empty((N, wl.Co), dtype=w_d.dtype, device=dev)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    nm = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
    wp = sp.spconv_pack_weights(w_d)
    sp.spconv_forward_packed(f_d, nm, w_d, wp, b_d, out=out)
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated(dev) - base
    vp = nm.valid_pairs
    for _ in range(3):
        sp.spconv_forward_packed(f_d, nm, w_d, wp, b_d, out=out)
    stream = torch.cuda.current_stream(dev)
    pl = per_launch(torch, lambda: sp.spconv_forward_packed(f_d, nm, w_d, wp, b_d, out=out), stream, dev, 10)
    b_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        tb = time.perf_counter()
        nm_b = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
        b_ms.append((time.perf_counter() - tb) * 1e3)
    del nm_b
    flops = fwd_flops(wl, vp)
    ms = pl["flushed"]["median_ms"]
    achieved = flops / (ms * 1e-3) / 1e12
    res = {"N": N, "valid_pairs": vp, "K": wl.K, "dilation": wl.dilation, "Ci": wl.Ci, "Co": wl.Co,
           "dtype": wl.dtype, "forward_ms_flushed_median": ms, "forward_ms_warm_median": pl["warm"]["median_ms"],
           "forward_ms_flushed_min": pl["flushed"]["min_ms"], "forward_tflops": achieved,
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                        "frac": achieved / PEAK_TFLOPS[wl.dtype]},
           "algorithmic_bytes": fwd_alg_bytes(wl, N),
           "peak_extra_hbm_bytes": int(peak_extra), "peak_extra_hbm_bytes_per_voxel": peak_extra / N,
           "materialised_gather_bytes": int(wl.K) * N * wl.Ci * (2 if wl.dtype == "bf16" else 4),
           "build_ms_median": sorted(b_ms)[1]}
    prof = profile_summary(wl)
    if prof:
        res["counters"] = {k: prof[k] for k in ("kernel", "traffic_bytes_per_launch", "hbm_gbs", "hbm_frac",
                                                "mfma_busy_frac", "executed_over_useful") if k in prof}
    if with_cpu:
        host = (f_d.cpu(), w_d.cpu(), b_d.cpu())
        runs = 3 if wl.index <= 3 else 1
        res["cpu_baseline"] = cpu_baseline(coords, *host, wl, vp, cpu_budget, runs, full_map=False)
    del nm, wp, f_d, w_d, b_d, out, c_d
    torch.cuda.empty_cache()
    return res


def shard_run(sp, torch, W, dev, name, parts):
    """One GPU's share of a P-way spatial split: Morton ranges of the global
    schedule balanced by valid pairs; the heaviest range's rows plus their
    halo (neighbours owned by other ranges) are built and convolved on this
    GPU, the halo rows appended after the own rows.  Values are drawn on the
    device (the timing does not depend on them)."""
    wl = W.by_name(name)
    c_all = torch.from_numpy(W.geometry(wl)).to(dev)
    N = c_all.shape[0]
    nm = sp.spconv_build_nmap(c_all, wl.K, wl.dilation)
    nbr, order = nm.export()
    del nm
    cnt = (nbr != N).sum(0, dtype=torch.int64)                    # valid pairs per caller row
    cum = torch.cumsum(cnt[order.long()], 0)
    total = int(cum[-1])
    cuts = [0] + [int(torch.searchsorted(cum, total * i // parts)) for i in range(1, parts)] + [N]
    loads = [int(cum[b - 1]) - (int(cum[a - 1]) if a else 0) for a, b in zip(cuts[:-1], cuts[1:])]
    s = max(range(parts), key=lambda i: loads[i])
    own = order[cuts[s]:cuts[s + 1]].long()
    inside = torch.zeros(N + 1, dtype=torch.bool, device=dev)
    inside[own] = True
    inside[N] = True                                               # the sentinel
    nb = nbr[:, own].reshape(-1).long()
    halo = torch.unique(nb[~inside[nb]])
    del nbr, nb, inside
    rows = torch.cat([own, halo])
    c_s = c_all[rows].contiguous()
    del c_all
    Ns, H = own.numel(), halo.numel()
    f_s, w_s, b_s = device_values(torch, wl, Ns + H, dev, 777)
    wp = sp.spconv_pack_weights(w_s)
    o_s = torch.empty((Ns + H, wl.Co), dtype=w_s.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        sp.spconv_forward_packed(f_s, sp.spconv_build_nmap(c_s, wl.K, wl.dilation), w_s, wp, b_s, out=o_s)
    torch.cuda.synchronize()
    tb = time.perf_counter()
    nm_s = sp.spconv_build_nmap(c_s, wl.K, wl.dilation)
    build_ms = (time.perf_counter() - tb) * 1e3
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record(stream)
    for _ in range(10):
        sp.spconv_forward_packed(f_s, nm_s, w_s, wp, b_s, out=o_s)
    e_ev.record(stream)
    torch.cuda.synchronize()
    fwd_ms = s_ev.elapsed_time(e_ev) / 10
    return {"workload": f"{name} split {parts} ways; shard {s} (the most valid pairs)",
            "own_rows": Ns, "halo_rows": H, "halo_fraction": H / Ns,
            "own_valid_pairs": loads[s], "computed_valid_pairs": nm_s.valid_pairs,
            "build_ms": build_ms, "forward_ms": fwd_ms,
            "tflops_own": 2.0 * loads[s] * wl.Ci * wl.Co / (fwd_ms * 1e-3) / 1e12,
            "what": "own rows + appended halo rows built and convolved on one GPU; tflops_own counts only "
                    "the own rows' valid pairs (halo rows' outputs are discarded)"}


def calibrate_copy(torch, dev, mib):
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def profile_run(a, sp, torch, W, dev):
    """The program rocprof_harness.py profiles: --fwd-iters steps as the
    timed region runs them (neighbour map, weight pack, forward), then
    --wgrad-iters weight gradients back to back on the last map, then the
    optional copy calibration.  (Forwards back to back with nothing between
    them run the chip at a lower clock after a few milliseconds: the step
    keeps the forward's conditions those of the timed region.)"""
    wl = W.by_name(a.workload)
    coords = W.geometry(wl)
    N = coords.shape[0]
    c_d = torch.from_numpy(coords).to(dev)
    f_d, w_d, b_d = device_values(torch, wl, N, dev, 1000 + wl.index)
    out = torch.empty((N, wl.Co), dtype=w_d.dtype, device=dev)
    wp = torch.empty(sp.spconv_pack_weights_size(wl.K, wl.Ci, wl.Co, dtype_code(sp, wl)),
                     dtype=torch.uint8, device=dev)
    nm = None
    for _ in range(max(a.fwd_iters, 1)):
        nm = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
        sp.spconv_pack_weights(w_d, out=wp)
        sp.spconv_forward_packed(f_d, nm, w_d, wp, b_d, out=out)
    if a.wgrad_iters:
        g = torch.Generator(device=dev)
        g.manual_seed(2000 + wl.index)
        dout = torch.randn((N, wl.Co), generator=g, device=dev).to(w_d.dtype)
        wws = torch.empty(sp.spconv_wgrad_workspace_size(N, wl.K, wl.Ci, wl.Co, dtype_code(sp, wl)),
                          dtype=torch.uint8, device=dev)
        dwo = torch.empty((wl.K, wl.Ci, wl.Co), dtype=w_d.dtype, device=dev)
        for _ in range(a.wgrad_iters):
            sp.spconv_wgrad(f_d, dout, nm, out=dwo, workspace=wws)
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": wl.name, "N": N, "valid_pairs": nm.valid_pairs, "forwards": a.fwd_iters,
                      "wgrads": a.wgrad_iters,
                      "flops_per_forward": fwd_flops(wl, nm.valid_pairs),
                      "algorithmic_bytes_per_forward": fwd_alg_bytes(wl, N),
                      "algorithmic_bytes_per_wgrad": wgrad_alg_bytes(wl, N),
                      "kernel_source_sha256_16": source_hash(),
                      "wgrad_source_sha256_16": source_hash(WGRAD_SRC)}), flush=True)
    if a.calibrate_copy_mib:
        calibrate_copy(torch, dev, a.calibrate_copy_mib)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import workloads as W
    import submanifold_sparse_convolution_spconv_amd as sp

    dev = torch.device("cuda:0")
    if a.profile_run:
        profile_run(a, sp, torch, W, dev)
        return
    wl = W.by_name(a.workload)
    coords = W.geometry(wl)
    N = coords.shape[0]
    feats, w, bias = W.values(wl, N)
    c_d = torch.from_numpy(coords).to(dev)
    f_d, w_d, b_d = feats.to(dev), w.to(dev), bias.to(dev)
    out = torch.empty((N, wl.Co), dtype=w_d.dtype, device=dev)
    # the weights are repacked inside every step (as they would be after a
    # weight update); the packed buffer itself is allocated once
    wpack = torch.empty(sp.spconv_pack_weights_size(wl.K, wl.Ci, wl.Co, dtype_code(sp, wl)),
                        dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        nm = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
        sp.spconv_pack_weights(w_d, out=wpack)
        sp.spconv_forward_packed(f_d, nm, w_d, wpack, b_d, out=out)
        return nm

    # peak extra device memory of one step, beyond inputs and output
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    free0, _ = torch.cuda.mem_get_info(dev)
    nm = step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated(dev) - base + wpack.numel()   # + the packed weights
    free1, _ = torch.cuda.mem_get_info(dev)
    vp = nm.valid_pairs
    del nm

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        nm = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
        sp.spconv_pack_weights(w_d, out=wpack)
        ev[i][0].record(stream)
        sp.spconv_forward_packed(f_d, nm, w_d, wpack, b_d, out=out)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t_steps = time.perf_counter() - t0
    fwd_ms_in_steps = sum(s.elapsed_time(e) for s, e in ev) / a.steps

    # forward alone, back to back on a built map
    nm = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record(stream)
    for _ in range(a.fwd_iters):
        sp.spconv_forward_packed(f_d, nm, w_d, wpack, b_d, out=out)
    e_ev.record(stream)
    torch.cuda.synchronize()
    fwd_ms = s_ev.elapsed_time(e_ev) / a.fwd_iters

    # forward per launch, 20 runs each: flushed and warm
    pl = per_launch(torch, lambda: sp.spconv_forward_packed(f_d, nm, w_d, wpack, b_d, out=out), stream, dev)

    # the unpacked forward (spconv_forward: w as given), back to back
    s_ev.record(stream)
    for _ in range(a.fwd_iters):
        sp.spconv_forward(f_d, nm, w_d, b_d, out=out)
    e_ev.record(stream)
    torch.cuda.synchronize()
    fwd_unpacked_ms = s_ev.elapsed_time(e_ev) / a.fwd_iters

    # the build on its own: host time of the call (it waits for its own
    # kernels) on an idle stream, median of 5
    b_ms = []
    for _ in range(5):
        torch.cuda.synchronize()
        tb = time.perf_counter()
        nm_b = sp.spconv_build_nmap(c_d, wl.K, wl.dilation)
        b_ms.append((time.perf_counter() - tb) * 1e3)
    del nm_b

    # secondary run on the raster (np.argwhere) order of the same voxels: the
    # builder's Morton schedule has to give the same locality
    c_r = torch.from_numpy(W.geometry(wl, shuffle=False)).to(dev)
    for _ in range(2):
        sp.spconv_forward_packed(f_d, sp.spconv_build_nmap(c_r, wl.K, wl.dilation), w_d, wpack, b_d, out=out)
    torch.cuda.synchronize()
    r_build, r_fwd = [], []
    for _ in range(5):
        tb = time.perf_counter()
        nm_r = sp.spconv_build_nmap(c_r, wl.K, wl.dilation)
        r_build.append((time.perf_counter() - tb) * 1e3)
        s_ev.record(stream)
        sp.spconv_forward_packed(f_d, nm_r, w_d, wpack, b_d, out=out)
        e_ev.record(stream)
        torch.cuda.synchronize()
        r_fwd.append(s_ev.elapsed_time(e_ev))
    del nm_r, c_r

    # input gradient on the same map (dout drawn once, seeded): mirror + pack
    # the weights into a workspace, then the forward kernels with Ci and Co
    # exchanged; back to back, HIP events on the launch stream
    g = torch.Generator().manual_seed(4242)
    dout = torch.randn((N, wl.Co), generator=g, dtype=torch.float32).to(w_d.dtype).to(dev)
    dws = torch.empty(sp.spconv_dgrad_workspace_size(wl.K, wl.Ci, wl.Co, dtype_code(sp, wl)),
                      dtype=torch.uint8, device=dev)
    dfe = torch.empty((N, wl.Ci), dtype=w_d.dtype, device=dev)
    for _ in range(3):
        sp.spconv_dgrad(dout, nm, w_d, out=dfe, workspace=dws)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for _ in range(a.fwd_iters):
        sp.spconv_dgrad(dout, nm, w_d, out=dfe, workspace=dws)
    e_ev.record(stream)
    torch.cuda.synchronize()
    dgrad_ms = s_ev.elapsed_time(e_ev) / a.fwd_iters

    # weight gradient on the same map and inputs: split-K partials + ordered
    # reduction, back to back
    wws = torch.empty(sp.spconv_wgrad_workspace_size(N, wl.K, wl.Ci, wl.Co, dtype_code(sp, wl)),
                      dtype=torch.uint8, device=dev)
    dwo = torch.empty((wl.K, wl.Ci, wl.Co), dtype=w_d.dtype, device=dev)
    for _ in range(3):
        sp.spconv_wgrad(f_d, dout, nm, out=dwo, workspace=wws)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for _ in range(a.fwd_iters):
        sp.spconv_wgrad(f_d, dout, nm, out=dwo, workspace=wws)
    e_ev.record(stream)
    torch.cuda.synchronize()
    wgrad_ms = s_ev.elapsed_time(e_ev) / a.fwd_iters
    ws = profile_summary(wl, "wgrad")
    wgrad_counters = None if ws is None else {
        k: ws.get(k) for k in ("kernel", "avg_duration_us", "reduce_avg_duration_us", "traffic_bytes_per_call",
                               "traffic_over_algorithmic", "mfma_busy_frac", "executed_over_useful")}

    # mixed dtypes on the same map: feats in the other dtype, cast to w's
    # dtype by a separate pass into a workspace (fp32 feats into bf16 w), and
    # in the gather (no workspace); each back to back
    f_mx = f_d.to(torch.float32 if wl.dtype == "bf16" else torch.bfloat16)
    mx_ws = torch.empty(sp.spconv_forward_mixed_workspace_size(
        N, wl.Ci, sp.SPCONV_F32 if f_mx.dtype == torch.float32 else sp.SPCONV_BF16, dtype_code(sp, wl)),
        dtype=torch.uint8, device=dev)
    mixed_ms = {}
    for form, ws in (("cast_pass", mx_ws), ("gather_cast", None)):
        for _ in range(3):
            sp.spconv_forward_mixed(f_mx, nm, w_d, b_d, out=out, workspace=ws, wpack=wpack)
        torch.cuda.synchronize()
        s_ev.record(stream)
        for _ in range(a.fwd_iters):
            sp.spconv_forward_mixed(f_mx, nm, w_d, b_d, out=out, workspace=ws, wpack=wpack)
        e_ev.record(stream)
        torch.cuda.synchronize()
        mixed_ms[form] = s_ev.elapsed_time(e_ev) / a.fwd_iters
    del f_mx, mx_ws, dws, dfe, wws, dwo, dout

    flops = fwd_flops(wl, vp)
    ms_per_step = t_steps * 1e3 / a.steps
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = flops / (fwd_ms_in_steps * 1e-3) / 1e12
    prof = profile_summary(wl)
    roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak,
                "traffic": float(prof["traffic_bytes_per_launch"]) if prof and "traffic_bytes_per_launch" in prof
                else None,
                "kernel": prof["kernel"] if prof else None}
    if prof:
        for k in ("hbm_gbs", "hbm_frac", "mfma_busy_frac", "executed_over_useful", "avg_duration_us"):
            if k in prof:
                roofline[k] = float(prof[k])
    res = {
        "metric": METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: seeded surface voxels (shells + planes) in a "
                               f"{wl.grid}^3 grid, K={wl.K} dilation {wl.dilation}, "
                               f"Ci={wl.Ci} Co={wl.Co} {wl.dtype}, fp32 accumulate",
                   "N": N, "valid_pairs": vp, "K": wl.K, "Ci": wl.Ci, "Co": wl.Co,
                   "step": "build neighbour map + pack weights + fused forward"},
        "peak_extra_hbm_bytes": int(peak_extra),
        "peak_extra_hbm_bytes_per_voxel": peak_extra / N,
        "materialised_gather_bytes": int(wl.K) * N * wl.Ci * (2 if wl.dtype == "bf16" else 4),
        "mem_get_info_delta_bytes": int(free0 - free1),
        "build_ms": sorted(b_ms)[2],
        "forward_ms": fwd_ms_in_steps,
        "forward_ms_back_to_back": fwd_ms,
        "forward_tflops": achieved,
        "forward_per_launch": pl,
        "forward_unpacked_ms_back_to_back": fwd_unpacked_ms,
        "raster_order": {"build_ms_median": sorted(r_build)[2], "forward_ms_median": sorted(r_fwd)[2],
                         "what": "the same voxels in raster order instead of shuffled (build host time, "
                                 "forward HIP events)"},
        "dgrad": {"ms": dgrad_ms, "tflops": flops / (dgrad_ms * 1e-3) / 1e12,
                  "what": "spconv_dgrad on the same map: weight mirror + pack + forward over dout "
                          "(Ci and Co exchanged), back to back"},
        "wgrad": {"ms": wgrad_ms, "tflops": flops / (wgrad_ms * 1e-3) / 1e12,
                  "algorithmic_bytes": wgrad_alg_bytes(wl, N),
                  "counters": wgrad_counters,
                  "what": "spconv_wgrad on the same map: split-K partials over row chunks + ordered "
                          "reduction, back to back"},
        "forward_mixed": {"ms": mixed_ms["cast_pass"], "tflops": flops / (mixed_ms["cast_pass"] * 1e-3) / 1e12,
                          "ms_gather_cast": mixed_ms["gather_cast"],
                          "what": "spconv_forward_mixed on the same map, feats in "
                                  + ("float32" if wl.dtype == "bf16" else "bfloat16")
                                  + " cast to w's dtype: ms = with the workspace (a cast pass where one exists), "
                                    "ms_gather_cast = cast in the gather; back to back"},
        "roofline": roofline,
    }
    del nm, f_d, w_d, b_d, out, wpack, c_d
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(coords, feats, w, bias, wl, vp, a.cpu_seconds, 3, full_map=True)
    if a.configs:
        res["configs"] = {}
        for name in a.configs.split(","):
            res["configs"][name] = config_run(sp, torch, W, dev, name, a.cpu_seconds / 2, not a.no_cpu_baseline)
            print(f"# config {name}: forward {res['configs'][name]['forward_ms_flushed_median']:.4f} ms",
                  file=sys.stderr, flush=True)
    if a.shard_workload:
        res["shard"] = shard_run(sp, torch, W, dev, a.shard_workload, a.shard_parts)
    print(json.dumps(res), flush=True)
    if a.calibrate_copy_mib:
        calibrate_copy(torch, dev, a.calibrate_copy_mib)


if __name__ == "__main__":
    main()
