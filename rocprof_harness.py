"""rocprofv3 harness: matrix-core utilisation and HBM traffic of the forward
against MI355X's published peaks, written as short text summaries under
profiles/.

For each workload it runs `bench.py --profile-run` (a few steps as bench.py
times them: neighbour map, weight pack, forward; for the --wgrad workloads a
few weight gradients back to back; then a plain device copy of known size)
four times under rocprofv3, each pass a run of its own:

  1. --kernel-trace --stats             per-kernel durations
  2. --pmc FETCH_SIZE                   bytes read from HBM per dispatch (KiB)
  3. --pmc WRITE_SIZE                   bytes written to HBM per dispatch (KiB)
  4. --pmc SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_<dtype> SQ_VALU_MFMA_BUSY_CYCLES
           SQ_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE

and reduces the CSVs to, for the forward kernel (the kernel named k_fwd*
with the most total time):
  * average duration and the effective rate 2*valid_pairs*Ci*Co / duration
    against the dense peak of the dtype (bf16 2516.6, fp32 157.3 TFLOP/s);
  * HBM traffic per launch: FETCH_SIZE and WRITE_SIZE scaled by what the same
    counters read for the copy (bytes copied / counter), their rate against
    8 TB/s and their ratio to the algorithmic bytes;
  * matrix-core busy fraction: SQ_VALU_MFMA_BUSY_CYCLES over
    (SIMDs x GRBM_GUI_ACTIVE per XCD), and executed / useful MFMA work
    (MOPS x 512 FLOP against 2*valid_pairs*Ci*Co).
For the weight gradient the same figures are written for its main kernel
(k_wgrad*, not the chunk reduction), with the HBM traffic of a whole call:
the main kernel's and the reduction's bytes added (the algorithmic bytes of a
call: feats and dout once, the K x N neighbour indices, dw once).
Each summary records its kernel source's hash, so bench.py uses its counter
figures only while that source is unchanged.

  python rocprof_harness.py --workloads surf256,surf1024,surf512d2 --wgrad surf256 --out gpurun_out/prof

The harness itself never touches the GPU: it only starts rocprofv3 as a child
process (with the profiled program after `--`) and reads what it wrote.
"""
import argparse
import csv
import glob
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
SIMDS = 256 * 4
XCDS = 8
COPY_MIB = 256
MFMA_FLOP_PER_MOP = 512


def run(cmd, log, timeout):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout, cwd=ROOT,
                           env=dict(os.environ, TMPDIR="/tmp"))
    if r.returncode != 0:
        tail = open(log).read()[-2000:]
        raise RuntimeError(f"{cmd[0]} exited {r.returncode}:\n{tail}")


def bench_cmd(wl, iters, copy, wgrad_iters=0):
    c = [sys.executable, "-u", "bench.py", "--profile-run", "--workload", wl, "--fwd-iters", str(iters)]
    if wgrad_iters:
        c += ["--wgrad-iters", str(wgrad_iters)]
    if copy:
        c += ["--calibrate-copy-mib", str(COPY_MIB)]
    return c


def find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def col(r, *names):
    for n in names:
        if n in r:
            return r[n]
    raise KeyError(f"none of {names} in {list(r)}")


def short(name):
    """'void spc::(anonymous namespace)::k_fwd_bf16_ws<128>(...)' -> 'k_fwd_bf16_ws<128>';
    names of other libraries' kernels are kept whole."""
    m = re.search(r"\b(k_\w+(?:<[^()]*?>)?)\s*\(", name)
    return m.group(1) if m else name.strip()


def kernel_durations(trace_csv):
    """{short kernel name: [durations in us, in dispatch order]}"""
    out = {}
    for r in rows(trace_csv):
        n = short(col(r, "Kernel_Name", "KernelName"))
        d = (int(col(r, "End_Timestamp", "EndNs")) - int(col(r, "Start_Timestamp", "BeginNs"))) / 1e3
        out.setdefault(n, []).append(d)
    return out


def counters(counter_csv):
    """({short kernel name: [{counter: value} per dispatch, in dispatch order]},
    [(kernel name, {counter: value}) for every dispatch, in dispatch order])"""
    per, flat = {}, {}
    for r in rows(counter_csv):
        n = short(col(r, "Kernel_Name", "KernelName"))
        disp = int(col(r, "Dispatch_Id", "Dispatch_ID", "Index"))
        name, val = col(r, "Counter_Name", "CounterName"), float(col(r, "Counter_Value", "CounterValue"))
        per.setdefault(n, {}).setdefault(disp, {})[name] = val
        flat.setdefault(disp, (n, {}))[1][name] = val
    return {n: [d[k] for k in sorted(d)] for n, d in per.items()}, [flat[k] for k in sorted(flat)]


def mean(v):
    return sum(v) / len(v)


def profile(wl_name, out_dir, iters, prof_dir, reduce_only=False, wgrad_iters=0):
    import workloads as W
    wl = W.by_name(wl_name)
    base = os.path.join(out_dir, wl_name)
    os.makedirs(base, exist_ok=True)
    env_note = "cd /tmp && export TMPDIR=/tmp (rocprofv3's scratch), then from the repository root:"
    passes = {
        "trace": ["--kernel-trace", "--stats"],
        "fetch": ["--pmc", "FETCH_SIZE"],
        "write": ["--pmc", "WRITE_SIZE"],
        "mfma": ["--pmc", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_" + ("BF16" if wl.dtype == "bf16" else "F32"),
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
                 "GRBM_GUI_ACTIVE"],
    }
    cmds = {}
    info = None
    for name, opts in passes.items():
        d = os.path.join(base, name)
        cmd = ["rocprofv3", *opts, "--output-format", "csv", "-d", d, "-o", "run", "--",
               *bench_cmd(wl_name, iters, copy=name in ("fetch", "write"), wgrad_iters=wgrad_iters)]
        cmds[name] = " ".join(cmd[:cmd.index("--")] + ["--"] + [os.path.basename(cmd[cmd.index("--") + 1])]
                              + cmd[cmd.index("--") + 2:])
        if not reduce_only:
            t0 = time.time()
            run(cmd, os.path.join(base, name + ".log"), timeout=300)
            print(f"  pass {name}: {time.time() - t0:.1f}s", flush=True)
        for line in open(os.path.join(base, name + ".log")):
            if line.startswith("{\"profile_run\""):
                info = json.loads(line)
    if info is None:
        raise RuntimeError("bench.py --profile-run printed no summary line")

    dur = kernel_durations(find(os.path.join(base, "trace"), "kernel_trace.csv"))
    fwd = max((n for n in dur if n.startswith("k_fwd")), key=lambda n: sum(dur[n]))
    d_us = mean(dur[fwd])
    flops = info["flops_per_forward"]
    alg_bytes = info["algorithmic_bytes_per_forward"]
    achieved = flops / (d_us * 1e-6) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]

    fc, f_flat = counters(find(os.path.join(base, "fetch"), "counter_collection.csv"))
    wc, w_flat = counters(find(os.path.join(base, "write"), "counter_collection.csv"))

    def copy_reading(flat, key):
        """(kernel, mean counter) of the calibration copy: the run's last
        three dispatches, which are the three copies of COPY_MIB MiB."""
        last = flat[-3:]
        return last[0][0], mean([x[key] for _, x in last])
    copy_kib = COPY_MIB * 1024.0
    copy_kernel, f_copy = copy_reading(f_flat, "FETCH_SIZE")
    _, w_copy = copy_reading(w_flat, "WRITE_SIZE")
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    f_kib = mean([x["FETCH_SIZE"] for x in fc[fwd]])
    w_kib = mean([x["WRITE_SIZE"] for x in wc[fwd]])
    traffic = (f_kib * f_scale + w_kib * w_scale) * 1024.0
    hbm_gbs = traffic / (d_us * 1e-6) / 1e9

    mc = counters(find(os.path.join(base, "mfma"), "counter_collection.csv"))[0][fwd]
    avg = {k: mean([x[k] for x in mc if k in x]) for k in mc[0]}
    mops_key = [k for k in avg if k.startswith("SQ_INSTS_VALU_MFMA_MOPS")][0]
    executed = avg[mops_key] * MFMA_FLOP_PER_MOP
    busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * avg["GRBM_GUI_ACTIVE"] / XCDS)

    path = os.path.join(prof_dir, f"fwd_{wl.dtype}_{wl_name}_rocprof.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 summary of the forward on {wl_name} (N = {info['N']:,}, K = {wl.K}, dilation "
                f"{wl.dilation}, Ci = {wl.Ci}, Co = {wl.Co}, {wl.dtype}; {info['valid_pairs']:,} valid pairs),\n")
        f.write(f"# written by rocprof_harness.py; each pass its own run ({env_note}):\n")
        for n, c in cmds.items():
            f.write(f"#   {c}\n")
        f.write(f"# Averages over the {len(dur[fwd])} dispatches of the forward kernel per run ({iters} steps of\n"
                f"# map, pack and forward, as bench.py times them).  Byte counters are scaled by what they read for a\n"
                f"# {COPY_MIB} MiB device copy in the same run ({copy_kernel[:60]}): FETCH x {f_scale:.3f}, "
                f"WRITE x {w_scale:.3f}.\n")
        f.write(f"kernel: {fwd}\n")
        f.write(f"kernel_source_sha256_16: {info['kernel_source_sha256_16']}\n")
        f.write(f"avg_duration_us: {d_us:.2f}\n")
        f.write(f"flops_per_launch: {flops:.6e}\n")
        f.write(f"achieved_tflops: {achieved:.1f}\n")
        f.write(f"peak_tflops: {peak}\n")
        f.write(f"mfma_frac_of_peak: {achieved / peak:.4f}\n")
        f.write(f"fetch_kib_per_dispatch: {f_kib:.1f}\n")
        f.write(f"write_kib_per_dispatch: {w_kib:.1f}\n")
        f.write(f"fetch_scale: {f_scale:.3f}\n")
        f.write(f"write_scale: {w_scale:.3f}\n")
        f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
        f.write(f"algorithmic_bytes_per_launch: {alg_bytes:.0f}\n")
        f.write(f"traffic_over_algorithmic: {traffic / alg_bytes:.3f}\n")
        f.write(f"hbm_gbs: {hbm_gbs:.1f}\n")
        f.write(f"hbm_frac: {hbm_gbs / PEAK_HBM_GBS:.4f}\n")
        for k in sorted(avg):
            f.write(f"{k}: {avg[k]:.4e}\n")
        f.write(f"executed_flops_per_launch: {executed:.6e}\n")
        f.write(f"executed_over_useful: {executed / flops:.3f}\n")
        f.write(f"mfma_busy_frac: {busy:.4f}\n")
        f.write("# mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs): the share\n"
                "# of the kernel's SIMD-cycles in which the matrix pipes run (useful or not);\n"
                "# executed = MOPS x 512 FLOP.  Other kernels of the trace run (average us, calls):\n")
        for n in sorted(dur, key=lambda n: -sum(dur[n])):
            f.write(f"#   {n[:90]}: {mean(dur[n]):.1f} us x {len(dur[n])}\n")
    print(open(path).read(), flush=True)
    if not wgrad_iters:
        return path

    # the weight gradient: its main kernel, and the chunk reduction's traffic
    wg = max((n for n in dur if n.startswith("k_wgrad") and not n.startswith("k_wgrad_reduce")),
             key=lambda n: sum(dur[n]))
    red = [n for n in dur if n.startswith("k_wgrad_reduce")]
    g_us = mean(dur[wg])
    r_us = mean(dur[red[0]]) if red else 0.0
    g_alg = info["algorithmic_bytes_per_wgrad"]
    g_achieved = flops / (g_us * 1e-6) / 1e12

    def call_bytes(n):
        return (mean([x["FETCH_SIZE"] for x in fc[n]]) * f_scale + mean([x["WRITE_SIZE"] for x in wc[n]]) * w_scale) * 1024.0
    g_bytes = call_bytes(wg)
    r_bytes = call_bytes(red[0]) if red else 0.0
    gm = counters(find(os.path.join(base, "mfma"), "counter_collection.csv"))[0][wg]
    gavg = {k: mean([x[k] for x in gm if k in x]) for k in gm[0]}
    g_exec = gavg[mops_key] * MFMA_FLOP_PER_MOP
    g_busy = gavg["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * gavg["GRBM_GUI_ACTIVE"] / XCDS)
    gpath = os.path.join(prof_dir, f"wgrad_{wl.dtype}_{wl_name}_rocprof.txt")
    with open(gpath, "w") as f:
        f.write(f"# rocprofv3 summary of the weight gradient on {wl_name} (N = {info['N']:,}, K = {wl.K}, "
                f"dilation {wl.dilation}, Ci = {wl.Ci}, Co = {wl.Co}, {wl.dtype}; {info['valid_pairs']:,} valid "
                f"pairs),\n")
        f.write(f"# written by rocprof_harness.py from the same runs as the forward's summary ({env_note}):\n")
        for n, c in cmds.items():
            f.write(f"#   {c}\n")
        f.write(f"# Averages over the {len(dur[wg])} calls per run ({wgrad_iters} back to back after the "
                f"forwards).  Byte counters scaled as in\n# the forward's summary: FETCH x {f_scale:.3f}, "
                f"WRITE x {w_scale:.3f}.  traffic_bytes_per_call = main kernel + chunk reduction.\n")
        f.write(f"kernel: {wg}\n")
        f.write(f"reduce_kernel: {red[0] if red else 'none'}\n")
        f.write(f"kernel_source_sha256_16: {info['wgrad_source_sha256_16']}\n")
        f.write(f"avg_duration_us: {g_us:.2f}\n")
        f.write(f"reduce_avg_duration_us: {r_us:.2f}\n")
        f.write(f"flops_per_call: {flops:.6e}\n")
        f.write(f"achieved_tflops: {g_achieved:.1f}\n")
        f.write(f"peak_tflops: {peak}\n")
        f.write(f"mfma_frac_of_peak: {g_achieved / peak:.4f}\n")
        f.write(f"kernel_traffic_bytes: {g_bytes:.0f}\n")
        f.write(f"reduce_traffic_bytes: {r_bytes:.0f}\n")
        f.write(f"traffic_bytes_per_call: {g_bytes + r_bytes:.0f}\n")
        f.write(f"algorithmic_bytes_per_call: {g_alg:.0f}\n")
        f.write(f"traffic_over_algorithmic: {(g_bytes + r_bytes) / g_alg:.3f}\n")
        f.write(f"hbm_gbs: {g_bytes / (g_us * 1e-6) / 1e9:.1f}\n")
        for k in sorted(gavg):
            f.write(f"{k}: {gavg[k]:.4e}\n")
        f.write(f"executed_flops_per_call: {g_exec:.6e}\n")
        f.write(f"executed_over_useful: {g_exec / flops:.3f}\n")
        f.write(f"mfma_busy_frac: {g_busy:.4f}\n")
    print(open(gpath).read(), flush=True)
    return path


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--workloads", default="surf256,surf1024,surf512d2")
    p.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    p.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    p.add_argument("--iters", type=int, default=8)
    p.add_argument("--wgrad", default="surf256", help="workloads whose weight gradient is profiled too")
    p.add_argument("--wgrad-iters", type=int, default=8)
    p.add_argument("--reduce-only", action="store_true", help="reduce the CSVs of an earlier run under --out")
    a = p.parse_args()
    sys.path.insert(0, ROOT)
    os.makedirs(a.profiles, exist_ok=True)
    for wl in a.workloads.split(","):
        profile(wl, a.out, a.iters, a.profiles, a.reduce_only,
                a.wgrad_iters if wl in a.wgrad.split(",") else 0)


if __name__ == "__main__":
    main()
