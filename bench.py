"""Benchmark: chunked Gated DeltaNet prefill forward + backward on one MI355X.

One step = gdn_chunk_fwd + gdn_chunk_bwd (the whole hot path) over one batch of
synthetic inputs already resident in HBM.  Default workload: B=1, T=32768,
H=16, dk=dv=128, chunk 64, bf16 (inputs as in gdn_inputs, h0 = 0, dhT = 0).

Prints ONE JSON line with tokens/s (B*T per step, all heads), the fraction of
the bf16 MFMA peak reached by the step's algorithmic FLOPs, per-kernel times
measured with HIP events on the launch stream during the timed region, a
roofline entry for the dominant kernel, and the fp64 CPU oracle timed on a
bounded sample of the same workload on this host's cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunked prefill fwd+bwd tokens/s and % bf16 MFMA peak, H=16 d=128 T=32k"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CH = 64


def flops_per_token_head(dk, dv, C=CH):
    """Algorithmic FLOP model (full C x C tiles, no recompute)."""
    fwd = 6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + (2.0 / 3.0) * C * C
    bwd = 12 * dk * dv + 4 * C * (3 * dk + 2 * dv) + 4 * C * C
    return fwd, bwd


def kernel_models(dk, dv, esz):
    """Per token-head algorithmic FLOPs and HBM bytes each kernel is responsible for.

    fwd:  the forward chunk algebra; reads q, k, v, g, beta and writes o.
    rev:  the state-gradient chain (diag(Gam)Q)^T dO and W^T dU; reads q, k, g, beta, dO.
    grad: the rest of the backward; reads q, k, v, dO, g, beta, writes dq, dk, dv, dbeta, dg.
    The replay and the lead-in chunks of the chains are recomputation and count
    no algorithmic work.
    """
    fwd, bwd = flops_per_token_head(dk, dv)
    rev = 4 * dk * dv
    return {
        "fwd": (fwd, (2 * dk + dv) * esz + 4 + esz + dv * esz),
        "rev": (rev, (2 * dk + dv) * esz + 4 + esz),
        "grad": (bwd - rev, (2 * dk + 2 * dv) * esz + 4 + esz + (2 * dk + dv) * esz + esz + 4),
    }


def kernel_sources_sha256():
    """Digest of the HIP sources (the key under which measured counters stay
    valid): their code, with comments and blank space removed, so that a
    comment edit keeps the counters; any change to the code drops them."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_deltanet_chunked_delta_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(d, "*.hip")) + glob.glob(os.path.join(d, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)  # block comments
        src = re.sub(r"//[^\n]*", " ", src)                # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    record (already scaled by the copy-kernel reference), or None if there is no record or the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return rec["traffic_bytes_per_launch"]


def host_info():
    """Threads this process may run on and the CPU model (from /proc/cpuinfo)."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return nproc, model


def cpu_baseline(x_full, seconds_target=15.0):
    """Time the fp64 oracle (forward, then backward) on the first tokens of the workload."""
    from oracle import ref
    import gdn_inputs  # noqa: F401

    def run(Ts):
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:, :Ts])
        q, k, v, g, b, do = (sl(a) for a in (x_full.q, x_full.k, x_full.v, x_full.g, x_full.beta, x_full.do))
        t0 = time.perf_counter()
        ref.fwd(q, k, v, g, b, x_full.scale)
        ref.bwd(q, k, v, g, b, x_full.scale, do)
        return time.perf_counter() - t0

    T = x_full.q.shape[1]
    Ts = min(T, 256)
    dt = run(Ts)
    while dt < seconds_target / 4 and Ts < T:
        Ts = min(T, int(Ts * min(8.0, max(2.0, seconds_target / max(dt, 1e-3)))))
        dt = run(Ts)
    B, _, H, _ = x_full.q.shape
    nproc, model = host_info()
    return {"value": B * Ts / dt, "unit": "tokens/s", "cores": ref.threads(), "kind": "oracle",
            "nproc": nproc, "cpu_model": model,
            "sample": f"first {Ts} of {T} tokens (B={B}, all {H} heads), fp64 token recurrence forward "
                      f"then its reverse-mode backward, {dt:.1f} s"}


def summarize_pmc(paths):
    """Per-kernel means of rocprofv3 --pmc counter_collection.csv files (one or more passes):
    a markdown table with every counter's mean per dispatch and, where the counters are
    present, instructions per wave and the busy fractions of the matrix cores
    (SQ_VALU_MFMA_BUSY_CYCLES over the kernel's cycles x 1024 SIMDs), the vector ALUs
    (4 SQ_ACTIVE_INST_VALU over the same) and the LDS (SQ_LDS_IDX_ACTIVE over the
    kernel's cycles x 256 CUs).  The kernel's cycles are GRBM_GUI_ACTIVE / 8: the
    counter is summed over MI355X's eight accelerator dies (XCDs)."""
    import csv
    import re
    def demangle(n):
        # this library's kernels: _ZN3gdn[12_GLOBAL__N_1]<len><name>I<template args>EEvNS_...
        m = re.match(r"_ZN3gdn(?:12_GLOBAL__N_1)?(\d+)(\w+)", n)
        if not m:
            return n
        ln = int(m.group(1))
        base, rest = m.group(2)[:ln], m.group(2)[ln:]
        if not rest.startswith("I"):
            return base
        out = []
        for t in re.finditer(r"DF16b|L[bi]\d+E|f(?=L|E)", rest):
            tok = t.group(0)
            out.append("bf16" if tok == "DF16b" else ("f32" if tok == "f" else tok[2:-1]))
        return f"{base}<{','.join(out)}>"

    vals = {}      # kernel -> counter -> [values]
    meta = {}      # kernel -> (grid, workgroup, lds, vgpr, agpr)
    rows = []
    for path in paths:
        with open(path, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    names = sorted({r["Kernel_Name"] for r in rows})
    demangled = {n: demangle(n) for n in names}
    if True:
        if True:
            for row in rows:
                name = demangled[row["Kernel_Name"]]
                short = re.sub(r"\(.*\)$", "", name).replace("void ", "")
                short = re.sub(r"gdn::(?:\(anonymous namespace\)::)?", "", short)
                short = short.replace("__hip_bfloat16", "bf16").replace("__bf16", "bf16")
                short = short.replace("true", "1").replace("false", "0")
                if "at::native" in name or "elementwise" in name or "fill" in name.lower():
                    short = "torch: " + re.sub(r"<.*", "", short.split("::")[-1])
                d = vals.setdefault(short, {})
                d.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                meta[short] = (row.get("Grid_Size"), row.get("Workgroup_Size"), row.get("LDS_Block_Size"),
                               row.get("VGPR_Count"), row.get("Accum_VGPR_Count"))
    counters = sorted({c for d in vals.values() for c in d})
    lines = ["| kernel | dispatches | grid | wg | LDS | VGPR/AGPR | " + " | ".join(counters) + " | per wave |",
             "|---" * (6 + len(counters) + 1) + "|"]
    for k in sorted(vals, key=lambda kk: -max(len(v) for v in vals[kk].values())):
        d = vals[k]
        n = max(len(v) for v in d.values())
        mean = {c: sum(v) / len(v) for c, v in d.items()}
        per = []
        waves = mean.get("SQ_WAVES")
        if waves:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD",
                      "SQ_INSTS_VMEM_WR"):
                if c in mean:
                    per.append(f"{c[9:]} {mean[c] / waves:,.0f}")
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui:
            gui /= 8.0  # summed over the eight XCDs
            per.append(f"cycles {gui:,.0f}")
            for c, lab, units in (("SQ_VALU_MFMA_BUSY_CYCLES", "MFMA busy", 1024), ("SQ_ACTIVE_INST_VALU", "VALU busy",
                                                                                    1024 / 4),
                                  ("SQ_LDS_IDX_ACTIVE", "LDS busy", 256)):
                if c in mean:
                    per.append(f"{lab} {100 * mean[c] / (gui * units):.1f}%")
        g, wg, lds, vg, ag = meta[k]
        lines.append(f"| `{k}` | {n} | {g} | {wg} | {lds} | {vg}/{ag} | "
                     + " | ".join(f"{mean[c]:,.0f}" if c in mean else "" for c in counters)
                     + " | " + ", ".join(per) + " |")
    return "\n".join(lines)


def bench_decode(args, log):
    """One gdn_decode_step per step over N sequences x 16 heads (d = 128, bf16 inputs, fp32
    state updated in place).  HBM-bound: the state is read and written once per step."""
    import torch
    import gdn_inputs
    from gated_deltanet_chunked_delta_amd import binding as gb
    N, H, D = args.decode_batch, 16, 128
    dev = torch.device("cuda:0")
    x = gdn_inputs.generate(B=N, T=1, H=H, Dk=D, Dv=D, dtype="bf16", seed=20260099, h0_std=0.1)
    bf = torch.bfloat16
    t = lambda a, d=bf: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d).contiguous()
    q, k, v, beta = (t(a[:, 0]) for a in (x.q, x.k, x.v, x.beta))
    g = t(x.g[:, 0], torch.float32)
    state = t(x.h0, torch.float32)
    o = torch.empty((N, H, D), dtype=bf, device=dev)
    step = lambda: gb.gdn_decode_step(q, k, v, g, beta, x.scale, state, o=o)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    # back to back: the state may stay in the 256 MB last-level cache between steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / args.steps
    # each step after writing 1 GiB elsewhere (L2 and last-level cache flushed), as a
    # serving loop sees it; the median step is the reported figure
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    gb.gdn_profile_reset()
    gb.gdn_profile_enable(True)
    times = []
    for _ in range(args.steps):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    gb.gdn_profile_enable(False)
    prof = gb.gdn_profile_read()
    ms = float(np.median(times))
    kern_s = prof["decode"][0] / prof["decode"][1] * 1e-3
    # algorithmic bytes per (sequence, head): fp32 state in and out, q, k, v, g, beta in, o out
    b_sh = 2 * D * D * 4 + (3 * D) * 2 + 4 + 2 + D * 2
    f_sh = 2 * D * D * 3 + 2 * D * D  # p = h^T k, the update, o = h'^T q
    gbs = b_sh * N * H / kern_s / 1e9
    out = {
        "metric": "GDN recurrent decode step tokens/s, H=16 d=128", "value": N * 1e3 / ms, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode_{N}x{H}", "N": N, "H": H, "dk": D, "dv": D, "state": "fp32 in place",
                   "timing": "median step, caches flushed before each"},
        "back_to_back": {"ms_per_step": ms_warm, "value": N * 1e3 / ms_warm, "unit": "tokens/s"},
        "kernels": {k_: {"avg_ms": v_[0] / v_[1], "launches_per_step": v_[1] / args.steps} for k_, v_ in prof.items()},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "kernel": "decode", "traffic": None,
                     "algorithmic_per_launch": {"flop": f_sh * N * H, "bytes": b_sh * N * H}},
    }
    if not args.no_cpu_baseline:
        from oracle import ref
        log("timing the CPU oracle")
        reps, dt = 0, 0.0
        t0 = time.perf_counter()
        while dt < args.cpu_seconds / 3:
            ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
            reps += 1
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": N * reps / dt, "unit": "tokens/s", "cores": ref.threads(), "kind": "oracle",
                               "sample": f"{reps} repetitions of the same {N} x {H} single-token step, fp64, {dt:.1f} s"}
    print(json.dumps(out))


# Phase names of the instrumented kernels' clocks (the order of their slots).
CLOCK_PHASES = {
    "fwd": ["before the first chunk", "staging", "P; T lands", "-W, Ut", "state chain (U, O, h')", "output stores",
            "after the last chunk"],
    "rev": ["before the first chunk", "staging (T lands)", "scale P^T, -W^T", "dU, state-gradient update",
            "after the last chunk"],
    "grad": ["", "staging (K, Q, record)", "K K^T * D and P; U, dO, T land", "dU, G_P", "G_W, dQ1, U dh'^T",
             "X_W, dQ, G_T", "Z", "G_A, E", "dK, row sums", "gradient stores"],
}


def phase_clock_report(lib, config):
    """Markdown tables of the per-phase shader-clock cycles that the instrumented
    library recorded for the last launch of each kernel (wave 0 of each of the
    first 512 workgroups; the barriers keep a workgroup's waves in step)."""
    import ctypes
    for fn in ("gdn_clock_read_fwd", "gdn_clock_read_rev", "gdn_clock_read_grad"):
        if not hasattr(lib, fn):
            sys.exit("--phase-clock needs the instrumented library: python -m gated_deltanet_chunked_delta_amd.build "
                     "--phase-clock, then GDN_LIB=gated_deltanet_chunked_delta_amd/libgdn_clock.so")
    blocks = 512
    fwd = np.zeros((2, blocks, 8, 8), dtype=np.uint32)
    rev = np.zeros((blocks, 8, 8), dtype=np.uint32)
    grad = np.zeros((blocks, 8, 10), dtype=np.uint32)
    for fn, buf in (("gdn_clock_read_fwd", fwd), ("gdn_clock_read_rev", rev), ("gdn_clock_read_grad", grad)):
        f = getattr(lib, fn)
        f.argtypes = [ctypes.c_void_p]
        if f(buf.ctypes.data) != 0:
            sys.exit(f"{fn} failed")
    out = [f"Phase clock, workload {config}: shader-clock cycles (s_memtime), wave 0 of each recorded workgroup.", ""]

    def chain(name, rec, phases):
        w0 = rec[:, 0, :].astype(np.float64)
        used = w0[:, 7] > 0
        w0 = w0[used]
        nch = w0[:, 7]
        total = w0[:, :len(phases)].sum(1)
        out.append(f"**{name}** ({used.sum()} workgroups, {nch.mean():.1f} chunks each on average; "
                   f"workgroup cycles median {np.median(total):,.0f}, max {total.max():,.0f})")
        out.append("")
        out.append("| phase | cycles per chunk (mean over workgroups) | share |")
        out.append("|---|---|---|")
        per = [w0[:, i].sum() / nch.sum() for i in range(len(phases))]
        for i, ph in enumerate(phases):
            if 1 <= i <= len(phases) - 2:
                out.append(f"| {i} {ph} | {per[i]:,.0f} | {per[i] / sum(per[1:len(phases) - 1]):.0%} |")
            else:
                out.append(f"| {i} {ph} (per workgroup) | {w0[:, i].mean():,.0f} | |")
        out.append("")

    chain("forward (`gdn_fwd_seg<...,1,0,0>`)", fwd[0], CLOCK_PHASES["fwd"])
    chain("replay (`gdn_fwd_seg<...,0,0,1>`)", fwd[1], CLOCK_PHASES["fwd"])
    chain("reverse chain (`gdn_rev_seg`)", rev, CLOCK_PHASES["rev"])
    w0 = grad[:, 0, :].astype(np.float64)
    used = w0[:, 1:].sum(1) > 0
    w0 = w0[used]
    total = w0[:, 1:].sum(1)
    out.append(f"**gradient kernel (`gdn_grad_kernel`)** ({used.sum()} workgroups, one chunk each; cycles median "
               f"{np.median(total):,.0f}, max {total.max():,.0f})")
    out.append("")
    out.append("| phase | cycles (median over workgroups) | share |")
    out.append("|---|---|---|")
    med = [np.median(w0[:, i]) for i in range(10)]
    for i in range(1, 10):
        out.append(f"| {i} {CLOCK_PHASES['grad'][i]} | {med[i]:,.0f} | {med[i] / sum(med[1:]):.0%} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="metric_32k")
    ap.add_argument("--direction", default="fwdbwd", choices=["fwdbwd", "fwd", "bwd", "decode"],
                    help="decode: one recurrent step for --decode-batch sequences x 16 heads, d = 128 "
                         "(its own JSON line; not the headline metric)")
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--cp-mode", type=int, default=0)
    ap.add_argument("--prep", action="store_true",
                    help="in-kernel pre-processing: raw q, k (rescaled rows) normalised inside the kernels, "
                         "gate and beta passed as logits (g = -0.1 softplus(a), beta = sigmoid(b))")
    ap.add_argument("--save-states", action="store_true",
                    help="the forward keeps the chunk states and the backward reads them (no replay)")
    ap.add_argument("--no-save-t", action="store_true",
                    help="the forward does not keep the chunk matrices T; the backward solves for them")
    ap.add_argument("--api", default="abi", choices=["abi", "fla"],
                    help="abi: the library's entry points; fla: the FLA-convention autograd entry "
                         "(fla_compat.chunk_gated_delta_rule forward + torch.autograd.grad)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy (out = x * 1, fp32) of this many MiB three "
                         "times: the reference kernel that scales HBM byte counters under rocprofv3 --pmc")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-protocol", action="store_true",
                    help="skip the per-direction timing protocol (median / min / max over --protocol-iters "
                         "iterations, each after a 1 GiB write that flushes L2 and the last-level cache)")
    ap.add_argument("--protocol-iters", type=int, default=30)
    ap.add_argument("--phase-clock", action="store_true",
                    help="with the instrumented library (python -m gated_deltanet_chunked_delta_amd.build "
                         "--phase-clock; GDN_LIB=gated_deltanet_chunked_delta_amd/libgdn_clock.so): run the step "
                         "and print each kernel's cycles per phase (per chunk for the chains) as markdown")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print a per-kernel markdown summary of rocprofv3 --pmc counter_collection.csv "
                         "files and exit (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    log = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)
    log("importing torch")
    import torch
    if args.direction == "decode":
        return bench_decode(args, log)
    import gdn_inputs
    from gated_deltanet_chunked_delta_amd import binding as gb

    dev = torch.device("cuda:0")
    log(f"generating {args.config}")
    x = gdn_inputs.config(args.config, grad=True)
    prep_kw = {}
    if args.prep:
        # raw inputs of the same workload: rows rescaled, gate / beta as logits
        rng = np.random.default_rng(12345)
        rnd = gdn_inputs.round_bf16 if x.dtype == "bf16" else (lambda a: a.astype(np.float32))
        x.q = rnd(x.q * rng.uniform(0.25, 4.0, size=x.q.shape[:-1] + (1,)))
        x.k = rnd(x.k * rng.uniform(0.25, 4.0, size=x.k.shape[:-1] + (1,)))
        x.g = rng.standard_normal(x.g.shape).astype(np.float32)
        x.beta = rnd(rng.standard_normal(x.beta.shape))
        prep_kw = dict(qk_norm=True, gate_act=True,
                       gate_scale=torch.full((x.q.shape[2],), 0.1, dtype=torch.float32, device=dev))
    B, T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    t = lambda a, d=dt: torch.from_numpy(a).to(dev).to(d).contiguous()
    q, k, v, beta, do = (t(a) for a in (x.q, x.k, x.v, x.beta, x.do))
    g = t(x.g, torch.float32)
    h0 = None if x.h0 is None else t(x.h0, torch.float32)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens).to(dev)
    host = x.cu_seqlens
    ntok = int(B * T) if cu is None else int(x.cu_seqlens[-1])

    # The step follows the backward as specified: it takes the forward's inputs
    # and replays the forward states; the forward keeps every chunk's matrix T
    # (64 x 64 fp32 per 64 tokens and head) for it, as the autograd wrapper does
    # (--no-save-t: the backward solves for T itself).  --save-states times the
    # alternative in which the forward also keeps the chunk states (Dk*Dv
    # values per 64 tokens and head) for the backward; the default run also
    # reports that variant in a separate, labelled object.
    keep = False
    save_t = not args.no_save_t and args.direction == "fwdbwd"

    if args.api == "fla":
        if args.direction != "fwdbwd" or args.prep or args.no_save_t:
            sys.exit("--api fla times the forward + backward of the default workload only")
        from gated_deltanet_chunked_delta_amd.fla_compat import chunk_gated_delta_rule as fla_entry
        leaves = [a.detach().requires_grad_(True) for a in (q, k, v, g, beta)]

    def step_fla():
        o, _ = fla_entry(*leaves, scale=x.scale, cu_seqlens=cu)
        torch.autograd.grad([o], leaves, [do])

    def step():
        if args.api == "fla":
            return step_fla()
        states = chunk_t = None
        if args.direction in ("fwdbwd", "fwd"):
            res = gb.gdn_chunk_fwd(q, k, v, g, beta, x.scale, h0=h0, cu_seqlens=cu, cu_seqlens_host=host,
                                   cp_mode=args.cp_mode, save_states=keep, save_t=save_t, **prep_kw)
            states = res[2] if keep else None
            chunk_t = res[-1] if save_t else None
        if args.direction in ("fwdbwd", "bwd"):
            gb.gdn_chunk_bwd(q, k, v, g, beta, x.scale, do, h0=h0, cu_seqlens=cu, cu_seqlens_host=host,
                             cp_mode=args.cp_mode, need_dh0=h0 is not None, states=states, chunk_t=chunk_t,
                             **prep_kw)

    stream = torch.cuda.current_stream(dev)

    if args.phase_clock:
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        print(phase_clock_report(gb.lib(), args.config))
        return

    def timed_run(profile):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        if profile:
            gb.gdn_profile_reset()
            gb.gdn_profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        prof = None
        if profile:
            gb.gdn_profile_enable(False)
            prof = gb.gdn_profile_read()
        return e0.elapsed_time(e1) / args.steps, prof

    # The step time comes from a run with no per-kernel events in the stream;
    # a second run of the same steps, each kernel bracketed by the library's HIP
    # events, gives the per-kernel durations (the roofline entry's kernel time).
    log("warmup + timed steps")
    keep = args.save_states and args.direction == "fwdbwd"
    ms, _ = timed_run(False)
    log(f"timed {args.steps} steps")
    ms_prof, prof = timed_run(True)
    log(f"timed {args.steps} steps with per-kernel events")
    variant = None
    if args.direction == "fwdbwd" and not args.save_states and args.api == "abi":
        keep = True
        ms_v, _ = timed_run(False)
        keep = False
        variant = {"states": "saved by fwd (no replay in bwd)",
                   "chunk_T": "saved by fwd" if save_t else "solved in bwd",
                   "ms_per_step": ms_v, "value": ntok * 1e3 / ms_v, "unit": "tokens/s"}
        log(f"timed {args.steps} steps with saved states")

    # Timing protocol per direction: the forward alone (keeping T, as in the
    # step), the backward alone (given that T), and both; 5 warm-ups, then the
    # median, min and max of --protocol-iters iterations, each timed by its own
    # event pair on the launch stream after a 1 GiB write that evicts L2 and the
    # last-level cache (the write is enqueued before the first event).
    protocol = None
    fwd_f, bwd_f = flops_per_token_head(dk, dv)
    if not args.no_protocol and args.api == "abi" and args.direction == "fwdbwd":
        log(f"timing protocol: {args.protocol_iters} iterations per direction, 1 GiB write before each")
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        kw = dict(h0=h0, cu_seqlens=cu, cu_seqlens_host=host, cp_mode=args.cp_mode, **prep_kw)

        def p_fwd():
            return gb.gdn_chunk_fwd(q, k, v, g, beta, x.scale, save_t=True, **kw)[-1]

        t_kept = p_fwd()

        def p_bwd():
            gb.gdn_chunk_bwd(q, k, v, g, beta, x.scale, do, need_dh0=h0 is not None, chunk_t=t_kept, **kw)

        def p_both():
            tt = p_fwd()
            gb.gdn_chunk_bwd(q, k, v, g, beta, x.scale, do, need_dh0=h0 is not None, chunk_t=tt, **kw)

        protocol = {"method": f"5 warm-ups, then {args.protocol_iters} iterations, each after a 1 GiB device "
                              "write (L2 and last-level cache evicted), timed by HIP events on the launch "
                              "stream; median, min, max",
                    "flop_per_token_head": {"fwd": fwd_f, "bwd": bwd_f, "fwdbwd": fwd_f + bwd_f}}
        for name, fn, fl in (("fwd", p_fwd, fwd_f), ("bwd", p_bwd, bwd_f), ("fwdbwd", p_both, fwd_f + bwd_f)):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(args.protocol_iters):
                flush.fill_(1.0)
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record(stream)
                fn()
                b_.record(stream)
                torch.cuda.synchronize()
                ts.append(a_.elapsed_time(b_))
            med = float(np.median(ts))
            tf = fl * ntok * H / (med * 1e-3) / 1e12
            protocol[name] = {"median_ms": med, "min_ms": float(np.min(ts)), "max_ms": float(np.max(ts)),
                              "tokens_per_s": ntok * 1e3 / med, "tflops": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS}
        del flush
        log("timing protocol done")

    per_th = {"fwdbwd": fwd_f + bwd_f, "fwd": fwd_f, "bwd": bwd_f}[args.direction]
    tflops = per_th * ntok * H / (ms * 1e-3) / 1e12
    kernels = {name: {"avg_ms": tot / n, "launches_per_step": n / args.steps}
               for name, (tot, n) in prof.items()}

    # roofline entry for the kernel with the largest share of the step
    esz = 2 if x.dtype == "bf16" else 4
    models = kernel_models(dk, dv, esz)
    dom = max(prof, key=lambda nm: prof[nm][0])
    avg_s = prof[dom][0] / prof[dom][1] * 1e-3
    f_th, b_th = models.get(dom, (0.0, 0.0))
    units = ntok * H
    flop_rate = f_th * units / avg_s / 1e12
    byte_rate = b_th * units / avg_s / 1e9
    if f_th / max(b_th, 1) >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": flop_rate, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byte_rate, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(dom, args.config)
    roof["algorithmic_per_launch"] = {"flop": f_th * units, "bytes": b_th * units}

    out = {
        "metric": METRIC, "value": ntok * 1e3 / ms, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if x.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.config, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": CH,
                   "direction": args.direction, "cp_mode": args.cp_mode, "tokens_per_step": ntok,
                   "states": "saved by fwd" if (args.save_states or args.api == "fla") else "recomputed in bwd",
                   "api": "fla_compat autograd" if args.api == "fla" else "C ABI",
                   "chunk_T": "saved by fwd" if save_t else "solved in bwd",
                   "preprocessing": "in-kernel q/k L2 norm + gate/beta activation" if args.prep else "none"},
        "tflops": tflops, "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "kernels": kernels, "ms_per_step_with_kernel_events": ms_prof, "roofline": roof,
    }
    if protocol is not None:
        out["fwd_ms"] = protocol["fwd"]["median_ms"]
        out["bwd_ms"] = protocol["bwd"]["median_ms"]
        out["frac_bf16_peak_fwd"] = protocol["fwd"]["frac_bf16_peak"]
        out["frac_bf16_peak_bwd"] = protocol["bwd"]["frac_bf16_peak"]
        out["protocol"] = protocol
    if variant is not None:
        out["variant_saved_states"] = variant
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy reference: 3 x {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
