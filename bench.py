"""Benchmark: Mamba-2 SSD chunked scan, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mamba2_2p7b]
                    [--seqlen L] [--batch B] [--with-states] [--dt-softplus]
                    [--dtype fp8] [--fwd-only]
    python bench.py --op conv1d [--workload mamba2_2p7b] [--batch B] [--seqlen L]

A step is one ssd_fwd + ssd_bwd over one batch of the workload's seeded
synthetic inputs (already resident in HBM).  --seqlen / --batch change the
workload's sequence length / batch (a length that is not a multiple of the
chunk adds a shorter last chunk); --with-states starts the forward from a
seeded initial state and gives the backward a seeded final-state cotangent,
returning the initial-state gradient as well (one GPU's share of a sequence
split across GPUs); --dt-softplus passes the raw step and the per-head bias
and lets the library apply softplus(dt_raw + dt_bias) (and return ddt_bias);
--dtype changes the storage mode (fp8: x, B, C as E4M3 codes, dy and the
gradients bf16); --fwd-only times the forward pass alone.  Prints ONE JSON line on stdout;
diagnostics (per-kernel times) go to stderr.

Timing: W untimed warmup steps, then exactly K timed steps.  A 1 GiB write
before every timed step evicts the L2s and the 256 MB Infinity Cache, so each
step starts cold; each step is bracketed by events on the launch stream, and
the headline ms_per_step is the median of the K cold steps.  The same K steps
run back to back on warm caches afterwards (timing.warm_ms_per_step).

targets: per-kernel fractions of HBM and bf16 MFMA peak from the per-kernel
probe times (also on flushed caches): the chunk GEMM kernels against 50 % of
the MFMA peak beside the cap HBM alone puts on each, the two state-passing
scans against 60 % of HBM peak, and the step against its own HBM floor
(compulsory I/O of both passes plus five passes over the chunk states).

The roofline object describes the kernel with the largest share of the step:
its algorithmic bytes and flops per launch (formulas in kernel_model below)
over its average launch duration, measured with HIP events that libssd records
around that kernel on the launch stream during the timed steps.

--op conv1d times the causal depthwise conv1d before the scan instead (one
ssd_conv1d_fwd + ssd_conv1d_bwd per step, with bias, SiLU and a halo) on the
workload's conv shape (channels = nheads*headdim + 2*ngroups*dstate).

cpu_baseline: the float64 oracle on a bounded slice of the same workload
(one batch row, a subset of heads), timed on this host's cores and scaled
linearly in heads and batch to the workload's tokens/s.
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

METRIC = "SSD fwd+bwd tokens/s per GPU + % of bf16 MFMA peak / % HBM peak"
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, GB/s
# dense matrix-core peaks; in fp8 mode only C.B^T runs on the FP8 matrix
# cores, every other product (and the dominant kernels) on the bf16 ones
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 2500.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic traffic and work per launch of each kernel.
def head_slices(s) -> int:
    """Head slices of the group-level backward launches, as the library plans
    them: about 512 workgroups per kind of 64-row block, at most 4 slices, at
    most one per head, every slice non-empty."""
    base = s.batch * (-(-s.seqlen // s.chunk)) * s.ngroups * (s.chunk // 64)
    hpg = s.nheads // s.ngroups
    sl = max(1, min(-(-512 // base), 4, hpg))
    per = -(-hpg // sl)
    return -(-hpg // per)


def kernel_model(s, esz):
    """Bytes and flops per launch over the whole chunks (a shorter last chunk
    runs as a separate launch of each kernel, which the probes do not time)."""
    b, L, H, P, N, G, Q = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk
    K = L // Q
    T = b * K * Q
    eszx = 1 if s.dtype == "fp8" else esz   # x, B, C storage
    nt = Q // 16
    tiles = nt * (nt + 1) // 2
    X = T * H * P * esz              # one x-sized tensor in the step dtype (y, dy, dx)
    BCO = T * G * N * esz            # one of dB / dC (the step dtype)
    XI = T * H * P * eszx            # x as stored
    BC = T * G * N * eszx            # one of B / C
    DT = T * H * esz                 # dt / ddt in the caller's layout
    CS = b * H * K * Q * 4           # cs, or the float32 step the cumsum writes in cs's layout
    ST4 = b * K * H * P * N * 4      # chunk states, fp32
    STe = b * K * H * P * N * esz    # chunk states, storage dtype
    WT = b * K * G * tiles * 256 * esz
    nbp = (Q // 64) * (Q // 64 + 1) // 2
    S = head_slices(s)
    # dW as the head-sum launch writes it: one slice in the storage dtype, else fp32 per slice
    DW = b * K * G * nbp * 64 * 64 * (esz if S == 1 and esz == 2 else 4 * S)
    PART = 2 * S * T * G * N * 4     # fp32 head-slice partials of dC and dB (written, then read once)
    tri = Q * (Q + 1) // 2
    bkh, bkg = b * K * H, b * K * G
    m = {
        # dt in, cs and the float32 step out; B, C in, C.B^T tiles out
        "cumsum_bmm": (DT + 2 * CS + 2 * BC + WT, 2 * bkg * tri * N),
        "chunk_state": (XI + BC + 2 * CS + STe, 2 * bkh * Q * P * N),
        "state_passing": (2 * STe + b * H * P * N * 4, 0),
        "chunk_scan": (XI + X + 2 * CS + BC + STe + WT, 2 * bkh * (Q * N * P + tri * P)),
        # dy, C, cs, Hin in; dH_loc and the state-to-output term (one fp32 row per unit) out
        "chunk_state_bwd": (X + BC + CS + 2 * STe + bkh * Q * 4, 4 * bkh * Q * P * N),
        "state_passing_bwd": (2 * STe, 0),
        # x, dy, the step, cs, B, C, Gk, Hin (for <Gk, Hin>) in; dx out (+ dl assembly: ddt out).
        # C.B^T is formed again per head in fp32 (the tri * N term)
        "chunk_scan_bwd": (XI + 2 * X + DT + 2 * CS + 2 * BC + 2 * STe,
                           2 * bkh * (Q * N * P + 2 * tri * P + tri * N)),
        # dW, dC and dB head sums in one launch: x, dy, cs, the step, Hin and G in; dW and the
        # dC / dB head-slice partials out
        "dw_heads": (XI + X + 2 * CS + 2 * STe + DW + PART, 2 * bkh * tri * P + 4 * bkh * Q * P * N),
        # dC and dB: dW, the partials, B, C in; dC, dB out
        "bc_final": (DW + PART + 2 * BC + 2 * BCO, 4 * bkg * tri * N),
        "da_dd": (2 * b * K * H * 4 + 2 * H * 4, 0),
    }
    return m


def source_hash() -> str:
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "state_space_model_mamba2_amd", "csrc")
    for f in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


class Hip:
    """The few HIP runtime calls bench needs for events (plumbing)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e

    def elapsed_ms(self, a, b) -> float:
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def make_probe(kernel_id, start, stop):
    from state_space_model_mamba2_amd import _lib
    return _lib.Probe(kernel_id, 0, start.value, stop.value)


def run_step(ssd, dev, chunk, fscr, bscr, fprobe=None, bprobe=None):
    s0, dfs = dev.get("initial_state"), dev.get("dfinal_state")
    sp = dev.get("softplus", False)
    y, fs, ctx = ssd.fwd(dev["x"], dev["dt_raw"] if sp else dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], chunk,
                         initial_state=s0, dt_softplus=sp, dt_bias=dev["dt_bias"] if sp else None,
                         scratch=fscr, probe=fprobe)
    if dev.get("fwd_only", False):
        return y, fs, None
    g = ssd.bwd(dev["dy"], ctx, dfinal_state=dfs, want_dinitial_state=s0 is not None, scratch=bscr, probe=bprobe)
    return y, fs, g


def per_kernel_times(ssd, dev, chunk, fscr, bscr, hip, flush, reps=5):
    """Average duration of every kernel (probed one kernel per step), each
    step started on flushed caches like the timed steps."""
    from state_space_model_mamba2_amd import _lib
    import torch
    out = {}
    fwd_ids = range(0, _lib.N_FWD_KERNELS)
    for kid, name in enumerate(_lib.KERNELS):
        if dev.get("fwd_only", False) and kid not in fwd_ids:
            continue
        evs = [(hip.event(), hip.event()) for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            flush.fill_(float(i))
            p = make_probe(kid, a, b)
            run_step(ssd, dev, chunk, fscr, bscr, fprobe=p if kid in fwd_ids else None,
                     bprobe=None if kid in fwd_ids else p)
        torch.cuda.synchronize()
        out[name] = sum(hip.elapsed_ms(a, b) for a, b in evs) / reps
        for a, b in evs:
            hip.destroy(a)
            hip.destroy(b)
    return out


def copy_rate_gbps(flush):
    """Rate of a plain 1 GiB device-to-device copy: the achievable-HBM reference."""
    import torch
    src = torch.empty_like(flush).fill_(1.0)
    ts = []
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        flush.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    del src
    return 2 * flush.numel() * 4 / (ts[len(ts) // 2] / 1e3) / 1e9


def shader_clock_mhz():
    """Current shader clock level from the driver's sysfs table, if readable."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if line.rstrip().endswith("*"):
                    return line.split(":", 1)[1].strip().rstrip("*").strip()
        except OSError:
            pass
    return None


def cpu_model() -> str | None:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads() -> int:
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def cpu_baseline(shape, inp_full, batch_rows: int, heads: int):
    """Time the float64 oracle on the first `batch_rows` batch rows and the
    first `heads` heads (rounded to whole groups) of the workload's inputs;
    scale linearly in batch and heads to the workload's tokens/s."""
    import numpy as np
    from oracle import seq
    from state_space_model_mamba2_amd.inputs import bf16_bits_to_f32

    H, G = shape.nheads, shape.ngroups
    hpg = H // G
    heads = max(hpg, min(H, heads) // hpg * hpg)
    gs = heads // hpg
    nb = max(1, min(batch_rows, shape.batch))

    def f64(a):
        a = np.ascontiguousarray(a)
        return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)

    x = f64(inp_full.x[:nb, :, :heads])
    dt = f64(inp_full.dt[:nb, :, :heads])
    A, D = f64(inp_full.A[:heads]), f64(inp_full.D[:heads])
    B = f64(inp_full.B[:nb, :, :gs])
    C = f64(inp_full.C[:nb, :, :gs])
    dy = f64(inp_full.dy[:nb, :, :heads])
    threads = host_threads()
    t0 = time.perf_counter()
    seq.ssd_fwd(x, dt, A, B, C, D, nthreads=threads)
    seq.ssd_bwd(x, dt, A, B, C, D, dy, nthreads=threads)
    t = time.perf_counter() - t0
    scale = (shape.batch / nb) * (H / heads)
    tok_s = shape.batch * shape.seqlen / (t * scale)
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"float64 oracle fwd+bwd on batch rows 0..{nb - 1} of {shape.batch}, heads 0..{heads - 1} "
                      f"of {H} ({gs} group(s)), seqlen {shape.seqlen}: {t:.1f} s wall on {threads} threads; "
                      f"tokens/s scaled linearly by x{scale:g} (batch x heads) to the full workload"}


# HIP kernels that make up each timed kernel of the step (a probe brackets
# all of them); names may come mangled or demangled from rocprofv3.
def kernel_matches(bench_kernel: str, name: str) -> bool:
    fwd_flag = "Lb0E" in name or "false>" in name
    bwd_flag = "Lb1E" in name or "true>" in name
    rules = {
        "cumsum_bmm": "k_cumsum_bmm" in name,
        "chunk_state": "k_chunk_state" in name and fwd_flag,
        "state_passing": "k_state_passing" in name and fwd_flag,
        "chunk_scan": "k_chunk_scan_fwd" in name,
        "chunk_state_bwd": "k_chunk_state" in name and bwd_flag,
        "state_passing_bwd": "k_state_passing" in name and bwd_flag,
        "chunk_scan_bwd": "k_chunk_scan_bwd" in name or "k_dl_assemble" in name,
        "dw_heads": "k_dw_heads" in name or "k_head_sums" in name,
        "bc_final": "k_bc_final" in name,
        "da_dd": "k_da_dd" in name,
    }
    return rules.get(bench_kernel, False)


COPY_KERNEL = "__amd_rocclr_copyBuffer"  # the blit kernel behind a device-to-device copy


def _counter_rows(d: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no rocprofv3 counter_collection.csv under {d}")
    return rows


def _per_dispatch_kib(rows, counter: str, match) -> float:
    """Sum over the matching HIP kernels of their mean per-dispatch counter value (KiB)."""
    by_kernel = {}
    for r in rows:
        if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
            continue
        d = by_kernel.setdefault(r["Kernel_Name"], {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not by_kernel:
        raise SystemExit(f"no dispatch with counter {counter} matched")
    return sum(sum(v.values()) / len(v) for v in by_kernel.values())


def write_traffic(pmc_dir: str, kernel: str, workload: str, copy_bytes: int, commands: list) -> None:
    """HBM traffic per launch of `kernel` from two rocprofv3 --pmc passes
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for a device-to-device copy of `copy_bytes` bytes (which
    reads and writes exactly that many bytes)."""
    fetch = _per_dispatch_kib(_counter_rows(os.path.join(pmc_dir, "fetch")), "FETCH_SIZE",
                              lambda n: kernel_matches(kernel, n))
    write = _per_dispatch_kib(_counter_rows(os.path.join(pmc_dir, "write")), "WRITE_SIZE",
                              lambda n: kernel_matches(kernel, n))
    cf = _per_dispatch_kib(_counter_rows(os.path.join(pmc_dir, "copy_fetch")), "FETCH_SIZE", lambda n: COPY_KERNEL in n)
    cw = _per_dispatch_kib(_counter_rows(os.path.join(pmc_dir, "copy_write")), "WRITE_SIZE", lambda n: COPY_KERNEL in n)
    f_fetch = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    traffic = fetch * 1024.0 * f_fetch + write * 1024.0 * f_write
    out = {"kernel": kernel, "workload": workload, "source_hash": source_hash(),
           "fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_factor": f_fetch, "write_factor": f_write,
           "read_bytes": fetch * 1024.0 * f_fetch, "written_bytes": write * 1024.0 * f_write,
           "traffic_bytes": traffic, "commands": commands}
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def summarize_stats(csv_path: str, command: str, title: str) -> str:
    """Markdown table from a rocprofv3 --kernel-trace --stats *_kernel_stats.csv."""
    import csv
    with open(csv_path) as fh:
        rows = list(csv.DictReader(fh))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "rocprofv3 kernel statistics (durations in microseconds):", "",
             "| kernel | name as reported (truncated) | calls | total us | average us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    import re
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = r["Name"]
        m = re.search(r"(k_[a-z_0-9]+)", n)
        short = m.group(1) if m else n.split("(")[0].split("<")[0].replace("void ", "")[:40]
        # the kernels' bool template flag names the variant
        # (mangled Lb0E / Lb1E, or false / true in a demangled name)
        flag = re.search(r"L(b[01])E", n)
        bit = int(flag.group(1)[1]) if flag else (1 if ", true" in n else 0 if ", false" in n else None)
        labels = {"k_chunk_state": ("forward", "backward"), "k_state_passing": ("forward", "backward")}
        if bit is not None and short in labels:
            short += f" ({labels[short][bit]})"
        lines.append(f"| {short} | `{n[:70]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_hash") != source_hash():
        return None
    return d.get("traffic_bytes")


def conv_bench(args):
    """Causal depthwise conv1d: fwd + bwd per step.  Each direction is also
    timed alone over `steps` back-to-back calls with events on the launch
    stream (one call is short next to the Python launch overhead, so events
    around single calls would count the host's gaps); roofline against HBM."""
    import numpy as np
    import torch
    from state_space_model_mamba2_amd import _lib, inputs, ssd

    _lib.load()
    cw = dict(inputs.CONV_WORKLOADS[args.workload])
    cw.update({k: v for k, v in (("seqlen", args.seqlen), ("batch", args.batch)) if v is not None})
    b, L, C, W, dtype = cw["batch"], cw["seqlen"], cw["channels"], cw["width"], cw["dtype"]
    esz = 2 if dtype == "bf16" else 4
    log(f"[bench] conv1d {args.workload}: {cw}")
    ci = inputs.generate_conv(b, L, C, W, dtype, seed=0)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    x, w, bias, prev, dy = dev(ci.x), dev(ci.w), dev(ci.bias), dev(ci.x_prev), dev(ci.dy)

    fwd = lambda: ssd.conv1d_fwd(x, w, bias, prev)
    bwd = lambda: ssd.conv1d_bwd(x, w, dy, bias, prev, want_dx_prev=True)

    def timed(fn, n):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z) / n

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    fwd_ms = timed(fwd, args.steps)
    bwd_ms = timed(bwd, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    X = b * L * C * esz
    fwd_bytes = 2 * X + C * (W + 1) * 4                     # x in, y out, w, bias
    bwd_bytes = 3 * X + 2 * C * (W + 1) * 4                 # x, dy in, dx out, w, bias in, dw, dbias out
    dom, dom_ms, nbytes = ("conv1d_bwd", bwd_ms, bwd_bytes) if bwd_ms >= fwd_ms else ("conv1d_fwd", fwd_ms, fwd_bytes)
    achieved = nbytes / (dom_ms / 1e3) / 1e9
    log(f"[bench] conv1d fwd {fwd_ms:.4f} ms ({fwd_bytes / fwd_ms / 1e6:.0f} GB/s), "
        f"bwd {bwd_ms:.4f} ms ({bwd_bytes / bwd_ms / 1e6:.0f} GB/s), step {ms:.4f} ms")
    out = {"metric": "causal conv1d fwd+bwd tokens/s per GPU", "value": b * L / (ms / 1e3), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
           "config": {"workload": f"conv1d_{args.workload}", "batch": b, "seqlen": L, "channels": C, "width": W,
                      "silu": True, "parallelism": "single-gpu"},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": dom, "kernel_ms": dom_ms,
                        "algorithmic_bytes": nbytes},
           "kernel_ms": {"conv1d_fwd": fwd_ms, "conv1d_bwd": bwd_ms}, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--op", choices=["ssd", "conv1d"], default="ssd")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba2_2p7b")
    ap.add_argument("--seqlen", type=int, default=None, help="override the workload's sequence length")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    ap.add_argument("--with-states", action="store_true",
                    help="seeded initial state and final-state cotangent; dinitial_state returned")
    ap.add_argument("--dt-softplus", action="store_true",
                    help="raw step + per-head bias; the library applies the softplus")
    ap.add_argument("--dtype", choices=["f32", "bf16", "fp8"], default=None, help="override the storage mode")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward pass alone")
    ap.add_argument("--cpu-heads", type=int, default=80, help="heads in the oracle CPU-baseline slice")
    ap.add_argument("--cpu-batch", type=int, default=4, help="batch rows in the oracle CPU-baseline slice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernel", default=None,
                    help="only run warmup + steps (for rocprofv3); no breakdown, no CPU baseline")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration mode: time a plain device copy of this many bytes and exit")
    ap.add_argument("--write-traffic", metavar="PMC_DIR", default=None,
                    help="(no GPU) write profiles/traffic_<kernel>_<workload>.json from the rocprofv3 --pmc "
                         "passes under PMC_DIR/{fetch,write,copy_fetch,copy_write}; needs --traffic-kernel "
                         "and --copy-bytes of the calibration copy")
    ap.add_argument("--traffic-kernel", default="chunk_scan_bwd")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="the profiling commands, recorded in the JSON")
    ap.add_argument("--summarize-stats", metavar="CSV", default=None,
                    help="(no GPU) print a markdown summary of a rocprofv3 *_kernel_stats.csv")
    ap.add_argument("--stats-command", default="")
    ap.add_argument("--stats-title", default="")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args.write_traffic, args.traffic_kernel, args.workload, args.copy_bytes, args.traffic_command)
        return
    if args.summarize_stats:
        sys.stdout.write(summarize_stats(args.summarize_stats, args.stats_command, args.stats_title))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the SSD scan here is a "
              f"single-GPU build and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.op == "conv1d":
        conv_bench(args)
        return

    import torch
    from state_space_model_mamba2_amd import _lib, inputs, ssd

    if args.copy_bytes:
        n = args.copy_bytes // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        dt_s = (time.perf_counter() - t0) / 10
        print(json.dumps({"copy_bytes": n * 4, "ms": dt_s * 1e3, "GBps": 2 * n * 4 / dt_s / 1e9}))
        return

    _lib.load()  # fail loudly if the HIP library is missing
    over = {k: v for k, v in (("seqlen", args.seqlen), ("batch", args.batch), ("dtype", args.dtype))
            if v is not None}
    shape = inputs.workload(args.workload, **over)
    esz = 4 if shape.dtype == "f32" else 2
    log(f"[bench] workload {args.workload}: {shape}")
    t0 = time.perf_counter()
    inp = inputs.generate(shape, seed=0)
    dev = ssd.to_device(inp, "cuda")
    if args.dt_softplus:
        dev["softplus"] = True
    if args.fwd_only:
        dev["fwd_only"] = True
    if args.with_states:
        s0, dfs = inputs.generate_states(shape, seed=0)
        dev["initial_state"] = torch.from_numpy(s0).cuda()
        dev["dfinal_state"] = torch.from_numpy(dfs).cuda()
    torch.cuda.synchronize()
    log(f"[bench] inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")

    code = {"f32": _lib.SSD_F32, "bf16": _lib.SSD_BF16, "fp8": _lib.SSD_FP8}[shape.dtype]
    shp = ssd.shape_of(dev["x"], dev["B"], shape.chunk, code, _lib.SSD_DT_SOFTPLUS if args.dt_softplus else 0)
    lib = _lib.load()
    fscr = torch.empty(lib.ssd_fwd_scratch_bytes(ctypes.byref(shp)), dtype=torch.uint8, device="cuda")
    bscr = torch.empty(lib.ssd_bwd_scratch_bytes(ctypes.byref(shp)), dtype=torch.uint8, device="cuda")

    hip = Hip()
    model = kernel_model(shape, esz)
    # written before every timed step: 1 GiB evicts the L2s and the 256 MB Infinity Cache
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    for _ in range(args.warmup):
        run_step(ssd, dev, shape.chunk, fscr, bscr)
    torch.cuda.synchronize()

    if args.profile_kernel is None:
        breakdown = per_kernel_times(ssd, dev, shape.chunk, fscr, bscr, hip, flush)
        dom = max(breakdown, key=breakdown.get)
    else:
        breakdown, dom = {}, args.profile_kernel
    dom_id = _lib.KERNEL_ID[dom]
    is_fwd = dom_id < _lib.N_FWD_KERNELS

    # Timed region: exactly `steps` steps, each started on flushed caches (the
    # flush is outside the step's events) and timed with events on the launch
    # stream; the dominant kernel is bracketed by its own events in each step.
    # The headline is the median cold step.
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, ((a, b), (sa, sb)) in enumerate(zip(evs, step_evs)):
        flush.fill_(float(i))
        p = make_probe(dom_id, a, b)
        sa.record()
        run_step(ssd, dev, shape.chunk, fscr, bscr, fprobe=p if is_fwd else None, bprobe=None if is_fwd else p)
        sb.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(hip.elapsed_ms(a, b) for a, b in evs) / len(evs)
    cold = sorted(sa.elapsed_time(sb) for sa, sb in step_evs)
    ms_per_step = cold[len(cold) // 2]
    tokens = shape.batch * shape.seqlen
    value = tokens / (ms_per_step / 1e3)

    # Secondary: the same number of steps back to back on warm caches.
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        run_step(ssd, dev, shape.chunk, fscr, bscr)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t1) * 1e3 / args.steps

    peak_mfma = MFMA_PEAK_TFLOPS[shape.dtype]
    ridge = peak_mfma * 1e12 / (HBM_PEAK_GBS * 1e9)

    def fracs(k, ms):
        nb, nf = model[k]
        t = ms / 1e3
        return {"ms": ms, "hbm_frac": nb / t / 1e9 / HBM_PEAK_GBS, "mfma_frac": nf / t / 1e12 / peak_mfma,
                # what HBM alone allows the matrix cores: arithmetic intensity x 8 TB/s over the peak
                "mfma_cap_frac": min(1.0, (nf / nb) / ridge) if nb else None,
                "algorithmic_bytes": nb, "algorithmic_flops": nf}

    nbytes, nflops = model[dom]
    t_s = dom_ms / 1e3
    mfma_frac = nflops / t_s / 1e12 / peak_mfma if nflops else 0.0
    hbm_frac = nbytes / t_s / 1e9 / HBM_PEAK_GBS
    ai = nflops / nbytes if nbytes else 0.0
    if ai > ridge:
        roof = {"bound": "mfma", "achieved": nflops / t_s / 1e12, "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": mfma_frac}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / t_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm_frac}
    plain = not over and not args.with_states and not args.dt_softplus
    roof["traffic"] = load_traffic(dom, args.workload) if plain else None
    roof["kernel"] = dom
    roof["kernel_ms"] = dom_ms
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = nflops
    roof["mfma_frac"] = mfma_frac
    roof["hbm_frac"] = hbm_frac

    targets = None
    if breakdown:
        log("[bench] per-kernel average duration (ms, flushed caches), algorithmic GB/s and TFLOP/s:")
        tot = sum(breakdown.values())
        for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1]):
            nb, nf = model[k]
            log(f"  {k:18s} {v:8.4f} ms {100 * v / tot:5.1f}%  {nb / v / 1e6:8.1f} GB/s ({100 * nb / v / 1e6 / HBM_PEAK_GBS:5.1f}%)"
                f"  {nf / v / 1e9:7.1f} TFLOP/s ({100 * nf / v / 1e9 / peak_mfma:5.1f}%)")
        log(f"  sum of kernels {tot:.4f} ms vs step {ms_per_step:.4f} ms")
        per = {k: fracs(k, v) for k, v in breakdown.items()}
        gemm = [k for k in ("chunk_state", "chunk_scan", "chunk_state_bwd", "chunk_scan_bwd", "dw_heads") if k in per]
        scan = [k for k in ("state_passing", "state_passing_bwd") if k in per]
        # the step's own floor: compulsory I/O of both passes plus five passes over
        # the chunk states (forward write and read of the entry states; backward
        # write and read of their gradients, and a read of the entry states),
        # at the storage element size the states are kept in
        b_, L_, H_, P_, N_, G_ = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
        K_ = -(-L_ // shape.chunk)
        X = b_ * L_ * H_ * P_ * esz
        XI = b_ * L_ * H_ * P_ * (1 if shape.dtype == "fp8" else esz)
        BCb = b_ * L_ * G_ * N_ * (1 if shape.dtype == "fp8" else esz)
        DTb = b_ * L_ * H_ * esz
        FS = b_ * H_ * P_ * N_ * 4
        io = (XI + DTb + 2 * BCb + X + FS) + (0 if args.fwd_only else (X + XI + DTb + 2 * BCb + X + DTb + 2 * BCb))
        passes = (2 if args.fwd_only else 5) * b_ * K_ * H_ * P_ * N_ * esz
        step_floor_ms = (io + passes) / (HBM_PEAK_GBS * 1e9) * 1e3
        targets = {
            "chunk_gemm_mfma": {"target_frac": 0.50, "peak_tflops": peak_mfma,
                                "kernels": {k: {"mfma_frac": per[k]["mfma_frac"], "mfma_cap_frac": per[k]["mfma_cap_frac"]}
                                            for k in gemm}},
            "state_passing_hbm": {"target_frac": 0.60, "peak_gbps": HBM_PEAK_GBS,
                                  "kernels": {k: {"hbm_frac": per[k]["hbm_frac"]} for k in scan},
                                  "met": all(per[k]["hbm_frac"] >= 0.60 for k in scan)},
            "step_hbm_floor": {"bytes": io + passes, "ms": step_floor_ms, "frac": step_floor_ms / ms_per_step},
            "kernels": per,
        }

    timing = None
    if args.profile_kernel is None:
        timing = {"cold_ms_per_step_median": ms_per_step, "cold_ms_per_step_max": cold[-1],
                  "cold_ms_per_step_min": cold[0], "warm_ms_per_step": warm_ms,
                  "wall_ms_per_step_incl_flush": wall * 1e3 / args.steps,
                  "copy_GBps": copy_rate_gbps(flush), "shader_clock": shader_clock_mhz()}
        roof["frac_of_copy"] = roof["achieved"] / timing["copy_GBps"] if roof["unit"] == "GB/s" else None
        log(f"[bench] step median cold {ms_per_step:.4f} ms, warm (back to back) {warm_ms:.4f} ms;"
            f" 1 GiB copy {timing['copy_GBps']:.0f} GB/s; shader clock {timing['shader_clock']}")
    del flush

    cpu = None
    if not args.no_cpu_baseline and args.profile_kernel is None and not args.fwd_only:
        log("[bench] timing the float64 oracle on a bounded sample ...")
        cpu = cpu_baseline(shape, inp, args.cpu_batch, args.cpu_heads)
        log(f"[bench] {cpu['sample']}")

    out = {
        "metric": "SSD fwd tokens/s per GPU" if args.fwd_only else METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": shape.batch, "seqlen": shape.seqlen,
                   "nheads": shape.nheads, "headdim": shape.headdim, "dstate": shape.dstate,
                   "ngroups": shape.ngroups, "chunk": shape.chunk, "parallelism": "single-gpu",
                   "initial_state": bool(args.with_states), "dt_softplus": bool(args.dt_softplus),
                   "state_storage": "f32" if shape.dtype == "f32" else "bf16",
                   "caches": "flushed before every timed step"},
        "roofline": roof,
        "targets": targets,
        "cpu_baseline": cpu,
        "kernel_ms": breakdown or None,
        "timing": timing,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
