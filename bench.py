"""Throughput benchmark of the MI355X NSA forward (one GPU).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                [--no-cpu-baseline] [--profile-only] [--no-extra]

A step is one whole forward pass (pool, compressed attention + top-k,
selection + window + gated combine) over one batch of seeded synthetic input
already resident in HBM; the selection-branch backward of the same input (the
rest of the hot path) is timed after it and reported beside the forward.
Prints ONE JSON line (rank 0, N = 1):
  value      = forward tokens/s = batch * seq_len / (seconds per forward step)
  roofline   = the selection/window/combine kernel (the dominant one): useful
               attention FLOPs per launch / its average duration, measured with
               HIP events recorded around it on its own stream in K steps run
               right after the timed ones (the events would perturb the timed
               steps), against the bf16 dense MFMA peak
  cpu_baseline = the fp64 oracle timed on the host (every core this process
               may use; nproc and CPU model stated) on a bounded sample of the
               same workload: whole forward passes, about ten seconds of them
  workloads  = nested results (same fields) of the other seq-8192 and
               long-context shapes: the 1.3B layer (B4 T8192 Hq16 Hkv4 D128),
               the MQA ablation (B4 T8192 Hq16 Hkv1 D128: all branches, the
               compression output pruned, the window alone) and the 32k layer
               (B1 T32768 Hq16 Hkv4 D128, forward plus selection backward)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NSA fwd tokens/sec at seq 8192 GQA-4 bf16; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def useful_counts(wl):
    """Per (b, h): sums over t of |K_sel(t)|, |K_win(t)|, n_c(t) -- the keys the
    method itself must attend (closed form of the selection rules)."""
    T, k, W = wl.seq_len, wl.top_k, wl.window
    sel = win = cmp = 0
    for t in range(T):
        c = t // 64
        if c == 0:
            sel += t + 1
        else:
            sel += (t % 64 + 1) + 64 + 64 * min(c - 1, k - 2)
        win += min(W, t + 1)
        cmp += (t + 1) // 64
    return sel, win, cmp


def useful_flops(wl, branches="all"):
    """Useful forward FLOPs: 4 D per (query, head, attended key).  With the
    compression output pruned only its scores (Q Kc^T, 2 D per pooled key) are
    still needed for the selection; window-only needs the window alone."""
    sel, win, cmp = useful_counts(wl)
    per = 4 * wl.head_dim * wl.batch * wl.n_q_heads
    if branches == "window":
        sel, cmp = 0, 0
    elif branches == "no-cmp":
        cmp = cmp / 2
    return {"sel_win": per * (sel + win), "cmp": per * cmp, "total": per * (sel + win + cmp)}


def useful_bwd_flops(wl):
    """Selection-branch backward: 10 D FLOPs per (query, head, selected key s <= t)
    (dP = dO V^T, dV += P^T dO, dQ += dS K, dK += dS^T Q, 2 D each, plus the
    recomputed S = Q K^T)."""
    sel, _, _ = useful_counts(wl)
    return 10 * wl.head_dim * wl.batch * wl.n_q_heads * sel


def useful_full_bwd_flops(wl):
    """Gradient of all three branches: 10 D FLOPs per (query, head, attended key)
    over the selected, window and visible pooled keys (the pooled keys' gradient
    back through the mean-pool is not counted)."""
    sel, win, cmp = useful_counts(wl)
    return 10 * wl.head_dim * wl.batch * wl.n_q_heads * (sel + win + cmp)


def algorithmic_bytes(wl):
    """HBM bytes the whole forward must move at least once (inputs read once,
    output written once)."""
    es = 2 if wl.dtype == "bf16" else 4
    B, T, Hq, Hkv, D = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    return es * (B * T * Hq * D * 2 + 2 * B * T * Hkv * D + B * T * Hq * 3)


def host_cores():
    """Cores this process may run on (the host's CPU share)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, arrs_f64, min_seconds=10.0, max_passes=50):
    """The fp64 oracle on the host, on every core this process may use: whole
    forward passes of the same workload, repeated until at least min_seconds
    of wall time have been measured."""
    import oracle

    threads = int(os.environ.get("NSA_ORACLE_THREADS", "0")) or host_cores()
    passes, t_total = 0, 0.0
    while passes < max_passes and (passes == 0 or t_total < min_seconds):
        t0 = time.perf_counter()
        oracle.forward(arrs_f64["q"], arrs_f64["k"], arrs_f64["v"], arrs_f64["gates"],
                       top_k=wl.top_k, window=wl.window, scale=wl.scale, threads=threads)
        t_total += time.perf_counter() - t0
        passes += 1
    tokens = wl.batch * wl.seq_len
    return {"value": round(tokens * passes / t_total, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{passes} full forward pass(es) of {wl.name} (batch {wl.batch} x "
                      f"{wl.seq_len} positions, all heads, fp64), {t_total:.1f} s total"}


# --- HBM traffic of the dominant kernel from committed rocprofv3 counters -----
PROFILES = os.path.join(ROOT, "profiles")
K3_SOURCES = ["sparse_attention_long_compress_amd/csrc/sel_win.hip",
              "sparse_attention_long_compress_amd/csrc/sel_compact.hip",
              "sparse_attention_long_compress_amd/csrc/nsa_device.h",
              "sparse_attention_long_compress_amd/csrc/nsa_launch.h"]


def k3_kernel(wl, branches="all"):
    """Name of the selection/window kernel the library runs for this workload
    (asked from the library itself: nsa_forward_kernel)."""
    import sparse_attention_long_compress_amd as nsa

    flags = {"all": 0, "no-cmp": nsa.SKIP_CMP_OUT,
             "window": nsa.SKIP_CMP_OUT | nsa.SKIP_SEL}[branches]
    p = nsa.make_params(wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                        top_k=wl.top_k, window=wl.window,
                        dtype=nsa.NSA_BF16 if wl.dtype == "bf16" else nsa.NSA_FP32,
                        scale=wl.scale, flags=flags)
    return nsa.forward_kernel(p)


def kernel_source_hash(paths=K3_SOURCES):
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_summary(path):
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def committed_traffic(workload, kernel):
    """Bytes per launch of the selection/window kernel from profiles/, or None
    when the summary is missing or the kernel source changed since it was taken."""
    summ = read_summary(os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt"))
    if not summ or summ.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(summ["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, kernel):
    """Text summary of FETCH_SIZE / WRITE_SIZE (KiB per dispatch) for `kernel`,
    scaled by what the same counters read for a copy kernel of known size."""
    import csv

    def per_dispatch(path, name_part, counter):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter]
        return sum(vals) / len(vals), len(vals)

    def biggest(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        return max(float(r["Counter_Value"]) for r in rows)

    f_kib, nf = per_dispatch(fetch_csv, kernel, "FETCH_SIZE")
    w_kib, nw = per_dispatch(write_csv, kernel, "WRITE_SIZE")
    cf = copy_bytes / 1024.0 / biggest(copy_fetch_csv, "FETCH_SIZE")
    cw = copy_bytes / 1024.0 / biggest(copy_write_csv, "WRITE_SIZE")
    traffic = (f_kib * cf + w_kib * cw) * 1024.0
    lines = [f"kernel: {kernel}", f"source_hash: {kernel_source_hash()}",
             f"fetch_kib_per_dispatch: {f_kib:.1f}  (mean of {nf} dispatches)",
             f"write_kib_per_dispatch: {w_kib:.1f}  (mean of {nw} dispatches)",
             f"copy_kernel_bytes: {copy_bytes}",
             f"copy_fetch_factor: {cf:.4f}", f"copy_write_factor: {cw:.4f}",
             f"traffic_bytes_per_launch: {traffic:.0f}"]
    return "\n".join(lines)


def copy_calibration(nbytes):
    """A plain device copy of known size (one elementwise kernel per call), for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = nbytes // 4
    a = torch.ones(n, device="cuda", dtype=torch.float32)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()


def decode_bench(nsa, torch, np, wl, steps, warmup, batch=64):
    """One decode step (nsa_decode) for `batch` sequences of the workload's
    shape at full cache length (the workload's seq_len), timed with HIP events
    on the current stream.  Algorithmic HBM bytes per step: for every
    (sequence, KV group) the K and V rows of the union of its selected blocks
    and its window (keys <= t), its pooled keys and values, plus q, gates and
    out; taken from the step's own selection."""
    Lmax = wl.seq_len
    Hq, Hkv, D = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(wl.seed + 7)
    k = torch.randn((batch, Lmax, Hkv, D), dtype=tdt, device="cuda", generator=gen)
    v = torch.randn((batch, Lmax, Hkv, D), dtype=tdt, device="cuda", generator=gen)
    q = torch.randn((batch, Hq, D), dtype=tdt, device="cuda", generator=gen)
    gates = torch.sigmoid(torch.randn((batch, Hq, 3), device="cuda", generator=gen)).to(tdt)
    kc, vc = nsa.pool(k, v)
    lens = torch.full((batch,), Lmax, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    res = nsa.decode(q, k, v, kc, vc, lens, gates, top_k=wl.top_k, window=wl.window,
                     scale=wl.scale, want_indices=True)
    idx = res["indices"].cpu().numpy()
    t = Lmax - 1
    own, nc = t // 64, Lmax // 64
    jw_lo = max(0, t - wl.window + 1) // 64
    es = 2 if wl.dtype == "bf16" else 4
    blocks = 0
    for b in range(batch):
        for g in range(Hkv):
            sel = {int(j) for j in idx[b, g] if j >= 0}
            blocks += len(sel | set(range(jw_lo, own + 1)))
    nbytes = (blocks * 64 * D * 2 * es + batch * Hkv * nc * D * 2 * es
              + batch * Hq * (2 * D + 3) * es)
    for _ in range(warmup):
        nsa.decode(q, k, v, kc, vc, lens, gates, top_k=wl.top_k, window=wl.window,
                   scale=wl.scale, out=out)
    torch.cuda.synchronize()
    # one event pair around all the steps (events between steps perturb them)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        nsa.decode(q, k, v, kc, vc, lens, gates, top_k=wl.top_k, window=wl.window,
                   scale=wl.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) * 1e-3 / steps
    gbs = nbytes / dt / 1e9
    return {"kernel": "decode_mfma_kernel" if wl.dtype == "bf16" else "decode_kernel",
            "batch": batch, "cache_len": Lmax,
            "step_us": round(dt * 1e6, 2), "tokens_per_s": round(batch / dt, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": int(nbytes)}}


def prepare(wl, with_dout):
    """Seeded synthetic inputs of the workload, rounded once to its dtype,
    resident in HBM (plus the rounded CPU copy for the oracle)."""
    import torch

    from sparse_attention_long_compress_amd.synth import draw, to_dtype

    arrs = draw(wl, with_dout=with_dout)
    cpu = to_dtype(arrs, wl.dtype)
    dev = {k: v.to("cuda") for k, v in cpu.items()}
    torch.cuda.synchronize()
    return dev, cpu


def time_forward(nsa, torch, np, wl, dev, steps, warmup, branches="all"):
    """Forward steps of the workload timed with the host clock (bracketed by
    synchronisations): the throughput.  Then the same number of steps again
    with HIP events recorded by the library around each of its three kernels
    on the launch stream: the per-kernel durations (recording those events
    costs about 35 us of a 190 us step, so they are kept out of the
    throughput region)."""
    bflags = {"all": 0, "no-cmp": nsa.SKIP_CMP_OUT,
              "window": nsa.SKIP_CMP_OUT | nsa.SKIP_SEL}[branches]
    p = nsa.params_for(dev["q"], dev["k"], top_k=wl.top_k, window=wl.window, scale=wl.scale,
                       flags=bflags)
    ws = nsa.alloc_workspace(p, dev["q"].device)
    out = torch.empty_like(dev["q"])

    def step(events=None):
        nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                    window=wl.window, scale=wl.scale, out=out, workspace=ws, events=events,
                    flags=bflags)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # events (created by torch on the current stream's device; raw handles go to the library)
    evs = []
    for _ in range(steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in row:
            e.record()  # materialise the underlying hipEvent_t
        evs.append(row)
    torch.cuda.synchronize()
    for i in range(steps):
        step(events=[e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    k1 = np.mean([r[0].elapsed_time(r[1]) for r in evs]) * 1e-3
    k2 = np.mean([r[1].elapsed_time(r[2]) for r in evs]) * 1e-3
    k3 = np.mean([r[2].elapsed_time(r[3]) for r in evs]) * 1e-3
    ev_step = np.mean([r[0].elapsed_time(r[3]) for r in evs]) * 1e-3
    fl = useful_flops(wl, branches)
    tokens = wl.batch * wl.seq_len
    achieved = fl["sel_win"] / k3 / 1e12
    kern = k3_kernel(wl, branches)
    return {
        "wall": wall, "ws": ws,
        "tokens_per_s": round(tokens / wall, 1),
        "ms_per_step": round(wall * 1e3, 4),
        "useful_tflops": round(fl["total"] / wall / 1e12, 2),
        "pct_bf16_peak": round(100 * fl["total"] / wall / 1e12 / PEAK_BF16_TFLOPS, 2),
        "stage_us": {"pool": round(k1 * 1e6, 2), "cmp_select": round(k2 * 1e6, 2),
                     "sel_win_combine": round(k3 * 1e6, 2), "events_total": round(ev_step * 1e6, 2)},
        "roofline": {"kernel": kern, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": committed_traffic(wl.name, kern) if branches == "all" else None},
    }


def time_select_bwd(nsa, torch, np, wl, dev, ws, steps, warmup):
    """The selection-branch backward of the same input, fed by the forward's
    saved indices, log-sum-exp and o_sel; HIP events around each call."""
    p = nsa.params_for(dev["q"], dev["k"], top_k=wl.top_k, window=wl.window, scale=wl.scale)
    res_f = nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                        window=wl.window, scale=wl.scale, workspace=ws, want_indices=True,
                        want_lse=True, want_o_sel=True)
    wsb = nsa.alloc_workspace(p, dev["q"].device, backward=True)
    grads = (torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"]))

    def bstep():
        nsa.select_bwd(dev["q"], dev["k"], dev["v"], dev["gates"], res_f["indices"],
                       res_f["lse_sel"], res_f["o_sel"], dev["dout"], top_k=wl.top_k,
                       scale=wl.scale, workspace=wsb, out=grads)

    for _ in range(warmup):
        bstep()
    torch.cuda.synchronize()
    # one event pair around all the calls (events between calls perturb them)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        bstep()
    e1.record()
    torch.cuda.synchronize()
    bwd = e0.elapsed_time(e1) * 1e-3 / steps
    fb = useful_bwd_flops(wl)
    return bwd, {"us": round(bwd * 1e6, 2), "useful_tflops": round(fb / bwd / 1e12, 2),
                 "pct_bf16_peak": round(100 * fb / bwd / 1e12 / PEAK_BF16_TFLOPS, 2)}


def public(d):
    return {k: v for k, v in d.items() if k not in ("wall", "ws")}


def extra_configs(nsa, torch, np, steps, warmup):
    """The other seq-8192 / long-context workloads, each a nested result:
    1.3B (B4 T8192 Hq16 Hkv4 D128) forward; the MQA ablation (B4 T8192 Hq16
    Hkv1 D128) with all branches, the compression output pruned, and the
    window alone; the 32k forward plus selection backward (B1 T32768 Hq16
    Hkv4 D128)."""
    from sparse_attention_long_compress_amd.synth import WORKLOADS

    out = {}
    wl = WORKLOADS["1b3-gqa4"]
    print(f"# timing {wl.name}", file=sys.stderr, flush=True)
    dev, _ = prepare(wl, False)
    out[wl.name] = public(time_forward(nsa, torch, np, wl, dev, steps, warmup))
    del dev
    torch.cuda.empty_cache()
    wl = WORKLOADS["mqa-ablation"]
    print(f"# timing {wl.name}", file=sys.stderr, flush=True)
    dev, _ = prepare(wl, False)
    runs = {}
    for br in ("all", "no-cmp", "window"):
        runs[br] = public(time_forward(nsa, torch, np, wl, dev, steps, warmup, br))
    runs["window_only_speedup"] = round(runs["all"]["ms_per_step"] / runs["window"]["ms_per_step"], 2)
    out[wl.name] = runs
    del dev
    torch.cuda.empty_cache()
    wl = WORKLOADS["32k-fwd-bwd"]
    print(f"# timing {wl.name}", file=sys.stderr, flush=True)
    dev, _ = prepare(wl, True)
    f = time_forward(nsa, torch, np, wl, dev, steps, warmup)
    bwd, b = time_select_bwd(nsa, torch, np, wl, dev, f["ws"], steps, warmup)
    r = public(f)
    r["selection_backward"] = b
    r["fwd_plus_bwd_tokens_per_s"] = round(wl.batch * wl.seq_len / (f["wall"] + bwd), 1)
    out[wl.name] = r
    del dev, f
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="340m-gqa4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + steps and exit without the oracle (for rocprofv3)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                       "COPY_WRITE_CSV"),
                    help="print the traffic summary of the workload's selection/window kernel "
                         "from rocprofv3 CSVs and exit")
    ap.add_argument("--copy-bytes", type=int, default=256 << 20)
    ap.add_argument("--ab-single", action="store_true",
                    help="only time the two-pass selection backward against the single-pass one "
                         "with atomics (nsa_select_bwd_single) and print one JSON line")
    ap.add_argument("--branches", choices=("all", "no-cmp", "window"), default="all",
                    help="branches in the output: all; no-cmp (compression output pruned, its scores "
                         "still drive the selection); window (sliding window only) -- the pruned-branch "
                         "layers of the MQA ablation.  Other than 'all' implies --no-backward --no-decode")
    ap.add_argument("--no-decode", action="store_true",
                    help="leave out the decode-step measurement (nsa_decode, 64 sequences at "
                         "full cache length)")
    ap.add_argument("--no-backward", action="store_true",
                    help="time the forward only (the selection-branch backward and a training "
                         "step -- forward with saved tensors plus the full backward -- are timed "
                         "by default)")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the nested results of the 1.3B, MQA-ablation and 32k workloads")
    args = ap.parse_args()
    if args.pmc_summary:
        from sparse_attention_long_compress_amd.synth import WORKLOADS as _W
        print(pmc_summary(*args.pmc_summary, copy_bytes=args.copy_bytes,
                          kernel=k3_kernel(_W[args.workload])))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards over batch or KV groups with no exchange; see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_long_compress_amd as nsa
    from sparse_attention_long_compress_amd.synth import WORKLOADS, as_f64

    wl = WORKLOADS[args.workload]
    if args.branches != "all":
        args.no_backward = True
        args.no_decode = True
        args.no_extra = True
    if args.workload != "340m-gqa4" or args.profile_only or args.ab_single:
        args.no_extra = True
    dev, cpu = prepare(wl, not args.no_backward or args.ab_single)
    p = nsa.params_for(dev["q"], dev["k"], top_k=wl.top_k, window=wl.window, scale=wl.scale)

    if args.ab_single:
        ws = nsa.alloc_workspace(p, dev["q"].device)
        res_f = nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                            window=wl.window, scale=wl.scale, workspace=ws, want_indices=True,
                            want_lse=True, want_o_sel=True)
        fargs = (dev["q"], dev["k"], dev["v"], dev["gates"], res_f["indices"], res_f["lse_sel"],
                 res_f["o_sel"], dev["dout"])
        grads = (torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"]))
        ab = {}
        for name, fn, mode in (("two_pass", nsa.select_bwd, True),
                               ("single_pass_atomic", nsa.select_bwd_single, "single")):
            wsx = nsa.alloc_workspace(p, dev["q"].device, backward=mode)
            for _ in range(args.warmup):
                fn(*fargs, top_k=wl.top_k, scale=wl.scale, workspace=wsx, out=grads)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn(*fargs, top_k=wl.top_k, scale=wl.scale, workspace=wsx, out=grads)
            e1.record()
            torch.cuda.synchronize()
            ab[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / args.steps, 2)
            del wsx
        ab["single_over_two_pass"] = round(ab["single_pass_atomic_us"] / ab["two_pass_us"], 2)
        print(json.dumps({"selection_backward_ab": ab, "workload": wl.name, "steps": args.steps}),
              flush=True)
        return

    fwd = time_forward(nsa, torch, np, wl, dev, args.steps, args.warmup, args.branches)
    wall, ws = fwd["wall"], fwd["ws"]

    # the rest of the hot path: the selection-branch backward of the same input
    bwd = bres = None
    if not args.no_backward:
        bwd, bres = time_select_bwd(nsa, torch, np, wl, dev, ws, args.steps, args.warmup)

    # a training step: the forward that saves every tensor the full backward
    # needs, then the gradient of all three branches and the gates
    train = None
    if not args.no_backward:
        wsf = nsa.alloc_workspace(p, dev["q"].device, backward="full")
        saved = nsa.forward_train(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                                  window=wl.window, scale=wl.scale, workspace=ws)
        fgrads = (torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"]),
                  torch.empty_like(dev["gates"]))

        def fstep():
            nsa.forward_train(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                              window=wl.window, scale=wl.scale, workspace=ws, out=saved["out"])

        def bwstep():
            nsa.backward(dev["q"], dev["k"], dev["v"], dev["gates"], saved, dev["dout"],
                         top_k=wl.top_k, window=wl.window, scale=wl.scale, workspace=wsf,
                         out=fgrads)

        def loop_time(fn):
            # one event pair around all the calls (events between calls perturb them)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / args.steps

        for _ in range(args.warmup):
            fstep()
            bwstep()
        torch.cuda.synchronize()
        train = (loop_time(fstep), loop_time(bwstep))
        del wsf, saved, fgrads

    tokens = wl.batch * wl.seq_len
    if args.profile_only:
        dec = None if args.no_decode else decode_bench(nsa, torch, np, wl, args.steps, args.warmup)
        st = fwd["stage_us"]
        print(json.dumps({"profile_only": True, "ms_per_step": wall * 1e3,
                          "decode_us": None if dec is None else dec["step_us"],
                          "k1_us": st["pool"], "k2_us": st["cmp_select"],
                          "k3_us": st["sel_win_combine"],
                          "sel_bwd_us": None if bwd is None else bwd * 1e6,
                          "train_fwd_us": None if train is None else train[0] * 1e6,
                          "full_bwd_us": None if train is None else train[1] * 1e6}), flush=True)
        return

    res = {
        "metric": METRIC,
        "value": fwd["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fwd["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, sigmoid(N(0,1)) gates)",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "block": 64, "top_k": wl.top_k,
                   "window": wl.window, "branches": args.branches, "parallelism": "none (1 GPU)"},
        "useful_tflops": fwd["useful_tflops"],
        "pct_bf16_peak": fwd["pct_bf16_peak"],
        "stage_us": fwd["stage_us"],
        "roofline": fwd["roofline"],
    }
    if bwd is not None:
        bres["fwd_plus_bwd_ms"] = round((wall + bwd) * 1e3, 4)
        bres["fwd_plus_bwd_tokens_per_s"] = round(tokens / (wall + bwd), 1)
        res["selection_backward"] = bres
    if train is not None:
        ff, fbf = useful_flops(wl)["total"], useful_full_bwd_flops(wl)
        step_s = train[0] + train[1]
        res["training_step"] = {
            "forward_us": round(train[0] * 1e6, 2), "full_backward_us": round(train[1] * 1e6, 2),
            "full_backward_useful_tflops": round(fbf / train[1] / 1e12, 2),
            "step_ms": round(step_s * 1e3, 4), "tokens_per_s": round(tokens / step_s, 1),
            "pct_bf16_peak": round(100 * (ff + fbf) / step_s / 1e12 / PEAK_BF16_TFLOPS, 2)}
    if not args.no_decode:
        res["decode"] = decode_bench(nsa, torch, np, wl, args.steps, args.warmup)
    del fwd, ws, dev
    torch.cuda.empty_cache()
    if not args.no_extra:
        res["workloads"] = extra_configs(nsa, torch, np, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        f64 = {k: as_f64(v) for k, v in cpu.items()}
        res["cpu_baseline"] = cpu_baseline(wl, f64)
        res["cpu_baseline"]["gpu_over_cpu"] = round(res["value"] / res["cpu_baseline"]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
