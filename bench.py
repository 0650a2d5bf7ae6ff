"""Benchmark of the block-sparse attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-gsrs-loop]
    python bench.py --cpu-full NAME [--cpu-threads T]     (CPU oracle only, whole workload)

A step is one pass of the whole path over one batch of seeded synthetic
video tokens already resident in HBM: the block-importance estimator
(mean-pool, pooled scores, row softmax, Top-p, CSR) followed by the sparse
forward with exact per-block attention mass (and, on the training workload,
the backward).  The default workload is the largest single-GPU one, the
HunyuanVideo-like layer (B 1, H 24, N 118,800, D 128, block 128).  Prints one
JSON line; besides the step it times the reduced-search loop of the GSRS page
(Figure 4 and Figure 7 captions) over the Wan2.1-like workload's five
denoising steps.

value = executed forward FLOP (4 D sum over selected pairs |Q_i||K_j|) per
step divided by the step time, in TFLOP/s.  The roofline object reports the
forward kernel alone, timed with HIP events on its stream.
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
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd TFLOP/s (executed + dense-equiv) and % bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
KERNEL_SOURCES = ["block_sparse_attention_16_amd/csrc/forward_bf16.hip"]


def executed_pairs(N: int, block: int, BH: int, row_ptr: np.ndarray, col_idx: np.ndarray) -> int:
    """Sum over selected (i, j) of |Q_i| * |K_j| (valid token pairs)."""
    nb = -(-N // block)
    sizes = np.minimum(block, N - np.arange(nb) * block).astype(np.int64)
    csum = np.concatenate([[0], np.cumsum(sizes[col_idx])])
    keys_per_row = csum[row_ptr[1:]] - csum[row_ptr[:-1]]
    return int((np.tile(sizes, BH) * keys_per_row).sum())


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


ESTIMATOR_SOURCES = ["block_sparse_attention_16_amd/csrc/estimate.hip"]


def load_estimator_traffic(workload: str):
    """Counted HBM bytes of one estimator call (its four kernels) from the
    committed rocprofv3 counter runs, if taken on the current estimator
    source; else None."""
    path = os.path.join(ROOT, "profiles", "estimator_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != source_hash(ESTIMATOR_SOURCES):
        return None
    return entry.get("hbm_bytes_per_call")


def load_traffic(kernel: str, workload: str, flop_per_launch: float):
    """HBM bytes per forward launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "fwd_kernel_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != source_hash(KERNEL_SOURCES):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(x, w, scale, top_p, budget_s: float, exec_flop_total: float):
    """Time the CPU oracle on a bounded, seeded sample of the workload.

    A third of the budget runs the oracle's estimator on whole heads (seeded
    order); the rest runs the oracle's forward on seeded rows of those heads,
    over the oracle's own masks.  The rate is the sampled rows' executed FLOP
    over their forward time plus their share of the estimator time.  The
    whole-workload time is extrapolated from the same sample: estimator time
    per head times the heads, plus forward time per executed FLOP times the
    workload's executed FLOP (taken from the GPU's mask)."""
    from oracle import bsa_oracle as O
    cores = blas_threads()
    rng = np.random.default_rng(12345)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    masks, t_est = [], 0.0
    t0 = time.perf_counter()
    for hi in rng.permutation(len(heads)):
        b, h = heads[int(hi)]
        ts = time.perf_counter()
        rp_h, ci_h, _ = O.estimate_mask(x["q"], x["k"], w.block, top_p, scale,
                                        keep_prefix_tokens=w.keep_prefix_tokens, heads=[(b, h)])
        t_est += time.perf_counter() - ts
        masks.append((b, h, rp_h, ci_h))
        if time.perf_counter() - t0 > budget_s / 3:
            break
    est_per_row = t_est / (len(masks) * w.nb)
    sizes = np.minimum(w.block, w.N - np.arange(w.nb) * w.block)
    pairs = [(m, i) for m in range(len(masks)) for i in range(w.nb)]
    flop, t_fwd, n = 0.0, 0.0, 0
    t1 = time.perf_counter()
    for pi in rng.permutation(len(pairs)):
        m, i = pairs[int(pi)]
        b, h, rp_h, ci_h = masks[m]
        sl = (slice(b, b + 1), slice(h, h + 1))
        ts = time.perf_counter()
        O.sparse_forward(x["q"][sl], x["k"][sl], x["v"][sl], w.block, rp_h, ci_h, scale, rows=[i])
        t_fwd += time.perf_counter() - ts
        flop += 4.0 * w.D * sizes[i] * sizes[ci_h[rp_h[i]:rp_h[i + 1]]].sum()
        n += 1
        if time.perf_counter() - t1 > budget_s * 2 / 3:
            break
    dt = t_fwd + n * est_per_row
    whole = t_est / len(masks) * len(heads) + t_fwd / max(flop, 1.0) * exec_flop_total
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 numpy oracle on {cpu_model()}: estimator on {len(masks)} of {len(heads)} heads "
                      f"({t_est:.1f} s), forward on {n} seeded rows of those heads over the oracle's masks "
                      f"({t_fwd:.1f} s); rate = their FLOP / (forward time + their share of the estimator time)",
            "cpu_model": cpu_model(),
            "whole_workload_s_extrapolated": round(whole, 1),
            "seconds": t_est + t_fwd, "rows": n}


def cpu_full(name: str, threads: int) -> int:
    """The whole oracle on one workload, on the host alone: the estimator on
    every head, then the forward (O, LSE, block mass) on every row of its own
    mask, and on the training workload the backward; every denoising step of a
    multi-step workload (later steps searching step 1's blocks).  Prints one
    JSON line with the seconds, the BLAS threads and the CPU model."""
    from workloads import get, make_inputs
    from oracle import bsa_oracle as O
    w = get(name)
    if threads > 0:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=threads)          # for the rest of this process
    scale = float(np.float32(1.0 / np.sqrt(w.D)))
    t_est = t_fwd = t_bwd = 0.0
    flop = 0.0
    cand = None
    for s in range(1, w.steps + 1):
        x = make_inputs(w, step=s, dtype="bf16", want_grad=w.backward)
        p = float(np.float32(w.top_p[s - 1]))
        ts = time.perf_counter()
        rp, ci, _ = O.estimate_mask(x["q"], x["k"], w.block, p, scale, candidate=cand,
                                    keep_prefix_tokens=w.keep_prefix_tokens)
        t_est += time.perf_counter() - ts
        print(json.dumps({"cpu_full": name, "step": s, "estimator_s": round(time.perf_counter() - ts, 2)}),
              flush=True)
        ts = time.perf_counter()
        for b in range(w.B):
            for h in range(w.H):
                r0 = (b * w.H + h) * w.nb
                srp = rp[r0:r0 + w.nb + 1] - rp[r0]
                sci = ci[rp[r0]:rp[r0 + w.nb]]
                sl = (slice(b, b + 1), slice(h, h + 1))
                O.sparse_forward(x["q"][sl], x["k"][sl], x["v"][sl], w.block, srp, sci, scale)
                if w.backward:
                    tb = time.perf_counter()
                    O.sparse_backward(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl], w.block, srp, sci, scale)
                    t_bwd += time.perf_counter() - tb
                print(json.dumps({"cpu_full": name, "step": s, "head": [b, h], "elapsed_s":
                                  round(time.perf_counter() - ts, 1)}), file=sys.stderr, flush=True)
        t_fwd += time.perf_counter() - ts
        flop += 4.0 * w.D * executed_pairs(w.N, w.block, w.B * w.H, rp, ci)
        if w.reduced_search and s == 1:
            cand = (rp, ci)
    t_fwd -= t_bwd
    print(json.dumps({"cpu_full": name, "kind": "oracle", "cores": threads if threads > 0 else blas_threads(),
                      "cpu_model": cpu_model(), "steps": w.steps, "estimator_s": round(t_est, 2),
                      "forward_s": round(t_fwd, 2), "backward_s": round(t_bwd, 2) if w.backward else None,
                      "total_s": round(t_est + t_fwd + t_bwd, 2), "executed_fwd_tflop": flop / 1e12,
                      "fwd_tflops": round(flop / max(t_fwd, 1e-9) / 1e12, 5)}), flush=True)
    return 0


def gsrs_loop(torch, bsa, dev, reps: int) -> dict:
    """The reduced-search loop of the GSRS page (Figure 4 caption: search steps
    restricted to the baseline mask, then reuse; Figure 7 caption: search
    overhead) over the Wan2.1-like workload's five denoising steps.

    Step 1 is a full search (estimator over every block) and a forward with
    exact block mass.  Steps 2-5 each narrow the previous step's mask by its
    block masses at the step's Top-p (bsa_select_from_mass) and run the forward
    with mass on the narrowed mask; the reduced-search estimator (scoring only
    step 1's blocks) is timed beside them at the same Top-p.  A final
    non-search step reuses step 5's mask for a forward alone.  Times are HIP
    events on the library's stream, the mean of ``reps`` passes over the loop
    (after one untimed pass)."""
    from workloads import get, make_inputs, bf16_bits
    w = get("wan")

    def up(arr):
        return torch.from_numpy(bf16_bits(arr).view(np.int16)).view(torch.bfloat16).to(dev)

    steps = []
    for s in range(1, w.steps + 1):
        x = make_inputs(w, step=s, dtype="bf16")
        steps.append(tuple(up(x[n]) for n in "qkv"))
        del x
    R, cap = w.B * w.H * w.nb, w.B * w.H * w.nb * w.nb
    shape = bsa.make_shape(w.B, w.H, w.N, w.D, w.block, 0)
    ws_e = torch.empty(bsa.bsa_workspace_size(shape, 0, 0), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(bsa.bsa_workspace_size(shape, 1, cap), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(bsa.bsa_workspace_size(shape, 3, 0), dtype=torch.uint8, device=dev)
    masks = [bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int32,
                                                                                     device=dev))
             for _ in range(w.steps)]
    red = bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int32, device=dev))
    masses = [torch.empty(cap, dtype=torch.float32, device=dev) for _ in range(w.steps)]
    o = torch.empty_like(steps[0][0])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ps = [float(np.float32(p)) for p in w.top_p]
    names = ["search"] + ["narrow"] * (w.steps - 1)
    acc = {k: np.zeros(w.steps) for k in ("search_ms", "fwd_ms", "reduced_ms")}
    reuse_ms = loop_ms = 0.0

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    for rep in range(reps + 1):
        marks = []
        t_loop0 = ev()
        for s in range(w.steps):
            q, k, v = steps[s]
            a = ev()
            if s == 0:
                bsa.bsa_estimate_mask(q, k, ps[0], w.block, out=masks[0], workspace=ws_e)
            else:
                bsa.bsa_select_from_mass(q, masks[s - 1], masses[s - 1], ps[s], w.block, out=masks[s],
                                         workspace=ws_s)
            b = ev()
            bsa.bsa_forward(q, k, v, masks[s], w.block, out=o, lse=lse, mass=masses[s], workspace=ws_f)
            c = ev()
            marks.append((a, b, c))
        q, k, v = steps[-1]
        r0 = ev()
        bsa.bsa_forward(q, k, v, masks[-1], w.block, want_mass=False, out=o, lse=lse, workspace=ws_f)
        r1 = ev()
        t_loop1 = ev()
        red_marks = []
        for s in range(1, w.steps):                      # reduced search beside the narrowing
            q, k, _ = steps[s]
            a = ev()
            bsa.bsa_estimate_mask(q, k, ps[s], w.block, candidate=masks[0], out=red, workspace=ws_e)
            red_marks.append((a, ev()))
        torch.cuda.synchronize()
        if rep == 0:
            continue
        for s, (a, b, c) in enumerate(marks):
            acc["search_ms"][s] += a.elapsed_time(b) / reps
            acc["fwd_ms"][s] += b.elapsed_time(c) / reps
        for s, (a, b) in enumerate(red_marks, start=1):
            acc["reduced_ms"][s] += a.elapsed_time(b) / reps
        reuse_ms += r0.elapsed_time(r1) / reps
        loop_ms += t_loop0.elapsed_time(t_loop1) / reps
    nnz = [int(m.row_ptr[-1].item()) for m in masks]
    full = acc["search_ms"][0]
    narrow = float(np.mean(acc["search_ms"][1:]))
    reduced = float(np.mean(acc["reduced_ms"][1:]))
    out = {"workload": f"{w.name}: {w.note}", "top_p": [round(p, 4) for p in ps],
           "steps": [{"step": s + 1, "search": names[s], "search_ms": round(acc["search_ms"][s], 4),
                      "fwd_mass_ms": round(acc["fwd_ms"][s], 4), "nnz": nnz[s],
                      "block_density": round(nnz[s] / (R * w.nb), 4)} for s in range(w.steps)],
           "reduced_search_ms": [round(t, 4) for t in acc["reduced_ms"][1:]],
           "reuse_step_fwd_ms": round(reuse_ms, 4),
           "loop_ms": round(loop_ms, 4),
           "search_overhead_ratio_full_vs_narrow": round(full / narrow, 2),
           "search_overhead_ratio_full_vs_reduced": round(full / reduced, 2),
           "search_share_of_loop": round((full + narrow * (w.steps - 1)) / loop_ms, 4)}
    del steps, masks, masses, red, ws_e, ws_f, ws_s, o, lse
    torch.cuda.empty_cache()
    return out


def density_sweep(torch, bsa, steps: int, warmup: int) -> int:
    """Forward latency against block density on seeded random masks (the
    density sweep of the GSRS page's Figure 5 shape; context, not the metric)."""
    B, H, N, D, bs = 1, 24, 115200, 128, 128
    nb = -(-N // bs)
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    q, k, v = (torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).to(dev) for _ in range(3))
    rng = np.random.default_rng(0)
    R = B * H * nb
    for dens in (0.05, 0.1, 0.2, 0.3, 0.5, 1.0):
        rows = []
        for r in range(R):
            i = r % nb
            kk = max(1, int(round(dens * nb)))
            if kk >= nb:
                sel = np.arange(nb)
            else:
                others = rng.choice(np.delete(np.arange(nb), i), size=kk - 1, replace=False)
                sel = np.sort(np.concatenate([[i], others]))           # the diagonal block is always kept
            rows.append(sel)
        counts = np.array([len(x) for x in rows])
        rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        ci = np.concatenate(rows).astype(np.int32)
        mask = bsa.csr_from_host(rp, ci, dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        ws = torch.empty(bsa.bsa_workspace_size(bsa.make_shape(B, H, N, D, bs, 0), 1, ci.size), dtype=torch.uint8,
                         device=dev)
        for _ in range(max(1, warmup)):
            bsa.bsa_forward(q, k, v, mask, bs, want_mass=False, out=o, lse=lse, workspace=ws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            bsa.bsa_forward(q, k, v, mask, bs, want_mass=False, out=o, lse=lse, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flop = 4.0 * D * executed_pairs(N, bs, B * H, rp.astype(np.int64), ci.astype(np.int64))
        print(json.dumps({"sweep": "block density", "density": dens, "nnz": int(ci.size), "fwd_ms": round(ms, 4),
                          "executed_tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                          "pct_bf16_peak": round(100 * flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
                          "shape": {"B": B, "H": H, "N": N, "D": D, "block": bs}}), flush=True)
        del mask, ws
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hunyuan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gsrs-loop", action="store_true",
                    help="skip the reduced-search loop over the Wan2.1-like workload's five steps")
    ap.add_argument("--cpu-full", metavar="WORKLOAD", default=None,
                    help="run only the whole CPU oracle on WORKLOAD (no GPU) and print its time")
    ap.add_argument("--cpu-threads", type=int, default=0, help="BLAS threads for --cpu-full (0: all)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--density-sweep", action="store_true",
                    help="instead of the step: forward latency and TFLOP/s over seeded random block masks of "
                         "density 5-100%% at B=1, H=24, N=115200, D=128, block 128 (one JSON line per density)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the timed region, run one plain device-to-device copy of BYTES bytes "
                         "(reference point for HBM byte counters under rocprofv3 --pmc)")
    a = ap.parse_args(argv)
    if a.cpu_full:
        return cpu_full(a.cpu_full, a.cpu_threads)
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus must be 1 (the path shards over "
                                   "heads with no exchange, and no multi-GPU run is implemented)"}))
        return 2

    import torch
    import block_sparse_attention_16_amd as bsa
    from workloads import get, make_inputs, bf16_bits

    if a.density_sweep:
        return density_sweep(torch, bsa, a.steps, a.warmup)

    w = get(a.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(w, dtype="bf16", want_grad=w.backward)

    def up(arr):
        return torch.from_numpy(bf16_bits(arr).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
    g = up(x["g"]) if w.backward else None
    top_p = float(np.float32(w.top_p[0]))
    scale = float(np.float32(1.0 / np.sqrt(w.D)))
    R = w.B * w.H * w.nb
    cap = R * w.nb
    mask = bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int32, device=dev))
    shape = bsa.make_shape(w.B, w.H, w.N, w.D, w.block, 0)
    ws_e = torch.empty(bsa.bsa_workspace_size(shape, 0, 0), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(bsa.bsa_workspace_size(shape, 1, cap), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    mass = torch.empty(cap, dtype=torch.float32, device=dev)
    if w.backward:
        ws_b = torch.empty(max(bsa.bsa_workspace_size(shape, 2, cap), 256), dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        # fp32 copy of O from the forward: delta for the backward without a recomputing pass
        o32 = torch.empty(q.shape, dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream()
    ev = []

    def step(record: bool):
        e0 = torch.cuda.Event(enable_timing=True) if record else None
        e1 = torch.cuda.Event(enable_timing=True) if record else None
        e2 = torch.cuda.Event(enable_timing=True) if record else None
        e3 = torch.cuda.Event(enable_timing=True) if record else None
        if record:
            e0.record(stream)
        bsa.bsa_estimate_mask(q, k, top_p, w.block, candidate=None, keep_prefix_tokens=w.keep_prefix_tokens,
                              out=mask, workspace=ws_e)
        if record:
            e1.record(stream)
        bsa.bsa_forward(q, k, v, mask, w.block, out=o, lse=lse, mass=mass, workspace=ws_f,
                        o32=o32 if w.backward else None)
        if record:
            e2.record(stream)
        if w.backward:
            bsa.bsa_backward(q, k, v, o, g, lse, mask, w.block, workspace=ws_b, dq=dq, dk=dk, dv=dv, o32=o32)
        if record:
            e3.record(stream)
            ev.append((e0, e1, e2, e3))

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(a.steps):
        step(True)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps
    # per-step event times; means feed the roofline (comparable with rocprofv3's
    # average duration), medians are reported beside them
    est_t = [e0.elapsed_time(e1) for e0, e1, _, _ in ev]
    fwd_t = [e1.elapsed_time(e2) for _, e1, e2, _ in ev]
    bwd_t = [e2.elapsed_time(e3) for _, _, e2, e3 in ev] if w.backward else None
    est_ms, fwd_ms = float(np.mean(est_t)), float(np.mean(fwd_t))
    bwd_ms = float(np.mean(bwd_t)) if w.backward else None

    if a.copy_calibration > 0:
        src = torch.empty(a.copy_calibration // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Mask narrowing from the forward's exact block mass (reduced search of a
    # later step): timed on its own, outside the step, at the next step's
    # threshold (the same one for single-step workloads).
    p_next = float(np.float32(w.top_p[1] if len(w.top_p) > 1 else w.top_p[0]))
    narrowed = bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int32,
                                                                                       device=dev))
    ws_s = torch.empty(bsa.bsa_workspace_size(shape, 3, 0), dtype=torch.uint8, device=dev)
    nsel = 10
    bsa.bsa_select_from_mass(q, mask, mass, p_next, w.block, w.keep_prefix_tokens, out=narrowed, workspace=ws_s)
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(nsel):
        bsa.bsa_select_from_mass(q, mask, mass, p_next, w.block, w.keep_prefix_tokens, out=narrowed, workspace=ws_s)
    s1.record(stream)
    torch.cuda.synchronize()
    sel_ms = s0.elapsed_time(s1) / nsel
    nnz_narrow = int(narrowed.row_ptr[-1].item())

    # Reduced search (multi-step workloads): later steps score only the blocks
    # step 1 kept; timed on its own at step 2's threshold.
    red = None
    if w.reduced_search and len(w.top_p) > 1:
        p2 = float(np.float32(w.top_p[1]))
        cand_out = bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev),
                           torch.empty(cap, dtype=torch.int32, device=dev))
        bsa.bsa_estimate_mask(q, k, p2, w.block, candidate=mask, keep_prefix_tokens=w.keep_prefix_tokens,
                              out=cand_out, workspace=ws_e)
        s0.record(stream)
        for _ in range(nsel):
            bsa.bsa_estimate_mask(q, k, p2, w.block, candidate=mask, keep_prefix_tokens=w.keep_prefix_tokens,
                                  out=cand_out, workspace=ws_e)
        s1.record(stream)
        torch.cuda.synchronize()
        red = {"ms": round(s0.elapsed_time(s1) / nsel, 4), "top_p": p2,
               "entries_out": int(cand_out.row_ptr[-1].item())}
        del cand_out

    # Hierarchical block scoring (block logits over 4 key sub-blocks), timed on
    # its own at the step's threshold.
    hier_g = 4
    ws_h = torch.empty(bsa.bsa_workspace_size(shape, 5, 0), dtype=torch.uint8, device=dev)
    hier_out = bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int32,
                                                                                       device=dev))
    bsa.bsa_estimate_mask(q, k, top_p, w.block, keep_prefix_tokens=w.keep_prefix_tokens, out=hier_out,
                          workspace=ws_h, sub_blocks=hier_g)
    s0.record(stream)
    for _ in range(nsel):
        bsa.bsa_estimate_mask(q, k, top_p, w.block, keep_prefix_tokens=w.keep_prefix_tokens, out=hier_out,
                              workspace=ws_h, sub_blocks=hier_g)
    s1.record(stream)
    torch.cuda.synchronize()
    hier = {"ms": round(s0.elapsed_time(s1) / nsel, 4), "sub_blocks": hier_g, "top_p": top_p,
            "entries_out": int(hier_out.row_ptr[-1].item())}
    del hier_out, ws_h

    # Token permutation (space-filling-curve order in for Q, K, V; the inverse
    # order out for O), timed on its own: an HBM-streaming gather/scatter.
    from workloads.hilbert import hilbert_order
    T_, Hg_, Wg_ = w.grid
    perm_h = np.concatenate([np.arange(w.text_prefix), w.text_prefix + np.asarray(hilbert_order((T_, Hg_, Wg_)))])
    perm_d = torch.from_numpy(perm_h.astype(np.int32)).to(dev)
    pq, pk, pv, po = (torch.empty_like(t) for t in (q, k, v, o))

    def permute_all():
        bsa.bsa_permute_tokens(q, perm_d, out=pq)
        bsa.bsa_permute_tokens(k, perm_d, out=pk)
        bsa.bsa_permute_tokens(v, perm_d, out=pv)
        bsa.bsa_permute_tokens(o, perm_d, inverse=True, out=po)

    permute_all()
    s0.record(stream)
    for _ in range(nsel):
        permute_all()
    s1.record(stream)
    torch.cuda.synchronize()
    perm_ms = s0.elapsed_time(s1) / nsel
    perm_bytes = 4 * 2.0 * q.numel() * q.element_size()
    del pq, pk, pv, po

    # Structured head mask (spatial heads over the video frames) generated on the GPU.
    kinds = torch.full((w.B * w.H,), 1, dtype=torch.int32, device=dev)
    smask = bsa.bsa_structured_mask(q, kinds, w.block, prefix_tokens=w.text_prefix, frame_tokens=Hg_ * Wg_)
    s0.record(stream)
    for _ in range(nsel):
        bsa.bsa_structured_mask(q, kinds, w.block, prefix_tokens=w.text_prefix, frame_tokens=Hg_ * Wg_, out=smask)
    s1.record(stream)
    torch.cuda.synchronize()
    struct_ms = s0.elapsed_time(s1) / nsel
    struct_nnz = int(smask.row_ptr[-1].item())
    del smask

    rp, ci = mask.to_host()
    nnz = int(rp[-1])
    pairs = executed_pairs(w.N, w.block, w.B * w.H, rp, ci)
    exec_flop = 4.0 * w.D * pairs
    dense_flop = w.dense_fwd_flop()
    step_flop = exec_flop * (3.5 if w.backward else 1.0)     # fwd + bwd (2.5x fwd) on the training step
    value = step_flop / (ms * 1e-3) / 1e12
    fwd_tflops = exec_flop / (fwd_ms * 1e-3) / 1e12
    est_bytes = 2.0 * w.B * w.H * w.N * w.D * 2 + 4.0 * (R + 1) + 4.0 * nnz
    traffic = load_traffic("fwd_kernel", w.name, exec_flop)
    est_counted = load_estimator_traffic(w.name)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "H": w.H, "N": w.N, "D": w.D, "block": w.block,
                   "top_p": w.top_p[0], "keep_prefix_tokens": w.keep_prefix_tokens,
                   "step": "estimate + forward(+mass)" + (" + backward" if w.backward else "")},
        "executed_tflop_per_step": exec_flop / 1e12,
        "dense_equiv_tflop_per_step": dense_flop / 1e12,
        "dense_equiv_tflops": round(dense_flop * (3.5 if w.backward else 1.0) / (ms * 1e-3) / 1e12, 3),
        "fwd_kernel": {"ms": round(fwd_ms, 4), "ms_median": round(float(np.median(fwd_t)), 4),
                       "executed_tflops": round(fwd_tflops, 3),
                       "dense_equiv_tflops": round(dense_flop / (fwd_ms * 1e-3) / 1e12, 3),
                       "pct_bf16_peak": round(100 * fwd_tflops / BF16_PEAK_TFLOPS, 2)},
        "estimator": {"ms": round(est_ms, 4), "ms_median": round(float(np.median(est_t)), 4),
                      "algorithmic_bytes": est_bytes,
                      "gbps": round(est_bytes / (est_ms * 1e-3) / 1e9, 1),
                      "pct_hbm_peak": round(100 * est_bytes / (est_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                      "counted_bytes": est_counted,
                      "counted_gbps": (round(est_counted / (est_ms * 1e-3) / 1e9, 1) if est_counted else None)},
        "block_density": nnz / (R * w.nb),
        "token_pair_density": pairs / (w.B * w.H * float(w.N) ** 2),
        "nnz": nnz,
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 3), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "fwd_kernel"},
    }
    sel_bytes = 4.0 * (R + 1) + 8.0 * nnz + 4.0 * (R + 1) + 4.0 * nnz_narrow
    out["select_from_mass"] = {"ms": round(sel_ms, 4), "top_p": p_next, "entries_in": nnz, "entries_out": nnz_narrow,
                               "algorithmic_bytes": sel_bytes,
                               "gbps": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1)}
    if red is not None:
        red_bytes = 2.0 * w.B * w.H * w.N * w.D * 2 + 8.0 * (R + 1) + 4.0 * nnz + 4.0 * red["entries_out"]
        red["gbps"] = round(red_bytes / (red["ms"] * 1e-3) / 1e9, 1)
        out["estimator_reduced_search"] = red
    hier_bytes = 2.0 * w.B * w.H * w.N * w.D * 2 + 4.0 * (R + 1) + 4.0 * hier["entries_out"]
    hier["gbps"] = round(hier_bytes / (hier["ms"] * 1e-3) / 1e9, 1)
    out["estimator_hierarchical"] = hier
    out["permute_tokens"] = {"ms": round(perm_ms, 4), "tensors": "gather q, k, v + scatter o",
                             "bytes": perm_bytes, "gbps": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1),
                             "pct_hbm_peak": round(100 * perm_bytes / (perm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
    out["structured_mask"] = {"ms": round(struct_ms, 4), "pattern": "spatial heads", "nnz": struct_nnz,
                              "block_density": struct_nnz / (R * w.nb)}
    if w.backward:
        out["bwd_ms"] = round(bwd_ms, 4)
        out["bwd_ms_median"] = round(float(np.median(bwd_t)), 4)
        out["bwd_executed_tflops"] = round(2.5 * exec_flop / (bwd_ms * 1e-3) / 1e12, 3)
    if not a.no_gsrs_loop:
        print("bench: reduced-search loop over the Wan2.1-like steps", file=sys.stderr, flush=True)
        out["gsrs_loop"] = gsrs_loop(torch, bsa, dev, reps=3)
    if not a.no_cpu_baseline:
        print("bench: CPU oracle sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(x, w, scale, top_p, a.cpu_budget, exec_flop)
        out["cpu_baseline"] = {k2: cb[k2] for k2 in ("value", "unit", "cores", "kind", "sample", "cpu_model",
                                                      "whole_workload_s_extrapolated")}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
