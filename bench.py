"""Throughput of block-sparse factorized attention, forward + backward, on one GPU.

A step is one pass of the whole path over one batch of synthetic input:
sa_fwd (O, lse) followed by sa_bwd (dQ, dK, dV), with inputs already resident
in HBM.  The layouts are built once before timing (they depend only on the
pattern, the length and the block size); their build time is reported.

Metric: effective TFLOP/s counted over allowed blocks -- every listed T x T
block counts 4*T*T*d flops forward and 2.5 times that backward, whether or
not all of its elements are allowed -- and its fraction of the MI355X dense
bf16 MFMA peak (2.5 PFLOP/s).

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd(+bwd) effective TFLOP/s over allowed blocks; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="img64",
                    help="tiny | img32 | text | img64 | audio (default img64, N=12288)")
    ap.add_argument("--dense", action="store_true", help="run the dense causal comparison layout")
    ap.add_argument("--residue-view", action="store_true",
                    help="run strided-B heads in their residue view (a dense causal attention per residue "
                         "class mod l); the metric then counts the residue view's blocks")
    ap.add_argument("--compact-view", action="store_true",
                    help="run fixed-B heads in their compact view (blocks of the summary keys only); the "
                         "metric then counts the compact view's blocks")
    ap.add_argument("--no-views-path", action="store_true",
                    help="skip the views path: by default, after the timed steps, the same step is also timed with "
                         "strided-B heads in the residue view and fixed-B heads in the compact view (reported as "
                         "views_path; its launches have other grid sizes than the timed ones, which is how a "
                         "kernel trace tells them apart)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch (exploration)")
    ap.add_argument("--heads", type=int, default=0, help="override the workload's head count (exploration)")
    ap.add_argument("--n", type=int, default=0, help="override the workload's sequence length (exploration)")
    ap.add_argument("--split", type=int, default=None,
                    help="chunking of long lists for this run (sa_set_split: 0 per call, -1 none, k > 0 forced)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads in the oracle sample (default: sized to ~10-30 s)")
    ap.add_argument("--length-scaling", action="store_true",
                    help="time fwd and fwd+bwd for n = 2^12 .. 2^20 with strided heads of stride l = sqrt(n) "
                         "(head A raster, head B in its residue view) and fit the exponent of n")
    ap.add_argument("--memory", action="store_true",
                    help="64 stacked layers of 4-head attention at n = 12288 through the autograd wrapper: "
                         "memory kept for the backward pass against dense n x n weights")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (to scale HBM counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size, profiled with the same counters as the
    kernels so that FETCH_SIZE / WRITE_SIZE can be scaled to bytes."""
    import torch
    nbytes = 512 << 20
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}), flush=True)


def traffic_from_profile(kernel_file, kernel, workload):
    """HBM bytes per launch measured by the counter runs under profiles/, if
    they were taken on the current source of the kernel's file (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "block_sparse_factorized_amd", "csrc", kernel_file)
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for e in json.load(open(path)).get("entries", []):
        if e["kernel"] == kernel and e["workload"] == workload and e["source_sha256"] == sha:
            return e["hbm_bytes_per_launch"]
    return None


def counters_from_profile(kernel_file, kernel, workload):
    """MFMA busy of a kernel from the rocprofv3 counter runs under profiles/
    (counters.json), if they were taken on the current source of the
    kernel's file (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters.json")
    src = os.path.join(ROOT, "block_sparse_factorized_amd", "csrc", kernel_file)
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for e in json.load(open(path)).get("entries", []):
        if e["kernel"] == kernel and e["workload"] == workload and e["source_sha256"] == sha:
            return e
    return None


def measured_peaks():
    """The machine's own denominators (libsa_peaks.so, include/sa_peaks.h):
    the sustained bf16 MFMA rate of a kernel that does nothing else, and the
    device-to-device copy bandwidth (bytes read + written per second)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_sparse_factorized_amd", "_lib", "libsa_peaks.so")
    lib = ctypes.CDLL(path)
    lib.sap_mfma_bf16_tflops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sap_mfma_bf16_tflops.restype = ctypes.c_double
    lib.sap_copy_gbs.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.sap_copy_gbs.restype = ctypes.c_double
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mfma = lib.sap_mfma_bf16_tflops(cus * 8, 2048, stream)
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    copy = lib.sap_copy_gbs(b.data_ptr(), a.data_ptr(), nbytes, 10, stream)
    del a, b
    return {"mfma_bf16_tflops": mfma if mfma > 0 else None, "hbm_copy_gbs": copy if copy > 0 else None,
            "how": "bf16 32x32x16 MFMA loop (8 chains per wave), %d workgroups x 4 waves; 1 GiB device copy x 10" % (cus * 8)}


def residue_blocks(lay):
    """(blocks per residue class, residue classes) of a residue view: a dense
    causal attention over n/l rows in blocks of 64."""
    nb = -(-(lay.n // lay.l) // 64)
    return nb, lay.l


def listed_blocks(lay):
    """Blocks the kernels walk for one head: the layout's listing, the
    residue view's dense causal blocks over every residue class, or the
    compact view's blocks."""
    v = lay.view_info()
    return v["nnz"] * (lay.l if v["kind"] == "residue" else 1)


def compact_live_quadrants(lay):
    """Live 32 x 32 quadrants of a fixed-B compact view: query row i sees the
    first cnt(i) summary keys, so quadrant (query half rh, key half ch) of
    block (qb, kb) is live when some row of half rh has cnt > 64 kb + 32 ch."""
    import numpy as np
    n, l, c = lay.n, lay.l, lay.c
    i = np.arange(n, dtype=np.int64)
    cnt = (i + 1) // l * c + np.maximum(0, (i + 1) % l - (l - c))
    half_max = cnt.reshape(-1, 32).max(1)  # widest row of every 32-row half
    nkb = -(-(n // l * c) // 64)
    kb = np.arange(nkb, dtype=np.int64)
    live = half_max[:, None, None] > (64 * kb[None, :, None] + 32 * np.arange(2)[None, None, :])
    return int(live.sum())


def counted_flops(layouts, batch, T, d):
    """Forward flops counted over the listed blocks, summed over (batch, head)."""
    blocks = sum(listed_blocks(lay) for lay in layouts) * batch
    return blocks * 4.0 * T * T * d, blocks


def live_quadrants(layouts, batch, T):
    """32 x 32 quadrants of the listed blocks that hold an allowed element,
    summed over (batch, head).  The block-64 kernels skip the others, so
    their matrix cores execute this many quadrants' products; the counted
    metric charges four quadrants for every listed block."""
    import numpy as np
    total = 0
    for lay in layouts:
        if getattr(lay, "residue_view", False):
            nb, nr = residue_blocks(lay)  # dense causal: 3 live quadrants on the diagonal
            total += nr * (3 * nb + 4 * (nb * (nb - 1) // 2))
            continue
        if getattr(lay, "compact_view", False):
            total += compact_live_quadrants(lay)
            continue
        ex = lay.export()
        mid = np.asarray(ex["mask_id"])
        if T != 64:  # only block-64 kernels skip quadrants
            total += 4 * len(mid)
            continue
        words = np.asarray(ex["mask_words"]).reshape(-1, 64)  # row r of a mask = word r
        if len(words):
            lo = (words & np.uint64(0xFFFFFFFF)) != 0
            hi = (words >> np.uint64(32)) != 0
            per_mask = (lo[:, :32].any(1).astype(np.int64) + hi[:, :32].any(1) + lo[:, 32:].any(1)
                        + hi[:, 32:].any(1))
            total += int(np.where(mid < 0, 4, per_mask[np.maximum(mid, 0)]).sum())
        else:
            total += 4 * len(mid)
    return total * batch


def _block_rel_l2(g, r):
    """Largest relative L2 error over 64-row blocks, each against the larger
    of its own norm and a tenth of the RMS block norm."""
    import numpy as np
    nb = max(1, -(-g.shape[0] // 64))
    floor = 0.1 * np.linalg.norm(r) / np.sqrt(nb)
    worst = 0.0
    for a in range(0, g.shape[0], 64):
        den = max(np.linalg.norm(r[a:a + 64]), floor, 1e-30)
        worst = max(worst, float(np.linalg.norm(g[a:a + 64] - r[a:a + 64]) / den))
    return worst


def cpu_baseline(w, x, pats, lays, T, max_heads, outputs=None, runs=3):
    """The fp64 oracle on the host's cores over a bounded sample of heads of
    the same workload, fwd + bwd, scaled to the same counted-flop metric
    (blocks counted as for the GPU run); the median of `runs` timed passes.
    The first pass's results are also compared with the GPU outputs of the
    timed steps (`outputs`: host copies of o, lse and, with the backward,
    dq, dk, dv), which gives the run's own parity figures."""
    import numpy as np
    import oracle
    from workloads import to_f64

    sample = []
    for b in range(w.batch):
        for h in range(w.heads):
            sample.append((b, h))
    # interleave A and B heads so any prefix is representative
    sample.sort(key=lambda bh: (bh[1] // 2, bh[0], bh[1] % 2))
    sample = sample[:max_heads]
    counted = 0.0
    elements = 0
    args = {bh: [to_f64(x[t][bh[0], bh[1]]) for t in (("q", "k", "v", "do") if w.backward else ("q", "k", "v"))]
            for bh in sample}
    for (b, h) in sample:
        counted += listed_blocks(lays[h]) * 4.0 * T * T * w.d * (3.5 if w.backward else 1.0)
    times = []
    err = {"o_max_abs": 0.0, "o_rel_l2": 0.0, "lse_max_abs": 0.0, "empty_rows_exact": True}
    if w.backward:
        err.update({"dq_rel_l2": 0.0, "dk_rel_l2": 0.0, "dv_rel_l2": 0.0, "grad_block_rel_l2": 0.0})
    for run in range(runs):
        t0 = time.perf_counter()
        results = {}
        for (b, h) in sample:
            p, l, c = pats[h]
            if w.backward:
                results[(b, h)] = oracle.head_bwd(p, l, c, *args[(b, h)], 1.0)
            else:
                results[(b, h)] = (None, None, None) + tuple(oracle.head_fwd(p, l, c, *args[(b, h)], 1.0))
        times.append(time.perf_counter() - t0)
        if run > 0 or outputs is None:
            continue
        rel = lambda g, r: float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
        for (b, h), (rdq, rdk, rdv, ro, rlse) in results.items():
            go = to_f64(outputs["o"][b, h])
            glse = outputs["lse"][b, h].double().numpy()
            fin = np.isfinite(rlse)
            err["o_max_abs"] = max(err["o_max_abs"], float(np.abs(go - ro).max()))
            err["o_rel_l2"] = max(err["o_rel_l2"], rel(go, ro))
            if fin.any():
                err["lse_max_abs"] = max(err["lse_max_abs"], float(np.abs(glse[fin] - rlse[fin]).max()))
            err["empty_rows_exact"] = bool(err["empty_rows_exact"] and np.array_equal(np.isfinite(glse), fin)
                                           and np.all(go[~fin] == 0.0))
            if w.backward:
                for nm, r in (("dq", rdq), ("dk", rdk), ("dv", rdv)):
                    g = to_f64(outputs[nm][b, h])
                    err[nm + "_rel_l2"] = max(err[nm + "_rel_l2"], rel(g, r))
                    err["grad_block_rel_l2"] = max(err["grad_block_rel_l2"], _block_rel_l2(g, r))
    secs = float(np.median(times))
    for (b, h) in sample:
        p, l, c = pats[h]
        elements += int(oracle.row_counts(p, w.n, l, c).sum())
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    parity = None
    if outputs is not None:
        # the acceptance bars: O max-abs 2e-2 (bf16) or 1e-4 (fp32), gradients 5e-2 relative L2
        o_bar = 2e-2 if w.dtype == "bf16" else 1e-4
        ok = err["o_max_abs"] <= o_bar and err["empty_rows_exact"]
        if w.backward:
            ok = ok and max(err["dq_rel_l2"], err["dk_rel_l2"], err["dv_rel_l2"]) <= 5e-2
        parity = dict(err, heads=len(sample), o_max_abs_bar=o_bar, grad_rel_l2_bar=5e-2 if w.backward else None,
                      passed=bool(ok), against="the fp64 oracle on the timed steps' outputs, whole heads")
    return {
        "value": counted / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d of %d heads of %s (b,h in A/B pairs), fwd%s in fp64, median of %d passes of %.1f s"
                  % (len(sample), w.batch * w.heads, w.name, "+bwd" if w.backward else "", runs, secs),
        "seconds": secs,
        "seconds_each": times,
        "cpu_model": cpu_model,
        # the oracle's own work: 4 d flops per allowed element forward, 10 d backward
        "allowed_element_gflops": elements * w.d * (14.0 if w.backward else 4.0) / secs / 1e9,
        "parity": parity,
    }


def views_step(w, pats, x, steps, warmup):
    """The same step with every strided-B head in its residue view and every
    fixed-B head (c a power of two) in its compact view -- the same allowed
    pairs, walked as dense blocks -- on its own output buffers: step time
    and the pattern's useful-pair rate.  None when no head has a view."""
    import torch
    import block_sparse_factorized_amd as sa
    if not w.backward or w.block != 64:  # the views are walked by the block-64 kernels only
        return None
    dev = torch.device("cuda:0")
    lays, cache, any_view = [], {}, False
    for (p, l, c) in pats:
        if (p, l, c) not in cache:
            lay = sa.sa_layout_build(p, w.n, l, c, block=w.block)
            if p == "strided_b" and w.n % l == 0:
                lay.set_residue_view(True)
                any_view = True
            elif p == "fixed_b" and w.n % l == 0 and (c & (c - 1)) == 0:
                lay.set_compact_view(True)
                any_view = True
            cache[(p, l, c)] = lay
        lays.append(cache[(p, l, c)])
    if not any_view:
        return None
    q, k, v, do = (x[t].to(dev) for t in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(max(sa.sa_bwd_workspace_size(w.batch, w.heads, w.n, w.d), 16), dtype=torch.uint8, device=dev)

    def step():
        sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse)
        sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    allowed = sum(lay.info()["allowed"] for lay in lays) * w.batch
    return {"ms_per_step": ms, "useful_pair_tflops": allowed * w.d * 14.0 / (ms * 1e-3) / 1e12,
            "views": sorted(set(lay.view_info()["kind"] for lay in lays) - {"layout"}),
            "what": "the same step with strided-B heads in the residue view and fixed-B heads in the compact "
                    "view (same allowed pairs, fewer and denser blocks); not the metric, which counts the "
                    "layouts' blocks"}


def length_scaling(args):
    """Step time against sequence length for the strided pattern with
    l = sqrt(n): the pages' O(n sqrt n) cost (batch 1, one head of each of
    strided A and B, d = 64, bf16, scale 1).  One JSON line."""
    import numpy as np
    import torch
    import block_sparse_factorized_amd as sa
    import workloads

    dev = torch.device("cuda:0")
    points = []
    for k in (12, 14, 16, 18, 20):
        n, l, d = 1 << k, 1 << (k // 2), 64
        a = sa.sa_layout_build("strided_a", n, l, block=64)
        b = sa.sa_layout_build("strided_b", n, l, block=64).set_residue_view(True)
        lays = [a, b]
        x = workloads.custom_inputs((1, 2, n, d), torch.bfloat16, seed=k)
        q, kk, v, do = (x[t].to(dev) for t in ("q", "k", "v", "do"))
        del x
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(sa.sa_bwd_workspace_size(1, 2, n, d), dtype=torch.uint8, device=dev)
        reps = max(3, min(args.steps, 20))

        def timed(fn):
            for _ in range(2):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(reps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / reps

        fwd_ms = timed(lambda: sa.sa_fwd(q, kk, v, lays, 1.0, o=o, lse=lse))
        step_ms = timed(lambda: (sa.sa_fwd(q, kk, v, lays, 1.0, o=o, lse=lse),
                                 sa.sa_bwd(q, kk, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv, workspace=ws)))
        pairs = a.info()["allowed"] + b.info()["allowed"]
        points.append({"n": n, "l": l, "allowed_pairs": pairs, "fwd_ms": fwd_ms, "fwd_bwd_ms": step_ms,
                       "blocks_walked": listed_blocks(a) + listed_blocks(b)})
        print("n = %d: fwd %.3f ms, fwd+bwd %.3f ms" % (n, fwd_ms, step_ms), file=sys.stderr, flush=True)
        del q, kk, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    # Exponent of n between consecutive lengths (the small ones do not fill
    # the GPU, so the exponent approaches the pages' 1.5 only at large n).
    local = []
    for p1, p2 in zip(points, points[1:]):
        e = lambda key: float(np.log(p2[key] / p1[key]) / np.log(p2["n"] / p1["n"]))
        local.append({"n_from": p1["n"], "n_to": p2["n"], "pairs": e("allowed_pairs"), "fwd": e("fwd_ms"),
                      "fwd_bwd": e("fwd_bwd_ms")})
    print(json.dumps({
        "metric": "step time vs sequence length, strided heads with l = sqrt(n)",
        "unit": "ms", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "length-scaling", "batch": 1, "heads": 2, "head_dim": 64, "block": 64,
                   "pattern": "strided A (raster) + strided B (residue view), l = sqrt(n)"},
        "points": points,
        "local_exponents": local,
    }), flush=True)


def memory_run(args):
    """Memory kept for the backward pass by 64 stacked self-attention layers
    (the pages' 154 GB example: 64 layers, 4 heads, n = 12288, stored
    attention weights in fp32 would take 64 * 4 * 12288^2 * 4 bytes), run
    through sparse_attention, which keeps only O and lse per layer.  One
    JSON line."""
    import torch
    import block_sparse_factorized_amd as sa
    import workloads

    dev = torch.device("cuda:0")
    layers, B, H, n, d, l = 64, 1, 4, 12288, 64, 128
    pats = [("strided_a", l, 1), ("strided_b", l, 1)] * (H // 2)
    lay_a, lay_b = sa.sa_layout_build("strided_a", n, l, block=64), sa.sa_layout_build("strided_b", n, l, block=64)
    lays = [lay_a, lay_b] * (H // 2)
    x0 = workloads.custom_inputs((B, H, n, d), torch.bfloat16, seed=64, with_dout=False)["q"].to(dev)
    x0.requires_grad_(True)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    t0 = time.perf_counter()
    x = x0
    for _ in range(layers):
        x = sa.sparse_attention(x, x, x, lays, 1.0)  # self-attention, no projections
    torch.cuda.synchronize()
    t_fwd = time.perf_counter() - t0
    kept = torch.cuda.memory_allocated(dev) - base
    t0 = time.perf_counter()
    x.backward(torch.ones_like(x))
    torch.cuda.synchronize()
    t_bwd = time.perf_counter() - t0
    peak = torch.cuda.max_memory_allocated(dev) - base
    act = B * H * n * d * 2              # one layer's output (bf16)
    lse = B * H * n * 4                  # its log-sum-exp (fp32)
    dense = B * H * n * n * 4            # its attention weights, fp32
    print(json.dumps({
        "metric": "memory kept for the backward pass, 64 layers of 4-head attention at n = 12288",
        "unit": "bytes", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "memory-64-layers", "layers": layers, "batch": B, "heads": H, "n": n,
                   "head_dim": d, "patterns": "strided A/B, l = 128", "block": 64},
        "kept_bytes": kept, "kept_bytes_per_layer": kept / layers,
        "expected_per_layer_output_plus_lse": act + lse,
        "peak_bytes_fwd_bwd": peak,
        "dense_weights_bytes_per_layer": dense, "dense_weights_bytes_total": dense * layers,
        "dense_over_kept": dense * layers / kept if kept else None,
        "fwd_s": t_fwd, "bwd_s": t_bwd,
    }), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.length_scaling:
        length_scaling(args)
        return
    if args.memory:
        memory_run(args)
        return

    import numpy as np
    import torch
    import block_sparse_factorized_amd as sa
    import workloads

    w = workloads.WORKLOADS[args.workload]
    shape_tag = ""
    if args.batch or args.heads or args.n:
        import dataclasses
        w = dataclasses.replace(w, batch=args.batch or w.batch, heads=args.heads or w.heads, n=args.n or w.n)
        shape_tag = "-b%dh%dn%d" % (w.batch, w.heads, w.n)
    if args.split is not None:
        sa.sa_set_split(args.split)
        shape_tag += "-split%d" % args.split
    dev = torch.device("cuda:0")
    pats = w.head_patterns(dense=args.dense)
    T, d = w.block, w.d

    t0 = time.perf_counter()
    cache = {}
    lays = []
    for (p, l, c) in pats:
        if (p, l, c) not in cache:
            cache[(p, l, c)] = sa.sa_layout_build(p, w.n, l, c, block=T)
            if args.residue_view and p == "strided_b":
                cache[(p, l, c)].set_residue_view(True)
            if args.compact_view and p == "fixed_b":
                cache[(p, l, c)].set_compact_view(True)
        lays.append(cache[(p, l, c)])
    layout_ms = (time.perf_counter() - t0) * 1e3

    label = (w.name + shape_tag + ("-dense" if args.dense else "") + ("-residue-view" if args.residue_view else "")
             + ("-compact-view" if args.compact_view else ""))
    views = args.residue_view or args.compact_view
    x = workloads.make_inputs(w)
    q, k, v, do = (x[t].to(dev) for t in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(max(sa.sa_bwd_workspace_size(w.batch, w.heads, w.n, d), 16), dtype=torch.uint8, device=dev)
    scale = 1.0

    # One step = forward + the two backward stages (the same kernels sa_bwd
    # launches: dQ with the row terms, then dK/dV), each bracketed by events
    # on torch's current stream -- the stream every launch goes to -- so every
    # kernel is timed live.
    names = ["fwd", "bwd_dq", "bwd_dkdv"] if w.backward else ["fwd"]

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        sa.sa_fwd(q, k, v, lays, scale, o=o, lse=lse)
        rec(1)
        if w.backward:
            sa.sa_bwd_dq_rowterms(q, k, v, o, lse, do, lays, scale, workspace=ws, dq=dq)
            rec(2)
            sa.sa_bwd_dkdv(q, k, v, do, lays, scale, ws, dk=dk, dv=dv)
            rec(3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = {nm: np.array([e[i].elapsed_time(e[i + 1]) for e in events]) for i, nm in enumerate(names)}

    fwd_flops, blocks = counted_flops(lays, w.batch, T, d)
    bwd_flops = 2.5 * fwd_flops if w.backward else 0.0
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # Counted (algorithmic) flops per launch, per listed block: forward 4*T*T*d;
    # backward 10*T*T*d split as dK/dV 8*T*T*d (S, dP, dV, dK) and dQ 2*T*T*d
    # (dQ itself; the S and dP it recomputes are not counted twice).
    per_block = {"fwd": 4.0, "bwd_dkdv": 8.0, "bwd_dq": 2.0}
    # Matrix-core flops the kernels execute, per live 32 x 32 quadrant
    # (forward S, PV; dK/dV S, dP, dV, dK; dQ S, dP, dQ).
    # The fp32 block-16 kernel skips nothing: it executes what is counted.
    quads = live_quadrants(lays, w.batch, T)
    per_quad = {"fwd": 4.0, "bwd_dkdv": 8.0, "bwd_dq": 6.0}
    kernels = {}
    for nm in names:
        avg_s = float(kernel_ms[nm].mean()) * 1e-3
        nb, nq = blocks, quads
        fl = per_block[nm] * T * T * d * nb
        ex = per_quad[nm] * 32 * 32 * d * nq if T == 64 else fl
        kernels[nm] = {"avg_us": avg_s * 1e6, "median_us": float(np.median(kernel_ms[nm])) * 1e3,
                       "p10_us": float(np.percentile(kernel_ms[nm], 10)) * 1e3,
                       "p90_us": float(np.percentile(kernel_ms[nm], 90)) * 1e3,
                       "counted_gflop": fl / 1e9, "tflops": fl / avg_s / 1e12 if fl else None,
                       "executed_gflop": ex / 1e9, "executed_tflops": ex / avg_s / 1e12 if ex else None}
    dominant = max(names, key=lambda nm: kernels[nm]["avg_us"])
    kern_sym = {
        "fwd": "fwd_bf16_t64_kernel<%d>" % d if w.dtype == "bf16" else "fwd_f32_t16_d64_kernel",
        "bwd_dkdv": "bwd_dkdv_kernel<%d>" % d,
        # (the library launches the dQ kernel's one-element form when a walked
        # layout has quadrants with at most one allowed element per lane:
        # strided B walked raster, fixed B with one summary column)
        "bwd_dq": "bwd_dq_kernel<%d, true, %s>" % (d, "true" if any(
            (p == "strided_b" and not args.residue_view) or (p == "fixed_b" and c == 1)
            for (p, l, c) in pats) else "false"),
    }
    dk_ = kernels[dominant]
    kern_file = "fwd.hip" if dominant == "fwd" else "bwd.hip"
    # The fastest walk of the same pairs, when the layouts have views (after
    # the timed steps, on its own buffers).
    fastest = views_step(w, pats, x, max(5, args.steps // 2), 3) if not args.no_views_path and not views else None
    # The machine's own denominators, measured after the timed steps.
    mp = measured_peaks() if w.dtype == "bf16" else None
    mpeak = mp["mfma_bf16_tflops"] if mp else None
    # Allowed (query, key) pairs over the elements of the walked blocks.
    allowed = sum(lay.info()["allowed"] for lay in lays) * w.batch
    traffic = traffic_from_profile(kern_file, kern_sym[dominant], label)
    ctr = counters_from_profile(kern_file, kern_sym[dominant], label)
    roofline = {
        "kernel": kern_sym[dominant],
        "bound": "mfma",
        "achieved": dk_["tflops"],
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": dk_["tflops"] / peak,
        "traffic": traffic,
        # the counters' HBM bytes over this run's launch time
        "achieved_hbm_gbs": traffic / (dk_["avg_us"] * 1e-6) / 1e9 if traffic else None,
        "counted_flops_per_launch": dk_["counted_gflop"] * 1e9,
        "avg_launch_us": dk_["avg_us"],
        # What the matrix cores actually execute (empty quadrants skipped).
        "executed_mfma_tflops": dk_["executed_tflops"],
        "executed_frac": dk_["executed_tflops"] / peak,
        # rocprofv3 counters of the same kernel and workload (profiles/mfma_busy.md):
        # SQ_VALU_MFMA_BUSY_CYCLES over the XCD's GPU-busy cycles times 1024 SIMDs,
        # and over the traced duration at 2.4 GHz; null once the source changed
        "mfma_busy": ctr["mfma_busy_grbm"] if ctr else None,
        "mfma_busy_at_2400mhz": ctr["mfma_busy_at_2400mhz"] if ctr else None,
        "frac_of_measured_peak": dk_["tflops"] / mpeak if mpeak else None,
    }
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": label,
            "batch": w.batch, "heads": w.heads, "n": w.n, "head_dim": d, "block": T,
            "pattern": "dense causal" if args.dense else w.pattern, "l": w.l, "c": w.c,
            "scale": scale, "allowed_blocks": blocks, "backward": w.backward,
            "residue_view": bool(args.residue_view),
            "compact_view": bool(args.compact_view),
        },
        "frac_of_peak": value / peak,
        "measured_peaks": mp,
        "frac_of_measured_peak": value / mpeak if mpeak else None,
        "useful_element_fraction": allowed / (blocks * T * T) if blocks else None,
        # the pattern's own work: 4 d flops per allowed (query, key) pair
        # forward and 10 d backward, over the step time
        "useful_pair_tflops": allowed * w.d * (14.0 if w.backward else 4.0) / (ms_per_step * 1e-3) / 1e12,
        # With a residue or compact view, the raster layouts' block count over
        # the same step time (a reference only: the views walk fewer blocks).
        "raster_counted_tflops": (sum(lay.info()["nnz"] for lay in lays) * w.batch * 4.0 * T * T * d
                                  * (3.5 if w.backward else 1.0) / (ms_per_step * 1e-3) / 1e12)
        if views else None,
        "live_quadrant_fraction": quads / (4.0 * blocks) if blocks else None,
        "kernels": kernels,
        "fwd_frac_of_peak": kernels["fwd"]["tflops"] / peak,
        "fwd_frac_of_measured_peak": kernels["fwd"]["tflops"] / mpeak if mpeak else None,
        "layout_build_ms": layout_ms,
        "roofline": roofline,
        "views_path": dict(fastest, speedup_vs_layouts=ms_per_step / fastest["ms_per_step"]) if fastest else None,
        "cpu_baseline": None,
        "parity": None,
    }
    if not args.no_cpu_baseline:
        heads = args.cpu_heads or {"tiny": 2, "img32": 16, "text": 16, "img64": 32, "audio": 2}[w.name]
        outs = {"o": o.cpu(), "lse": lse.cpu()}
        if w.backward:
            outs.update(dq=dq.cpu(), dk=dk.cpu(), dv=dv.cpu())
        out["cpu_baseline"] = cpu_baseline(w, x, pats, lays, T, heads, outputs=outs)
        # the same run's correctness figures, next to the rate they qualify
        out["parity"] = out["cpu_baseline"].pop("parity")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
