"""Benchmark of the exact-attention forward on one MI355X.

A step is one fa2_fwd call over one batch of the long-sequence workload
B=1, H=32, N_q=N_k=16384, d=128 (bf16, non-causal, scale 1/sqrt(d)), inputs
resident in HBM.  Throughput counts 4*B*H*N_q*N_k*d FLOP per step (halved for
causal).  The same run also times the other named workloads (the causal
variants, the d=64 and d=128 training shapes, sliding window, backward, the
FP8 forward and the split-KV decode) and the fp64 oracle on a bounded sample of
the headline workload, and prints ONE JSON line.  With --fp8 the timed step is
the FP8 forward of the same workload (for its own profile).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu] [--calib-copy] [--fp8]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 256 * 4 * 1024 * 2.4e9 / 1e12   # 2516.6: 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS              # 5033.2: the 8-bit matrix rate is twice the bf16 rate
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s (bf16, causal/non-causal) and % of MI355X MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "exact_attention_85_amd", "csrc", "fa2_fwd.hip")
FP8_SRC = os.path.join(ROOT, "exact_attention_85_amd", "csrc", "fa2_fp8.hip")
BWD_SRC = os.path.join(ROOT, "exact_attention_85_amd", "csrc", "fa2_bwd.hip")
METRIC_FP8 = "attention fwd TFLOP/s (fp8 e4m3 inputs, per-head scaling) and % of MI355X fp8 MFMA peak"
METRIC_BWD = "attention bwd TFLOP/s (bf16, FLOPs counted as 2.5x the forward's) and % of MI355X MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TUNE_TABLE = os.path.join(ROOT, "exact_attention_85_amd", "csrc", "fa2_tune_table.h")


def kernel_source_sha(*paths) -> str:
    """sha256[:16] of the concatenated sources (fa2_fwd.hip alone by default)."""
    h = hashlib.sha256()
    for path in paths or (KERNEL_SRC,):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def env_info() -> dict:
    """Where the line was measured: the device, the runtime versions, and the kernel
    sources it ran (sha256[:16], the key the committed counter summaries carry)."""
    props = torch.cuda.get_device_properties(0)
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__,
            "kernel_sources": {os.path.basename(p): kernel_source_sha(p)
                               for p in (KERNEL_SRC, TUNE_TABLE, BWD_SRC, FP8_SRC)}}


def measured_traffic(key: str, src=(KERNEL_SRC,)):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on different sources (the kernel file, and for the bf16
    forward also the table that picks its configuration)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(key)
    if not e or e.get("kernel_source_sha") != kernel_source_sha(*src):
        return None
    return e.get("hbm_bytes_per_launch")


def time_launches(fn, steps: int, warmup: int):
    """Average milliseconds per call of fn over `steps` calls on torch's current
    stream, timed with events recorded on that stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def cpu_baseline(w, causal: bool, q, k, v, o, lse):
    """The fp64 oracle on a bounded sample of query rows of the workload, spread
    over all heads (about 15 s of host work), in TFLOP/s with the same FLOP count
    per row as the GPU figure.  The same oracle rows are compared with the timed
    run's O and LSE: returns (baseline, parity)."""
    import oracle

    bits = [workloads.bf16_bits(t) for t in (q, k, v)]  # whole tensors on the host
    flop_row = 4.0 * w.n_k * w.d / (2 if causal else 1)  # the metric's per-row count
    rng = np.random.default_rng(7)
    total_rows = w.B * w.H * w.n_q

    def run(n_rows):
        rows = np.sort(rng.choice(total_rows, size=n_rows, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attention_rows_bf16(*bits, rows, causal, w.scale)
        return time.perf_counter() - t0, rows, o_ref, l_ref

    # grow the sample until one run takes about 10-30 s (a small sample over-states the cost
    # per row: each thread converts the K/V heads its rows touch)
    n_rows = min(total_rows, 2048)
    dt, rows, o_ref, l_ref = run(n_rows)
    while dt < 10.0 and n_rows < total_rows:
        n_rows = int(min(total_rows, n_rows * min(8.0, 15.0 / max(dt, 1e-3))))
        dt, rows, o_ref, l_ref = run(n_rows)
    baseline = {"value": n_rows * flop_row / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": f"{n_rows} random query rows (all heads) of {w.name}, "
                          f"{'causal' if causal else 'non-causal'}, fp64 two-pass softmax, {dt:.1f} s"}
    # the timed run's outputs at those rows (flat row = (b*H + h)*N_q + i)
    idx = torch.from_numpy(rows).to(o.device)
    o_g = o.reshape(-1, w.d)[idx].float().cpu().double().numpy()
    l_g = lse.reshape(-1)[idx].cpu().double().numpy()
    d_o, d_l = np.abs(o_g - o_ref), np.abs(l_g - l_ref)
    ok = bool(np.all(np.isfinite(o_g)) and np.all(np.isfinite(l_g)) and d_o.max() <= 1e-2 and d_l.max() <= 1e-3)
    parity = {"rows": int(n_rows), "of_rows": int(total_rows), "max_abs_O": float(d_o.max()),
              "max_abs_LSE": float(d_l.max()), "tol_O": 1e-2, "tol_LSE": 1e-3, "pass": ok,
              "checked": "the timed run's O and LSE at the oracle rows of cpu_baseline"}
    return baseline, parity


def blockmask_causal_pairs(mask, n_q: int, n_k: int, block_q: int = 128, block_k: int = 64) -> int:
    """Visible (query, key) pairs of one head under a block mask and the causal band (key j <= i)."""
    i = np.arange(n_q)
    total = 0
    for qb, kb in zip(*np.nonzero(mask)):
        rows = i[qb * block_q:(qb + 1) * block_q]
        k0, k1 = kb * block_k, min(n_k, (kb + 1) * block_k)
        total += int(np.clip(np.minimum(rows + 1, k1) - k0, 0, None).sum())
    return total


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward on the same workload instead (inputs quantised per head "
                         "before the timed region)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward (fa2_bwd) of the same workload instead, FLOPs counted as 2.5x the "
                         "forward's (for its profile)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB read + 1 GiB write elementwise kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the attention forward "
              f"shards over heads with no exchange, so the one-GPU figure is the per-GPU throughput)",
              file=sys.stderr)
        sys.exit(2)

    import exact_attention_85_amd as fa2

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fa2.load_library()

    w = workloads.C4
    causal = False
    q, k, v = workloads.make_qkv(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.n_q), dtype=torch.float32, device=dev)

    if args.calib_copy:
        # counter calibration: an out-of-place multiply that reads 1 GiB and writes 1 GiB
        # (four times the 256 MB last-level cache, so it streams from HBM)
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.bwd:
        args.fp8 = False
        dout = workloads.make_tensor(w.index, 3, w.B, w.H, w.n_q, w.d, dev)
        fa2.forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse)
        wsb = torch.empty(fa2.bwd_workspace_bytes(w.B, w.H, w.n_q, w.n_k, w.d) // 4, dtype=torch.float32, device=dev)
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def step():
            fa2.backward(q, k, v, o, lse, dout, causal=causal, scale=w.scale, workspace=wsb, dq=gq, dk=gk, dv=gv)
    elif args.fp8:
        qc, dq = fa2.quantize_fp8(q)
        kc, dk = fa2.quantize_fp8(k)
        vt, dv = fa2.quantize_fp8(v, transposed=True)

        def step():
            fa2.forward_fp8(qc, kc, vt, dq, dk, dv, causal=causal, scale=w.scale, out=o, lse=lse)
    else:
        def step():
            fa2.forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one event between consecutive launches: the mean is first-to-last, and the
    # per-launch times give the median and minimum
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    events[0].record()
    for i in range(args.steps):
        step()
        events[i + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = events[0].elapsed_time(events[-1]) / args.steps
    per_launch = sorted(events[i].elapsed_time(events[i + 1]) for i in range(args.steps))
    ms_median, ms_min = per_launch[len(per_launch) // 2], per_launch[0]
    flop = w.flop(causal) * (2.5 if args.bwd else 1.0)
    tflops = flop / (ms * 1e-3) / 1e12
    assert torch.isfinite(lse).all().item(), "non-finite LSE"
    mode = " fp8" if args.fp8 else (" backward" if args.bwd else "")
    log(f"{w.name} non-causal{mode}: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s, wall {t_wall:.2f} s")

    peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    if args.bwd:
        kname, traffic = "bwd_kv_pp_kernel<128> + bwd_dq_pp_kernel<128>", measured_traffic(f"bwd:{w.name}:noncausal",
                                                                                      (BWD_SRC,))
        # read Q, O, dO (N_q x d) and K, V (N_k x d) in bf16 and LSE in fp32; write dQ, dK, dV in bf16
        alg_bytes = w.B * w.H * (2 * (3 * w.n_q + 2 * w.n_k) * w.d + 4 * w.n_q + 2 * (w.n_q + 2 * w.n_k) * w.d)
    elif args.fp8:
        kname, traffic = "fwd_fp8_kernel<128,4>", measured_traffic(f"fwd_fp8_kernel:{w.name}:noncausal", (FP8_SRC,))
        alg_bytes = w.B * w.H * (w.n_q * w.d + 2 * w.n_k * w.d + 2 * w.n_q * w.d + 4 * w.n_q)  # 1-byte Q, K, V codes
    else:
        kname, traffic = "fwd_pp_kernel<128>", measured_traffic(f"fwd_pp_kernel:{w.name}:noncausal",
                                                                (KERNEL_SRC, TUNE_TABLE))
        alg_bytes = w.io_bytes()
    result = {
        "metric": METRIC_FP8 if args.fp8 else (METRIC_BWD if args.bwd else METRIC), "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4), "ms_per_step_min": round(ms_min, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3" if args.fp8 else "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}_noncausal", "B": w.B, "H": w.H, "N_q": w.n_q, "N_k": w.n_k, "d": w.d,
                   "causal": False, "scale": w.scale, "inputs": "iid N(0,1) fp32 -> bf16 RNE, seeded"},
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": flop, "algorithmic_bytes_per_launch": alg_bytes},
    }

    if not args.no_extra:
        extra = []
        steps_x = max(5, args.steps // 2)
        for wx, cx in ((workloads.C4, True), (workloads.C3, False), (workloads.C3, True), (workloads.C2, False),
                       (workloads.C2, True), (workloads.C1, False)):
            qx, kx, vx = workloads.make_qkv(wx, dev)
            ox = torch.empty_like(qx)
            lx = torch.empty((wx.B, wx.H, wx.n_q), dtype=torch.float32, device=dev)
            msx = time_launches(lambda: fa2.forward(qx, kx, vx, causal=cx, scale=wx.scale, out=ox, lse=lx),
                                steps_x, args.warmup)
            tf = wx.flop(cx) / (msx * 1e-3) / 1e12
            extra.append({"workload": wx.name, "causal": cx, "ms": round(msx, 4), "TFLOP/s": round(tf, 2),
                          "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
            log(f"{wx.name} causal={cx}: {msx:.3f} ms, {tf:.1f} TFLOP/s")
            del qx, kx, vx, ox, lx
        # sliding window on the long-sequence shape: causal attention over the last 4096 positions;
        # FLOPs counted over the visible (query, key) pairs, 4*d per pair
        for (wl, wr) in ((4095, 0),):
            wx = workloads.C4
            qx, kx, vx = workloads.make_qkv(wx, dev)
            ox = torch.empty_like(qx)
            lx = torch.empty((wx.B, wx.H, wx.n_q), dtype=torch.float32, device=dev)
            msx = time_launches(lambda: fa2.forward_window(qx, kx, vx, wl, wr, scale=wx.scale, out=ox, lse=lx),
                                steps_x, args.warmup)
            i = np.arange(wx.n_q)
            lo = np.maximum(0, i - wl) if wl >= 0 else np.zeros_like(i)
            hi = np.minimum(wx.n_k, i + wr + 1) if wr >= 0 else np.full_like(i, wx.n_k)
            pairs = int(np.maximum(hi - lo, 0).sum())
            fl = 4.0 * wx.d * wx.B * wx.H * pairs
            tf = fl / (msx * 1e-3) / 1e12
            extra.append({"workload": f"{wx.name}_window_{wl}_{wr}", "window": [wl, wr], "ms": round(msx, 4),
                          "TFLOP/s": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "visible_pairs_per_head": pairs})
            log(f"{wx.name} window ({wl},{wr}): {msx:.3f} ms, {tf:.1f} TFLOP/s")
            del qx, kx, vx, ox, lx
        # block-sparse: a dilated causal window on the long-sequence shape (each query block sees the
        # key blocks of its own positions and every 2nd of the 128 key blocks before them); FLOPs
        # counted over the visible (query, key) pairs, 4*d per pair
        wx = workloads.C4
        qx, kx, vx = workloads.make_qkv(wx, dev)
        ox = torch.empty_like(qx)
        lx = torch.empty((wx.B, wx.H, wx.n_q), dtype=torch.float32, device=dev)
        mask = workloads.dilated_block_mask(wx.n_q, wx.n_k, 2, 64, True)
        mt = torch.from_numpy(mask).to(dev)
        msx = time_launches(lambda: fa2.forward_blocksparse(qx, kx, vx, mt, -1, 0, scale=wx.scale, out=ox, lse=lx),
                            steps_x, args.warmup)
        pairs = blockmask_causal_pairs(mask, wx.n_q, wx.n_k)
        fl = 4.0 * wx.d * wx.B * wx.H * pairs
        tf = fl / (msx * 1e-3) / 1e12
        extra.append({"workload": f"{wx.name}_dilated_r2_w64_causal", "mask_blocks": [int(mask.sum()), int(mask.size)],
                      "ms": round(msx, 4), "TFLOP/s": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "visible_pairs_per_head": pairs})
        log(f"{wx.name} block-sparse dilated r2 w64 causal: {msx:.3f} ms, {tf:.1f} TFLOP/s")
        del qx, kx, vx, ox, lx, mt
        # backward (deterministic two-pass dQ): FLOPs 2.5x the forward's (five products instead of two)
        for wx, cx in ((workloads.C3, False), (workloads.C3, True), (workloads.C4, False)):
            qx, kx, vx = workloads.make_qkv(wx, dev)
            dox = workloads.make_tensor(wx.index, 3, wx.B, wx.H, wx.n_q, wx.d, dev)
            ox, lx = fa2.forward(qx, kx, vx, causal=cx, scale=wx.scale)
            wsx = torch.empty(fa2.bwd_workspace_bytes(wx.B, wx.H, wx.n_q, wx.n_k, wx.d) // 4, dtype=torch.float32,
                              device=dev)
            gq, gk, gv = torch.empty_like(qx), torch.empty_like(kx), torch.empty_like(vx)
            msx = time_launches(lambda: fa2.backward(qx, kx, vx, ox, lx, dox, causal=cx, scale=wx.scale,
                                                     workspace=wsx, dq=gq, dk=gk, dv=gv), steps_x, args.warmup)
            tf = 2.5 * wx.flop(cx) / (msx * 1e-3) / 1e12
            extra.append({"workload": f"{wx.name}_backward", "causal": cx, "ms": round(msx, 4), "TFLOP/s": round(tf, 2),
                          "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flop": 2.5 * wx.flop(cx),
                          "workspace_bytes": wsx.numel() * 4})
            log(f"{wx.name} backward causal={cx}: {msx:.3f} ms, {tf:.1f} TFLOP/s")
            del qx, kx, vx, dox, ox, lx, wsx, gq, gk, gv
        # FP8 forward: inputs quantised per (batch, head) outside the timed region (the quantiser
        # is timed on its own: it reads bf16 and writes one byte per element)
        for wx, cx in ((workloads.C4, False), (workloads.C4, True), (workloads.C3, False)):
            qx, kx, vx = workloads.make_qkv(wx, dev)
            qc, dq = fa2.quantize_fp8(qx)
            kc, dk = fa2.quantize_fp8(kx)
            vt, dv = fa2.quantize_fp8(vx, transposed=True)
            ox = torch.empty_like(qx)
            lx = torch.empty((wx.B, wx.H, wx.n_q), dtype=torch.float32, device=dev)
            msx = time_launches(lambda: fa2.forward_fp8(qc, kc, vt, dq, dk, dv, causal=cx, scale=wx.scale, out=ox,
                                                        lse=lx), steps_x, args.warmup)
            tf = wx.flop(cx) / (msx * 1e-3) / 1e12
            row = {"workload": f"{wx.name}_fp8", "causal": cx, "dtype": "fp8_e4m3", "ms": round(msx, 4),
                   "TFLOP/s": round(tf, 2), "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                   "speedup_vs_bf16_kernel_same_shape": None}
            if wx is workloads.C4 and not cx:
                msq = time_launches(lambda: fa2.quantize_fp8(vx, transposed=True), steps_x, args.warmup)
                nbytes = 3 * wx.B * wx.H * wx.n_k * wx.d
                row["quantize_v_transposed"] = {"ms": round(msq, 4), "GB/s": round(nbytes / (msq * 1e-3) / 1e9, 1)}
            extra.append(row)
            log(f"{wx.name} fp8 causal={cx}: {msx:.3f} ms, {tf:.1f} TFLOP/s")
            del qx, kx, vx, qc, kc, vt, ox, lx
        bf16_ms = {(e["workload"], e.get("causal")): e["ms"] for e in extra if "dtype" not in e and "ms" in e}
        if not args.fp8:
            bf16_ms[(w.name, causal)] = ms
        for e in extra:
            if e.get("dtype") == "fp8_e4m3":
                ref = bf16_ms.get((e["workload"][:-4], e["causal"]))
                e["speedup_vs_bf16_kernel_same_shape"] = round(ref / e["ms"], 3) if ref else None
        # split-KV decode: bound by streaming K and V from HBM
        wd = workloads.C5
        qd, kd, vd = workloads.make_qkv(wd, dev)
        od = torch.empty_like(qd)
        ld = torch.empty((wd.B, wd.H, wd.n_q), dtype=torch.float32, device=dev)
        ws = torch.empty(fa2.splitkv_workspace_bytes(wd.B, wd.H, wd.n_q, wd.d, wd.num_splits) // 4,
                         dtype=torch.float32, device=dev)
        msd = time_launches(lambda: fa2.forward_splitkv(qd, kd, vd, num_splits=wd.num_splits, scale=wd.scale,
                                                        workspace=ws, out=od, lse=ld), steps_x, args.warmup)
        gbs = wd.io_bytes() / (msd * 1e-3) / 1e9
        extra.append({"workload": wd.name, "causal": False, "ms": round(msd, 4), "GB/s": round(gbs, 1),
                      "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                      "TFLOP/s": round(wd.flop(False) / (msd * 1e-3) / 1e12, 3),
                      "algorithmic_bytes": wd.io_bytes(),
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "traffic": measured_traffic(f"splitkv:{wd.name}")}})
        log(f"{wd.name}: {msd:.3f} ms, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s)")
        # the same decode with the split count fa2_num_splits picks (1 here: B*H fills the chip,
        # so fa2_fwd streams each head's keys in one workgroup and writes O directly)
        s_auto = fa2.num_splits(wd.B, wd.H, wd.n_q, wd.n_k, wd.d)
        if s_auto == 1:
            fn = lambda: fa2.forward(qd, kd, vd, scale=wd.scale, out=od, lse=ld)  # noqa: E731
        else:
            fn = lambda: fa2.forward_splitkv(qd, kd, vd, num_splits=s_auto, scale=wd.scale,  # noqa: E731
                                             workspace=ws, out=od, lse=ld)
        msa = time_launches(fn, steps_x, args.warmup)
        gba = wd.io_bytes() / (msa * 1e-3) / 1e9
        extra.append({"workload": wd.name.replace("_s16", "_auto"), "num_splits": s_auto, "causal": False,
                      "ms": round(msa, 4), "GB/s": round(gba, 1), "frac_of_hbm_peak": round(gba / PEAK_HBM_GBS, 4)})
        log(f"decode with fa2_num_splits -> {s_auto}: {msa:.3f} ms, {gba:.0f} GB/s")
        # the same decode over an FP8 K/V cache (codes quantised per head before the timed region)
        qc8, dq8 = fa2.quantize_fp8(qd)
        kc8, dk8 = fa2.quantize_fp8(kd)
        vc8, dv8 = fa2.quantize_fp8(vd)
        ms8 = time_launches(lambda: fa2.decode_fp8(qc8, kc8, vc8, dq8, dk8, dv8, scale=wd.scale, out=od, lse=ld),
                            steps_x, args.warmup)
        bytes8 = wd.B * wd.H * (2 * wd.n_k * wd.d + wd.d + 2 * wd.d + 4)  # K, V and Q codes in; O, LSE out
        gb8 = bytes8 / (ms8 * 1e-3) / 1e9
        extra.append({"workload": wd.name.replace("_s16", "_fp8"), "dtype": "fp8_e4m3", "causal": False,
                      "ms": round(ms8, 4), "GB/s": round(gb8, 1), "frac_of_hbm_peak": round(gb8 / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": bytes8, "speedup_vs_bf16_decode": round(msa / ms8, 3)})
        log(f"decode over FP8 K/V: {ms8:.3f} ms, {gb8:.0f} GB/s, {msa / ms8:.2f}x the bf16 decode")
        del qd, kd, vd, od, ld, ws, qc8, kc8, vc8
        result["workloads"] = extra

    if not args.no_cpu and not args.fp8 and not args.bwd:  # the oracle baseline is the bf16 forward
        result["cpu_baseline"], result["parity"] = cpu_baseline(w, causal, q, k, v, o, lse)
        log(f"oracle: {result['cpu_baseline']}")
        log(f"parity of the timed run: {result['parity']}")
    result["env"] = env_info()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
