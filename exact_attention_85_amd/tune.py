"""Autotuner of the forward configurations (kernel x workgroup order).

The synthesis page (section 3 item 3) faults FlashAttention-2 for choosing its
block sizes by hand from a few candidates, and (section 5 item 1) names a search
over block sizes, warp counts and stages per shape as the way forward.  This
module runs that search on the GPU it is given: it times every configuration
fa2_fwd_config offers on a grid of shapes (head dim x mask x sequence length, at
a fixed number of query tokens per launch), picks the fastest per shape, and
writes the table that fa2_fwd and fa2_fwd_window read
(exact_attention_85_amd/csrc/fa2_tune_table.h).

    python -m exact_attention_85_amd.tune [--out DIR] [--write] [--reps R] [--quick]

Outputs in DIR (default gpurun_out/tune): tune_fwd.json (every timing),
tune_fwd.md (the tables) and fa2_tune_table.h; --write also replaces the
table in the source tree (rebuild the library afterwards).  Timing: one
launch per configuration in turn, repeated R times, so that clock drift hits
every configuration alike; the median per configuration is kept.  Inputs are
the seeded N(0, 1) bf16 tensors of workloads.make_qkv_shape.
"""
import argparse
import datetime
import json
import os
import sys

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import exact_attention_85_amd as fa2  # noqa: E402
import workloads  # noqa: E402

TABLE_PATH = os.path.join(PKG, "csrc", "fa2_tune_table.h")
TOKENS = 1 << 19                        # query tokens per launch (B*H*N_q)
SEQ_LENS = (512, 1024, 2048, 4096, 8192, 16384)
PEAK_BF16_TFLOPS = 256 * 4 * 1024 * 2.4e9 / 1e12


def shape_grid(quick: bool):
    lens = (1024, 4096, 16384) if quick else SEQ_LENS
    for d in (64, 128):
        for banded in (0, 1):
            for n in lens:
                bh = max(1, TOKENS // n)
                H = min(bh, 32)
                yield d, banded, n, bh // H, H


def flop(B, H, n, d, banded):
    f = 4.0 * B * H * n * n * d
    return f / 2 if banded else f


def time_configs(B, H, n, d, banded, reps, configs):
    """Median milliseconds per launch of each configuration, timed in rotation."""
    q, k, v = workloads.make_qkv_shape(B, H, n, n, d, seed=n + d + banded, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    wr = 0 if banded else -1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for c in configs:  # warm-up, and every configuration must agree with the first
        fa2.forward_config(q, k, v, c, -1, wr, out=o, lse=lse)
    torch.cuda.synchronize()
    ref = None
    for c in configs:
        fa2.forward_config(q, k, v, c, -1, wr, out=o, lse=lse)
        torch.cuda.synchronize()
        if ref is None:
            ref = (o.clone(), lse.clone())
        elif (o.float() - ref[0].float()).abs().max().item() > 1e-2 or (lse - ref[1]).abs().max().item() > 1e-3:
            raise RuntimeError(f"configuration {fa2.config_name(c)} disagrees with {fa2.config_name(configs[0])}")
    times = {c: [] for c in configs}
    for _ in range(reps):
        for c in configs:
            ev[0].record()
            fa2.forward_config(q, k, v, c, -1, wr, out=o, lse=lse)
            ev[1].record()
            ev[1].synchronize()
            times[c].append(ev[0].elapsed_time(ev[1]))
    del q, k, v, o, lse
    return {c: float(np.median(t)) for c, t in times.items()}


NOISE = 0.025  # timings within 2.5 % of the fastest count as a tie (about the spread between runs)


def low_traffic(config: int) -> bool:
    """The renumbered head-major order runs each head's blocks on one XCD, so each head's K/V is
    fetched into one L2: HBM reads measured 1.0-1.7x the input bytes against 3.0-5.7x for the other
    orders (with the renumbering and query-block-major order every XCD sees every head)."""
    return fa2.config_name(config).endswith("_remap_headmajor")


def table_rows(results, noise=NOISE):
    """(d, banded) -> rows (nq_min, config): per measured length the fastest configuration,
    applying from the geometric midpoint to the previous measured length.  Configurations within
    `noise` of the fastest count as tied with it; among tied ones the previous length's choice
    comes first (so that the table does not switch on run-to-run noise), then the lower-traffic
    (renumbered) orders, then the faster.  Equal neighbours are merged."""
    rows = {}
    for (d, banded), per_n in sorted(results.items()):
        lens = sorted(per_n)
        out = []
        for i, n in enumerate(lens):
            t = per_n[n]
            fastest = min(t.values())
            tied = [c for c in t if t[c] <= fastest * (1 + noise)]
            prev = out[-1][1] if out else None
            best = min(tied, key=lambda c: (c != prev, not low_traffic(c), t[c]))
            nq_min = 1 if i == 0 else int(round((lens[i - 1] * n) ** 0.5))
            if not out or out[-1][1] != best:
                out.append((nq_min, best))
        rows[(d, banded)] = out
    return rows


def write_header(path, rows, source):
    lines = [
        "// Forward configuration per shape class: the rows fa2_fwd and fa2_fwd_window",
        "// look up (the synthesis page, section 3 item 3 and section 5 item 1: block",
        "// sizes, warp counts and similar launch choices searched per shape instead of",
        "// a few hand-picked ones).  Written by exact_attention_85_amd/tune.py from its",
        "// measurements; tune.py --write replaces this file.",
        "//",
        "// Each row: head dim, banded (causal or windowed), the smallest N_q the row",
        "// applies to, and the configuration (index into kFwdConfigs).  For a shape the",
        "// row with matching d and banded and the largest nq_min <= N_q applies.",
        "#pragma once",
        "",
        "namespace fa2 {",
        "",
        "struct TuneRow {",
        "  int d;",
        "  int banded;",
        "  int nq_min;",
        "  int config;",
        "};",
        "",
        f"// source: {source}",
        "constexpr TuneRow kTuneTable[] = {",
    ]
    for (d, banded), rs in sorted(rows.items()):
        for nq_min, c in rs:
            lines.append(f"    {{{d}, {banded}, {nq_min}, {c}}},  // {fa2.config_name(c)}")
    lines += ["};", "", "}  // namespace fa2", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def probe_summary(n=4096, launches=4):
    """Where the workgroups of `launches` probe launches ran: for each launch the offset o with
    XCD = (id + o) mod 8 for the most workgroups, and the fraction of workgroups that fits it."""
    out = []
    for _ in range(launches):
        xcd, _ = fa2.probe_xcc(n)
        xcd = xcd.numpy()
        off = np.bincount((xcd - np.arange(n)) % 8, minlength=8)
        o = int(np.argmax(off))
        out.append({"offset": o, "frac_round_robin": float(off[o]) / n,
                    "per_xcd": np.bincount(xcd, minlength=8).tolist()})
    return {"workgroups": n, "launches": out}


def probe_text(probe):
    ls = probe["launches"]
    fracs = ", ".join("%.1f %%" % (100 * x["frac_round_robin"]) for x in ls)
    return (f"Dispatch probe ({probe['workgroups']} one-wave workgroups, {len(ls)} launches): workgroup i ran on XCD "
            f"(i + o) mod 8 for {fracs} of the workgroups, offsets o = {[x['offset'] for x in ls]}; "
            f"per-XCD counts {ls[0]['per_xcd']}.")


def profile_one(name, shape, launches):
    """Launch one configuration `launches` times on one shape (a counter or trace run under
    rocprofv3 sees exactly these dispatches of the attention kernel) and print its timing."""
    d, banded, B, H, n = (int(x) for x in shape.split(","))
    torch.cuda.set_device(0)
    fa2.load_library()
    c = [fa2.config_name(i) for i in range(fa2.num_configs())].index(name)
    q, k, v = workloads.make_qkv_shape(B, H, n, n, d, seed=n + d + banded, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(launches):
        fa2.forward_config(q, k, v, c, -1, 0 if banded else -1, out=o, lse=lse)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(launches))
    f = flop(B, H, n, d, banded)
    print(json.dumps({"config": name, "d": d, "causal": bool(banded), "B": B, "H": H, "N": n,
                      "ms_median": round(ms[len(ms) // 2], 4), "ms_min": round(ms[0], 4),
                      "tflops_median": round(f / (ms[len(ms) // 2] * 1e-3) / 1e12, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "tune"))
    ap.add_argument("--write", action="store_true", help="replace csrc/fa2_tune_table.h")
    ap.add_argument("--reps", type=int, default=15)
    ap.add_argument("--quick", action="store_true", help="three lengths only")
    ap.add_argument("--from-json", default=None,
                    help="rebuild the table and summary from a tune_fwd.json of an earlier run (no GPU)")
    ap.add_argument("--profile", default=None, metavar="CONFIG",
                    help="only run configuration CONFIG (a name) on --shape, --launches times (for counters)")
    ap.add_argument("--shape", default="128,0,1,32,16384", help="d,causal,B,H,N for --profile")
    ap.add_argument("--launches", type=int, default=5)
    args = ap.parse_args()
    if args.profile:
        return profile_one(args.profile, args.shape, args.launches)
    os.makedirs(args.out, exist_ok=True)
    configs = list(range(fa2.num_configs()))
    names = [fa2.config_name(c) for c in configs]
    if args.from_json:
        with open(args.from_json) as f:
            saved = json.load(f)
        records, probe, source = saved["records"], saved["probe"], saved["source"]
        reps, quick = saved.get("reps", args.reps), saved.get("quick", False)
        results = {}
        for r in records:
            results.setdefault((r["d"], int(r["causal"])), {})[r["N"]] = {
                names.index(k): v for k, v in r["ms"].items()}
    else:
        reps, quick = args.reps, args.quick
        torch.cuda.set_device(0)
        fa2.load_library()
        props = torch.cuda.get_device_properties(0)
        results, records = {}, []
        for d, banded, n, B, H in shape_grid(quick):
            t = time_configs(B, H, n, d, banded, reps, configs)
            results.setdefault((d, banded), {})[n] = t
            f = flop(B, H, n, d, banded)
            best = min(t, key=t.get)
            rec = {"d": d, "causal": bool(banded), "N": n, "B": B, "H": H,
                   "ms": {fa2.config_name(c): round(t[c], 4) for c in configs},
                   "tflops": {fa2.config_name(c): round(f / (t[c] * 1e-3) / 1e12, 1) for c in configs},
                   "best": fa2.config_name(best)}
            records.append(rec)
            print(f"d={d} causal={bool(banded)} N={n} B={B} H={H}: best {rec['best']} "
                  f"{rec['tflops'][rec['best']]} TFLOP/s; " +
                  ", ".join(f"{k} {v}" for k, v in rec["tflops"].items()), flush=True)
        probe = probe_summary()
        stamp = datetime.datetime.now(datetime.timezone.utc).strftime("%Y-%m-%d %H:%M UTC")
        source = f"tune.py on {props.name} ({props.multi_processor_count} CUs), {stamp}, {reps} reps"
    rows = table_rows(results)
    chosen = {(d, b): rs for (d, b), rs in rows.items()}
    for r in records:  # the configuration the table picks at each measured length
        rs = chosen[(r["d"], int(r["causal"]))]
        r["table"] = fa2.config_name([c for m, c in rs if m <= r["N"]][-1])
    write_header(os.path.join(args.out, "fa2_tune_table.h"), rows, source)
    if args.write:
        write_header(TABLE_PATH, rows, source)
    if not args.from_json:
        with open(os.path.join(args.out, "tune_fwd.json"), "w") as f:
            json.dump({"source": source, "reps": reps, "quick": quick, "tokens_per_launch": TOKENS,
                       "records": records, "probe": probe,
                       "table": {f"d{d}_{'causal' if b else 'plain'}": [[m, fa2.config_name(c)] for m, c in r]
                                 for (d, b), r in rows.items()}}, f, indent=1)
    md = ["# Forward configurations measured by tune.py", "",
          f"Command: `python -m exact_attention_85_amd.tune --reps {reps}{' --quick' if quick else ''}`"
          f" ({source}).", f"{TOKENS} query tokens per launch (B*H = {TOKENS}/N), N_q = N_k = N, seeded N(0,1) bf16,"
          " scale 1/sqrt(d). TFLOP/s from the median of the launches of each configuration (timed in rotation);"
          f" causal FLOPs halved. Configurations within {100 * NOISE:.1f} % of the fastest count as tied; ties go to the"
          " previous length's choice, then to the XCD-renumbered head-major orders (fewest HBM bytes,"
          " `xcd_order_counters_c2_c3_c4.md`) (column `table`).", "",
          probe_text(probe) if "launches" in probe else
          f"Dispatch probe: {100 * probe['frac_on_xcd_id_mod_8']:.1f} % of {probe['workgroups']} workgroups ran on "
          f"XCD (id mod 8); per-XCD counts {probe['per_xcd']}.", "",
          "| d | causal | N | B x H | " + " | ".join(names) + " | fastest | table |",
          "|---|---|---|---|" + "---|" * len(names) + "---|---|"]
    for r in records:
        md.append(f"| {r['d']} | {'yes' if r['causal'] else 'no'} | {r['N']} | {r['B']} x {r['H']} | " +
                  " | ".join(f"{r['tflops'][nm]}" for nm in names) + f" | {r['best']} | {r['table']} |")
    md += ["", "Table written (nq_min -> configuration):", ""]
    for (d, b), rs in sorted(rows.items()):
        md.append(f"* d = {d}, {'causal' if b else 'plain'}: " +
                  ", ".join(f"N_q >= {m}: {fa2.config_name(c)}" for m, c in rs))
    with open(os.path.join(args.out, "tune_fwd.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md[-6:]), flush=True)


if __name__ == "__main__":
    main()
