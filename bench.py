#!/usr/bin/env python3
"""Throughput of the compressed sparse attention hot path on one MI355X.

A step is one pass of the whole hot path (fp4 round trip of the step's new
latent and indexer-k rows, ring write, window columns, indexer scores + top-k,
sparse attention with the sink) over one batch: B independent sequences of a
workload, every input resident in HBM before the timed region.

Default workload: decode, m = 1 at start_pos = 32767, 64 heads x 512, window
128, ratio 4 (8192 compressed rows), indexer 64 x 128 with top-512, batched
over B = 2048 independent sequences (eight attention workgroups per compute
unit and call, two at a time, so that the launch, dispatch and
per-workgroup start-up cost is spread over more queries); one step streams
~2.8 GB, far past the 256 MB last-level cache.

Prints ONE JSON line (stdout): metric tokens/s, roofline of the dominant
kernel (HIP-event time on the library's stream), and the oracle timed on the
host cores as a CPU baseline.  Everything else goes to stderr.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, datasheet

DEFAULT_B = {"tiny_decode": 1, "decode": 2048, "long_decode": 512, "causal_prefill": 1, "chunked_prefill": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def describe(w):
    s = (f"{w.name}: m={w.m} start_pos={w.start_pos} H={w.H} D={w.D} win={w.win} ratio={w.ratio} "
         f"n_c={w.n_c}")
    if w.Hi:
        s += f" indexer {w.Hi}x{w.Di} top-{w.K}"
    else:
        s += f" all visible compressed rows (<= {w.K})"
    return s


def counts(w, B, call, kcache="bf16"):
    """Algorithmic bytes and flops of one library call for one step of B
    sequences: what the method must read and write (bf16 storage, each needed
    row once, valid (query, row) pairs only).  The implementation's workspace
    traffic is not counted.  bound: the roofline the call is judged against."""
    m, win, D = w.m, w.win, w.D
    V = [min(w.n_c, (w.start_pos + t + 1) // w.ratio) for t in range(m)]
    Wv = [min(win, w.start_pos + t + 1) for t in range(m)]
    C = [min(w.K, v) for v in V]
    pairs = sum(Wv) + sum(C)
    n_new = w.n_c - w.first_new_row
    dense = m > 1
    if call == "quant_latent":
        return {"bytes": B * n_new * D * 4, "flops": 0, "bound": "hbm"}
    krow = w.Di // 2 + w.Di // 32 if kcache == "fp4" else w.Di * 2  # stored bytes of an indexer k row
    if call == "quant_index_k":
        return {"bytes": B * n_new * (w.Di * 2 + krow), "flops": 0, "bound": "hbm"}
    if call == "ring_write":
        return {"bytes": B * min(m, win) * D * 4, "flops": 0, "bound": "hbm"}
    if call == "window_idx":
        return {"bytes": B * m * win * 4, "flops": 0, "bound": "hbm"}
    if call == "decode_prepare":  # the four set-up calls of a decode step in one launch
        return {"bytes": sum(counts(w, B, c, kcache)["bytes"]
                             for c in ("quant_latent", "quant_index_k", "ring_write", "window_idx")),
                "flops": 0, "bound": "hbm"}
    if call == "visible_idx":
        return {"bytes": B * m * w.K * 4, "flops": 0, "bound": "hbm"}
    if call == "index_scores_topk":
        by = B * (max(V) * krow + m * w.Hi * w.Di * 2 + m * w.Hi * 4 + m * w.K * 4)
        fl = B * sum(V) * w.Hi * w.Di * 2
        return {"bytes": by, "flops": fl, "bound": "mfma" if dense else "hbm"}
    if call == "sparse_attn_sink":
        rows = (w.m if w.start_pos == 0 else (win + m if m > 1 else None))
        row_bytes = (rows + w.n_c) * D * 2 if rows is not None else pairs * D * 2
        by = B * (row_bytes + 2 * m * w.H * D * 2 + m * w.T * 4 + w.H * 4)
        fl = B * pairs * w.H * D * 4
        return {"bytes": by, "flops": fl, "bound": "mfma" if dense else "hbm"}
    raise KeyError(call)


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank space removed, so that
    only code changes invalidate counters taken earlier."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_compressed_kv_e2m1_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(workload, B, call, kcache):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = rec.get("entries", {}).get(f"{workload}/B{B}/{kcache}/{call}")
    return None if entry is None else entry.get("hbm_bytes_per_launch")


# Library call -> the kernels it launches (demangled-name prefixes).
CALL_KERNELS = {
    "quant_latent": ["quant_rows_kernel<0,"],
    "quant_index_k": ["quant_rows_kernel<1,", "quant_pack_kernel<1>"],
    "ring_write": ["ring_write_kernel"],
    "decode_prepare": ["decode_prepare_kernel"],
    "window_idx": ["window_idx_kernel"],
    "visible_idx": ["visible_idx_kernel"],
    "index_scores_topk": ["index_score_kernel", "topk_kernel"],
    "sparse_attn_sink": ["sparse_attn_kernel", "combine_kernel"],
}


def _kernel_short(name):
    name = re.sub(r"^void ", "", name)
    name = name.replace("sckv::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name).replace(" ", "")


def _steady_groups(rows, key):
    """Per kernel: the dispatches of its most frequent grid size (the step's
    launches; one-off set-up launches of other sizes drop out)."""
    groups = {}
    for r in rows:
        if "sckv::" not in r["Kernel_Name"]:
            continue
        groups.setdefault(_kernel_short(r["Kernel_Name"]), {}).setdefault(key(r), []).append(r)
    return {k: max(v.values(), key=len) for k, v in groups.items()}


def _csv_rows(folder, suffix):
    import csv  # noqa: PLC0415
    import glob  # noqa: PLC0415

    paths = glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)
    if len(paths) != 1:
        raise SystemExit(f"expected one *{suffix} under {folder}, found {paths}")
    return list(csv.DictReader(open(paths[0])))


def summarize_profiles(w, B, folder, commands, kcache="bf16"):
    """Turn rocprofv3 output under `folder` (trace/, FETCH_SIZE/, WRITE_SIZE/,
    copy_FETCH_SIZE/, copy_WRITE_SIZE/) into the text summary
    profiles/hot_path_kernels_<workload>_B<B>.txt and the HBM-traffic entries
    of profiles/traffic.json (counter KiB per dispatch, scaled so that a plain
    1 GiB device copy reads and writes 1 GiB)."""
    tr = _steady_groups(_csv_rows(os.path.join(folder, "trace"), "kernel_trace.csv"),
                        lambda r: (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"]))
    dur = {k: sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in v) / len(v) / 1e3
           for k, v in tr.items()}
    calls = {k: len(v) for k, v in tr.items()}
    res = {"FETCH_SIZE": None, "WRITE_SIZE": None}
    scale = {}
    for c in res:
        d = os.path.join(folder, c)
        if not os.path.isdir(d):
            continue
        g = _steady_groups(_csv_rows(d, "counter_collection.csv"), lambda r: r["Grid_Size"])
        res[c] = {k: sum(float(r["Counter_Value"]) for r in v) / len(v) * 1024 for k, v in g.items()}
        cdir = os.path.join(folder, "copy_" + c)
        if not os.path.isdir(cdir):  # one calibration next to several workloads' folders
            cdir = os.path.join(os.path.dirname(os.path.normpath(folder)), "copy_" + c)
        cp = _csv_rows(cdir, "counter_collection.csv")
        # the 1 GiB copy: the largest per-dispatch value of the copy kernel
        copy_bytes = max(float(r["Counter_Value"]) * 1024 for r in cp if "copyBuffer" in r["Kernel_Name"]
                         or "copy" in r["Kernel_Name"].lower())
        scale[c] = (1 << 30) / copy_bytes
    lines = [f"# rocprofv3 summary: compressed sparse attention hot path, {describe(w)}, B={B}"
             + (f", indexer k cache {kcache}" if w.Hi else ""), "#"]
    lines += ["# commands (repo root as working directory):"] + [f"#   {c}" for c in commands]
    lines += [f"# counter scale (1 GiB device copy): FETCH_SIZE x{scale.get('FETCH_SIZE', float('nan')):.3f}, "
              f"WRITE_SIZE x{scale.get('WRITE_SIZE', float('nan')):.3f}",
              "# steady-state dispatches only (most frequent grid size per kernel)", "#",
              f"{'kernel':<44} {'calls':>5} {'avg_us':>9} {'read_MB':>9} {'write_MB':>9}"]
    # only the kernels of the step's own calls (set-up launches are left out)
    from sparse_compressed_kv_e2m1_amd.step import step_call_names  # noqa: PLC0415
    names = step_call_names(w, kcache)
    mine = lambda k: any(k.startswith(p.replace(" ", "")) for c in names for p in CALL_KERNELS[c])  # noqa: E731
    dur = {k: v for k, v in dur.items() if mine(k)}
    for k in sorted(dur, key=lambda k: -dur[k]):
        rd = res["FETCH_SIZE"].get(k) if res["FETCH_SIZE"] else None
        wr = res["WRITE_SIZE"].get(k) if res["WRITE_SIZE"] else None
        rd = "-" if rd is None else f"{rd * scale['FETCH_SIZE'] / 1e6:.2f}"
        wr = "-" if wr is None else f"{wr * scale['WRITE_SIZE'] / 1e6:.2f}"
        lines.append(f"{k[:44]:<44} {calls[k]:>5} {dur[k]:>9.2f} {rd:>9} {wr:>9}")
    lines += ["#", f"{'library call':<20} {'avg_us':>9} {'alg_MB':>9} {'hbm_MB':>9}"]
    entries = {}
    for call in dict.fromkeys(names):
        pre = CALL_KERNELS[call]
        ks = [k for k in dur if any(k.startswith(p.replace(" ", "")) for p in pre)]
        if not ks:
            continue
        us = sum(dur[k] for k in ks)
        hbm = None
        if res["FETCH_SIZE"] and res["WRITE_SIZE"] and all(k in res[c] for c in res for k in ks):
            hbm = sum(res["FETCH_SIZE"].get(k, 0) * scale["FETCH_SIZE"] + res["WRITE_SIZE"].get(k, 0)
                      * scale["WRITE_SIZE"] for k in ks)
        alg = counts(w, B, call, kcache)["bytes"]
        lines.append(f"{call:<20} {us:>9.2f} {alg / 1e6:>9.2f} {'-' if hbm is None else f'{hbm / 1e6:.2f}':>9}")
        entries[f"{w.name}/B{B}/{kcache if w.Hi else 'none'}/{call}"] = {"kernels": ks, "avg_us": round(us, 3),
                                            "hbm_bytes_per_launch": None if hbm is None else int(hbm)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    kc = f"_kcache_{kcache}" if w.Hi else ""
    out = os.path.join(ROOT, "profiles", f"hot_path_kernels_{w.name}_B{B}{kc}.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(tj)) if os.path.exists(tj) else {}
    if rec.get("kernel_source_hash") != kernel_source_hash():
        rec = {"kernel_source_hash": kernel_source_hash(), "entries": {}}
    rec["note"] = ("HBM bytes per library call (all its kernels), rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by a "
                   "1 GiB copy; valid only for the kernel sources whose hash is kernel_source_hash")
    if res["FETCH_SIZE"] and res["WRITE_SIZE"]:
        rec["entries"].update(entries)
    json.dump(rec, open(tj, "w"), indent=1, sort_keys=True)
    log(f"wrote {out} and {tj}")


def cpu_baseline(w, seconds):
    """The oracle as it stands, single-threaded, on a bounded sample of the same
    workload (one sequence; decode: whole steps, prefill: sampled queries)."""
    import numpy as np  # noqa: PLC0415

    import sckv_synth as synth  # noqa: PLC0415
    from tests.helpers import oracle_step, sample_queries  # noqa: PLC0415

    x = synth.make_inputs(w, 1)
    tokens, t0 = 0, time.perf_counter()
    if w.m == 1:
        while True:
            oracle_step(w, x, 0)
            tokens += 1
            if time.perf_counter() - t0 >= seconds:
                break
        sample = f"{tokens} whole decode step(s) of one sequence"
    else:
        qs = sample_queries(w, extra=64, seed=1)
        for t in qs:
            oracle_step(w, x, 0, np.array([t]))
            tokens += 1
            if time.perf_counter() - t0 >= seconds:
                break
        sample = f"{tokens} query token(s) of one {w.m}-token step (index lists + attention per query)"
    el = time.perf_counter() - t0
    return {"value": tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle", "sample": sample,
            "seconds": round(el, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--instances", type=int, default=None, help="B independent sequences per step")
    ap.add_argument("--kcache", choices=["fp4", "bf16"], default="fp4",
                    help="indexer k cache storage: packed fp4 codes + E8M0 bytes (default) or bf16 rows")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single", action="store_true", help="skip the B = 1 latency run (for profiling)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of one step (measured: within noise of the call-by-call "
                         "launches for prefill, ~1.5%% slower for decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale for HBM byte counters)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="only write the profiles/ summary of the rocprofv3 output under DIR (no GPU)")
    ap.add_argument("--command", action="append", default=[], help="profiling command to record (--summarize)")
    args = ap.parse_args()
    if args.summarize:
        import sckv_synth as synth  # noqa: PLC0415

        w = synth.WORKLOADS[args.workload]
        summarize_profiles(w, args.instances or DEFAULT_B[args.workload], args.summarize, args.command, args.kcache)
        return
    if args.copy_calibration:
        import torch  # noqa: PLC0415

        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 5}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the multi-GPU "
              "sharding of this path is a design note, not an implementation.", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: PLC0415

    import sckv_synth as synth  # noqa: PLC0415
    from sparse_compressed_kv_e2m1_amd.step import PathState  # noqa: PLC0415

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    B = args.instances or DEFAULT_B[args.workload]
    log(f"bench: workload {w.name} B={B}: generating inputs on the device")
    x = synth.make_inputs(w, B, device="cuda")
    st = PathState(w, x, B, kcache=args.kcache)
    del x
    st.setup()
    calls = st.calls()
    st._calls = calls
    torch.cuda.synchronize()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()

    # whole steps, launched call by call, or (--graph) replayed from a HIP
    # graph of one step (the same library calls, without per-launch host work)
    stream = torch.cuda.current_stream()
    run_step = st.step
    launch = "eager"
    if args.graph:
        graph = st.capture_graph()
        run_step = graph.replay
        launch = "hip graph"
        for _ in range(args.warmup):
            run_step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    log(f"bench: {args.steps} steps, {ms:.4f} ms/step (events), wall {wall * 1e3 / args.steps:.4f} ms/step")

    # per call, events on the same stream around each library call
    per = {name: [] for name, _ in calls}
    for _ in range(args.steps):
        for name, f in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            per[name].append((a, b))
    torch.cuda.synchronize()
    per_ms = {n: sum(a.elapsed_time(b) for a, b in v) / len(v) for n, v in per.items()}
    log("bench: per call ms " + json.dumps({k: round(v, 5) for k, v in per_ms.items()}))

    # single sequence latency (B = 1) on the same workload
    single = None
    if B > 1 and not args.no_single:
        x1 = synth.make_inputs(w, 1, device="cuda")
        s1 = PathState(w, x1, 1, kcache=args.kcache)
        s1.setup()
        for _ in range(args.warmup):
            s1.step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            s1.step()
        b.record(stream)
        torch.cuda.synchronize()
        ms1 = a.elapsed_time(b) / args.steps
        single = {"instances": 1, "ms_per_step": round(ms1, 5), "tokens_per_s": round(w.m / (ms1 / 1e3), 1)}
        del s1, x1

    tokens = B * w.m
    value = tokens / (ms / 1e3)
    dom = max(per_ms, key=per_ms.get)
    cnt = counts(w, B, dom, args.kcache)
    if cnt["bound"] == "hbm":
        achieved = cnt["bytes"] / (per_ms[dom] / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = cnt["flops"] / (per_ms[dom] / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = dom
    roof["ms_per_launch"] = round(per_ms[dom], 5)
    roof["algorithmic_bytes"] = cnt["bytes"]
    roof["algorithmic_flops"] = cnt["flops"]
    roof["traffic"] = traffic_for(w.name, B, dom, args.kcache if w.Hi else "none")

    line = {
        "metric": "sparse-attn tokens/s (decode & prefill) + % of HBM/MFMA roofline, 1 MI355X",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), device generator)",
        "config": {"workload": describe(w), "instances": B, "tokens_per_step": tokens,
                   "indexer_k_cache": args.kcache if w.Hi else None, "step_launch": launch},
        "roofline": roof,
        "per_call_ms": {k: round(v, 5) for k, v in per_ms.items()},
        "single_instance": single,
    }
    if not args.no_cpu_baseline:
        log(f"bench: timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
