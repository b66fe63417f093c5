"""Benchmark of the segmented-gather multi-LoRA hot path on one MI355X.

One step = one batch through the whole path: lora_prepare_meta, then per
layer lora_shrink + lora_expand (add_inputs=1), on seeded synthetic inputs
already resident in HBM.  Default workload: ``decode`` (N=256 tokens,
H=4096, r=16, 32 LoRAs, q/k/v slices 4096/1024/1024, 10% of tokens -1).

Cold caches: when one input set fits in the 256 MB last-level cache, the
bench rotates through enough independent copies (>= 1 GiB in total) that
every step reads data that is not cache resident.  Steps are replayed from a
HIP graph (one graph holds one step per copy), as a serving loop replays its
decode step; ``--eager`` launches every call from Python instead.

Prints ONE JSON line.  ``roofline`` refers to the kernel with the largest
average duration; its duration is measured with HIP events on the stream the
kernels run on, over graph replays of that kernel alone right after the
timed region.  ``traffic`` comes from committed rocprofv3 PMC summaries
(profiles/) when their kernel source hash matches the current sources.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA shrink+expand tokens/sec at 1 GPU; achieved HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per launch (inputs/outputs of active tokens
    and active LoRAs only; each x row once, each active LoRA's weights once)."""
    import numpy as np
    m = wl.mapping.numpy()
    n = m.size
    act = m[m >= 0]
    ta, la = int(act.size), int(np.unique(act).size)
    out = {"prepare": 16 * n, "shrink": [], "expand": [], "T_a": ta, "L_a": la}
    for L in wl.layers:
        sp = L.spec
        S, r, H, O = len(sp.slices), sp.rank, sp.hidden, sum(sp.slices)
        out["shrink"].append(0 if sp.expand_only else 2 * ta * H + 2 * la * S * r * H + 8 * S * ta * r)
        bias = 2 * la * O if L.bias is not None else 0
        out["expand"].append(4 * S * ta * r + 2 * la * r * O + bias + 2 * ta * O * 2)
    return out


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "segmented_gather_lora_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class DeviceSet:
    """One independent copy of the workload's inputs in HBM."""

    def __init__(self, wl, src=None):
        import torch
        import segmented_gather_lora_amd as sgl
        n = wl.mapping.numel()
        self.n = n
        self.mapping = wl.mapping.to("cuda") if src is None else src.mapping.clone()
        self.meta = sgl.LoraMeta(wl.spec.max_loras, n)
        self.layers = []
        for li, L in enumerate(wl.layers):
            sp = L.spec
            if src is None:
                d = dict(x=L.x.to("cuda"), a=[t.to("cuda") for t in L.lora_a], b=[t.to("cuda") for t in L.lora_b],
                         bias=None if L.bias is None else [t.to("cuda") for t in L.bias], y=L.y0.to("cuda"))
            else:
                s = src.layers[li]
                d = dict(x=s["x"].clone(), a=[t.clone() for t in s["a"]], b=[t.clone() for t in s["b"]],
                         bias=None if s["bias"] is None else [t.clone() for t in s["bias"]], y=s["y"].clone())
            if sp.expand_only:
                d["buf"] = d["x"]   # the layer's input is the expand input
            else:
                d["buf"] = torch.zeros((len(sp.slices), n, sp.rank), dtype=torch.float32, device="cuda")
            d["scale"] = sp.scale
            d["expand_only"] = sp.expand_only
            self.layers.append(d)

    def prepare(self):
        import segmented_gather_lora_amd as sgl
        sgl.lora_prepare_meta(self.mapping, self.meta)

    def shrink(self, li):
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_shrink(d["x"], d["a"], d["buf"], self.meta, d["scale"])

    def expand(self, li):
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_expand(d["buf"], d["b"], d["bias"], d["y"], self.meta, offset_start=0, add_inputs=True)

    def linear(self, li):
        """shrink + expand of one layer in one lora_shrink_expand call."""
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_shrink_expand(d["x"], d["a"], d["b"], d["bias"], d["buf"], d["y"], self.meta, d["scale"],
                               offset_start=0, add_inputs=True)

    def prepare_linear(self, li):
        """prepare + shrink + expand of one layer in one lora_prepare_shrink_expand call."""
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_prepare_shrink_expand(self.mapping, d["x"], d["a"], d["b"], d["bias"], d["buf"], d["y"], self.meta,
                                       d["scale"], offset_start=0, add_inputs=True)

    def step(self, path: str = "prepare_fused"):
        first = 0
        if path == "prepare_fused" and not self.layers[0]["expand_only"]:
            self.prepare_linear(0)
            first = 1
        else:
            self.prepare()
        for li in range(first, len(self.layers)):
            if self.layers[li]["expand_only"]:
                self.expand(li)
            elif path in ("fused", "prepare_fused"):
                self.linear(li)
            else:
                self.shrink(li)
                self.expand(li)


def set_bytes(wl) -> int:
    tot = wl.mapping.numel() * 4
    for L in wl.layers:
        tot += L.x.numel() * L.x.element_size() + L.y0.numel() * 2
        tot += sum(t.numel() for t in L.lora_a) * 2 + sum(t.numel() for t in L.lora_b) * 2
        if not L.spec.expand_only:
            tot += 4 * len(L.spec.slices) * wl.mapping.numel() * L.spec.rank
    return tot


def capture(fn, reps: int = 1):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    return g


def time_graph(g, replays: int) -> float:
    """Average ms per replay, HIP events on the replay stream."""
    import torch
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / replays


def cpu_baseline(wl, budget_s: float) -> dict:
    """The oracle, as it is, on this host's cores: prepare + shrink + expand on
    a bounded sample of the workload's tokens."""
    import numpy as np
    import oracle
    import workloads
    cores = len(os.sched_getaffinity(0))
    cores = max(1, min(cores, 16))
    m = wl.mapping.numpy()
    n = m.size

    def run(tokens):
        oracle.prepare(m, wl.spec.max_loras)
        for L in wl.layers:
            sp = L.spec
            if sp.expand_only:
                buf = np.ascontiguousarray(L.x.numpy()[:, tokens])
            else:
                xb = workloads.bf16_bits(L.x)[tokens]
                buf = np.zeros((len(sp.slices), tokens.size, sp.rank), np.float32)
                oracle.shrink(xb, [workloads.bf16_bits(a) for a in L.lora_a], buf, m[tokens], sp.scale,
                              wl.spec.max_loras, nthreads=cores)
            y = np.ascontiguousarray(workloads.bf16_bits(L.y0)[tokens])
            bias = None if L.bias is None else [workloads.bf16_bits(b) for b in L.bias]
            oracle.expand(buf, [workloads.bf16_bits(b) for b in L.lora_b], bias, y, m[tokens],
                          wl.spec.max_loras, add_inputs=True, nthreads=cores)

    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(n, size=min(n, 4 * cores), replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    run(probe)
    per_tok = (time.perf_counter() - t0) / probe.size
    k = int(min(n, max(probe.size, budget_s / max(per_tok, 1e-9))))
    tokens = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)
    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while True:
        run(tokens)
        reps += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s or reps >= 100000 or k < n:
            break
    sample = ("%d of %d tokens (seeded uniform sample), prepare on the full mapping, %d pass(es)"
              % (k, n, reps)) if k < n else ("the full batch of %d tokens, %d pass(es)" % (n, reps))
    return {"value": k * reps / elapsed, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": sample, "seconds": round(elapsed, 2)}


def summarize_pmc(workload: str, fetch_csv: str, write_csv: str, out_json: str, command: str) -> None:
    """Per-dispatch HBM traffic of each lora kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), scaled by what the same
    counters read for a plain 256 MiB device copy in the same run."""
    import csv
    import collections

    import workloads
    specs = workloads.WORKLOADS[workload].layers
    # layers issuing a kernel of each kind, in the order a step issues them
    layers_of = {"shrink": [i for i, L in enumerate(specs) if not L.expand_only],
                 "expand": list(range(len(specs))), "prepare": [0], "preplinear": [0], "copy": [0]}
    # the default path's later layers call lora_shrink_expand
    layers_of["linear"] = [i for i in layers_of["shrink"] if i > 0] or [0]

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        if rows and "Dispatch_Id" in rows[0]:
            rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = collections.defaultdict(list)
        seen = collections.Counter()
        for r in rows:
            name = r["Kernel_Name"]
            kind = ("prepare" if "prepare_kernel" in name else
                    "shrink" if ("shrink_kernel" in name or "shrink_lds_kernel" in name) else
                    "expand" if "expand_kernel" in name else
                    ("preplinear" if "true>" in name.split(",")[-1] else "linear")
                    if ("fused_kernel" in name or "lora_major_kernel" in name) else
                    "copy" if ("copyBuffer" in name or "elementwise" in name or "copy" in name.lower()) else None)
            if kind:
                lays = layers_of[kind]
                li = lays[seen[kind] % len(lays)]   # the k-th dispatch of a kind belongs to layer k mod count
                seen[kind] += 1
                key = kind if kind in ("prepare", "copy") else "%s%d" % (kind, li)
                vals[key].append(float(r["Counter_Value"]) * 1024.0)
        return vals

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(256 << 20)
    # the copy kernel is the largest-traffic dispatch of the copy kind
    cf = max(f["copy"]) if f.get("copy") else None
    cw = max(w["copy"]) if w.get("copy") else None
    fscale = copy_bytes / cf if cf else 1.0
    wscale = copy_bytes / cw if cw else 1.0
    rec = {"workload": workload, "kernel_hash": kernel_source_hash(), "command": command,
           "copy_fetch_scale": fscale, "copy_write_scale": wscale, "traffic_bytes": {}, "raw": {}}
    for k in sorted(f):
        if k != "copy" and w.get(k):
            fb = sum(f[k]) / len(f[k])
            wb = sum(w[k]) / len(w[k])
            rec["raw"][k] = {"fetch_bytes": fb, "write_bytes": wb, "dispatches": len(f[k])}
            rec["traffic_bytes"][k] = round(fb * fscale + wb * wscale)
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def summarize_mfma(workload: str, pmc_csv: str, out_md: str, command: str) -> None:
    """MFMA use per lora kernel from one rocprofv3 --pmc run of
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA operations / 512),
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (both summed over the
    device's instances; GRBM_GUI_ACTIVE over its 8 XCDs), next to the
    algorithmic flops of the shrink (2*T*H*S*r) and expand (2*T*r*O, twice:
    the buffer enters as bf16 hi and lo parts)."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(pmc_csv)):
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        if name.startswith("lora::"):
            vals[name[len("lora::"):]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    import workloads
    wl = workloads.make_workload(workload)
    ta = int((wl.mapping.numpy() >= 0).sum())
    sp = wl.layers[0].spec
    algo = {"shrink": 2.0 * ta * sp.hidden * len(sp.slices) * sp.rank,
            "expand": 2.0 * 2 * ta * sp.rank * sum(sp.slices)}
    lines = ["# MFMA use: %s workload" % workload, "", "Command:", "", "    " + command, "",
             "| kernel | dispatches | MFMA bf16 GFLOP | algorithmic GFLOP | MFMA busy % of SIMD cycles |",
             "|---|---|---|---|---|"]
    for k, v in sorted(vals.items()):
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0.0])
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", [0.0])
        gui = v.get("GRBM_GUI_ACTIVE", [1.0])
        flops = 512.0 * sum(mops) / len(mops)
        util = 100.0 * (sum(busy) / len(busy)) / ((sum(gui) / len(gui)) / 8.0 * 1024.0)
        kind = "shrink" if "shrink" in k else "expand" if "expand" in k else None
        lines.append("| %s | %d | %.3f | %s | %.1f |" % (k, len(mops), flops / 1e9,
                     "%.3f" % (algo[kind] / 1e9) if kind else "-", util))
    lines += ["", "MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
              "the run is a short eager profile under the counter collector, so its cycle counts "
              "include the collector's overhead."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def one_launch(wl, li: int, with_prepare: bool) -> bool:
    """Whether lora_shrink_expand (or lora_prepare_shrink_expand) runs layer
    li in one launch; outside that range the call makes the separate calls.
    The library answers (host only, no device work)."""
    import segmented_gather_lora_amd as sgl
    n = wl.mapping.numel()
    sp = wl.layers[li].spec
    if n < 1:
        return False
    return sgl.lora_shrink_expand_launches(n, wl.spec.max_loras, len(sp.slices), sp.rank, with_prepare) == 1


def summarize_stats(workload: str, stats_csv: str, out_md: str, command: str) -> None:
    """Markdown table of a rocprofv3 --kernel-trace --stats summary
    (kernel_stats.csv): calls and durations per kernel."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel statistics: %s workload" % workload, "", "Command:", "", "    " + command, "",
             "kernel_hash: " + kernel_source_hash(), "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "").replace("|", "/")
        if name.endswith(")") and "(" in name:   # drop the parameter list
            name = name[:name.rindex("(")]
        lines.append("| %s | %s | %.3f | %.3f | %.3f | %.1f |" % (
            name[:80], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic(workload: str, kernel: str):
    path = os.path.join(ROOT, "profiles", "pmc_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes", {}).get(kernel)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python (no HIP graph)")
    ap.add_argument("--path", choices=("prepare_fused", "fused", "separate"), default="prepare_fused",
                    help="prepare_fused: lora_prepare_shrink_expand for the first layer, lora_shrink_expand for "
                         "the others; fused: lora_prepare_meta, then lora_shrink_expand per layer; separate: "
                         "lora_prepare_meta, then lora_shrink and lora_expand per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate through (0 = auto)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many eager steps and a 256 MiB calibration copy, then exit (counter runs)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON", "COMMAND"),
                    help="write the per-kernel traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "OUT_MD", "COMMAND"),
                    help="write the kernel statistics of one rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_CSV", "OUT_MD", "COMMAND"),
                    help="write the per-kernel MFMA use of one rocprofv3 --pmc run and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc)
        return
    if args.summarize_stats:
        summarize_stats(args.workload, *args.summarize_stats)
        return
    if args.summarize_mfma:
        summarize_mfma(args.workload, *args.summarize_mfma)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from segmented_gather_lora_amd import _build
    _build.ensure_built()
    import segmented_gather_lora_amd  # noqa: F401
    import workloads

    torch.cuda.set_device(0)
    wl = workloads.make_workload(args.workload)
    n = wl.mapping.numel()
    ab = algorithmic_bytes(wl)
    sb = set_bytes(wl)
    if args.rotate:
        rotate = args.rotate
    else:
        rotate = max(1, math.ceil((1 << 30) / sb)) if sb < LLC_BYTES else 1
    print("# workload %s: N=%d, %.1f MB per input set, rotating %d set(s)" % (args.workload, n, sb / 1e6, rotate),
          file=sys.stderr, flush=True)
    first = DeviceSet(wl)
    sets = [first] + [DeviceSet(wl, src=first) for _ in range(rotate - 1)]
    nl = len(wl.layers)

    # warm-up (eager; loads the code objects), then capture one step per set
    path = args.path
    for i in range(max(args.warmup, rotate)):
        sets[i % rotate].step(path)
    torch.cuda.synchronize()

    if args.profile_steps:
        # short eager run for hardware-counter collection, plus a plain copy
        # of known size that calibrates the byte counters
        for i in range(args.profile_steps):
            sets[i % rotate].step(path)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("# profile run done", file=sys.stderr)
        return

    steps = max(args.steps // rotate, 1) * rotate
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            sets[i % rotate].step(path)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        g = capture(lambda: [s.step(path) for s in sets])
        for _ in range(max(1, args.warmup // rotate)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps // rotate):
            g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / steps
    value = n * steps / elapsed
    print("# timed %d steps in %.3f s" % (steps, elapsed), file=sys.stderr, flush=True)

    # per-kernel average durations: graphs of >= 32 launches of one kernel kind
    # cycling over the input sets (graph launch overhead amortised)
    launches = max(32, rotate)
    reps = max(2, 400 // launches)

    def per_launch(fn):
        g1 = capture(lambda: [fn(sets[i % rotate]) for i in range(launches)])
        g1.replay()
        return time_graph(g1, reps) / launches

    kern = {"prepare": per_launch(lambda s: s.prepare())}
    for li in range(nl):
        if not wl.layers[li].spec.expand_only:
            kern["shrink%d" % li] = per_launch(lambda s: s.shrink(li))
            kern["linear%d" % li] = per_launch(lambda s: s.linear(li))
        kern["expand%d" % li] = per_launch(lambda s: s.expand(li))
    if not wl.layers[0].spec.expand_only:
        kern["preplinear0"] = per_launch(lambda s: s.prepare_linear(0))
    torch.cuda.synchronize()
    bytes_of = {"prepare": ab["prepare"]}
    for li in range(nl):
        if not wl.layers[li].spec.expand_only:
            bytes_of["shrink%d" % li] = ab["shrink"][li]
            bytes_of["linear%d" % li] = ab["shrink"][li] + ab["expand"][li]
        bytes_of["expand%d" % li] = ab["expand"][li]
    if "preplinear0" in kern:
        bytes_of["preplinear0"] = ab["prepare"] + ab["shrink"][0] + ab["expand"][0]
    # the calls the timed step makes
    used = []
    for li in range(nl):
        if wl.layers[li].spec.expand_only:
            used.append("expand%d" % li)
        elif li == 0 and path == "prepare_fused":
            used.append("preplinear0")
        elif path in ("fused", "prepare_fused"):
            used.append("linear%d" % li)
        else:
            used += ["shrink%d" % li, "expand%d" % li]
    if "preplinear0" not in used:
        used.insert(0, "prepare")
    # A one-launch call outside its range runs as its separate kernels; the
    # roofline is then taken on the slowest of those kernels, not on the call.
    kernels = []
    for k in used:
        if k.startswith(("linear", "preplinear")) and not one_launch(wl, int(k[-1]), k.startswith("prep")):
            kernels += ["shrink%s" % k[-1], "expand%s" % k[-1]]
        else:
            kernels.append(k)
    dom = max((k for k in kernels if k != "prepare"), key=lambda k: kern[k])
    achieved = bytes_of[dom] / (kern[dom] * 1e-3) / 1e9
    kname = {"shrink": "lora_shrink", "expand": "lora_expand", "linear": "lora_shrink_expand",
             "prepli": "lora_prepare_shrink_expand"}[dom[:6]]
    if dom[:6] in ("shrink", "expand") and dom not in used:
        kname += " (in %s)" % ("lora_prepare_shrink_expand" if "preplinear0" in used and dom.endswith("0")
                               else "lora_shrink_expand")
    traffic = load_traffic(args.workload, dom)
    separate = [k for k in kern if k[:6] in ("shrink", "expand")]
    se_ms = sum(kern[k] for k in separate)
    se_bytes = sum(bytes_of[k] for k in separate)
    calls_ms = sum(kern[k] for k in used)
    calls_bytes = sum(bytes_of[k] for k in used)

    # a plain 256 MiB device-to-device copy, timed with events on the current
    # stream: the read + write bandwidth a simple streaming kernel reaches here
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = torch.cuda.current_stream()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    copies = 5
    c0.record(st)
    for _ in range(copies):
        dst.copy_(src)
    c1.record(st)
    c1.synchronize()
    copy_gbps = 2.0 * src.numel() * copies / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    spec = wl.spec
    layers_cfg = [{"hidden": L.spec.hidden, "slices": list(L.spec.slices), "rank": L.spec.rank,
                   "scale": L.spec.scale, "bias": L.bias is not None, "expand_only": L.spec.expand_only}
                  for L in wl.layers]
    parts = []
    for li, L in enumerate(wl.layers):
        if L.spec.expand_only:
            parts.append("expand")
        elif li == 0 and path == "prepare_fused":
            parts.append("prepare_shrink_expand")
        else:
            parts.append("shrink_expand" if path != "separate" else "shrink + expand")
    step_desc = ("" if "preplinear0" in used else "prepare + ") + " + ".join(parts)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "num_tokens": n, "max_loras": spec.max_loras, "layers": layers_cfg,
                   "active_tokens": ab["T_a"], "active_loras": ab["L_a"], "parallelism": "none",
                   "launch": "eager" if args.eager else "hip_graph", "input_sets_rotated": rotate,
                   "step": step_desc},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": bytes_of[dom], "avg_us": round(kern[dom] * 1e3, 3),
                     "measured_copy_GBps": round(copy_gbps, 1), "frac_of_copy": round(achieved / copy_gbps, 4)},
        "kernels_us": {k: round(v * 1e3, 3) for k, v in kern.items()},
        "step_calls": {"path": args.path, "us": round(calls_ms * 1e3, 3),
                        "tokens_per_s": round(n / (calls_ms * 1e-3), 1),
                        "GBps": round(calls_bytes / (calls_ms * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(calls_bytes / (calls_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "shrink_expand": {"us": round(se_ms * 1e3, 3), "tokens_per_s": round(n / (se_ms * 1e-3), 1),
                          "GBps": round(se_bytes / (se_ms * 1e-3) / 1e9, 1),
                          "frac_of_peak": round(se_bytes / (se_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
