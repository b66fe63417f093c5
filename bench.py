"""Benchmark of the segmented-gather multi-LoRA hot path on one MI355X.

One step = one batch through the whole path on seeded synthetic inputs that
are already resident in HBM: the batch's metadata (LoRAKernelMeta.prepare_tensors)
and, per layer, PunicaWrapperGPU.add_lora_linear -- shrink into a fresh fp32
buffer, then expand into y with add_inputs -- made as lora_prepare_shrink_expand
for the first layer and lora_shrink_expand for the others (one launch for
decode-like batches, the separate kernels otherwise).  Those calls write the
buffer as a fresh one ("="), so a step needs no clearing pass.

The headline line is the largest configuration, ``large`` (N=16384 tokens,
H=8192, r=128, 128 LoRAs, q/k/v slices 8192/1024/1024), timed for exactly
``--steps`` steps after ``--warmup`` untimed ones.  The same run adds one
record per other workload (decode, prefill, Zipf per layer, the all -1 batch,
logits, embedding), each timed over about ``--sub-ms`` milliseconds, and the
practical ceilings of this part: a 256 MiB device copy, a streaming read of
each workload's step bytes, and an empty launch.

Cold caches: when one input set fits in the 256 MB last-level cache, the
bench rotates through enough independent copies (>= 1 GiB in total) that
every step reads data that is not cache resident.  Steps are replayed from HIP
graphs (``--eager`` launches every call from Python instead).

Prints ONE JSON line.  ``roofline`` refers to the kernel with the largest
average duration in the timed step; durations are measured with HIP events on
the stream the kernels run on, over graph replays of one call at a time.
``traffic`` comes from committed rocprofv3 PMC summaries (profiles/) when
their kernel source hash matches the current sources.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import math
import os
import shlex
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA shrink+expand tokens/sec at 1 GPU; achieved HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20
HEADLINE = "large"
SUBS = ("decode", "prefill", "zipf", "large_nolora", "logits", "embedding")
PROBE_WG = 2048          # workgroups of the streaming-read probe
EMPTY_WG = 1024          # workgroups of the empty-launch probe (the decode kernel's grid)


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per launch: inputs and outputs of active
    tokens and active LoRAs only (each x row once, each active LoRA's weights
    once per call).  The linear calls write the fp32 buffer once (a fresh
    buffer) and the expand reads it once; lora_shrink on its own reads and
    writes it ("+=").  The metadata: the mapping read, the id copy and the
    sorted indices written (12 B per token)."""
    import numpy as np
    m = wl.mapping.numpy()
    n = m.size
    act = m[m >= 0]
    ta, la = int(act.size), int(np.unique(act).size)
    out = {"prepare": 12 * n, "shrink": [], "shrink_fresh": [], "expand": [], "T_a": ta, "L_a": la}
    for L in wl.layers:
        sp = L.spec
        S, r, H, O = len(sp.slices), sp.rank, sp.hidden, sum(sp.slices)
        base = 0 if sp.expand_only else 2 * ta * H + 2 * la * S * r * H
        out["shrink"].append(0 if sp.expand_only else base + 8 * S * ta * r)
        out["shrink_fresh"].append(0 if sp.expand_only else base + 4 * S * ta * r)
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


# ------------------------------------------------------------------ dispatch plan

class Plan:
    """The library calls a run makes, in order, with the kinds of the kernels
    each launches (from the library's own launch-count queries): rocprofv3's
    kernel trace is matched against it to give per-workload, per-layer
    durations."""

    def __init__(self):
        self.calls = []          # [workload, phase, tag, kernel kinds, times]
        self.phase = "setup"
        self.workload = ""

    def add(self, tag: str, kinds, times: int = 1):
        kinds = list(kinds)
        if self.calls and self.calls[-1][:4] == [self.workload, self.phase, tag, kinds]:
            self.calls[-1][4] += times
        else:
            self.calls.append([self.workload, self.phase, tag, kinds, times])

    def replay(self, seq, times: int):
        """A captured sequence of (tag, kinds) replayed `times` times."""
        for _ in range(times):
            for tag, k in seq:
                self.add(tag, k)

    def dump(self, path: str):
        with open(path, "w") as fh:
            json.dump({"calls": self.calls}, fh)


PLAN = Plan()


class DeviceSet:
    """One independent copy of the workload's inputs in HBM."""

    def __init__(self, wl, src=None):
        import torch
        import segmented_gather_lora_amd as sgl
        n = wl.mapping.numel()
        self.wl = wl
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
        PLAN.add("prepare", prepare_kinds(self.n, self.wl.spec.max_loras))

    def shrink(self, li):
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_shrink(d["x"], d["a"], d["buf"], self.meta, d["scale"])
        PLAN.add("shrink%d" % li, ["shrink"])

    def expand(self, li):
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_expand(d["buf"], d["b"], d["bias"], d["y"], self.meta, offset_start=0, add_inputs=True)
        PLAN.add("expand%d" % li, ["expand"])

    def linear(self, li):
        """add_lora_linear of one layer: one lora_shrink_expand call."""
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_shrink_expand(d["x"], d["a"], d["b"], d["bias"], d["buf"], d["y"], self.meta, d["scale"],
                               offset_start=0, add_inputs=True)
        PLAN.add("linear%d" % li, call_kinds(self.wl, li, False))

    def prepare_linear(self, li):
        """prepare + add_lora_linear of one layer: one lora_prepare_shrink_expand call."""
        import segmented_gather_lora_amd as sgl
        d = self.layers[li]
        sgl.lora_prepare_shrink_expand(self.mapping, d["x"], d["a"], d["b"], d["bias"], d["buf"], d["y"], self.meta,
                                       d["scale"], offset_start=0, add_inputs=True)
        PLAN.add("preplinear%d" % li, call_kinds(self.wl, li, True))

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
                # the separate calls, with the fresh buffer cleared in the step
                self.layers[li]["buf"].zero_()
                self.shrink(li)
                self.expand(li)


def launches(wl, li: int, with_prepare: bool) -> int:
    """Kernel launches of lora_shrink_expand (lora_prepare_shrink_expand) for
    layer li: the library answers (host only, no device work)."""
    import segmented_gather_lora_amd as sgl
    n = wl.mapping.numel()
    sp = wl.layers[li].spec
    if n < 1:
        return 0
    return sgl.lora_shrink_expand_launches(n, wl.spec.max_loras, sp.hidden, len(sp.slices), sp.rank, with_prepare)


def one_launch(wl, li: int, with_prepare: bool) -> bool:
    return launches(wl, li, with_prepare) == 1


def prepare_kinds(n: int, max_loras: int):
    """Kernels of lora_prepare_meta for n tokens: one sorting launch, or the
    rank and place launches of the several-workgroup sort."""
    import segmented_gather_lora_amd as sgl
    return ["prepare"] if sgl.lora_prepare_meta_launches(n, max_loras) == 1 else ["prepare_rank", "prepare_place"]


def call_kinds(wl, li: int, with_prepare: bool):
    """Kernels of lora_shrink_expand (lora_prepare_shrink_expand) for layer li,
    in launch order."""
    if launches(wl, li, with_prepare) == 1:
        return ["one_launch"]
    zero = ["zero"] if launches(wl, li, False) == 3 else []
    return (prepare_kinds(wl.mapping.numel(), wl.spec.max_loras) if with_prepare else []) + zero + ["shrink", "expand"]


def cold_sets(call_bytes: int, set_bytes_: int) -> int:
    """Input sets a call cycles over when it is timed on its own: enough that
    twice the last-level cache streams between two uses of one set (at least
    two sets; at most 64 or 16 GiB of sets)."""
    need = 1 + math.ceil(2 * LLC_BYTES / max(call_bytes, 1))
    cap = max(2, min(64, (16 << 30) // max(set_bytes_, 1)))
    return max(2, min(cap, need))


def set_bytes(wl) -> int:
    tot = wl.mapping.numel() * 4
    for L in wl.layers:
        tot += L.x.numel() * L.x.element_size() + L.y0.numel() * 2
        tot += sum(t.numel() for t in L.lora_a) * 2 + sum(t.numel() for t in L.lora_b) * 2
        if not L.spec.expand_only:
            tot += 4 * len(L.spec.slices) * wl.mapping.numel() * L.spec.rank
    return tot


def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    saved = PLAN.phase
    PLAN.phase = "capture"          # capture records launches; nothing runs
    n0 = len(PLAN.calls)
    with torch.cuda.graph(g, stream=s):
        fn()
    seq = [(c[2], c[3]) for c in PLAN.calls[n0:] for _ in range(c[4])]
    del PLAN.calls[n0:]
    PLAN.phase = saved
    torch.cuda.current_stream().wait_stream(s)
    return g, seq


def time_graph(g, seq, replays: int) -> float:
    """Average ms per replay, HIP events on the replay stream."""
    import torch
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    e1.synchronize()
    PLAN.replay(seq, replays)
    return e0.elapsed_time(e1) / replays


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(wl, budget_s: float) -> dict:
    """The oracle, as it is, on this host: prepare on the full mapping, then
    shrink + expand of every layer on a bounded, seeded sample of the
    workload's tokens; once on one thread and once on every core this process
    may run on (len(os.sched_getaffinity(0)), stated)."""
    import numpy as np
    import oracle
    import workloads
    cores = len(os.sched_getaffinity(0))
    m = wl.mapping.numpy()
    n = m.size
    bits = {}
    for li, L in enumerate(wl.layers):
        bits[li] = dict(x=None if L.spec.expand_only else workloads.bf16_bits(L.x),
                        a=[workloads.bf16_bits(a) for a in L.lora_a], b=[workloads.bf16_bits(b) for b in L.lora_b],
                        bias=None if L.bias is None else [workloads.bf16_bits(b) for b in L.bias],
                        y=workloads.bf16_bits(L.y0))

    def run(tokens, threads):
        oracle.prepare(m, wl.spec.max_loras)
        for li, L in enumerate(wl.layers):
            sp, bb = L.spec, bits[li]
            if sp.expand_only:
                buf = np.ascontiguousarray(L.x.numpy()[:, tokens])
            else:
                buf = np.zeros((len(sp.slices), tokens.size, sp.rank), np.float32)
                oracle.shrink(bb["x"][tokens], bb["a"], buf, m[tokens], sp.scale, wl.spec.max_loras, nthreads=threads)
            y = np.ascontiguousarray(bb["y"][tokens])
            oracle.expand(buf, bb["b"], bb["bias"], y, m[tokens], wl.spec.max_loras, add_inputs=True,
                          nthreads=threads)

    def leg(threads, seed):
        rng = np.random.default_rng(seed)
        probe = np.sort(rng.choice(n, size=min(n, 2 * threads), replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        run(probe, threads)
        per_tok = (time.perf_counter() - t0) / probe.size
        k = int(min(n, max(probe.size, 0.8 * budget_s / max(per_tok, 1e-9))))
        tokens = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        run(tokens, threads)
        el = time.perf_counter() - t0
        return k, el

    k1, e1 = leg(1, 0)
    kn, en = leg(cores, 1)
    return {"value": round(kn / en, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d tokens (seeded uniform sample) through shrink + expand of every layer, "
                      "prepare on the full mapping; %d threads" % (kn, n, cores),
            "seconds": round(en, 2),
            "single_thread": {"value": round(k1 / e1, 1), "unit": "tokens/s", "cores": 1,
                              "sample": "%d of %d tokens" % (k1, n), "seconds": round(e1, 2)}}


# ------------------------------------------------------------------ rocprofv3 summaries

def _kind_of(name: str):
    if "prepare_kernel" in name:
        return "prepare"
    if "prepare_rank_kernel" in name:
        return "prepare_rank"
    if "prepare_place_kernel" in name:
        return "prepare_place"
    if "zero_rows_kernel" in name:
        return "zero"
    if "shrink_kernel" in name or "shrink_lds_kernel" in name or "shrink_sk_kernel" in name:
        return "shrink"
    if "expand_kernel" in name:
        return "expand"
    if "fused_kernel" in name or "lora_major_kernel" in name:
        return "one_launch"
    if "probe_read_kernel" in name:
        return "probe_read"
    if "probe_empty_kernel" in name:
        return "probe_empty"
    return None


def summarize_trace(trace_csv: str, plan_json: str, out_md: str, command: str) -> dict:
    """Per-workload, per-layer kernel durations from one rocprofv3
    --kernel-trace run of bench.py --dispatch-plan: the library's dispatches,
    in dispatch order, are matched one by one against the calls bench made."""
    import csv
    rows = [r for r in csv.DictReader(open(trace_csv)) if _kind_of(r["Kernel_Name"])]
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Start_Timestamp"
    rows.sort(key=lambda r: int(r[key]))
    plan = json.load(open(plan_json))["calls"]
    expect = []
    for wl, phase, tag, kinds, times in plan:
        for _ in range(times):
            for kind in kinds:
                expect.append((wl, phase, tag, kind))
    if len(expect) != len(rows):
        raise SystemExit("trace has %d library dispatches, the plan %d" % (len(rows), len(expect)))
    stats = collections.defaultdict(list)
    names = {}
    for (wl, phase, tag, kind), r in zip(expect, rows):
        got = _kind_of(r["Kernel_Name"])
        if got != kind:
            raise SystemExit("dispatch %s: expected a %s kernel for %s/%s, trace has %s"
                             % (r[key], kind, wl, tag, r["Kernel_Name"][:80]))
        if phase not in ("timed", "per_call"):
            continue
        layer = "".join(ch for ch in tag if ch.isdigit())
        label = kind if kind.startswith(("prepare", "probe")) else "%s%s" % (kind, layer)
        k2 = (wl, phase, tag, label)
        stats[k2].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        names[k2] = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    lines = ["# rocprofv3 kernel trace by workload and layer", "", "Command:", "", "    " + command, "",
             "kernel_hash: " + kernel_source_hash(), "",
             "Library dispatches matched one by one, in dispatch order, with the calls bench.py made "
             "(its --dispatch-plan).  `timed`: the timed steps; `per_call`: graphs of one call at a time, "
             "whose HIP-event average is bench's `kernels_us`.", "",
             "| workload | phase | call | kernel | dispatches | average us | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    out = {}
    for k2 in sorted(stats):
        v = stats[k2]
        avg = sum(v) / len(v) / 1e3
        lines.append("| %s | %s | %s | %s %s | %d | %.3f | %.3f | %.3f |" % (
            k2[0], k2[1], k2[2], k2[3], names[k2][:60], len(v), avg, min(v) / 1e3, max(v) / 1e3))
        out["%s/%s/%s/%s" % k2] = round(avg, 3)
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return out


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    """Markdown table of a rocprofv3 --kernel-trace --stats summary
    (kernel_stats.csv): calls and durations per kernel name, over the whole
    run (every workload that launches the kernel)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "    " + command, "",
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


def summarize_pmc(workload: str, fetch_csv: str, write_csv: str, out_json: str, command: str) -> None:
    """Per-dispatch HBM traffic of each lora kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch) of bench.py
    --profile-steps, scaled by what the same counters read for a plain
    256 MiB device copy in the same run.  Dispatches are attributed to layers
    in dispatch order: the k-th dispatch of a kind in a step belongs to the
    k-th layer that issues that kind."""
    import csv
    import workloads
    specs = workloads.WORKLOADS[workload].layers
    layers_of = {"shrink": [i for i, L in enumerate(specs) if not L.expand_only],
                 "expand": list(range(len(specs))), "prepare": [0], "prepare_rank": [0], "prepare_place": [0],
                 "preplinear": [0], "copy": [0]}
    layers_of["linear"] = [i for i in layers_of["shrink"] if i > 0] or [0]
    # the zeroing of buf's rows runs only for layers whose call splits the shrink over K
    wl = workloads.make_workload(workload)
    layers_of["zero"] = [i for i in layers_of["shrink"] if launches(wl, i, False) == 3] or [0]

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        if rows and "Dispatch_Id" in rows[0]:
            rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = collections.defaultdict(list)
        seen = collections.Counter()
        for r in rows:
            name = r["Kernel_Name"]
            kind = _kind_of(name)
            if kind == "one_launch":
                kind = "preplinear" if "true>" in name.split(",")[-1] else "linear"
            elif kind is None and ("copyBuffer" in name or "elementwise" in name or "copy" in name.lower()):
                kind = "copy"
            if kind in layers_of:
                lays = layers_of[kind]
                li = lays[seen[kind] % len(lays)]
                seen[kind] += 1
                key = kind if kind.startswith("prepare") or kind == "copy" else "%s%d" % (kind, li)
                vals[key].append(float(r["Counter_Value"]) * 1024.0)
        return vals

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(256 << 20)
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
    """MFMA and VALU use per lora kernel from one rocprofv3 --pmc run of
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA operations / 512),
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU and GRBM_GUI_ACTIVE (summed over
    the device's instances; GRBM_GUI_ACTIVE over its 8 XCDs), next to the
    algorithmic flops of the shrink (2*T*H*S*r) and expand (2*T*r*O, twice:
    the buffer enters as bf16 hi and lo parts)."""
    import csv
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
    algo["one_launch"] = algo["shrink"] + algo["expand"]
    lines = ["# MFMA and VALU use: %s workload" % workload, "", "Command:", "", "    " + command, "",
             "kernel_hash: " + kernel_source_hash(), "",
             "| kernel | dispatches | MFMA bf16 GFLOP | algorithmic GFLOP | MFMA busy % of SIMD cycles | "
             "VALU instructions (M) |", "|---|---|---|---|---|---|"]
    for k, v in sorted(vals.items()):
        def avg(c, d=0.0):
            x = v.get(c, [d])
            return sum(x) / len(x)
        flops = 512.0 * avg("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        gui = avg("GRBM_GUI_ACTIVE", 1.0)
        util = 100.0 * avg("SQ_VALU_MFMA_BUSY_CYCLES") / (gui / 8.0 * 1024.0)
        kind = _kind_of(k)
        lines.append("| %s | %d | %.3f | %s | %.1f | %s |" % (
            k, len(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])), flops / 1e9,
            "%.3f" % (algo[kind] / 1e9) if kind in algo else "-", util,
            "%.2f" % (avg("SQ_INSTS_VALU") / 1e6) if "SQ_INSTS_VALU" in v else "-"))
    lines += ["", "MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
              "the run is a short eager profile under the counter collector, so its cycle counts "
              "include the collector's overhead."]
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


# ------------------------------------------------------------------ measurement

def copy_gbps() -> float:
    """A plain 256 MiB device-to-device copy (read + write bytes per second)."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = torch.cuda.current_stream()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(st)
    for _ in range(5):
        dst.copy_(src)
    c1.record(st)
    c1.synchronize()
    return 2.0 * src.numel() * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9


def probe_read(nbytes: int, copies: int) -> dict:
    """Streaming-read probe over `copies` rotated buffers of nbytes each (cold
    reads when the set exceeds the last-level cache): average us per launch
    and GB/s, replayed from a HIP graph like the step."""
    import torch
    import segmented_gather_lora_amd as sgl
    nbytes = max(16, nbytes // 16 * 16)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(PROBE_WG, dtype=torch.float32, device="cuda")

    def run():
        for b in bufs:
            sgl.lora_probe_read(b, PROBE_WG, sink)
            PLAN.add("probe_read", ["probe_read"])
    run()
    g, seq = capture(run)
    g.replay()
    PLAN.replay(seq, 1)
    reps = max(2, int(math.ceil(50e-3 / max(1e-6, nbytes * copies / 5e12))))
    ms = time_graph(g, seq, reps) / copies
    del bufs
    return {"us": round(ms * 1e3, 3), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes,
            "workgroups": PROBE_WG}


def probe_empty() -> float:
    import segmented_gather_lora_amd as sgl

    def run():
        for _ in range(64):
            sgl.lora_probe_empty(EMPTY_WG)
            PLAN.add("probe_empty", ["probe_empty"])
    run()
    g, seq = capture(run)
    g.replay()
    PLAN.replay(seq, 1)
    return time_graph(g, seq, 10) / 64 * 1e3


def run_workload(name: str, args, steps: int | None, warmup: int, sub_ms: float) -> dict:
    """Time one workload: `steps` steps exactly (None: about sub_ms of steps),
    then one call at a time for the per-kernel durations."""
    import torch
    import workloads
    PLAN.workload = name
    PLAN.phase = "setup"
    wl = workloads.make_workload(name)
    n = wl.mapping.numel()
    ab = algorithmic_bytes(wl)
    sb = set_bytes(wl)
    rotate = args.rotate or (max(1, math.ceil((1 << 30) / sb)) if sb < LLC_BYTES else 1)
    print("# %s: N=%d, %.1f MB per input set, rotating %d set(s)" % (name, n, sb / 1e6, rotate),
          file=sys.stderr, flush=True)
    first = DeviceSet(wl)
    sets = [first] + [DeviceSet(wl, src=first) for _ in range(rotate - 1)]
    nl = len(wl.layers)
    path = args.path

    PLAN.phase = "warmup"
    for i in range(max(warmup, rotate)):
        sets[i % rotate].step(path)
    torch.cuda.synchronize()

    if args.profile_steps:
        PLAN.phase = "profile"
        for i in range(args.profile_steps):
            sets[i % rotate].step(path)
        torch.cuda.synchronize()
        return {}

    # a graph holds per_graph steps cycling over the sets (at least 16 steps,
    # a multiple of the rotation); a second graph holds the remainder, so the
    # timed region is exactly `steps` steps
    per_graph = rotate * max(1, math.ceil(16 / rotate))
    if args.eager:
        steps = steps or 200
        torch.cuda.synchronize()
        PLAN.phase = "timed"
        t0 = time.perf_counter()
        for i in range(steps):
            sets[i % rotate].step(path)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        g, seq = capture(lambda: [sets[i % rotate].step(path) for i in range(per_graph)])
        PLAN.phase = "warmup"
        g.replay()
        PLAN.replay(seq, 1)
        torch.cuda.synchronize()
        if steps is None:   # about sub_ms of steps, in whole graphs
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            PLAN.replay(seq, 1)
            est = (time.perf_counter() - t0) / per_graph
            steps = per_graph * max(1, int(math.ceil(sub_ms * 1e-3 / max(est, 1e-7) / per_graph)))
        full, rem = divmod(steps, per_graph)
        gr = sr = None
        if rem:
            gr, sr = capture(lambda: [sets[i % rotate].step(path) for i in range(rem)])
            gr.replay()
            PLAN.replay(sr, 1)
        # the warmup steps once more, from the graph, right before the timed
        # region: the GPU idles during the captures above, and the first
        # replays after an idle stretch run slower than the ones after them
        for _ in range(max(1, math.ceil(warmup / per_graph))):
            g.replay()
            PLAN.replay(seq, 1)
        torch.cuda.synchronize()
        PLAN.phase = "timed"
        t0 = time.perf_counter()
        for _ in range(full):
            g.replay()
        if gr is not None:
            gr.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        PLAN.replay(seq, full)
        if gr is not None:
            PLAN.replay(sr, 1)
    ms_per_step = 1e3 * elapsed / steps
    print("# %s: timed %d steps in %.4f s" % (name, steps, elapsed), file=sys.stderr, flush=True)

    # per-call average durations: graphs of >= 32 launches of one call kind
    # cycling over enough input sets that a launch finds none of its inputs
    # in the last-level cache, as inside a step (which streams the other
    # calls' data in between)
    PLAN.phase = "per_call"
    pc_sets = {}
    reps = 2

    def per_call(fn, call_bytes, key):
        k = cold_sets(call_bytes, sb)
        while len(sets) < k:
            sets.append(DeviceSet(wl, src=first))
        pc_sets[key] = k
        ncalls = max(32, k)
        g1, s1 = capture(lambda: [fn(sets[i % k]) for i in range(ncalls)])
        g1.replay()
        PLAN.replay(s1, 1)
        # about 20 ms of replays right before the timed ones (the first
        # replays after the GPU has idled run slower), then about 20 ms timed
        n_rep = max(reps, math.ceil(20.0 / max(time_graph(g1, s1, 1), 1e-3)))
        for _ in range(n_rep):
            g1.replay()
        PLAN.replay(s1, n_rep)
        return time_graph(g1, s1, n_rep) / ncalls

    kern = {"prepare": per_call(lambda s: s.prepare(), ab["prepare"], "prepare")}
    for li in range(nl):
        if not wl.layers[li].spec.expand_only:
            kern["shrink%d" % li] = per_call(lambda s: s.shrink(li), ab["shrink"][li], "shrink%d" % li)
            kern["linear%d" % li] = per_call(lambda s: s.linear(li), ab["shrink_fresh"][li] + ab["expand"][li],
                                             "linear%d" % li)
        kern["expand%d" % li] = per_call(lambda s: s.expand(li), ab["expand"][li], "expand%d" % li)
    if not wl.layers[0].spec.expand_only:
        kern["preplinear0"] = per_call(lambda s: s.prepare_linear(0),
                                       ab["prepare"] + ab["shrink_fresh"][0] + ab["expand"][0], "preplinear0")
    torch.cuda.synchronize()

    bytes_of = {"prepare": ab["prepare"]}
    for li in range(nl):
        if not wl.layers[li].spec.expand_only:
            bytes_of["shrink%d" % li] = ab["shrink"][li]
            bytes_of["shrink_fresh%d" % li] = ab["shrink_fresh"][li]
            bytes_of["linear%d" % li] = ab["shrink_fresh"][li] + ab["expand"][li]
        bytes_of["expand%d" % li] = ab["expand"][li]
    if "preplinear0" in kern:
        bytes_of["preplinear0"] = ab["prepare"] + ab["shrink_fresh"][0] + ab["expand"][0]
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
    # A one-launch call outside its range runs as its separate kernels: the
    # roofline is then taken on the slowest of those kernels.
    kernels = []
    for k in used:
        if k.startswith(("linear", "preplinear")) and not one_launch(wl, int(k[-1]), k.startswith("prep")):
            kernels += ["shrink%s" % k[-1], "expand%s" % k[-1]]
        else:
            kernels.append(k)
    step_bytes = sum(bytes_of[k] for k in used)
    tokens_per_s = n / (ms_per_step * 1e-3)
    rec = {"workload": name, "num_tokens": n, "max_loras": wl.spec.max_loras,
           "active_tokens": ab["T_a"], "active_loras": ab["L_a"],
           "layers": [{"hidden": L.spec.hidden, "slices": list(L.spec.slices), "rank": L.spec.rank,
                       "scale": L.spec.scale, "bias": L.bias is not None, "expand_only": L.spec.expand_only}
                      for L in wl.layers],
           "input_sets_rotated": rotate, "per_call_input_sets": pc_sets, "steps": steps, "ms_per_step": round(ms_per_step, 5),
           "tokens_per_s": round(tokens_per_s, 1), "step_bytes": step_bytes,
           "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
           "step_frac_of_peak": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "kernels_us": {k: round(v * 1e3, 3) for k, v in kern.items()}}
    if ab["T_a"] == 0:
        rec["roofline"] = None   # the all -1 batch moves no data: launch-latency bound
    else:
        # the shrink of a linear call writes a fresh buffer: its bytes use the
        # write-only buffer term
        def kbytes(k):
            if k.startswith("shrink") and k not in used:
                return bytes_of["shrink_fresh" + k[6:]]
            return bytes_of[k]
        dom = max((k for k in kernels if k != "prepare"), key=lambda k: kern[k])
        achieved = kbytes(dom) / (kern[dom] * 1e-3) / 1e9
        kname = {"shrink": "lora_shrink", "expand": "lora_expand", "linear": "lora_shrink_expand",
                 "prepli": "lora_prepare_shrink_expand"}[dom[:6]]
        if dom[:6] in ("shrink", "expand") and dom not in used:
            kname += " (in %s)" % ("lora_prepare_shrink_expand" if "preplinear0" in used and dom.endswith("0")
                                   else "lora_shrink_expand")
        rec["roofline"] = {"bound": "hbm", "kernel": kname, "call": dom, "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": load_traffic(name, dom), "algorithmic_bytes": kbytes(dom),
                           "avg_us": round(kern[dom] * 1e3, 3)}
        # every kernel of the step against the peak
        rec["kernel_frac"] = {k: round(kbytes(k) / (kern[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                              for k in kernels if k != "prepare"}
    parts = []
    for li, L in enumerate(wl.layers):
        if L.spec.expand_only:
            parts.append("expand")
        elif li == 0 and path == "prepare_fused":
            parts.append("prepare_shrink_expand")
        else:
            parts.append("shrink_expand" if path != "separate" else "zero buf + shrink + expand")
    rec["step"] = ("" if "preplinear0" in used else "prepare + ") + " + ".join(parts)
    if not args.no_ceilings and ab["T_a"] > 0:
        rec["read_probe"] = probe_read(step_bytes, rotate)
        rec["frac_of_read_probe"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9 / rec["read_probe"]["GBps"], 4)
    del sets, first
    torch.cuda.empty_cache()
    rec["_wl"] = wl
    return rec


# LDS-staged shrink configurations the library defines (LORA_SHRINK_STAGED=1..)
STAGED_CFGS = 19


def sweep(name: str, what: str, out_md: str, grid=None, wl=None) -> None:
    """Time every tiling of one kernel on a full-size workload (the library's
    tuning overrides; each changes the tiling only, never the result): the
    LDS-staged shrink configurations x K splits and their stream-K forms, or
    the expand tile sizes x column-block run lengths and the share walk.
    Cold inputs, HIP-graph replays of one call."""
    import torch
    import workloads
    if wl is None:
        wl = workloads.make_workload(name)
    sb = set_bytes(wl)
    ab = algorithmic_bytes(wl)
    first = DeviceSet(wl)
    sets = [first]
    env = ("LORA_SHRINK_STAGED", "LORA_SHRINK_KSPLIT", "LORA_SHRINK_VARIANT", "LORA_SHRINK_SK",
           "LORA_EXPAND_TILE_TOKENS", "LORA_EXPAND_RUN", "LORA_EXPAND_SHARE")
    if grid is not None:
        grid = [dict(g) for g in grid]
    elif what == "shrink":
        # units of every staged configuration with 1-4 K chunks, and the stream-K form of each
        grid = [dict(LORA_SHRINK_SK="1", LORA_SHRINK_VARIANT="3", LORA_SHRINK_STAGED=str(c), LORA_SHRINK_KSPLIT=str(k))
                for c in range(1, STAGED_CFGS + 1) for k in (1, 2, 3, 4)]
        grid += [dict(LORA_SHRINK_SK="2", LORA_SHRINK_VARIANT="3", LORA_SHRINK_STAGED=str(c))
                 for c in range(1, STAGED_CFGS + 1)]
    else:
        # units of a run of column blocks, and equal shares of the block list
        grid = [dict(LORA_EXPAND_SHARE="2", LORA_EXPAND_TILE_TOKENS=str(t), LORA_EXPAND_RUN=str(r))
                for t in (16, 32, 64) for r in (1, 2, 4, 8, 16)]
        grid += [dict(LORA_EXPAND_SHARE="1", LORA_EXPAND_TILE_TOKENS=str(t)) for t in (16, 32, 64)]
    if {} not in grid:
        grid.append({})   # the automatic choice
    command = "python bench.py " + " ".join(shlex.quote(a) for a in sys.argv[1:])
    lines = ["# %s tilings: %s workload" % (what, name), "", "Command:", "", "    " + command, "",
             "kernel_hash: " + kernel_source_hash(), "",
             "us per launch (HIP events over about 20 ms of graph replays after about 20 ms of warm ones, "
             "cycling over enough input sets that a launch finds none of its inputs in the last-level cache); "
             "`auto` = the launcher's choice.", ""]
    for li, L in enumerate(wl.layers):
        if what == "shrink" and L.spec.expand_only:
            continue
        rotate = cold_sets(ab["shrink"][li] if what == "shrink" else ab["expand"][li], sb)
        while len(sets) < rotate:
            sets.append(DeviceSet(wl, src=first))
        for d in sets:
            d.prepare()
        torch.cuda.synchronize()
        n = max(8, rotate)
        res = []
        for g in grid:
            for k in env:
                os.environ.pop(k, None)
            os.environ.update(g)
            fn = (lambda d: d.shrink(li)) if what == "shrink" else (lambda d: d.expand(li))
            fn(sets[0])
            torch.cuda.synchronize()
            gr, seq = capture(lambda: [fn(sets[i % rotate]) for i in range(n)])
            gr.replay()
            PLAN.replay(seq, 1)
            # about 20 ms of replays right before the timed ones (the first
            # replays after the GPU has idled run slower), then about 20 ms timed
            reps = max(3, math.ceil(20.0 / max(time_graph(gr, seq, 1), 1e-3)))
            for _ in range(reps):
                gr.replay()
            PLAN.replay(seq, reps)
            us = time_graph(gr, seq, reps) / n * 1e3
            del gr
            label = " ".join("%s=%s" % (k[5:].lower(), v) for k, v in g.items() if k != "LORA_SHRINK_VARIANT") or "auto"
            res.append((us, label))
            print("# %s layer %d %s: %.2f us" % (what, li, label, us), file=sys.stderr, flush=True)
        for k in env:
            os.environ.pop(k, None)
        res.sort()
        auto = [u for u, lab in res if lab == "auto"][0]
        lines += ["## layer %d (best %.2f us, auto %.2f us; %d input sets)" % (li, res[0][0], auto, rotate), "",
                  "| tiling | us |", "|---|---|"] + ["| %s | %.2f |" % (lab, u) for u, lab in res] + [""]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="headline steps timed, exactly")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, help="the headline workload")
    ap.add_argument("--sub", default=",".join(SUBS),
                    help="comma-separated workloads reported next to the headline ('none': no others)")
    ap.add_argument("--sub-ms", type=float, default=100.0, help="timed milliseconds per other workload")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python (no HIP graph)")
    ap.add_argument("--path", choices=("prepare_fused", "fused", "separate"), default="prepare_fused",
                    help="prepare_fused: lora_prepare_shrink_expand for the first layer, lora_shrink_expand for "
                         "the others; fused: lora_prepare_meta, then lora_shrink_expand per layer; separate: "
                         "lora_prepare_meta, then per layer a cleared buffer, lora_shrink and lora_expand")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds per oracle leg (1 thread, all cores)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the read, copy and empty-launch probes")
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate through (0 = auto)")
    ap.add_argument("--dispatch-plan", default="", help="write the library calls made, in order, to this JSON")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many eager steps of --workload and a 256 MiB calibration copy, then exit "
                         "(counter runs)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON", "COMMAND"),
                    help="write the per-kernel traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_CSV", "PLAN_JSON", "OUT_MD", "COMMAND"),
                    help="write per-workload, per-layer kernel durations of a rocprofv3 --kernel-trace run")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "OUT_MD", "COMMAND"),
                    help="write the kernel statistics of one rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_CSV", "OUT_MD", "COMMAND"),
                    help="write the per-kernel MFMA use of one rocprofv3 --pmc run and exit")
    ap.add_argument("--sweep", nargs=2, metavar=("KERNEL", "OUT_MD"),
                    help="time every tiling of KERNEL (shrink or expand) on --workload and write a table")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_mfma:
        summarize_mfma(args.workload, *args.summarize_mfma)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: the segmented-gather LoRA path here has no multi-GPU part "
              "(requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from segmented_gather_lora_amd import _build
    _build.ensure_built()
    import segmented_gather_lora_amd  # noqa: F401

    torch.cuda.set_device(0)
    if args.sweep:
        sweep(args.workload, *args.sweep)
        return
    if args.profile_steps:
        run_workload(args.workload, args, None, args.warmup, 0)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("# profile run done", file=sys.stderr)
        return

    head = run_workload(args.workload, args, args.steps, args.warmup, 0)
    wl = head.pop("_wl")
    subs = {}
    names = [] if args.sub in ("", "none") else [s for s in args.sub.split(",") if s and s != args.workload]
    for s in names:
        r = run_workload(s, args, None, min(args.warmup, 10), args.sub_ms)
        r.pop("_wl")
        subs[s] = r
    ceil = {}
    if not args.no_ceilings:
        PLAN.workload, PLAN.phase = "probes", "per_call"
        ceil = {"copy_256MiB_GBps": round(copy_gbps(), 1), "empty_launch_us": round(probe_empty(), 3),
                "empty_launch_workgroups": EMPTY_WG}

    roof = dict(head["roofline"])
    if ceil:
        roof["measured_copy_GBps"] = ceil["copy_256MiB_GBps"]
        roof["frac_of_copy"] = round(roof["achieved"] / ceil["copy_256MiB_GBps"], 4)
    if "read_probe" in head:
        roof["measured_read_GBps"] = head["read_probe"]["GBps"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "num_tokens": head["num_tokens"], "max_loras": head["max_loras"],
                   "layers": head["layers"], "active_tokens": head["active_tokens"],
                   "active_loras": head["active_loras"], "parallelism": "none",
                   "launch": "eager" if args.eager else "hip_graph", "input_sets_rotated": head["input_sets_rotated"],
                   "step": head["step"], "path": args.path},
        "roofline": roof,
        "step_GBps": head["step_GBps"],
        "step_frac_of_peak": head["step_frac_of_peak"],
        "kernels_us": head["kernels_us"],
        "kernel_frac": head.get("kernel_frac"),
        "workloads": subs,
        "ceilings": ceil,
    }
    if "read_probe" in head:
        line["ceilings"]["read_probe_" + head["workload"]] = head["read_probe"]
        line["frac_of_read_probe"] = head["frac_of_read_probe"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    if args.dispatch_plan:
        PLAN.dump(args.dispatch_plan)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
