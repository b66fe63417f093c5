"""Host logic of bench.py (CPU only): which calls run as one launch, and the
summaries written from rocprofv3 output."""
import csv
import json
import types

import pytest

import bench


@pytest.fixture(scope="module", autouse=True)
def _library_built():
    """The launch-count query is a host-only call into the library."""
    from segmented_gather_lora_amd import _build
    _build.ensure_built()


def _wl(n, max_loras, layers, hidden=4096):
    """A stand-in workload: n tokens, max_loras, and (slices, rank) per layer."""
    mapping = types.SimpleNamespace(numel=lambda: n)
    spec = types.SimpleNamespace(max_loras=max_loras)
    ls = [types.SimpleNamespace(spec=types.SimpleNamespace(slices=s, rank=r, hidden=hidden, expand_only=False))
          for s, r in layers]
    return types.SimpleNamespace(mapping=mapping, spec=spec, layers=ls)


def test_launch_count_query(monkeypatch):
    """The library's own answer (host only) at the edges of the one-launch range."""
    import segmented_gather_lora_amd as sgl
    q = sgl.lora_shrink_expand_launches
    assert q(256, 32, 4096, 3, 16, True) == 1 and q(256, 32, 4096, 3, 16, False) == 1
    assert q(2048, 1022, 4096, 3, 16, True) == 1 and q(2049, 1022, 4096, 3, 16, True) == 3
    assert q(2049, 1022, 4096, 3, 16, False) == 1
    # outside the range: shrink + expand, plus the zeroing of buf's rows when the shrink is split over K
    sep = (2, 3)
    assert q(23 * 33, 32, 4096, 3, 16, False) == 1 and q(23 * 33 + 1, 32, 4096, 3, 16, False) in sep
    assert q(256, 32, 4096, 1, 64, False) == 1 and q(256, 32, 4096, 1, 72, False) in sep
    assert q(256, 32, 4096, 3, 32, False) in sep
    assert q(23 * 1024, 1023, 4096, 1, 8, False) == 1 and q(23 * 1024 + 1, 1023, 4096, 1, 8, False) in sep
    # large batches with wide ids are prepared in two launches (rank, then place)
    p = sgl.lora_prepare_meta_launches
    assert p(0, 128) == 1 and p(4095, 1023) == 1 and p(4096, 1023) == 1 and p(8192, 1023) == 2 and p(2097152, 1) == 2
    assert p(8192, 8) == 1 and p(8192, 128) == 2 and p(16384, 128) == 2 and p(4096, 64) == 1
    for bad in [(-1, 8), (8, 0), (8, 1024)]:
        with pytest.raises(sgl.LoraError):
            p(*bad)
    assert q(16384, 128, 8192, 3, 128, False) == 2 and q(16384, 128, 8192, 3, 128, True) == 4
    assert q(8192, 8, 4096, 3, 64, True) == 3
    # the stream-K shrink (batches of 1024 tokens or more) adds its parts up without atomics
    assert q(4096, 64, 14336, 1, 32, False) == 2 and q(4096, 64, 14336, 1, 32, True) == 3
    # without it, a split-K shrink into a fresh buffer zeroes the active rows first (Zipf's down layer)
    monkeypatch.setenv("LORA_SHRINK_SK", "1")
    assert q(4096, 64, 14336, 1, 32, False) == 3 and q(4096, 64, 14336, 1, 32, True) == 4
    monkeypatch.delenv("LORA_SHRINK_SK")
    for bad in [(0, 32, 4096, 3, 16), (256, 0, 4096, 3, 16), (256, 32, 4096, 0, 16), (256, 32, 4096, 3, 12),
                (256, 32, 12, 3, 16)]:
        with pytest.raises(sgl.LoraError):
            q(*bad, True)


def test_one_launch_range():
    qkv16 = [((4096, 1024, 1024), 16)]
    assert bench.one_launch(_wl(256, 32, qkv16), 0, True)           # 256 / 33 ids: 8 per id
    # at most 2048 tokens with the prepare
    assert bench.one_launch(_wl(2048, 1022, qkv16), 0, True)
    assert not bench.one_launch(_wl(2049, 1022, qkv16), 0, True)
    assert bench.one_launch(_wl(2049, 1022, qkv16), 0, False)
    # fewer than 24 tokens per id on average (ceil(n / min(n, max_loras + 1)))
    assert bench.one_launch(_wl(23 * 33, 32, qkv16), 0, False)
    assert not bench.one_launch(_wl(23 * 33 + 1, 32, qkv16), 0, False)
    # S * r <= 64 and r <= 64
    assert bench.one_launch(_wl(256, 32, [((64,), 64)]), 0, False)
    assert not bench.one_launch(_wl(256, 32, [((64,), 72)]), 0, False)
    assert not bench.one_launch(_wl(256, 32, [((64, 64, 64), 32)]), 0, False)
    assert not bench.one_launch(_wl(0, 32, qkv16), 0, False)


def test_gpus_above_one_exits_with_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_algorithmic_bytes_formulas():
    """Per-call bytes from the step's definition on a hand-checkable case."""
    import torch
    m = torch.tensor([0, -1, 1, 0, 2, -1], dtype=torch.int32)
    L = types.SimpleNamespace(spec=types.SimpleNamespace(slices=(16, 8), rank=8, hidden=32, expand_only=False),
                              bias=None)
    wl = types.SimpleNamespace(mapping=m, layers=[L])
    ab = bench.algorithmic_bytes(wl)
    ta, la, S, r, H, O = 4, 3, 2, 8, 32, 24
    assert ab["T_a"] == ta and ab["L_a"] == la and ab["prepare"] == 12 * 6
    assert ab["shrink"] == [2 * ta * H + 2 * la * S * r * H + 8 * S * ta * r]
    assert ab["shrink_fresh"] == [2 * ta * H + 2 * la * S * r * H + 4 * S * ta * r]
    assert ab["expand"] == [4 * S * ta * r + 2 * la * r * O + 2 * ta * O * 2]


def test_plan_merges_and_replays():
    p = bench.Plan()
    p.workload, p.phase = "w", "timed"
    A, B = ["prepare", "shrink", "expand"], ["shrink", "expand"]
    p.replay([("preplinear0", A), ("linear1", B)], 2)
    p.add("expand0", ["expand"], times=4)
    p.add("expand0", ["expand"])
    assert p.calls == [["w", "timed", "preplinear0", A, 1], ["w", "timed", "linear1", B, 1],
                       ["w", "timed", "preplinear0", A, 1], ["w", "timed", "linear1", B, 1],
                       ["w", "timed", "expand0", ["expand"], 5]]


def _write_trace(path, names_durations):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for i, (name, dur) in enumerate(names_durations):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 500


def test_summarize_trace_matches_plan(tmp_path):
    """Library dispatches (foreign kernels ignored) matched one by one with the
    plan; per workload, phase, call and kernel averages."""
    A, B = ["prepare", "shrink", "expand"], ["zero", "shrink", "expand"]
    plan = {"calls": [["zipf", "warmup", "preplinear0", A, 1],
                      ["zipf", "timed", "preplinear0", A, 1], ["zipf", "timed", "linear1", B, 1],
                      ["zipf", "timed", "preplinear0", A, 1], ["zipf", "timed", "linear1", B, 1],
                      ["decode", "per_call", "preplinear0", ["one_launch"], 2],
                      ["large", "timed", "prepare", ["prepare_rank", "prepare_place"], 1]]}
    json.dump(plan, open(tmp_path / "plan.json", "w"))
    P, Z = "void lora::prepare_kernel(lora::PrepareArgs)", "void lora::zero_rows_kernel(lora::ShrinkArgs)"
    S0, S1 = "void lora::shrink_lds_kernel<4, 2, 2, 4>(lora::ShrinkArgs)", "void lora::shrink_lds_kernel<2,2,2,4>(x)"
    E = "void lora::expand_kernel<1, 2, true, false>(lora::ExpandArgs)"
    LM = "void lora::lora_major_kernel<3, 1, true, true>(lora::FusedArgs)"
    rows = [(P, 7), (S0, 20), (E, 100), ("torch_fill", 3),
            (P, 6), (S0, 24), (E, 110), (Z, 2), (S1, 40), (E, 30),
            (P, 6), (S0, 26), (E, 130), (Z, 2), (S1, 44), (E, 34),
            (LM, 13000), (LM, 15000),
            ("void lora::prepare_rank_kernel(lora::PrepareArgs, int*, int)", 3000),
            ("void lora::prepare_place_kernel(lora::PrepareArgs, int*, int, int, int*, int)", 2000)]
    _write_trace(tmp_path / "t.csv", rows)
    out = bench.summarize_trace(str(tmp_path / "t.csv"), str(tmp_path / "plan.json"), str(tmp_path / "o.md"), "cmd")
    assert out["zipf/timed/preplinear0/shrink0"] == 0.025 and out["zipf/timed/preplinear0/expand0"] == 0.12
    assert out["zipf/timed/linear1/expand1"] == 0.032 and out["zipf/timed/linear1/zero1"] == 0.002
    assert out["zipf/timed/preplinear0/prepare"] == 0.006
    assert out["decode/per_call/preplinear0/one_launch0"] == 14.0
    assert out["large/timed/prepare/prepare_rank"] == 3.0 and out["large/timed/prepare/prepare_place"] == 2.0
    assert not any(k.startswith("zipf/warmup") for k in out)


def test_summarize_trace_rejects_a_mismatch(tmp_path):
    json.dump({"calls": [["w", "timed", "shrink0", ["shrink"], 1]]}, open(tmp_path / "plan.json", "w"))
    _write_trace(tmp_path / "t.csv", [("void lora::expand_kernel<1,1,true,true>(a)", 5)])
    with pytest.raises(SystemExit):
        bench.summarize_trace(str(tmp_path / "t.csv"), str(tmp_path / "plan.json"), str(tmp_path / "o.md"), "c")


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_summarize_pmc_attributes_layers_in_dispatch_order(tmp_path):
    # two Zipf steps: prepare, shrink L0, expand L0, shrink L1, expand L1; then a 256 MiB copy
    step = [("lora::prepare_kernel", 1), ("lora::shrink_lds_kernel<2, 2, 2, 4>", 10),
            ("lora::expand_kernel<1, 2, true, false>", 100), ("lora::shrink_lds_kernel<4, 2, 2, 4>", 1000),
            ("lora::expand_kernel<1, 2, true, false>", 10000)]
    fetch = step + step + [("__amd_rocclr_copyBuffer", 131072)]          # reads half: scale 2
    write = [(n, 2 * v) for n, v in step + step] + [("__amd_rocclr_copyBuffer", 262144)]   # exact: scale 1
    _write_pmc(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_pmc(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "o.json"
    bench.summarize_pmc("zipf", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out), "cmd")
    rec = json.load(open(out))
    assert rec["copy_fetch_scale"] == 2.0 and rec["copy_write_scale"] == 1.0
    tb = rec["traffic_bytes"]
    # fetch KiB * 1024 * 2 + write KiB * 1024 * 1 = 4 * KiB * 1024
    assert tb == {"prepare": 4096, "shrink0": 40960, "expand0": 409600, "shrink1": 4096000,
                  "expand1": 40960000}
    assert rec["kernel_hash"] == bench.kernel_source_hash()
    assert all(v["dispatches"] == 2 for v in rec["raw"].values())


def test_summarize_pmc_one_launch_call(tmp_path):
    step = [("lora::lora_major_kernel<3, 1, true, true>", 7)]
    _write_pmc(tmp_path / "f.csv", "FETCH_SIZE", step * 3 + [("__amd_rocclr_copyBuffer", 262144)])
    _write_pmc(tmp_path / "w.csv", "WRITE_SIZE", step * 3 + [("__amd_rocclr_copyBuffer", 262144)])
    out = tmp_path / "o.json"
    bench.summarize_pmc("decode", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out), "cmd")
    assert json.load(open(out))["traffic_bytes"] == {"preplinear0": 2 * 7 * 1024}


def test_cold_sets():
    """Input sets a call cycles over when timed alone: enough that twice the
    last-level cache streams between two uses of one set, within the caps."""
    llc = bench.LLC_BYTES
    assert bench.cold_sets(4 * llc, 10 * llc) == 2             # a call larger than the cache: two sets
    assert bench.cold_sets(llc // 4, llc) == 9                 # 1 + 2 * 4
    assert bench.cold_sets(1, 1 << 20) == 64                   # a tiny call: at most 64 sets
    assert bench.cold_sets(1, 8 << 30) == 2                    # at most 16 GiB of sets, at least two
    for cb in (1 << 20, 50 << 20, 200 << 20):
        k = bench.cold_sets(cb, 300 << 20)
        assert k == 2 or (k - 1) * cb >= 2 * llc or k * (300 << 20) > (16 << 30) - (300 << 20)
