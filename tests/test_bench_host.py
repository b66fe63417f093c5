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


def _wl(n, max_loras, layers):
    """A stand-in workload: n tokens, max_loras, and (slices, rank) per layer."""
    mapping = types.SimpleNamespace(numel=lambda: n)
    spec = types.SimpleNamespace(max_loras=max_loras)
    ls = [types.SimpleNamespace(spec=types.SimpleNamespace(slices=s, rank=r, expand_only=False)) for s, r in layers]
    return types.SimpleNamespace(mapping=mapping, spec=spec, layers=ls)


def test_launch_count_query():
    """The library's own answer (host only) at the edges of the one-launch range."""
    import segmented_gather_lora_amd as sgl
    q = sgl.lora_shrink_expand_launches
    assert q(256, 32, 3, 16, True) == 1 and q(256, 32, 3, 16, False) == 1
    assert q(2048, 1022, 3, 16, True) == 1 and q(2049, 1022, 3, 16, True) == 3
    assert q(2049, 1022, 3, 16, False) == 1
    assert q(23 * 33, 32, 3, 16, False) == 1 and q(23 * 33 + 1, 32, 3, 16, False) == 2
    assert q(256, 32, 1, 64, False) == 1 and q(256, 32, 1, 72, False) == 2 and q(256, 32, 3, 32, False) == 2
    assert q(23 * 1024, 1023, 1, 8, False) == 1 and q(23 * 1024 + 1, 1023, 1, 8, False) == 2
    for bad in [(0, 32, 3, 16), (256, 0, 3, 16), (256, 32, 0, 16), (256, 32, 3, 12)]:
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


def test_summarize_stats_names(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void lora::(anonymous namespace)::expand_kernel<1, 1, true, true>(lora::ExpandArgs)",
                    10, 80000, 8000, 30.0, 7000, 9000, 1])
        w.writerow(["void lora::(anonymous namespace)::lora_major_kernel<3, 1, true, true>(lora::FusedArgs)",
                    10, 130000, 13000, 70.0, 12000, 14000, 1])
    out = tmp_path / "s.md"
    bench.summarize_stats("decode", str(p), str(out), "cmd")
    text = open(out).read()
    assert "| lora::lora_major_kernel<3, 1, true, true> | 10 | 13.000 | 12.000 | 14.000 | 70.0 |" in text
    assert text.index("lora_major_kernel") < text.index("expand_kernel")    # sorted by total time
