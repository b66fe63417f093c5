"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Metadata must match bit for bit; the fp32 shrink buffer and the bf16 expand
output within the tolerances stated in _harness.py; tokens with id -1 and
columns outside the slices must be left bit-for-bit untouched.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import _harness as H

pytestmark = pytest.mark.gpu

# the oracle runs on every core this process may use
NTHREADS = max(1, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module", autouse=True)
def _setup():
    from segmented_gather_lora_amd import _build
    _build.ensure_built()
    torch.cuda.set_device(0)
    yield


def _prep(mapping: np.ndarray, max_loras: int, max_num_tokens=None):
    sgl = H.lib()
    meta = sgl.LoraMeta(max_loras, max_num_tokens or max(mapping.size, 1))
    sgl.lora_prepare_meta(torch.from_numpy(np.ascontiguousarray(mapping, np.int32)).to("cuda"), meta)
    torch.cuda.synchronize()
    return meta


# ------------------------------------------------------------------ metadata

@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_prepare_workload_mappings(name):
    spec = workloads.WORKLOADS[name]
    m = workloads.make_mapping(spec, torch.Generator().manual_seed(spec.seed)).numpy()
    print("prepare", name, m.size, flush=True)
    H.check_meta(_prep(m, spec.max_loras), m, spec.max_loras)


@pytest.mark.parametrize("seed,n,ml,neg", [
    (1, 1, 1, 0.0), (2, 63, 3, 0.3), (3, 64, 3, 0.3), (4, 65, 7, 0.3), (5, 1023, 32, 0.1),
    (6, 1024, 32, 0.0), (7, 1025, 128, 0.2), (8, 5000, 1023, 0.2), (9, 20000, 64, 0.05),
    (10, 3000, 1, 0.5), (11, 2049, 255, 0.0), (12, 777, 511, 0.9), (13, 70000, 1023, 0.1),
    (14, 16384, 2, 0.0), (15, 16385, 1023, 0.5),
    (16, 2097152, 1023, 0.1), (17, 2097152, 2, 0.0)])   # the largest batch the library takes
def test_prepare_random(seed, n, ml, neg):
    rng = np.random.default_rng(seed)
    m = rng.integers(0, ml, n).astype(np.int32)
    m[rng.random(n) < neg] = -1
    print("prepare random", seed, n, ml, flush=True)
    H.check_meta(_prep(m, ml), m, ml)


def test_prepare_skewed_and_sorted_inputs():
    # one id for everything; already sorted; reverse sorted; alternating
    for m in [np.zeros(4096, np.int32), np.sort(np.random.default_rng(1).integers(-1, 9, 3000)).astype(np.int32),
              np.sort(np.random.default_rng(2).integers(-1, 9, 3000))[::-1].astype(np.int32),
              (np.arange(2500) % 2).astype(np.int32)]:
        H.check_meta(_prep(m, 9), m, 9)


def test_prepare_worked_example_multiset():
    ids = np.array([-1] * 3 + [0] * 10 + [2] * 5 + [1] * 2, np.int32)
    m = ids[np.random.default_rng(7).permutation(ids.size)]
    got = H.check_meta(_prep(m, 3), m, 3)
    assert got["active_lora_ids"].tolist() == [-1, 0, 1, 2]
    assert got["num_tokens_per_lora"].tolist() == [3, 10, 2, 5]
    assert got["lora_token_start_loc"].tolist() == [0, 3, 13, 15, 20]


@pytest.mark.parametrize("n", [0, 1, 1000, 16384])
def test_prepare_no_lora_leaves_buffers(n):
    sgl = H.lib()
    meta = sgl.LoraMeta(5, 16384)
    v = meta.views()
    for k in ("token_lora_mapping", "token_indices_sorted"):
        v[k].fill_(12345)
    for k in ("active_lora_ids", "num_tokens_per_lora", "lora_token_start_loc"):
        v[k].fill_(7)
    sgl.lora_prepare_meta(torch.full((n,), -1, dtype=torch.int32, device="cuda"), meta)
    torch.cuda.synchronize()
    got = H.meta_numpy(meta, 16384)
    assert got["no_lora_flag"][0] == 1 and got["status"][0] == 0
    assert np.all(got["active_lora_ids"] == -1) and np.all(got["num_tokens_per_lora"] == 0)
    assert np.all(got["lora_token_start_loc"] == 0)
    assert np.all(got["token_lora_mapping"] == 12345) and np.all(got["token_indices_sorted"] == 12345)
    assert meta.num_tokens == n


def test_prepare_bad_ids_reported():
    m = np.array([0, 5, -2, 1, 1, 2, 77, -1], np.int32)
    H.check_meta(_prep(m, 3), m, 3)


def test_prepare_reuse_and_determinism():
    sgl = H.lib()
    meta = sgl.LoraMeta(64, 8192)
    big = np.random.default_rng(3).integers(-1, 64, 8192).astype(np.int32)
    small = np.array([3, 3, -1, 0], np.int32)
    for m in (big, small, big):
        sgl.lora_prepare_meta(torch.from_numpy(m).cuda(), meta)
        torch.cuda.synchronize()
        H.check_meta(meta, m, 64)
    a = H.meta_numpy(meta, 8192)
    sgl.lora_prepare_meta(torch.from_numpy(big).cuda(), meta)
    torch.cuda.synchronize()
    b = H.meta_numpy(meta, 8192)
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_host_mirror_of_flag():
    sgl = H.lib()
    meta = sgl.LoraMeta(4, 64)
    host = torch.full((1,), 99, dtype=torch.int32, pin_memory=True)
    meta.struct.host_no_lora = host.data_ptr()
    sgl.lora_prepare_meta(torch.full((10,), -1, dtype=torch.int32, device="cuda"), meta)
    torch.cuda.synchronize()
    assert int(host[0]) == 1
    sgl.lora_prepare_meta(torch.tensor([0, -1, 2], dtype=torch.int32, device="cuda"), meta)
    torch.cuda.synchronize()
    assert int(host[0]) == 0
    meta.struct.host_no_lora = None


# ------------------------------------------------------------------ shrink + expand

@pytest.mark.parametrize("add_inputs", [True, False])
@pytest.mark.parametrize("name,n", [("tiny", None), ("decode", 200), ("prefill", 600), ("zipf", 300),
                                    ("zipf", 1500), ("large", 160)])
def test_parity_all_tokens(name, n, add_inputs):
    """Every token at reduced N.  Zipf at 1500 tokens (about 23 per id at rank
    32) takes the expand kernel of 32-token tiles walking runs of 4 column
    blocks, the one the full Zipf shape runs."""
    wl = workloads.make_workload(name, num_tokens=n)
    print("parity", name, n, add_inputs, flush=True)
    st = H.run_and_check(wl, add_inputs=add_inputs)
    print(st, flush=True)


@pytest.mark.parametrize("name,sample", [("decode", None), ("prefill", 96), ("zipf", 96), ("large", 64)])
def test_parity_full_size_sampled(name, sample):
    wl = workloads.make_workload(name)
    print("full size", name, flush=True)
    st = H.run_and_check(wl, add_inputs=True, sample=sample, seed=11)
    print(st, flush=True)


@pytest.mark.slow
@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,add_inputs", [("prefill", True), ("prefill", False), ("zipf", True),
                                             ("large", True), ("large", False)])
def test_parity_full_size_every_token(name, add_inputs):
    """Every token of the full-size workloads through the calls the bench
    times (lora_prepare_shrink_expand for the first layer, lora_shrink_expand
    for the next; the separate kernels at these shapes), checked against the
    oracle on all host cores; add_inputs=false once per shape class."""
    wl = workloads.make_workload(name)
    print("full size every token", name, add_inputs, NTHREADS, flush=True)
    st = H.run_and_check(wl, add_inputs=add_inputs, prep=True, nthreads=NTHREADS)
    print(st, flush=True)


@pytest.mark.parametrize("bias", [False, True])
def test_largest_batch_sampled(bias):
    """The largest batch the library takes (2097152 tokens) over 1023 LoRAs:
    metadata bit-exact, shrink and expand on a seeded sample of tokens that
    covers the first and last token of segments."""
    wl = workloads.random_case(500 + bias, 2097152, 64, (64, 16), 16, 1023, neg_fraction=0.1, bias=bias)
    print("largest batch", bias, flush=True)
    H.run_and_check(wl, add_inputs=True, sample=512, seed=3)


def test_no_lora_full_size_touches_nothing():
    wl = workloads.make_workload("large_nolora")
    print("no-lora full size", flush=True)
    H.run_and_check(wl, add_inputs=True, sample=32)


@pytest.mark.parametrize("name,n", [("tiny", None), ("decode", None), ("prefill", 700), ("zipf", 400),
                                    ("large", 300)])
@pytest.mark.parametrize("add_inputs", [True, False])
def test_expand_only_synthetic_buffer(name, n, add_inputs):
    wl = workloads.make_workload(name, num_tokens=n)
    print("expand only", name, n, add_inputs, flush=True)
    print(H.run_expand_only(wl, add_inputs), flush=True)


@pytest.mark.parametrize("case", [
    dict(seed=101, n=1, hidden=64, slices=(8,), rank=8, max_loras=1, neg_fraction=0.0),
    dict(seed=102, n=37, hidden=72, slices=(24, 40), rank=24, max_loras=5, bias=True),
    dict(seed=103, n=130, hidden=200, slices=(264, 8, 520), rank=40, max_loras=9, bias=True),
    dict(seed=104, n=257, hidden=8, slices=(16,), rank=128, max_loras=3),
    dict(seed=105, n=90, hidden=136, slices=(8,) * 8, rank=16, max_loras=17, bias=True),
    dict(seed=106, n=500, hidden=1032, slices=(1032, 72), rank=56, max_loras=200),
    dict(seed=107, n=64, hidden=96, slices=(96,), rank=104, max_loras=2, neg_fraction=0.0),
])
def test_edge_shapes(case):
    wl = workloads.random_case(**case)
    print("edge", case, flush=True)
    H.run_and_check(wl, add_inputs=True)
    H.run_and_check(wl, add_inputs=False)


def test_offset_start_and_wide_rows():
    wl = workloads.random_case(111, 70, 64, (32, 16, 40), 16, 6, bias=True)
    H.run_and_check(wl, add_inputs=True, offset_start=24, ldy_extra=40)
    H.run_and_check(wl, add_inputs=False, offset_start=8, ldy_extra=8)


@pytest.mark.parametrize("tile,wk,ks", [(16, 1, 1), (16, 2, 3), (16, 4, 1), (32, 1, 2), (32, 2, 1),
                                        (32, 4, 4), (64, 1, 1), (64, 2, 2), (64, 4, 3)])
def test_shrink_tile_variants(tile, wk, ks, monkeypatch):
    monkeypatch.setenv("LORA_SHRINK_VARIANT", "2")
    monkeypatch.setenv("LORA_SHRINK_TILE_TOKENS", str(tile))
    monkeypatch.setenv("LORA_SHRINK_WAVES_K", str(wk))
    monkeypatch.setenv("LORA_SHRINK_KSPLIT", str(ks))
    wl = workloads.random_case(120 + tile + wk, 333, 520, (96, 40, 8), 24, 11, bias=True)
    print("shrink variant", tile, wk, ks, flush=True)
    H.run_and_check(wl, add_inputs=True)


@pytest.mark.parametrize("tt", [16, 48, 128, 256])
def test_expand_tile_variants(tt, monkeypatch):
    monkeypatch.setenv("LORA_EXPAND_TILE_TOKENS", str(tt))
    wl = workloads.random_case(130 + tt, 700, 64, (520, 264), 32, 5, bias=True, neg_fraction=0.1)
    print("expand variant", tt, flush=True)
    H.run_and_check(wl, add_inputs=True)


@pytest.mark.parametrize("run", [1, 2, 3, 8])
@pytest.mark.parametrize("tt,rank", [(16, 16), (64, 64), (64, 128)])
@pytest.mark.parametrize("add_inputs", [True, False])
def test_expand_run_variants(run, tt, rank, add_inputs, monkeypatch):
    """Units of one tile x a run of column blocks: slice widths whose block
    counts the run does not divide, partial last blocks, bias, an offset."""
    monkeypatch.setenv("LORA_EXPAND_RUN", str(run))
    monkeypatch.setenv("LORA_EXPAND_TILE_TOKENS", str(tt))
    wl = workloads.random_case(150 + run + tt + rank, 300, 64, (1800, 264, 8, 776), rank, 6, bias=True,
                               neg_fraction=0.15)
    print("expand run", run, tt, rank, add_inputs, flush=True)
    H.run_and_check(wl, add_inputs=add_inputs, offset_start=16, ldy_extra=8)


@pytest.mark.parametrize("grid", [0, 8, 2048])
@pytest.mark.parametrize("tt,rank", [(16, 16), (64, 64), (64, 128)])
@pytest.mark.parametrize("add_inputs", [True, False])
def test_expand_share_variants(grid, tt, rank, add_inputs, monkeypatch):
    """Equal shares of the (tile, column block) list: shares that start and
    end inside a slice or a tile, ragged slice widths, bias, an offset; with
    few workgroups (long shares) and more workgroups than blocks (empty ones)."""
    monkeypatch.setenv("LORA_EXPAND_SHARE", "1")
    monkeypatch.setenv("LORA_EXPAND_TILE_TOKENS", str(tt))
    if grid:
        monkeypatch.setenv("LORA_EXPAND_GRID", str(grid))
    wl = workloads.random_case(170 + tt + rank, 300, 64, (1800, 264, 8, 776), rank, 6, bias=True,
                               neg_fraction=0.15)
    print("expand share", grid, tt, rank, add_inputs, flush=True)
    H.run_and_check(wl, add_inputs=add_inputs, offset_start=16, ldy_extra=8)


def _gpu_outputs(wl, meta, buf0=None):
    sgl = H.lib()
    L = wl.layers[0]
    D = H.DevLayer(L)
    n = wl.mapping.numel()
    buf = torch.zeros((len(L.spec.slices), n, L.spec.rank), dtype=torch.float32, device="cuda")
    if buf0 is not None:
        buf.copy_(buf0)
    sgl.lora_shrink(D.x, D.a, buf, meta, L.spec.scale)
    y = D.y0.clone()
    sgl.lora_expand(buf, D.b, D.bias, y, meta, add_inputs=True)
    torch.cuda.synchronize()
    return buf.cpu().numpy(), H.bits(y)


def test_segment_order_invariance(monkeypatch):
    """Kernels must not assume ascending segments: metadata written by hand in
    the order of the pages' worked example ([-1, 0, 2, 1]) gives the same result."""
    monkeypatch.setenv("LORA_SHRINK_KSPLIT", "1")
    ids = np.array([-1] * 3 + [0] * 10 + [2] * 5 + [1] * 2, np.int32)
    m = ids[np.random.default_rng(9).permutation(ids.size)]
    wl = workloads.random_case(140, 20, 128, (64, 32), 16, 3, bias=True)
    wl.mapping.copy_(torch.from_numpy(m))
    meta = _prep(m, 3)
    buf_a, y_a = _gpu_outputs(wl, meta)
    v = meta.views()
    order = [-1, 0, 2, 1]
    srt = np.concatenate([np.nonzero(m == k)[0] for k in order]).astype(np.int32)
    cnt = [int((m == k).sum()) for k in order]
    v["active_lora_ids"].copy_(torch.tensor(order, dtype=torch.int32))
    v["num_tokens_per_lora"].copy_(torch.tensor(cnt, dtype=torch.int32))
    v["lora_token_start_loc"].copy_(torch.tensor([0] + list(np.cumsum(cnt)), dtype=torch.int32))
    assert v["lora_token_start_loc"].tolist() == [0, 3, 13, 18, 20]
    v["token_indices_sorted"][:20].copy_(torch.from_numpy(srt))
    buf_b, y_b = _gpu_outputs(wl, meta)
    assert np.array_equal(buf_a, buf_b) and np.array_equal(y_a, y_b)


def test_permutation_equivariance(monkeypatch):
    monkeypatch.setenv("LORA_SHRINK_KSPLIT", "1")
    wl = workloads.random_case(150, 300, 256, (128, 64), 32, 7, bias=True)
    m = wl.mapping.numpy()
    buf_a, y_a = _gpu_outputs(wl, _prep(m, 7))
    perm = np.random.default_rng(4).permutation(300)
    L = wl.layers[0]
    wl2 = workloads.Workload(wl.spec, wl.mapping[perm].clone(), [workloads.Layer(
        L.spec, L.x[perm].clone(), L.lora_a, L.lora_b, L.bias, L.y0[perm].clone())])
    buf_b, y_b = _gpu_outputs(wl2, _prep(m[perm], 7))
    assert np.array_equal(buf_b, buf_a[:, perm]) and np.array_equal(y_b, y_a[perm])


def test_shrink_accumulates_into_buffer():
    wl = workloads.random_case(160, 90, 192, (32, 16), 16, 4)
    L = wl.layers[0]
    m = wl.mapping.numpy()
    meta = _prep(m, 4)
    gen = torch.Generator().manual_seed(5)
    buf0 = torch.randn((2, 90, 16), generator=gen)
    sgl = H.lib()
    buf = buf0.cuda()
    sgl.lora_shrink(L.x.cuda(), [a.cuda() for a in L.lora_a], buf, meta, L.spec.scale)
    torch.cuda.synchronize()
    ref = buf0.numpy().copy()
    st, bound = oracle.shrink(workloads.bf16_bits(L.x), [workloads.bf16_bits(a) for a in L.lora_a], ref, m,
                              L.spec.scale, 4, with_bound=True)
    H.shrink_check(buf.cpu().numpy(), ref, bound)
    neg = m == -1
    assert np.array_equal(buf.cpu().numpy()[:, neg], buf0.numpy()[:, neg])


def test_bad_ids_are_not_touched():
    m = np.array([0, 9, 1, -5, 2, 2, 0, 100] * 4, np.int32)
    wl = workloads.random_case(170, m.size, 64, (16,), 8, 3)
    wl.mapping.copy_(torch.from_numpy(m))
    meta = _prep(m, 3)
    assert int(meta.views()["status"][0]) == H.lib().LORA_ERR_ID_RANGE
    buf, y = _gpu_outputs(wl, meta)
    bad = (m < -1) | (m >= 3)
    assert np.all(buf[:, bad] == 0)
    assert np.array_equal(y[bad], workloads.bf16_bits(wl.layers[0].y0)[bad])


def test_invalid_arguments_raise():
    sgl = H.lib()
    meta = _prep(np.zeros(8, np.int32), 2)
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    a = [torch.zeros((2, 16, 64), dtype=torch.bfloat16, device="cuda")]
    buf = torch.zeros((1, 8, 16), device="cuda")
    with pytest.raises(sgl.LoraError) as e:
        sgl.lora_shrink(x[:7], a, buf, meta, 1.0)
    assert e.value.status == sgl.LORA_ERR_NUM_TOKENS
    with pytest.raises(sgl.LoraError) as e:
        sgl.lora_shrink(x, [torch.zeros((2, 12, 64), dtype=torch.bfloat16, device="cuda")], buf, meta, 1.0)
    assert e.value.status == sgl.LORA_ERR_SHAPE
    with pytest.raises(sgl.LoraError):
        sgl.lora_prepare_meta(torch.zeros(9, dtype=torch.int32, device="cuda"), meta)
    # what the C ABI cannot see is refused by the binding before any launch
    b = [torch.zeros((2, 32, 16), dtype=torch.bfloat16, device="cuda")]
    y = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        sgl.lora_shrink(x.cpu(), a, buf, meta, 1.0)                           # a host tensor
    with pytest.raises(TypeError):
        sgl.lora_shrink(x.float(), a, buf, meta, 1.0)                         # wrong element type
    with pytest.raises(TypeError):
        sgl.lora_prepare_meta(torch.zeros(8, dtype=torch.int64, device="cuda"), meta)
    with pytest.raises(sgl.LoraError) as e:                                   # 1 LoRA for max_loras 2
        sgl.lora_shrink(x, [a[0][:1].contiguous()], buf, meta, 1.0)
    assert e.value.status == sgl.LORA_ERR_SHAPE
    with pytest.raises(sgl.LoraError) as e:                                   # B of another rank
        sgl.lora_expand(buf, [torch.zeros((2, 32, 8), dtype=torch.bfloat16, device="cuda")], None, y, meta)
    assert e.value.status == sgl.LORA_ERR_SHAPE
    with pytest.raises(sgl.LoraError) as e:                                   # y with too few rows
        sgl.lora_expand(buf, b, None, y[:5], meta)
    assert e.value.status == sgl.LORA_ERR_SHAPE
    with pytest.raises(sgl.LoraError) as e:                                   # y narrower than the slices
        sgl.lora_expand(buf, b, None, y, meta, offset_start=8)
    assert e.value.status == sgl.LORA_ERR_SHAPE
    with pytest.raises(sgl.LoraError) as e:                                   # a transposed (strided) x
        sgl.lora_shrink(torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda").t(), a, buf, meta, 1.0)
    assert e.value.status == sgl.LORA_ERR_SHAPE
    sgl.lora_expand(buf, b, None, y, meta)                                    # the valid call still runs
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", range(1, 20))
@pytest.mark.parametrize("ks", [1, 3])
def test_shrink_staged_variants(cfg, ks, monkeypatch):
    """Every LDS-staged shrink configuration on a ragged case: K not a
    multiple of 64, rows not a multiple of the row block, short segments;
    with 3 K chunks the pieces have fewer steps than the deeper tiles have
    stages (up to 12), so the ring is filled with reloads past the end."""
    monkeypatch.setenv("LORA_SHRINK_VARIANT", "3")
    monkeypatch.setenv("LORA_SHRINK_STAGED", str(cfg))
    monkeypatch.setenv("LORA_SHRINK_KSPLIT", str(ks))
    wl = workloads.random_case(200 + cfg, 517, 712, (72, 40, 104), 8, 6, bias=True, neg_fraction=0.15)
    print("staged shrink", cfg, ks, flush=True)
    H.run_and_check(wl, add_inputs=True)


def test_shrink_staged_full_rows(monkeypatch):
    """Staged kernel with 3 slices of rank 64 (192 rows), one long segment."""
    monkeypatch.setenv("LORA_SHRINK_VARIANT", "3")
    wl = workloads.random_case(230, 1000, 1024, (128, 64, 64), 64, 2, neg_fraction=0.0)
    H.run_and_check(wl, add_inputs=True)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 9, 10, 11, 14, 15])
@pytest.mark.parametrize("slices,rank,hidden", [((32,), 32, 1000), ((72, 40, 104), 32, 1000),
                                                ((64, 64, 64), 64, 520), ((256, 128, 128), 128, 712)])
@pytest.mark.parametrize("fused", [False, True])
def test_shrink_stream_k(cfg, slices, rank, hidden, fused, monkeypatch):
    """The stream-K shrink with every kind of staged tile, on 32 to 384
    weight rows (one or several row blocks), K not a multiple of 64, shares
    that cut tiles into two or more parts, -1 ids; accumulating into buf
    (lora_shrink) and writing a fresh one (lora_shrink_expand)."""
    monkeypatch.setenv("LORA_SHRINK_SK", "2")
    monkeypatch.setenv("LORA_SHRINK_STAGED", str(cfg))
    wl = workloads.random_case(300 + rank + len(slices), 1500, hidden, slices, rank, 6, bias=True,
                               neg_fraction=0.1)
    print("stream-K shrink", cfg, slices, rank, hidden, fused, flush=True)
    H.run_and_check(wl, add_inputs=True, fused=fused)


@pytest.mark.parametrize("n", [1023, 1024, 1100])
@pytest.mark.parametrize("fused", [False, True])
def test_shrink_walk_boundary(n, fused):
    """The automatic choice on both sides of the stream-K threshold (1024
    tokens: units below, stream-K from there on), with long segments (the
    LDS-staged kernel), 192 weight rows and K not a multiple of 64."""
    wl = workloads.random_case(360 + n, n, 1000, (64, 64, 64), 64, 4, bias=True, neg_fraction=0.05)
    print("shrink walk boundary", n, fused, flush=True)
    H.run_and_check(wl, add_inputs=True, fused=fused)
    H.run_and_check(wl, add_inputs=False, fused=fused)


@pytest.mark.parametrize("grid", [8, 64, 256])
def test_shrink_stream_k_many_parts(grid, monkeypatch):
    """Stream-K with more workgroups than the work needs: shares of a step or
    less, tiles cut into many parts, workgroups with nothing to do."""
    monkeypatch.setenv("LORA_SHRINK_SK", "2")
    monkeypatch.setenv("LORA_SHRINK_GRID", str(grid))
    wl = workloads.random_case(340 + grid, 1100, 712, (64, 64), 32, 3, neg_fraction=0.05)
    print("stream-K shrink grid", grid, flush=True)
    H.run_and_check(wl, add_inputs=True)
    H.run_and_check(wl, add_inputs=False, fused=True)


# ------------------------------------------------------------------ logits and embedding paths

@pytest.mark.parametrize("add_inputs", [True, False])
def test_logits_path_full_size(add_inputs):
    """The logits path at its full shape: shrink + expand over the per-prompt
    mapping into one vocab-wide slice (128256 columns); every prompt checked."""
    wl = workloads.make_workload("logits")
    print("logits full size", add_inputs, flush=True)
    print(H.run_and_check(wl, add_inputs=add_inputs), flush=True)


def test_logits_path_ragged_vocab():
    """A vocab width that is no multiple of the column block, with an offset."""
    wl = workloads.random_case(301, 37, 512, (32008,), 16, 5, neg_fraction=0.2)
    print("logits ragged vocab", flush=True)
    H.run_and_check(wl, add_inputs=True, offset_start=8, ldy_extra=16)


@pytest.mark.parametrize("add_inputs", [True, False])
@pytest.mark.parametrize("n,sample", [(333, None), (None, 1024)])
def test_embedding_path(n, sample, add_inputs):
    """The embedding path: expand only, one slice, from the fp32 [1][N][r] input."""
    wl = workloads.make_workload("embedding", num_tokens=n)
    print("embedding", n, sample, add_inputs, flush=True)
    print(H.run_and_check(wl, add_inputs=add_inputs, sample=sample, seed=5), flush=True)


# ------------------------------------------------------------------ graph-captured decode step

def test_graph_captured_decode_step():
    """prepare + shrink + expand captured once in a HIP graph on fixed buffers
    (metadata allocated at maximum size, the batch's ids copied into a fixed
    mapping buffer), then replayed for several batches, one of them all -1.
    Eager work and synchronizations run between the replays, and every replay
    is checked against the oracle on every token."""
    sgl = H.lib()
    base = workloads.make_workload("decode")
    L = base.layers[0]
    sp = L.spec
    n, ml = base.mapping.numel(), base.spec.max_loras
    S, r, O = len(sp.slices), sp.rank, sum(sp.slices)
    meta = sgl.LoraMeta(ml, n)
    host_flag = torch.full((1,), -7, dtype=torch.int32, pin_memory=True)
    meta.struct.host_no_lora = host_flag.data_ptr()
    D = H.DevLayer(L)
    mapping_dev = torch.empty(n, dtype=torch.int32, device="cuda")
    buf = torch.zeros((S, n, r), dtype=torch.float32, device="cuda")
    y = torch.empty((n, O), dtype=torch.bfloat16, device="cuda")

    def step():
        sgl.lora_prepare_meta(mapping_dev, meta)
        sgl.lora_shrink(D.x, D.a, buf, meta, sp.scale)
        sgl.lora_expand(buf, D.b, D.bias, y, meta, add_inputs=True)

    mapping_dev.copy_(base.mapping)
    y.copy_(D.y0)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    rng = np.random.default_rng(21)
    y0b = workloads.bf16_bits(L.y0)
    tokens = np.arange(n, dtype=np.int32)
    for rep in range(5):
        m = rng.integers(-1, ml, n).astype(np.int32)
        if rep == 2:
            m[:] = -1
        mapping_dev.copy_(torch.from_numpy(m))
        buf.zero_()
        y.copy_(D.y0)
        torch.cuda.synchronize()
        print("graph replay", rep, flush=True)
        g.replay()
        torch.cuda.synchronize()
        H.check_meta(meta, m, ml)
        assert int(host_flag[0]) == (1 if rep == 2 else 0)
        buf_g = buf.cpu().numpy()
        y_g = H.bits(y)
        buf_ref, y_ref, bound, mag = H.oracle_layer(L, m, ml, tokens, True)
        H.shrink_check(buf_g, buf_ref, bound)
        H.expand_check(y_g, y_ref, y0b, mag, True, H.propagated(L, m, buf_ref, bound))
        neg = m == -1
        assert np.all(buf_g[:, neg] == 0) and np.array_equal(y_g[neg], y0b[neg])
    meta.struct.host_no_lora = None


# ------------------------------------------------------------------ fused shrink -> expand

@pytest.mark.parametrize("layout", ["auto", "tile"])
@pytest.mark.parametrize("add_inputs", [True, False])
@pytest.mark.parametrize("name,n", [("decode", None), ("tiny", None), ("decode", 37), ("logits", None),
                                    ("zipf", 300), ("prefill", 600), ("large", 160)])
def test_fused_parity(name, n, add_inputs, layout, monkeypatch):
    """lora_shrink_expand against the oracle on every token: one launch for the
    decode-like shapes (decode, tiny, logits, a short Zipf batch; LoRA-major
    for decode, tiny and Zipf unless "tile" forces the tile-major kernel), the
    two kernels for the others (prefill, rank 128)."""
    if layout == "tile":
        monkeypatch.setenv("LORA_FUSED_LAYOUT", "tile")
    wl = workloads.make_workload(name, num_tokens=n)
    print("fused", name, n, add_inputs, flush=True)
    print(H.run_and_check(wl, add_inputs=add_inputs, fused=True), flush=True)


@pytest.mark.parametrize("case", [
    dict(seed=401, n=1, hidden=64, slices=(8,), rank=8, max_loras=1, neg_fraction=0.0),
    dict(seed=402, n=45, hidden=200, slices=(24, 40), rank=8, max_loras=7, bias=True),
    dict(seed=403, n=130, hidden=1032, slices=(264, 8, 520), rank=16, max_loras=9, bias=True),
    dict(seed=404, n=200, hidden=72, slices=(1800,), rank=64, max_loras=40),
    dict(seed=405, n=300, hidden=4104, slices=(512, 256), rank=32, max_loras=1023, neg_fraction=0.3),
    dict(seed=406, n=2600, hidden=512, slices=(128, 128), rank=24, max_loras=200),
    dict(seed=407, n=97, hidden=4096, slices=(8,) * 8, rank=8, max_loras=17, bias=True),
])
def test_fused_edge_shapes(case):
    """Ragged K, ranks 8..64, widths off the 256-column block, 1023 LoRAs, a
    batch past the sorted-index LDS copy, eight slices, bias and an offset."""
    wl = workloads.random_case(**case)
    print("fused edge", case["seed"], flush=True)
    H.run_and_check(wl, add_inputs=True, offset_start=8, ldy_extra=8, fused=True)


def test_fused_repeated_calls_and_no_lora():
    """Several fused calls on one prepared batch (the counters must come back
    to zero after each), then a no-LoRA batch, then a new batch."""
    sgl = H.lib()
    ml, n = 32, 256
    meta = sgl.LoraMeta(ml, 512)
    rng = np.random.default_rng(31)
    for m in (rng.integers(-1, ml, n).astype(np.int32), np.full(n, -1, np.int32),
              rng.integers(0, 3, 150).astype(np.int32)):
        mt = torch.from_numpy(m)
        sgl.lora_prepare_meta(mt.cuda(), meta)
        for layer in range(3):
            wl = workloads.random_case(500 + layer, m.size, 1024, (256, 64, 64), 16, ml, bias=layer == 1)
            wl.mapping.copy_(mt)
            L = wl.layers[0]
            D = H.DevLayer(L)
            # a fresh buffer each call: whatever it holds on entry is overwritten
            buf = torch.full((3, m.size, 16), float(layer) - 7.5, dtype=torch.float32, device="cuda")
            y = D.y0.clone()
            sgl.lora_shrink_expand(D.x, D.a, D.b, D.bias, buf, y, meta, L.spec.scale)
            torch.cuda.synchronize()
            H.check_sync_clear(meta, m.size)
            tokens = np.arange(m.size, dtype=np.int32)
            buf_ref, y_ref, bound, mag = H.oracle_layer(L, m, ml, tokens, True)
            buf_g, y_g = buf.cpu().numpy(), H.bits(y)
            act = m != -1
            H.shrink_check(buf_g[:, act], buf_ref[:, act], bound[:, act])
            assert np.all(buf_g[:, ~act] == np.float32(layer - 7.5)), "a -1 row of buf was touched"
            H.expand_check(y_g, y_ref, workloads.bf16_bits(L.y0), mag, True, H.propagated(L, m, buf_ref, bound))


def test_fused_graph_replay():
    """prepare + lora_shrink_expand captured once and replayed for several
    batches (one all -1), with eager work between replays."""
    sgl = H.lib()
    base = workloads.make_workload("decode")
    L = base.layers[0]
    sp = L.spec
    n, ml = base.mapping.numel(), base.spec.max_loras
    meta = sgl.LoraMeta(ml, n)
    D = H.DevLayer(L)
    mapping_dev = base.mapping.cuda()
    buf = torch.zeros((3, n, sp.rank), dtype=torch.float32, device="cuda")
    y = D.y0.clone()

    def step():
        sgl.lora_prepare_meta(mapping_dev, meta)
        sgl.lora_shrink_expand(D.x, D.a, D.b, D.bias, buf, y, meta, sp.scale)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    y0b = workloads.bf16_bits(L.y0)
    tokens = np.arange(n, dtype=np.int32)
    for rep in range(5):
        m = rng.integers(-1, ml, n).astype(np.int32)
        if rep == 3:
            m[:] = -1
        mapping_dev.copy_(torch.from_numpy(m))
        buf.fill_(rep + 0.25)   # a fresh buffer per call: its entry contents do not matter
        y.copy_(D.y0)
        torch.cuda.synchronize()
        print("fused graph replay", rep, flush=True)
        g.replay()
        torch.cuda.synchronize()
        H.check_meta(meta, m, ml)
        H.check_sync_clear(meta, n)
        buf_ref, y_ref, bound, mag = H.oracle_layer(L, m, ml, tokens, True)
        buf_g, y_g = buf.cpu().numpy(), H.bits(y)
        act = m != -1
        assert np.all(buf_g[:, ~act] == np.float32(rep + 0.25))
        H.shrink_check(buf_g[:, act], buf_ref[:, act], bound[:, act])
        H.expand_check(y_g, y_ref, y0b, mag, True, H.propagated(L, m, buf_ref, bound))


@pytest.mark.parametrize("layout", ["lora", "tile"])
@pytest.mark.parametrize("mode", ["owners_skip", "help_at_once"])
@pytest.mark.parametrize("name,n", [("decode", None), ("tiny", None)])
def test_fused_helping_path(name, n, mode, layout, monkeypatch):
    """The waiters' fallback, forced from the host: with owners leaving their
    parts, every part is run by waiters that take it by its flag; with no
    patience at all, owners and waiters race for every part.  Results and the
    counters' reset must be the same as on the normal path, in both layouts."""
    monkeypatch.setenv("LORA_FUSED_LAYOUT", layout)
    monkeypatch.setenv("LORA_FUSED_HELP_AFTER", "0")
    if mode == "owners_skip":
        monkeypatch.setenv("LORA_FUSED_OWNERS_SKIP", "1")
    wl = workloads.make_workload(name, num_tokens=n)
    print("fused helping", name, mode, flush=True)
    H.run_and_check(wl, add_inputs=True, fused=True)


# ------------------------------------------------------------------ prepare + fused shrink -> expand

@pytest.mark.parametrize("layout", ["auto", "tile"])
@pytest.mark.parametrize("add_inputs", [True, False])
@pytest.mark.parametrize("name,n", [("decode", None), ("tiny", None), ("decode", 37), ("logits", None),
                                    ("zipf", 300), ("large", 160), ("prefill", 600)])
def test_prepare_fused_parity(name, n, add_inputs, layout, monkeypatch):
    """lora_prepare_shrink_expand on poisoned metadata: the metadata written by
    the one launch is bit-exact and buf / y match the oracle on every token
    (the Zipf batch's second layer then uses lora_shrink_expand; rank 128 and
    prefill take the separate calls).  "auto" takes the LoRA-major kernel for
    decode, tiny, logits and the Zipf batch; "tile" forces the tile-major one."""
    if layout == "tile":
        monkeypatch.setenv("LORA_FUSED_LAYOUT", "tile")
    wl = workloads.make_workload(name, num_tokens=n)
    print("prepare+fused", name, n, add_inputs, layout, flush=True)
    print(H.run_and_check(wl, add_inputs=add_inputs, prep=True), flush=True)


@pytest.mark.parametrize("case", [
    dict(seed=701, n=2000, hidden=1032, slices=(96, 40), rank=16, max_loras=100, bias=True),
    dict(seed=702, n=512, hidden=4104, slices=(1024, 512, 512), rank=16, max_loras=32),
    dict(seed=703, n=64, hidden=64, slices=(8,), rank=8, max_loras=16, neg_fraction=0.0),
    dict(seed=704, n=300, hidden=8192, slices=(64,), rank=64, max_loras=24),
    dict(seed=705, n=1000, hidden=512, slices=(24, 40, 8, 8, 8, 8, 8, 8), rank=8, max_loras=48, bias=True),
])
@pytest.mark.parametrize("prep", [True, False])
def test_lora_major_shapes(case, prep, monkeypatch):
    """The LoRA-major one-launch kernel (forced: the call fails if it does not
    apply), with and without the prepare: about 20 tokens per id (two tiles
    each), ragged K over 9 parts, exactly 4 tokens per id with a single part,
    rank 64 over 16 parts, eight slices with bias, and an offset."""
    monkeypatch.setenv("LORA_FUSED_LAYOUT", "lora")
    wl = workloads.random_case(**case)
    print("lora-major", case["seed"], prep, flush=True)
    H.run_and_check(wl, add_inputs=True, offset_start=8, ldy_extra=8, prep=prep, fused=not prep)


@pytest.mark.parametrize("expanders", [1, 5])
@pytest.mark.parametrize("prep", [True, False])
def test_lora_major_expanders_walk_blocks(prep, expanders, monkeypatch):
    """LoRA-major expanders that walk several 256-column blocks each (fewer
    expander roles than blocks), on the decode shape and on two-tile ids."""
    monkeypatch.setenv("LORA_FUSED_LAYOUT", "lora")
    monkeypatch.setenv("LORA_LM_EXPANDERS", str(expanders))
    for wl in (workloads.make_workload("decode"),
               workloads.random_case(731, 1200, 1024, (512, 256), 16, 60, bias=True)):
        print("lora-major walk", prep, expanders, wl.spec.name, flush=True)
        H.run_and_check(wl, add_inputs=True, offset_start=8, ldy_extra=8, prep=prep, fused=not prep)


@pytest.mark.parametrize("prep", [True, False])
def test_lora_major_bad_ids_and_many_ids(prep, monkeypatch):
    """The LoRA-major kernel (forced) on 200 ids with ids out of range mixed
    in: prepare reports them and treats them as -1, and the kernel -- reading
    the raw mapping with a prepare, the cleaned copy without -- leaves their
    rows untouched."""
    monkeypatch.setenv("LORA_FUSED_LAYOUT", "lora")
    wl = workloads.random_case(721, 2000, 512, (64, 64), 16, 200, neg_fraction=0.1, bias=True)
    m = wl.mapping.numpy().copy()
    m[5::13] = 200
    m[9::29] = -7
    wl.mapping.copy_(torch.from_numpy(m))
    print("lora-major bad ids", prep, flush=True)
    H.run_and_check(wl, add_inputs=True, offset_start=8, ldy_extra=8, prep=prep, fused=not prep)


@pytest.mark.parametrize("prep", [True, False])
@pytest.mark.parametrize("add_inputs", [True, False])
def test_lora_major_skewed_batch(add_inputs, prep, monkeypatch):
    """One id holding 300 of 512 tokens (19 tiles for its part owners and
    expanders to walk) and every other id a few, with and without the
    prepare in the launch."""
    monkeypatch.setenv("LORA_FUSED_LAYOUT", "lora")
    wl = workloads.random_case(711, 512, 2048, (1024, 256, 256), 16, 32, neg_fraction=0.05)
    m = wl.mapping.numpy().copy()
    pos = np.random.default_rng(5).choice(512, 300, replace=False)
    m[pos] = 5
    wl.mapping.copy_(torch.from_numpy(m))
    print("lora-major skewed", add_inputs, prep, flush=True)
    H.run_and_check(wl, add_inputs=add_inputs, prep=prep, fused=not prep)


@pytest.mark.parametrize("layout", ["lora", "tile"])
@pytest.mark.parametrize("mode", ["owners_skip", "help_at_once"])
def test_prepare_fused_helping_path(mode, layout, monkeypatch):
    """The waiters' fallback in both one-launch kernels, forced from the host
    as for lora_shrink_expand."""
    monkeypatch.setenv("LORA_FUSED_LAYOUT", layout)
    monkeypatch.setenv("LORA_FUSED_HELP_AFTER", "0")
    if mode == "owners_skip":
        monkeypatch.setenv("LORA_FUSED_OWNERS_SKIP", "1")
    wl = workloads.make_workload("decode")
    print("prepare+fused helping", mode, layout, flush=True)
    H.run_and_check(wl, add_inputs=True, prep=True)


@pytest.mark.parametrize("case", [
    dict(seed=601, n=1, hidden=64, slices=(8,), rank=8, max_loras=1, neg_fraction=0.0),
    dict(seed=602, n=2048, hidden=256, slices=(64, 64), rank=16, max_loras=1023, neg_fraction=0.1),
    dict(seed=603, n=700, hidden=1032, slices=(264, 8, 520), rank=16, max_loras=200, bias=True),
    dict(seed=604, n=2049, hidden=128, slices=(128,), rank=32, max_loras=500),
    dict(seed=605, n=255, hidden=4104, slices=(512, 256), rank=32, max_loras=63, neg_fraction=0.95),
])
def test_prepare_fused_edge_shapes(case):
    """One token; 2048 tokens over 1023 LoRAs (the largest one-launch batch,
    every key slot used by the sort); 2049 tokens (the two calls); bias and
    an offset; a batch that is almost all -1."""
    wl = workloads.random_case(**case)
    print("prepare+fused edge", case["seed"], flush=True)
    H.run_and_check(wl, add_inputs=True, offset_start=8, ldy_extra=8, prep=True)


@pytest.mark.parametrize("kind", ["no_lora", "bad_ids"])
def test_prepare_fused_special_batches(kind):
    """An all -1 batch (no-LoRA flag, nothing touched) and ids out of range
    (reported, treated as -1), through the one launch."""
    sgl = H.lib()
    wl = workloads.make_workload("decode", num_tokens=200)
    m = wl.mapping.numpy().copy()
    if kind == "no_lora":
        m[:] = -1
    else:
        m[::7] = 32
        m[3::11] = -5
    wl.mapping.copy_(torch.from_numpy(m))
    st = H.run_and_check(wl, add_inputs=True, prep=True)
    print(kind, st, flush=True)


def test_prepare_fused_graph_replay():
    """One captured lora_prepare_shrink_expand replayed for several batches on
    fixed buffers (one all -1), with eager work between replays; metadata and
    results checked after every replay, and the host flag mirror."""
    sgl = H.lib()
    base = workloads.make_workload("decode")
    L = base.layers[0]
    sp = L.spec
    n, ml = base.mapping.numel(), base.spec.max_loras
    meta = sgl.LoraMeta(ml, n)
    host_flag = torch.full((1,), -7, dtype=torch.int32, pin_memory=True)
    meta.struct.host_no_lora = host_flag.data_ptr()
    D = H.DevLayer(L)
    mapping_dev = base.mapping.cuda()
    buf = torch.zeros((3, n, sp.rank), dtype=torch.float32, device="cuda")
    y = D.y0.clone()

    def step():
        sgl.lora_prepare_shrink_expand(mapping_dev, D.x, D.a, D.b, D.bias, buf, y, meta, sp.scale)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(43)
    y0b = workloads.bf16_bits(L.y0)
    tokens = np.arange(n, dtype=np.int32)
    for rep in range(5):
        m = rng.integers(-1, ml, n).astype(np.int32)
        if rep == 1:
            m[:] = -1
        mapping_dev.copy_(torch.from_numpy(m))
        buf.fill_(-rep - 0.5)   # a fresh buffer per call: its entry contents do not matter
        y.copy_(D.y0)
        H.poison_meta(meta)
        torch.cuda.synchronize()
        print("prepare+fused graph replay", rep, flush=True)
        g.replay()
        torch.cuda.synchronize()
        H.check_meta(meta, m, ml)
        H.check_sync_clear(meta, n)
        assert int(host_flag[0]) == (1 if rep == 1 else 0)
        buf_ref, y_ref, bound, mag = H.oracle_layer(L, m, ml, tokens, True)
        buf_g, y_g = buf.cpu().numpy(), H.bits(y)
        act = m != -1
        assert np.all(buf_g[:, ~act] == np.float32(-rep - 0.5))
        H.shrink_check(buf_g[:, act], buf_ref[:, act], bound[:, act])
        H.expand_check(y_g, y_ref, y0b, mag, True, H.propagated(L, m, buf_ref, bound))
    meta.struct.host_no_lora = None


def test_stream_k_graph_replay(monkeypatch):
    """A captured lora_prepare_shrink_expand with the stream-K shrink (1500
    tokens, long segments), replayed for several batches on fixed buffers
    (one all -1, one single id, one half -1) with eager work between
    replays: metadata, buffer and output checked against the oracle after
    every replay, and the stream-K counters left zero."""
    monkeypatch.setenv("LORA_SHRINK_SK", "2")
    sgl = H.lib()
    base = workloads.random_case(391, 1500, 712, (64, 64, 64), 64, 6, bias=True, neg_fraction=0.05)
    L = base.layers[0]
    sp = L.spec
    n, ml = base.mapping.numel(), base.spec.max_loras
    meta = sgl.LoraMeta(ml, n)
    D = H.DevLayer(L)
    mapping_dev = base.mapping.cuda()
    buf = torch.zeros((3, n, sp.rank), dtype=torch.float32, device="cuda")
    y = D.y0.clone()

    def step():
        sgl.lora_prepare_shrink_expand(mapping_dev, D.x, D.a, D.b, D.bias, buf, y, meta, sp.scale)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(391)
    y0b = workloads.bf16_bits(L.y0)
    tokens = np.arange(n, dtype=np.int32)
    for rep in range(4):
        m = rng.integers(-1, ml, n).astype(np.int32)
        if rep == 1:
            m[:] = -1
        elif rep == 2:
            m[:] = 3
        elif rep == 3:
            m[rng.random(n) < 0.5] = -1
        mapping_dev.copy_(torch.from_numpy(m))
        buf.fill_(-rep - 0.5)   # a fresh buffer per call: its entry contents do not matter
        y.copy_(D.y0)
        H.poison_meta(meta)
        torch.cuda.synchronize()
        print("stream-K graph replay", rep, flush=True)
        g.replay()
        torch.cuda.synchronize()
        H.check_meta(meta, m, ml)
        H.check_sk_clear(meta)
        buf_ref, y_ref, bound, mag = H.oracle_layer(L, m, ml, tokens, True)
        buf_g, y_g = buf.cpu().numpy(), H.bits(y)
        act = m != -1
        assert np.all(buf_g[:, ~act] == np.float32(-rep - 0.5))
        if act.any():
            H.shrink_check(buf_g[:, act], buf_ref[:, act], bound[:, act])
        H.expand_check(y_g, y_ref, y0b, mag, True, H.propagated(L, m, buf_ref, bound))


def _hip_runtime():
    """The HIP runtime library torch has loaded (the same instance, not a second copy)."""
    import ctypes
    with open("/proc/self/maps") as fh:
        paths = {ln.split()[-1] for ln in fh if "libamdhip64" in ln}
    assert paths, "libamdhip64 is not loaded"
    return ctypes.CDLL(sorted(paths)[0])


def _kernel_nodes(graph) -> int:
    import ctypes
    hip = _hip_runtime()
    g = ctypes.c_void_p(graph.raw_cuda_graph())
    count = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(g, None, ctypes.byref(count)) == 0
    nodes = (ctypes.c_void_p * count.value)()
    assert hip.hipGraphGetNodes(g, nodes, ctypes.byref(count)) == 0
    kinds = []
    for i in range(count.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        kinds.append(t.value)
    return sum(1 for k in kinds if k == 0)   # hipGraphNodeTypeKernel


@pytest.mark.parametrize("name,n,layer", [("decode", None, 0), ("tiny", None, 0), ("zipf", 1000, 0),
                                          ("zipf", 3000, 0), ("zipf", None, 1), ("prefill", 600, 0),
                                          ("large", 300, 0)])
@pytest.mark.parametrize("prep", [True, False])
def test_launch_count_query_matches_the_calls(name, n, layer, prep):
    """lora_shrink_expand_launches against the kernels a captured call really
    launches: one inside the one-launch range, else the separate calls (with
    the zeroing of buf's active rows before a split-K shrink)."""
    sgl = H.lib()
    wl = workloads.make_workload(name, num_tokens=n)
    L = wl.layers[layer]
    D = H.DevLayer(L)
    ntok = wl.mapping.numel()
    mapping = wl.mapping.to("cuda")
    meta = sgl.LoraMeta(wl.spec.max_loras, ntok)
    buf = torch.zeros((len(L.spec.slices), ntok, L.spec.rank), dtype=torch.float32, device="cuda")
    y = D.y0.clone()
    sgl.lora_prepare_meta(mapping, meta)
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph(keep_graph=True)
    except TypeError:
        pytest.skip("this torch cannot keep the captured graph")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        if prep:
            sgl.lora_prepare_shrink_expand(mapping, D.x, D.a, D.b, D.bias, buf, y, meta, L.spec.scale)
        else:
            sgl.lora_shrink_expand(D.x, D.a, D.b, D.bias, buf, y, meta, L.spec.scale)
    torch.cuda.current_stream().wait_stream(s)
    want = sgl.lora_shrink_expand_launches(ntok, wl.spec.max_loras, L.spec.hidden, len(L.spec.slices),
                                           L.spec.rank, prep)
    got = _kernel_nodes(g)
    print("launches", name, n, prep, want, got, flush=True)
    assert got == want
