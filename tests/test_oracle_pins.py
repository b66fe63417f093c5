"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle is checked against the pages'
worked example (LoRAKernelMeta.make comments), torch's CPU sort/unique/cumsum
(the library routines prepare_tensors itself calls), a numpy dense masked
brute force of the shrink/expand semantics (PunicaWrapperGPU.add_shrink /
add_expand docstrings, PunicaWrapperTPU._apply_bias), closed forms and
invariants.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from _numeric import bits_to_f64, f64_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------- metadata

def test_scan_pin_worked_example():
    g = _golden()
    p = g["printed"]
    out = oracle.start_loc(p["num_tokens_per_lora"], len(p["num_tokens_per_lora"]), g["max_loras"])
    assert out.tolist() == p["lora_token_start_loc"]          # max_loras + 2 = 5 entries


def test_scan_zero_tail():
    out = oracle.start_loc([4, 1], 2, 6)
    assert out.tolist() == [0, 4, 5, 0, 0, 0, 0, 0]


def test_prepare_pin_worked_example_multiset():
    g = _golden()
    want = g["prepare_from_multiset"]
    ids = [-1] * 3 + [0] * 10 + [2] * 5 + [1] * 2
    rng = np.random.default_rng(7)
    mapping = np.array(ids, np.int32)[rng.permutation(len(ids))]
    r = oracle.prepare(mapping, g["max_loras"])
    assert not r["no_lora"] and r["status"] == 0
    assert r["active_ids"].tolist() == want["active_lora_ids"]
    assert r["counts"].tolist() == want["num_tokens_per_lora"]
    assert r["start_loc"].tolist() == want["lora_token_start_loc"]
    # sorted: ids ascending, ties in token order
    srt = r["sorted"]
    keys = mapping[srt]
    assert np.all(np.diff(keys) >= 0)
    for k in np.unique(keys):
        assert np.all(np.diff(srt[keys == k]) > 0)
    assert r["mapping"].tolist() == mapping.tolist()


def _torch_meta(mapping: np.ndarray, max_loras: int):
    """The pages' own definition via torch CPU library routines."""
    t = torch.from_numpy(mapping.astype(np.int64))
    _, idx = torch.sort(t, stable=True)
    ids, counts = torch.unique(t, sorted=True, return_counts=True)
    cs = torch.cumsum(counts, 0)
    act = np.full(max_loras + 1, -1, np.int32)
    cnt = np.zeros(max_loras + 1, np.int32)
    sl = np.zeros(max_loras + 2, np.int32)
    act[:ids.numel()] = ids.numpy()
    cnt[:counts.numel()] = counts.numpy()
    sl[1:1 + cs.numel()] = cs.numpy()
    return idx.numpy().astype(np.int32), act, cnt, sl


@pytest.mark.parametrize("seed,n,max_loras,neg", [
    (1, 1, 1, 0.0), (2, 5, 3, 0.5), (3, 64, 3, 0.25), (4, 1000, 32, 0.1),
    (5, 4097, 128, 0.2), (6, 3000, 1, 0.0), (7, 777, 1023, 0.3), (8, 2048, 8, 0.0)])
def test_prepare_matches_torch_library(seed, n, max_loras, neg):
    rng = np.random.default_rng(seed)
    m = rng.integers(0, max_loras, n).astype(np.int32)
    m[rng.random(n) < neg] = -1
    if np.all(m == -1):
        m[0] = 0
    r = oracle.prepare(m, max_loras)
    idx, act, cnt, sl = _torch_meta(m, max_loras)
    assert not r["no_lora"] and r["status"] == 0
    assert np.array_equal(r["sorted"], idx)
    assert np.array_equal(r["active_ids"], act)
    assert np.array_equal(r["counts"], cnt)
    assert np.array_equal(r["start_loc"], sl)


def test_prepare_invariants():
    rng = np.random.default_rng(11)
    for n, ml in [(300, 5), (1, 2), (4096, 64)]:
        m = rng.integers(-1, ml, n).astype(np.int32)
        m[0] = 0
        r = oracle.prepare(m, ml)
        na = int((r["counts"] > 0).sum())
        assert r["counts"].sum() == n and r["start_loc"][na] == n
        assert np.all(r["start_loc"][na + 1:] == 0) and np.all(r["active_ids"][na:] == -1)
        assert sorted(r["sorted"].tolist()) == list(range(n))
        for k in range(na):
            seg = r["sorted"][r["start_loc"][k]:r["start_loc"][k + 1]]
            assert np.all(m[seg] == r["active_ids"][k]) and np.all(np.diff(seg) > 0)


@pytest.mark.parametrize("n", [0, 1, 17, 5000])
def test_prepare_no_lora(n):
    m = np.full(n, -1, np.int32)
    r = oracle.prepare(m, 4)
    assert r["no_lora"] and r["sorted"] is None and r["status"] == 0
    assert r["active_ids"].tolist() == [-1] * 5
    assert r["counts"].tolist() == [0] * 5
    assert r["start_loc"].tolist() == [0] * 6
    # torch.all over an empty tensor is True, as the oracle assumes for N = 0
    assert bool(torch.all(torch.from_numpy(m) == -1))


def test_prepare_bad_id_reported_and_treated_as_no_lora():
    m = np.array([0, 5, -2, 1, 1], np.int32)
    r = oracle.prepare(m, 3)
    assert r["status"] == oracle.ORACLE_BAD_ID
    assert r["mapping"].tolist() == [0, -1, -1, 1, 1]
    assert r["active_ids"].tolist() == [-1, 0, 1, -1]
    assert r["counts"].tolist() == [2, 1, 2, 0]


# ----------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_special_values():
    f = oracle.double_to_bf16
    assert f(1.0) == 0x3F80
    assert f(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even
    assert f(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert f(-2.5) == 0xC020
    assert f(2.0 ** -133) == 0x0001                # smallest subnormal
    assert f(2.0 ** -134) == 0x0000                # tie with 0 -> even
    assert f(1.5 * 2.0 ** -134) == 0x0001
    assert f(3.3895313892515355e38) == 0x7F7F      # largest finite
    assert f(2.0 ** 128) == 0x7F80
    assert f(-0.0) == 0x8000


def test_bf16_rounding_matches_torch_on_float32_values():
    # torch's float32 -> bfloat16 conversion rounds to nearest even; on inputs
    # exactly representable in float32 the oracle must agree bit for bit.
    g = torch.Generator().manual_seed(3)
    v = torch.cat([torch.randn(20000, generator=g) * 10.0 ** torch.randint(-30, 30, (20000,), generator=g),
                   (torch.randint(0, 1 << 16, (5000,), generator=g).to(torch.int32) << 16 | 0x8000).view(torch.float32)])
    v = v[torch.isfinite(v)]
    want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(x)) for x in v.tolist()], np.uint16)
    assert np.array_equal(got, want)


def test_independent_rounding_helper_agrees_with_oracle():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    got = np.array([oracle.double_to_bf16(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, f64_to_bf16_bits(v))


# ----------------------------------------------------------------- shrink / expand

def _brute_force(wl, layer_idx=0, buf_in=None, add_inputs=True, offset_start=0, ldy=None):
    """Dense masked form, in float64 with numpy matmuls:
    buf_i = scale * sum_l D_l X A_{i,l}^T ;  Y[:, off_i:off_i+O_i] = Y0 + sum_l D_l (buf_i B_{i,l}^T + 1 bias_{i,l}^T)
    with D_l the diagonal 0/1 mask of tokens whose id is l."""
    L = wl.layers[layer_idx]
    sp = L.spec
    m = wl.mapping.numpy()
    X = bits_to_f64(workloads.bf16_bits(L.x))
    n = X.shape[0]
    S = len(sp.slices)
    buf = np.zeros((S, n, sp.rank))
    for i in range(S):
        A = bits_to_f64(workloads.bf16_bits(L.lora_a[i]))
        for l in range(wl.spec.max_loras):
            D = np.diag((m == l).astype(np.float64))
            buf[i] += sp.scale * D @ X @ A[l].T
    buf32 = buf.astype(np.float32)
    if buf_in is not None:
        buf32 = buf_in
    O = sum(sp.slices)
    ldy = ldy or O
    y0 = np.zeros((n, ldy), np.float64)
    y0[:, offset_start:offset_start + O] = bits_to_f64(workloads.bf16_bits(L.y0))
    Y = y0.copy() if add_inputs else np.zeros_like(y0)
    off = offset_start
    for i, w in enumerate(sp.slices):
        B = bits_to_f64(workloads.bf16_bits(L.lora_b[i]))
        for l in range(wl.spec.max_loras):
            D = np.diag((m == l).astype(np.float64))
            term = D @ buf32[i].astype(np.float64) @ B[l].T
            if L.bias is not None:
                bias = bits_to_f64(workloads.bf16_bits(L.bias[i]))
                term += D @ np.ones((n, 1)) @ bias[l][None, :]
            Y[:, off:off + w] += term
        off += w
    ybits = f64_to_bf16_bits(Y)
    y0bits = np.zeros((n, ldy), np.uint16)
    y0bits[:, offset_start:offset_start + O] = workloads.bf16_bits(L.y0)
    active = m != -1
    ybits[~active] = y0bits[~active]
    return buf32, ybits, y0bits


def _oracle_run(wl, layer_idx=0, buf_in=None, add_inputs=True, offset_start=0, ldy=None):
    L = wl.layers[layer_idx]
    sp = L.spec
    m = wl.mapping.numpy()
    n = m.size
    S = len(sp.slices)
    buf = np.zeros((S, n, sp.rank), np.float32)
    st, bound = oracle.shrink(workloads.bf16_bits(L.x), [workloads.bf16_bits(a) for a in L.lora_a],
                              buf, m, sp.scale, wl.spec.max_loras, with_bound=True)
    assert st == 0
    if buf_in is not None:
        buf = buf_in.copy()
    O = sum(sp.slices)
    ldy = ldy or O
    y = np.zeros((n, ldy), np.uint16)
    y[:, offset_start:offset_start + O] = workloads.bf16_bits(L.y0)
    bias = None if L.bias is None else [workloads.bf16_bits(b) for b in L.bias]
    st, mag = oracle.expand(buf, [workloads.bf16_bits(b) for b in L.lora_b], bias, y, m,
                            wl.spec.max_loras, offset_start=offset_start, add_inputs=add_inputs,
                            with_mag=True)
    assert st == 0
    return buf, y, bound, mag


def _cases():
    return [
        workloads.make_workload("tiny"),
        workloads.random_case(21, 40, 64, (32, 16), 8, 4, bias=True, scale=0.75),
        workloads.random_case(22, 33, 48, (8, 24, 16), 16, 3, bias=True, scale=-1.5),
        workloads.random_case(23, 9, 8, (8,), 8, 2, neg_fraction=0.5),
    ]


@pytest.mark.parametrize("case", range(4))
@pytest.mark.parametrize("add_inputs", [True, False])
def test_oracle_matches_dense_masked_brute_force(case, add_inputs):
    wl = _cases()[case]
    buf_o, y_o, _, _ = _oracle_run(wl, add_inputs=add_inputs)
    buf_b, y_b, _ = _brute_force(wl, add_inputs=add_inputs)
    # both sums are exact-to-double; fp32 stores may differ only at a rounding tie
    np.testing.assert_allclose(buf_o, buf_b, rtol=2.0 ** -23, atol=1e-30)
    # expand from the same fp32 buffer: bf16 results agree bit for bit except
    # where the two double sums straddle a rounding boundary (at most 1 ulp)
    _, y_b2, _ = _brute_force(wl, buf_in=buf_o, add_inputs=add_inputs)
    diff = np.abs(y_o.astype(np.int64) - y_b2.astype(np.int64))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.999


def test_oracle_offset_start_and_wide_rows():
    wl = workloads.random_case(31, 20, 64, (16, 8), 8, 3, bias=True)
    buf_o, y_o, _, _ = _oracle_run(wl, offset_start=8, ldy=48)
    _, y_b, y0 = _brute_force(wl, buf_in=buf_o, offset_start=8, ldy=48)
    diff = np.abs(y_o.astype(np.int64) - y_b.astype(np.int64))
    assert diff.max() <= 1
    assert np.array_equal(y_o[:, :8], y0[:, :8]) and np.array_equal(y_o[:, 32:], y0[:, 32:])


def test_oracle_single_lora_reduces_to_two_matmuls():
    wl = workloads.random_case(41, 30, 64, (24,), 16, 2, neg_fraction=0.0)
    wl.mapping[:] = 1
    L = wl.layers[0]
    X = bits_to_f64(workloads.bf16_bits(L.x))
    A = bits_to_f64(workloads.bf16_bits(L.lora_a[0]))[1]
    B = bits_to_f64(workloads.bf16_bits(L.lora_b[0]))[1]
    buf, y, _, _ = _oracle_run(wl)
    ref_buf = (L.spec.scale * X @ A.T).astype(np.float32)
    np.testing.assert_allclose(buf[0], ref_buf, rtol=2.0 ** -23, atol=1e-30)
    ref_y = f64_to_bf16_bits(bits_to_f64(workloads.bf16_bits(L.y0)) + buf[0].astype(np.float64) @ B.T)
    assert np.abs(y.astype(np.int64) - ref_y.astype(np.int64)).max() <= 1


def test_oracle_closed_forms():
    wl = workloads.random_case(51, 16, 32, (16,), 8, 2, neg_fraction=0.0)
    L = wl.layers[0]
    # x rows are unit vectors e_k: buf = scale * A[id][:, k] exactly
    x = torch.zeros_like(L.x)
    ks = np.arange(16) % 32
    x[np.arange(16), ks] = 1.0
    L.x = x
    buf, _, _, _ = _oracle_run(wl)
    A = bits_to_f64(workloads.bf16_bits(L.lora_a[0]))
    m = wl.mapping.numpy()
    want = np.stack([L.spec.scale * A[m[t], :, ks[t]] for t in range(16)]).astype(np.float32)
    assert np.array_equal(buf[0], want)
    # zero B and no bias: add_inputs keeps y bit for bit, overwrite gives +0
    L.lora_b = [torch.zeros_like(b) for b in L.lora_b]
    _, y, _, _ = _oracle_run(wl, add_inputs=True)
    assert np.array_equal(y, workloads.bf16_bits(L.y0))
    _, y, _, _ = _oracle_run(wl, add_inputs=False)
    assert np.all(y == 0)


def test_oracle_neg_rows_untouched_and_no_lora():
    wl = workloads.random_case(61, 50, 32, (16, 16), 8, 3, bias=True, neg_fraction=0.4)
    m = wl.mapping.numpy()
    buf, y, bound, mag = _oracle_run(wl)
    neg = m == -1
    assert neg.any()
    assert np.all(buf[:, neg, :] == 0) and np.all(bound[:, neg, :] == 0)
    assert np.array_equal(y[neg], workloads.bf16_bits(wl.layers[0].y0)[neg])
    wl.mapping[:] = -1
    buf, y, _, _ = _oracle_run(wl, add_inputs=False)
    assert np.all(buf == 0) and np.array_equal(y, workloads.bf16_bits(wl.layers[0].y0))


def test_oracle_permutation_equivariance_and_scale_linearity():
    wl = workloads.random_case(71, 37, 64, (16, 8), 8, 4, bias=True)
    buf, y, _, _ = _oracle_run(wl)
    perm = np.random.default_rng(1).permutation(37)
    L = wl.layers[0]
    wl2 = workloads.Workload(wl.spec, wl.mapping[perm].clone(), [workloads.Layer(
        L.spec, L.x[perm].clone(), L.lora_a, L.lora_b, L.bias, L.y0[perm].clone())])
    buf2, y2, _, _ = _oracle_run(wl2)
    assert np.array_equal(buf2, buf[:, perm]) and np.array_equal(y2, y[perm])
    # metadata of the permuted mapping: same ids, counts and starts
    a, b = oracle.prepare(wl.mapping.numpy(), 4), oracle.prepare(wl2.mapping.numpy(), 4)
    for k in ("active_ids", "counts", "start_loc"):
        assert np.array_equal(a[k], b[k])
    # doubling the scale doubles the buffer exactly (power-of-two scaling)
    import dataclasses
    wl3 = workloads.Workload(wl.spec, wl.mapping, [workloads.Layer(
        dataclasses.replace(L.spec, scale=2 * L.spec.scale), L.x, L.lora_a, L.lora_b, L.bias, L.y0)])
    buf3, _, _, _ = _oracle_run(wl3)
    assert np.array_equal(buf3, 2 * buf)


def test_oracle_shrink_accumulates_and_token_subset():
    wl = workloads.random_case(81, 24, 32, (8,), 8, 3)
    L = wl.layers[0]
    m = wl.mapping.numpy()
    xb, ab = workloads.bf16_bits(L.x), [workloads.bf16_bits(a) for a in L.lora_a]
    buf = np.zeros((1, 24, 8), np.float32)
    oracle.shrink(xb, ab, buf, m, L.spec.scale, 3)
    buf2 = np.full((1, 24, 8), 0.5, np.float32)
    oracle.shrink(xb, ab, buf2, m, L.spec.scale, 3)
    act = m != -1
    np.testing.assert_allclose(buf2[:, act], buf[:, act] + 0.5, rtol=2.0 ** -23, atol=2.0 ** -24)
    assert np.all(buf2[:, ~act] == 0.5)
    # computing a subset of tokens gives the same rows
    buf3 = np.zeros((1, 24, 8), np.float32)
    toks = np.array([3, 17, 5], np.int32)
    _, bnd = oracle.shrink(xb, ab, buf3, m, L.spec.scale, 3, tokens=toks, with_bound=True)
    assert np.array_equal(buf3[:, toks], buf[:, toks]) and bnd.shape == (1, 3, 8)
