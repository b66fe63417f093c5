"""lora_shrink_expand_noalloc (the entry point for callers that cannot
allocate: its fp32 buffer is the library's static device array) against
lora_shrink_expand on the same inputs, two calls in a row with the second
batch smaller, through the C ABI; plus the size limit."""
import numpy as np
import pytest
import torch

import workloads
import _harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    from segmented_gather_lora_amd import _build
    _build.ensure_built()
    torch.cuda.set_device(0)
    yield


def _both(wl, add_inputs=True, offset_start=0):
    """y from lora_shrink_expand (caller's buffer) and from the no-alloc call,
    each from the same y0 on a freshly prepared batch."""
    sgl = H.lib()
    mapping = wl.mapping.numpy()
    n, ml = mapping.size, wl.spec.max_loras
    L = wl.layers[0]
    D = H.DevLayer(L)
    S, r, O = len(L.spec.slices), L.spec.rank, sum(L.spec.slices)
    meta = sgl.LoraMeta(ml, n)
    sgl.lora_prepare_meta(wl.mapping.to("cuda"), meta)
    ldy = offset_start + O
    y0 = torch.zeros((n, ldy), dtype=torch.bfloat16)
    y0[:, offset_start:] = L.y0
    buf = torch.full((S, n, r), H.BUF_POISON, dtype=torch.float32, device="cuda")
    ya = y0.to("cuda")
    sgl.lora_shrink_expand(D.x, D.a, D.b, D.bias, buf, ya, meta, L.spec.scale, offset_start=offset_start,
                           add_inputs=add_inputs)
    yb = y0.to("cuda")
    sgl.lora_shrink_expand_noalloc(D.x, D.a, D.b, D.bias, yb, meta, L.spec.scale, offset_start=offset_start,
                                   add_inputs=add_inputs)
    torch.cuda.synchronize()
    H.check_sync_clear(meta, n)
    return L, mapping, ml, H.bits(y0), H.bits(ya), H.bits(yb)


def _check(L, mapping, ml, y0b, ya, yb, add_inputs=True, offset_start=0):
    """The no-alloc call's y to the parity bar against lora_shrink_expand's y
    and against the oracle; -1 rows and columns outside the slices untouched."""
    n = mapping.size
    m = np.where((mapping < -1) | (mapping >= ml), -1, mapping).astype(np.int32)
    neg = m == -1
    assert np.array_equal(yb[neg], y0b[neg])
    assert np.array_equal(yb[:, :offset_start], y0b[:, :offset_start])
    tokens = np.arange(n, dtype=np.int32)
    buf_ref, y_ref, bound, mag = H.oracle_layer(L, m, ml, tokens, add_inputs, y_in=y0b, offset_start=offset_start)
    extra = H.propagated(L, m, buf_ref, bound)
    cols = slice(offset_start, None)
    # against the call it is a variant of: both sides carry the shrink's rounding
    H.expand_check(yb[:, cols], ya[:, cols], y0b[:, cols], mag, add_inputs, 2 * extra)
    H.expand_check(yb[:, cols], y_ref[:, cols], y0b[:, cols], mag, add_inputs, extra)


@pytest.mark.parametrize("first,second", [
    (("decode", None), ("decode", 100)),          # one launch (LoRA-major), then tile-major
    (("prefill", 700), ("tiny", None)),           # separate kernels, then a one-launch tiny batch
    (("zipf", None), ("zipf", 300)),              # down layer: split-K shrink into the array, then one launch
])
def test_noalloc_matches_lora_shrink_expand(first, second):
    for name, n in (first, second):
        wl = workloads.make_workload(name, num_tokens=n)
        if name == "zipf":
            wl = workloads.Workload(wl.spec, wl.mapping, [wl.layers[1]])   # the down layer (split K)
        print("noalloc", name, n, flush=True)
        _check(*_both(wl))


def test_noalloc_offset_and_overwrite():
    wl = workloads.random_case(731, 300, 1032, (264, 8, 520), 16, 9, bias=True)
    L, m, ml, y0b, ya, yb = _both(wl, add_inputs=False, offset_start=8)
    _check(L, m, ml, y0b, ya, yb, add_inputs=False, offset_start=8)


def test_noalloc_rejects_beyond_the_array():
    sgl = H.lib()
    n, h, r = 65537, 8, 128          # 1 slice: 65537 * 128 floats > 8388608
    meta = sgl.LoraMeta(1, n)
    sgl.lora_prepare_meta(torch.zeros(n, dtype=torch.int32, device="cuda"), meta)
    x = torch.zeros((n, h), dtype=torch.bfloat16, device="cuda")
    a = [torch.zeros((1, r, h), dtype=torch.bfloat16, device="cuda")]
    b = [torch.zeros((1, 8, r), dtype=torch.bfloat16, device="cuda")]
    y = torch.zeros((n, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sgl.LoraError) as e:
        sgl.lora_shrink_expand_noalloc(x, a, b, None, y, meta, 1.0)
    assert e.value.status == sgl.LORA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert int(y.abs().sum()) == 0
