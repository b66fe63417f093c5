"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU.  No call
here reaches a kernel launch (no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sgl():
    from segmented_gather_lora_amd import _build
    _build.ensure_built()
    import segmented_gather_lora_amd as m
    return m


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(lora_[a-z_]+)\s*\(", src))
    return names


def test_exports_every_declared_symbol(sgl):
    declared = _declared()
    assert declared == set(sgl.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", sgl._LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (lora_[a-z_]+)$", out, flags=re.M))
    assert declared <= exported
    for n in declared:
        assert getattr(sgl.lib, n) is not None


def test_status_strings(sgl):
    for code in range(-11, 1):
        s = sgl.lora_status_string(code)
        assert s and s != "unknown status"
    assert sgl.lora_status_string(-100) == "unknown status"


def test_meta_bytes_and_bind(sgl):
    assert sgl.lora_meta_bytes(0, 10) == 0
    assert sgl.lora_meta_bytes(1024, 10) == 0
    assert sgl.lora_meta_bytes(3, -1) == 0
    nb = sgl.lora_meta_bytes(3, 64)
    assert nb >= 4 * (64 + 64 + 4 + 4 + 5 + 2)
    base = 0x7f0000000000
    m = sgl.lora_meta_bind(base, nb, 3, 64)
    spans = [(m.token_lora_mapping, 4 * 64), (m.token_indices_sorted, 4 * 64), (m.active_lora_ids, 16),
             (m.num_tokens_per_lora, 16), (m.lora_token_start_loc, 20), (m.no_lora_flag, 4), (m.status, 4),
             (m.sync, 4 * 128 * (64 // 16 + 4 + 1))]
    spans.sort()
    for (p, sz), (q, _) in zip(spans, spans[1:]):
        assert p + sz <= q
    for p, sz in spans:
        assert p % 256 == 0 and base <= p and p + sz <= base + nb
    assert m.num_tokens == -1 and m.max_loras == 3 and m.max_num_tokens == 64 and not m.host_no_lora
    st = sgl.lora_meta_t()
    L = sgl.lib
    assert L.lora_meta_bind(base + 16, nb, 3, 64, ctypes.byref(st)) == sgl.LORA_ERR_BUFFER
    assert L.lora_meta_bind(base, nb - 1, 3, 64, ctypes.byref(st)) == sgl.LORA_ERR_BUFFER
    assert L.lora_meta_bind(None, nb, 3, 64, ctypes.byref(st)) == sgl.LORA_ERR_NULL
    assert L.lora_meta_bind(base, nb, 0, 64, ctypes.byref(st)) == sgl.LORA_ERR_MAX_LORAS


def _fake_meta(sgl, n_prepared):
    base = 0x7f0000000000
    m = sgl.lora_meta_bind(base, sgl.lora_meta_bytes(4, 128), 4, 128)
    m.num_tokens = n_prepared
    return m


def test_prepare_rejects(sgl):
    L = sgl.lib
    m = _fake_meta(sgl, -1)
    assert L.lora_prepare_meta(0x1000, 129, ctypes.byref(m), None) == sgl.LORA_ERR_NUM_TOKENS
    assert L.lora_prepare_meta(0x1000, -1, ctypes.byref(m), None) == sgl.LORA_ERR_NUM_TOKENS
    assert L.lora_prepare_meta(None, 5, ctypes.byref(m), None) == sgl.LORA_ERR_NULL
    assert L.lora_prepare_meta(0x1000, 5, None, None) == sgl.LORA_ERR_NULL
    m.max_loras = 2000
    assert L.lora_prepare_meta(0x1000, 5, ctypes.byref(m), None) == sgl.LORA_ERR_MAX_LORAS


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_shrink_rejects(sgl):
    L = sgl.lib
    A = _ptrs(0x10000, 0x20000, 0x30000)
    X, BUF = 0x40000, 0x50000
    m = _fake_meta(sgl, 32)
    ok = dict(x=X, ldx=64, n=32, h=64, a=A, s=3, r=16, buf=BUF)

    def call(**kw):
        a = dict(ok, **kw)
        return L.lora_shrink(a["x"], a["ldx"], a["n"], a["h"], a["a"], a["s"], a["r"], a["buf"],
                             ctypes.byref(kw.get("meta", m)), 1.0, None)
    assert call(n=31) == sgl.LORA_ERR_NUM_TOKENS
    assert call(meta=_fake_meta(sgl, -1)) == sgl.LORA_ERR_NUM_TOKENS
    assert call(s=0) == sgl.LORA_ERR_SLICES and call(s=9) == sgl.LORA_ERR_SLICES
    assert call(r=4) == sgl.LORA_ERR_SHAPE and call(r=12) == sgl.LORA_ERR_SHAPE and call(r=136) == sgl.LORA_ERR_SHAPE
    assert call(h=60) == sgl.LORA_ERR_SHAPE and call(ldx=56) == sgl.LORA_ERR_SHAPE and call(ldx=68) == sgl.LORA_ERR_SHAPE
    assert call(x=None) == sgl.LORA_ERR_NULL and call(buf=None) == sgl.LORA_ERR_NULL
    assert call(a=_ptrs(0x10000, None, 0x30000)) == sgl.LORA_ERR_NULL
    assert call(a=_ptrs(0x10000, 0x20008, 0x30000)) == sgl.LORA_ERR_ALIGN
    assert call(x=X + 8) == sgl.LORA_ERR_ALIGN and call(buf=BUF + 4) == sgl.LORA_ERR_ALIGN
    # nothing to do for an empty batch: returns without launching
    assert call(n=0, meta=_fake_meta(sgl, 0)) == sgl.LORA_OK


def test_expand_rejects(sgl):
    L = sgl.lib
    B = _ptrs(0x10000, 0x20000)
    W = (ctypes.c_int * 2)(64, 32)
    BUF, Y = 0x50000, 0x60000
    m = _fake_meta(sgl, 32)
    ok = dict(buf=BUF, n=32, r=16, b=B, bias=None, w=W, s=2, y=Y, ldy=96, off=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.lora_expand(a["buf"], a["n"], a["r"], a["b"], a["bias"], a["w"], a["s"], a["y"], a["ldy"],
                             a["off"], 1, ctypes.byref(kw.get("meta", m)), None)
    assert call(n=33) == sgl.LORA_ERR_NUM_TOKENS
    assert call(s=0) == sgl.LORA_ERR_SLICES
    assert call(w=(ctypes.c_int * 2)(64, 12)) == sgl.LORA_ERR_SHAPE
    assert call(w=(ctypes.c_int * 2)(64, 0)) == sgl.LORA_ERR_SHAPE
    assert call(ldy=88) == sgl.LORA_ERR_SHAPE
    assert call(off=8, ldy=96) == sgl.LORA_ERR_SHAPE       # 8 + 96 > 96
    assert call(off=4, ldy=104) == sgl.LORA_ERR_SHAPE
    assert call(r=20) == sgl.LORA_ERR_SHAPE
    assert call(b=_ptrs(0x10000, None)) == sgl.LORA_ERR_NULL
    assert call(bias=_ptrs(None, 0x70008)) == sgl.LORA_ERR_ALIGN
    assert call(y=Y + 2) == sgl.LORA_ERR_ALIGN and call(buf=BUF + 8) == sgl.LORA_ERR_ALIGN
    assert call(y=None) == sgl.LORA_ERR_NULL
    assert call(n=0, meta=_fake_meta(sgl, 0)) == sgl.LORA_OK


def test_shrink_expand_rejects(sgl):
    """The fused call checks both halves' arguments, before any launch."""
    L = sgl.lib
    A = _ptrs(0x10000, 0x20000)
    B = _ptrs(0x30000, 0x40000)
    W = (ctypes.c_int * 2)(64, 32)
    X, BUF, Y = 0x50000, 0x60000, 0x70000
    m = _fake_meta(sgl, 32)
    ok = dict(x=X, ldx=64, n=32, h=64, a=A, b=B, bias=None, w=W, s=2, r=16, buf=BUF, y=Y, ldy=96, off=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.lora_shrink_expand(a["x"], a["ldx"], a["n"], a["h"], a["a"], a["b"], a["bias"], a["w"], a["s"],
                                    a["r"], a["buf"], a["y"], a["ldy"], a["off"], 1,
                                    ctypes.byref(kw.get("meta", m)), 1.0, None)
    assert call(n=31) == sgl.LORA_ERR_NUM_TOKENS
    assert call(s=0) == sgl.LORA_ERR_SLICES
    assert call(h=60) == sgl.LORA_ERR_SHAPE and call(r=12) == sgl.LORA_ERR_SHAPE
    assert call(w=(ctypes.c_int * 2)(64, 12)) == sgl.LORA_ERR_SHAPE and call(ldy=88) == sgl.LORA_ERR_SHAPE
    assert call(a=_ptrs(0x10000, None)) == sgl.LORA_ERR_NULL and call(b=_ptrs(None, 0x40000)) == sgl.LORA_ERR_NULL
    assert call(x=X + 8) == sgl.LORA_ERR_ALIGN and call(y=Y + 2) == sgl.LORA_ERR_ALIGN
    mm = _fake_meta(sgl, 32)
    mm.sync = None
    assert call(meta=mm) == sgl.LORA_ERR_NULL
    assert call(n=0, meta=_fake_meta(sgl, 0)) == sgl.LORA_OK


def test_product_path_has_no_fallback():
    # the package imports nothing from the oracle and fails loudly without the library
    pkg = os.path.join(ROOT, "segmented_gather_lora_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("oracle/", ""), f
    init = open(os.path.join(pkg, "__init__.py")).read()
    assert "raise ImportError" in init
