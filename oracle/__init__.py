"""CPU oracle for the segmented-gather multi-LoRA path (ctypes over
``lora_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are its only users.  It shares no code with the
HIP library and never imports it.  The arithmetic lives in ``lora_oracle.c``;
this file only marshals numpy arrays.  Each function's docstring names the
page passage it follows (vLLM API documentation: the "lora_kernel_metadata"
page, class LoRAKernelMeta; the "punica_gpu" page, PunicaWrapperGPU; the
"punica_tpu" page, PunicaWrapperTPU).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")
_lib = None

ORACLE_OK = 0
ORACLE_BAD_ID = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) next to its source."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [dbl]
        lib.oracle_bf16_to_double.restype = dbl
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_start_loc.restype = None
        lib.oracle_start_loc.argtypes = [P, i32, i32, P]
        lib.oracle_prepare.restype = i32
        lib.oracle_prepare.argtypes = [P, i32, i32, P, P, P, P, P, P]
        lib.oracle_shrink.restype = i32
        lib.oracle_shrink.argtypes = [P, i64, i32, i32, P, i32, i32, i32, P, P, dbl, P, i32, P, i32]
        lib.oracle_expand.restype = i32
        lib.oracle_expand.argtypes = [P, i32, i32, P, P, P, i32, P, i64, i32, i32, P, i32, P, i32, P, i32]
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def double_to_bf16(v: float) -> int:
    """Round-to-nearest-even of a double to a bfloat16 bit pattern."""
    return int(_load().oracle_double_to_bf16(float(v)))


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits)))


def start_loc(counts: Sequence[int], n_active: int, max_loras: int) -> np.ndarray:
    """Segment starts (LoRAKernelMeta.make comments and prepare_tensors:
    first entry 0, then the running sum of the counts, zero padding)."""
    c = _c(counts, np.int32)
    out = np.empty(max_loras + 2, np.int32)
    _load().oracle_start_loc(_ptr(c), int(n_active), int(max_loras), _ptr(out))
    return out


def prepare(mapping: np.ndarray, max_loras: int, max_num_tokens: Optional[int] = None):
    """LoRAKernelMeta._reset + prepare_tensors.  Returns a dict with
    ``mapping``, ``sorted`` (None when the no-LoRA flag is set: the pages
    leave those buffers untouched), ``active_ids``, ``counts``,
    ``start_loc``, ``no_lora`` and ``status``."""
    m = _c(mapping, np.int32)
    n = m.size
    cap = max(n, max_num_tokens or 0, 1)
    mc = np.full(cap, np.iinfo(np.int32).min, np.int32)
    srt = np.full(cap, np.iinfo(np.int32).min, np.int32)
    act = np.empty(max_loras + 1, np.int32)
    cnt = np.empty(max_loras + 1, np.int32)
    sl = np.empty(max_loras + 2, np.int32)
    flag = np.zeros(1, np.int32)
    st = _load().oracle_prepare(_ptr(m), n, int(max_loras), _ptr(mc), _ptr(srt), _ptr(act),
                                _ptr(cnt), _ptr(sl), _ptr(flag))
    no_lora = bool(flag[0])
    return dict(mapping=None if no_lora else mc[:n], sorted=None if no_lora else srt[:n],
                active_ids=act, counts=cnt, start_loc=sl, no_lora=no_lora, status=int(st))


def shrink(x_bits: np.ndarray, lora_a_bits: Sequence[np.ndarray], buf: np.ndarray,
           mapping: np.ndarray, scale: float, max_loras: int,
           tokens: Optional[np.ndarray] = None, with_bound: bool = False, nthreads: int = 1):
    """PunicaWrapperGPU.add_shrink semantics (per slice
    ``buf[i] += (x @ A_i[id]) * scale``, fp32 buffer as in add_lora_linear).

    ``x_bits`` uint16 [N][H]; ``lora_a_bits`` per slice uint16
    [max_loras][r][H]; ``buf`` float32 [S][N][r], updated in place.
    Returns (status, bound) where bound is |scale| * sum |x * a| per computed
    element ([S][ntok][r]) or None."""
    x = _c(x_bits, np.uint16)
    n, h = x.shape
    s = len(lora_a_bits)
    a = [_c(t, np.uint16) for t in lora_a_bits]
    r = a[0].shape[1]
    assert buf.dtype == np.float32 and buf.flags.c_contiguous and buf.shape == (s, n, r)
    m = _c(mapping, np.int32)
    aptrs = (ctypes.c_void_p * s)(*[t.ctypes.data for t in a])
    tok = None if tokens is None else _c(tokens, np.int32)
    cnt = n if tok is None else tok.size
    bound = np.empty((s, cnt, r), np.float64) if with_bound else None
    st = _load().oracle_shrink(_ptr(x), h, n, h, aptrs, s, r, int(max_loras), _ptr(buf), _ptr(m),
                               float(scale), _ptr(tok), cnt, _ptr(bound), int(nthreads))
    return int(st), bound


def expand(buf: np.ndarray, lora_b_bits: Sequence[np.ndarray], bias_bits, y_bits: np.ndarray,
           mapping: np.ndarray, max_loras: int, offset_start: int = 0, add_inputs: bool = True,
           tokens: Optional[np.ndarray] = None, with_mag: bool = False, nthreads: int = 1):
    """PunicaWrapperGPU.add_expand semantics with the bias of
    PunicaWrapperTPU._apply_bias folded in: per slice, columns
    ``[off_i, off_i + O_i)`` of y get ``buf[i][t] @ B_i[id]^T + bias_i[id]``.

    ``buf`` float32 [S][N][r]; ``lora_b_bits`` per slice uint16
    [max_loras][O_i][r]; ``bias_bits`` None or per slice (None | uint16
    [max_loras][O_i]); ``y_bits`` uint16 [N][ldy], updated in place.
    Returns (status, mag) with mag = add_inputs*|y0| + |bias| + sum |buf*b|
    per computed element ([ntok][sum O_i]) or None."""
    b = _c(buf, np.float32)
    s, n, r = b.shape
    w = [_c(t, np.uint16) for t in lora_b_bits]
    assert len(w) == s
    widths = np.array([t.shape[1] for t in w], np.int32)
    bptrs = (ctypes.c_void_p * s)(*[t.ctypes.data for t in w])
    if bias_bits is None:
        biasptrs = None
        keep = []
    else:
        keep = [None if t is None else _c(t, np.uint16) for t in bias_bits]
        biasptrs = (ctypes.c_void_p * s)(*[None if t is None else t.ctypes.data for t in keep])
    assert y_bits.dtype == np.uint16 and y_bits.flags.c_contiguous
    ldy = y_bits.shape[1]
    m = _c(mapping, np.int32)
    tok = None if tokens is None else _c(tokens, np.int32)
    cnt = n if tok is None else tok.size
    mag = np.empty((cnt, int(widths.sum())), np.float64) if with_mag else None
    st = _load().oracle_expand(_ptr(b), n, r, bptrs, biasptrs, _ptr(widths), s, _ptr(y_bits), ldy,
                               int(offset_start), int(bool(add_inputs)), _ptr(m), int(max_loras),
                               _ptr(tok), cnt, _ptr(mag), int(nthreads))
    del keep
    return int(st), mag
