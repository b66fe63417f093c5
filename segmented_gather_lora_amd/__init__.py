"""Python binding of liblora_mi355x.so (segmented-gather multi-LoRA on MI355X).

Argument marshalling only: every step runs in the library's HIP kernels.
Torch tensors supply device memory and the current HIP stream.  The names
mirror the C ABI in include/lora_mi355x.h:

    lora_meta_bytes, lora_meta_bind, lora_prepare_meta, lora_shrink,
    lora_expand, lora_shrink_expand, lora_prepare_shrink_expand,
    lora_shrink_expand_noalloc, lora_status_string, and the measurement aids
    lora_shrink_expand_launches, lora_prepare_meta_launches, lora_probe_read,
    lora_probe_empty

plus ``LoraMeta``, a holder that owns one device region sized by
``lora_meta_bytes`` (LoRAKernelMeta.make on the "lora_kernel_metadata" page)
and exposes its arrays as tensor views.

The library is loaded on the first call; that call raises ImportError if the
library has not been built (``python -m segmented_gather_lora_amd._build``):
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

from ._build import LIB as _LIB_PATH

LORA_OK = 0
LORA_ERR_NULL = -1
LORA_ERR_NUM_TOKENS = -2
LORA_ERR_SHAPE = -3
LORA_ERR_MAX_LORAS = -4
LORA_ERR_BUFFER = -5
LORA_ERR_ALIGN = -6
LORA_ERR_SLICES = -7
LORA_ERR_LAUNCH = -8
LORA_ERR_ID_RANGE = -9
LORA_ERR_SYNC = -10
LORA_ERR_SCRATCH = -11

LORA_MAX_LORAS = 1023
LORA_MAX_SLICES = 8
LORA_MAX_RANK = 128

EXPORTED = ("lora_meta_bytes", "lora_meta_bind", "lora_prepare_meta", "lora_shrink",
            "lora_expand", "lora_shrink_expand", "lora_prepare_shrink_expand", "lora_shrink_expand_launches",
            "lora_prepare_meta_launches",
            "lora_status_string", "lora_probe_read", "lora_probe_empty", "lora_shrink_expand_noalloc")


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, lora_status_string(status), status))


class lora_meta_t(ctypes.Structure):
    _fields_ = [
        ("token_lora_mapping", ctypes.c_void_p),
        ("token_indices_sorted", ctypes.c_void_p),
        ("active_lora_ids", ctypes.c_void_p),
        ("num_tokens_per_lora", ctypes.c_void_p),
        ("lora_token_start_loc", ctypes.c_void_p),
        ("no_lora_flag", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("sync", ctypes.c_void_p),
        ("host_no_lora", ctypes.c_void_p),
        ("max_loras", ctypes.c_int32),
        ("max_num_tokens", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError("liblora_mi355x.so is not built (%s); run "
                          "`python -m segmented_gather_lora_amd._build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.lora_meta_bytes.restype = ctypes.c_size_t
    lib.lora_meta_bytes.argtypes = [i32, i32]
    lib.lora_meta_bind.restype = i32
    lib.lora_meta_bind.argtypes = [P, ctypes.c_size_t, i32, i32, ctypes.POINTER(lora_meta_t)]
    lib.lora_prepare_meta.restype = i32
    lib.lora_prepare_meta.argtypes = [P, i32, ctypes.POINTER(lora_meta_t), P]
    lib.lora_shrink.restype = i32
    lib.lora_shrink.argtypes = [P, i64, i32, i32, P, i32, i32, P, ctypes.POINTER(lora_meta_t),
                                ctypes.c_float, P]
    lib.lora_expand.restype = i32
    lib.lora_expand.argtypes = [P, i32, i32, P, P, P, i32, P, i64, i32, i32,
                                ctypes.POINTER(lora_meta_t), P]
    lib.lora_shrink_expand.restype = i32
    lib.lora_shrink_expand.argtypes = [P, i64, i32, i32, P, P, P, P, i32, i32, P, P, i64, i32, i32,
                                       ctypes.POINTER(lora_meta_t), ctypes.c_float, P]
    lib.lora_shrink_expand_noalloc.restype = i32
    lib.lora_shrink_expand_noalloc.argtypes = [P, i64, i32, i32, P, P, P, P, i32, i32, P, i64, i32, i32,
                                               ctypes.POINTER(lora_meta_t), ctypes.c_float, P]
    lib.lora_prepare_shrink_expand.restype = i32
    lib.lora_prepare_shrink_expand.argtypes = [P, i32, P, i64, i32, P, P, P, P, i32, i32, P, P, i64, i32, i32,
                                               ctypes.POINTER(lora_meta_t), ctypes.c_float, P]
    lib.lora_shrink_expand_launches.restype = i32
    lib.lora_shrink_expand_launches.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.lora_prepare_meta_launches.restype = i32
    lib.lora_prepare_meta_launches.argtypes = [i32, i32]
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_status_string.argtypes = [i32]
    lib.lora_probe_read.restype = i32
    lib.lora_probe_read.argtypes = [P, ctypes.c_size_t, i32, P, P]
    lib.lora_probe_empty.restype = i32
    lib.lora_probe_empty.argtypes = [i32, P]
    return lib


_handle = None


def _lib() -> ctypes.CDLL:
    """The library, loaded on first use (the builder imports this package
    before any library exists); raises ImportError when it is not built."""
    global _handle
    if _handle is None:
        _handle = _load()
    return _handle


def __getattr__(name):
    if name == "lib":
        return _lib()
    raise AttributeError(name)


def lora_status_string(status: int) -> str:
    return _lib().lora_status_string(int(status)).decode()


def lora_shrink_expand_launches(num_tokens: int, max_loras: int, hidden: int, num_slices: int, rank: int,
                                with_prepare: bool) -> int:
    """Kernel launches of lora_shrink_expand / lora_prepare_shrink_expand for
    such a layer: 1 inside the one-launch range, else the separate calls'
    count (host only)."""
    st = _lib().lora_shrink_expand_launches(int(num_tokens), int(max_loras), int(hidden), int(num_slices),
                                            int(rank), 1 if with_prepare else 0)
    if st < 0:
        raise LoraError(st, "lora_shrink_expand_launches")
    return st


def lora_prepare_meta_launches(num_tokens: int, max_loras: int) -> int:
    """Kernel launches of lora_prepare_meta for a batch of this size (host only)."""
    st = _lib().lora_prepare_meta_launches(int(num_tokens), int(max_loras))
    if st < 0:
        raise LoraError(st, "lora_prepare_meta_launches")
    return st


def lora_probe_read(src, workgroups: int, sink, stream=None) -> None:
    """Measurement aid: one streaming read of every byte of the device tensor
    `src` by `workgroups` workgroups (sink: device float32 [>= workgroups])."""
    import torch
    _need(src.is_cuda and src.is_contiguous(), LORA_ERR_SHAPE, "lora_probe_read", "src must be a contiguous device tensor")
    _need(sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= workgroups, LORA_ERR_SHAPE,
          "lora_probe_read", "sink must be a device float32 tensor of >= workgroups elements")
    nbytes = src.numel() * src.element_size()
    _check(_lib().lora_probe_read(src.data_ptr(), nbytes, int(workgroups), sink.data_ptr(), _stream(stream)),
           "lora_probe_read")


def lora_probe_empty(workgroups: int, stream=None) -> None:
    """Measurement aid: one launch of `workgroups` workgroups that do nothing."""
    _check(_lib().lora_probe_empty(int(workgroups), _stream(stream)), "lora_probe_empty")


def _check(st: int, where: str) -> None:
    if st != LORA_OK:
        raise LoraError(st, where)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _need(ok: bool, status: int, where: str, what: str) -> None:
    if not ok:
        raise LoraError(status, "%s: %s" % (where, what))


def _dev(t, dtype, meta, where: str, name: str) -> None:
    """A tensor the kernels read or write through a raw pointer: on meta's
    device, of the element type the C ABI takes, rows of unit element stride.
    What the C ABI cannot see is checked here, so that a host tensor or a
    wrong element type raises instead of reaching a kernel."""
    if not (t.is_cuda and t.device == meta.region.device):
        raise TypeError("%s: %s must be on %s (got %s)" % (where, name, meta.region.device, t.device))
    if t.dtype != dtype:
        raise TypeError("%s: %s must be %s (got %s)" % (where, name, dtype, t.dtype))
    _need(t.dim() == 0 or t.stride(-1) == 1 or t.numel() <= 1, LORA_ERR_SHAPE, where,
          "%s needs unit stride in its last dimension" % name)


def _weights(ts, meta, where: str, name: str, last: Optional[int], mid: Optional[Sequence] = None) -> None:
    """Per-slice weight tensors [>= max_loras][rows][last], contiguous: every
    id below max_loras indexes a whole matrix."""
    import torch
    for i, t in enumerate(ts):
        _dev(t, torch.bfloat16, meta, where, "%s[%d]" % (name, i))
        _need(t.dim() == 3 and t.is_contiguous(), LORA_ERR_SHAPE, where, "%s[%d] must be a contiguous 3-d tensor" % (name, i))
        _need(t.shape[0] >= meta.max_loras, LORA_ERR_SHAPE, where,
              "%s[%d] holds %d LoRAs, fewer than max_loras %d" % (name, i, t.shape[0], meta.max_loras))
        if last is not None:
            _need(t.shape[2] == last, LORA_ERR_SHAPE, where, "%s[%d] last dimension %d != %d" % (name, i, t.shape[2], last))
        if mid is not None:
            _need(t.shape[1] == mid[i], LORA_ERR_SHAPE, where, "%s[%d] rows %d != %d" % (name, i, t.shape[1], mid[i]))


def _bias(bias, widths, meta, where: str) -> None:
    import torch
    if bias is None:
        return
    _need(len(bias) == len(widths), LORA_ERR_SLICES, where, "one bias entry per slice")
    for i, t in enumerate(bias):
        if t is None:
            continue
        _dev(t, torch.bfloat16, meta, where, "bias[%d]" % i)
        _need(t.dim() == 2 and t.is_contiguous() and t.shape[0] >= meta.max_loras and t.shape[1] == widths[i],
              LORA_ERR_SHAPE, where, "bias[%d] must be contiguous [>= max_loras][%d]" % (i, widths[i]))


def _layer_checks(where: str, meta, n: int, x=None, lora_a=None, lora_b=None, bias=None, buf=None, y=None,
                  offset_start: int = 0) -> None:
    """The tensors of one layer call, checked before the library sees them.
    The token count is checked against the batch first, with the status the
    library gives it."""
    import torch
    _need(n == meta.num_tokens, LORA_ERR_NUM_TOKENS, where, "%d tokens, the batch has %d" % (n, meta.num_tokens))
    rank = None
    if buf is not None:
        _dev(buf, torch.float32, meta, where, "buf")
        _need(buf.dim() == 3 and buf.is_contiguous() and buf.shape[1] == n, LORA_ERR_SHAPE, where,
              "buf must be contiguous [S][%d][r]" % n)
        rank = buf.shape[2]
    if x is not None:
        _dev(x, torch.bfloat16, meta, where, "x")
        _need(x.dim() == 2 and x.shape[0] == n, LORA_ERR_SHAPE, where, "x must be [%d][H]" % n)
    if lora_a is not None:
        _weights(lora_a, meta, where, "lora_a", x.shape[1] if x is not None else None,
                 [rank] * len(lora_a) if rank is not None else None)
    if lora_b is not None:
        _weights(lora_b, meta, where, "lora_b", rank)
        widths = [int(t.shape[1]) for t in lora_b]
        _bias(bias, widths, meta, where)
        if y is not None:
            _dev(y, torch.bfloat16, meta, where, "y")
            _need(y.dim() == 2 and y.shape[0] >= n and y.shape[1] >= offset_start + sum(widths), LORA_ERR_SHAPE,
                  where, "y must be [>= %d][>= %d]" % (n, offset_start + sum(widths)))


def _ptr_array(tensors) -> ctypes.Array:
    return (ctypes.c_void_p * len(tensors))(*[None if t is None else t.data_ptr() for t in tensors])


def lora_meta_bytes(max_loras: int, max_num_tokens: int) -> int:
    return int(_lib().lora_meta_bytes(int(max_loras), int(max_num_tokens)))


def lora_meta_bind(dev_ptr: int, nbytes: int, max_loras: int, max_num_tokens: int) -> lora_meta_t:
    m = lora_meta_t()
    _check(_lib().lora_meta_bind(dev_ptr, nbytes, int(max_loras), int(max_num_tokens), ctypes.byref(m)),
           "lora_meta_bind")
    return m


class LoraMeta:
    """One device region holding a batch's kernel metadata (make() on the
    "lora_kernel_metadata" page: allocated once at maximum sizes, reused)."""

    def __init__(self, max_loras: int, max_num_tokens: int, device="cuda"):
        import torch
        nbytes = lora_meta_bytes(max_loras, max_num_tokens)
        if nbytes == 0:
            raise LoraError(LORA_ERR_MAX_LORAS, "lora_meta_bytes")
        # torch's caching allocator returns 512-byte aligned blocks; zero-filled
        # once so that the fused calls' counters start at zero
        self.region = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.struct = lora_meta_bind(self.region.data_ptr(), nbytes, max_loras, max_num_tokens)
        self.max_loras, self.max_num_tokens = max_loras, max_num_tokens

    def _view(self, field: str, n: int):
        off = getattr(self.struct, field) - self.region.data_ptr()
        return self.region[off:off + 4 * n].view(__import__("torch").int32)

    @property
    def num_tokens(self) -> int:
        return self.struct.num_tokens

    def views(self) -> dict:
        """Tensor views of the metadata arrays (sizes as make() allocates)."""
        L, T = self.max_loras, self.max_num_tokens
        return dict(token_lora_mapping=self._view("token_lora_mapping", T),
                    token_indices_sorted=self._view("token_indices_sorted", T),
                    active_lora_ids=self._view("active_lora_ids", L + 1),
                    num_tokens_per_lora=self._view("num_tokens_per_lora", L + 1),
                    lora_token_start_loc=self._view("lora_token_start_loc", L + 2),
                    no_lora_flag=self._view("no_lora_flag", 1),
                    status=self._view("status", 1),
                    sync=self._view("sync", 1))


def lora_prepare_meta(mapping, meta: LoraMeta, stream=None) -> None:
    """mapping: int32 device tensor [N] of LoRA ids (-1 = none)."""
    import torch
    n = mapping.numel()
    if n:
        _dev(mapping, torch.int32, meta, "lora_prepare_meta", "mapping")
        _need(mapping.is_contiguous(), LORA_ERR_SHAPE, "lora_prepare_meta", "mapping must be contiguous")
    _check(_lib().lora_prepare_meta(mapping.data_ptr() if n else None, n, ctypes.byref(meta.struct),
                                 _stream(stream)), "lora_prepare_meta")


def lora_shrink(x, lora_a: Sequence, buf, meta: LoraMeta, scale: float, stream=None) -> None:
    """buf[i][t] += scale * x[t] @ lora_a[i][id_t]^T.
    x bf16 [N][H] (row stride x.stride(0)); lora_a: bf16 [max_loras][r][H] per
    slice; buf fp32 [S][N][r] contiguous."""
    n, h = x.shape
    r = lora_a[0].shape[1]
    _layer_checks("lora_shrink", meta, n, x=x, lora_a=lora_a, buf=buf)
    _need(buf.shape[0] == len(lora_a) and buf.shape[2] == r, LORA_ERR_SHAPE, "lora_shrink", "buf must be [S][N][r]")
    ptrs = _ptr_array(lora_a)
    _check(_lib().lora_shrink(x.data_ptr(), x.stride(0), n, h, ptrs, len(lora_a), r, buf.data_ptr(),
                           ctypes.byref(meta.struct), float(scale), _stream(stream)), "lora_shrink")


def lora_expand(buf, lora_b: Sequence, bias: Optional[Sequence], y, meta: LoraMeta,
                offset_start: int = 0, add_inputs: bool = True, stream=None) -> None:
    """y[t, off_i:off_i+O_i] = (add_inputs ? y : 0) + buf[i][t] @ lora_b[i][id_t]^T + bias[i][id_t].
    buf fp32 [S][N][r]; lora_b bf16 [max_loras][O_i][r] per slice; bias None
    or per slice (None | bf16 [max_loras][O_i]); y bf16 [N][ldy]."""
    s, n, r = buf.shape
    _layer_checks("lora_expand", meta, n, lora_b=lora_b, bias=bias, buf=buf, y=y, offset_start=offset_start)
    _need(len(lora_b) == s, LORA_ERR_SLICES, "lora_expand", "one lora_b entry per buf slice")
    widths = (ctypes.c_int * s)(*[int(t.shape[1]) for t in lora_b])
    bptrs = _ptr_array(lora_b)
    biasptrs = None if bias is None else _ptr_array(bias)
    _check(_lib().lora_expand(buf.data_ptr(), n, r, bptrs, biasptrs, widths, s, y.data_ptr(), y.stride(0),
                           int(offset_start), int(bool(add_inputs)), ctypes.byref(meta.struct),
                           _stream(stream)), "lora_expand")


def lora_shrink_expand(x, lora_a: Sequence, lora_b: Sequence, bias: Optional[Sequence], buf, y,
                       meta: LoraMeta, scale: float, offset_start: int = 0, add_inputs: bool = True,
                       stream=None) -> None:
    """add_lora_linear in one call (one launch for decode-like batches): buf
    is written as a fresh buffer, buf[i][t] = scale * x[t] @ lora_a[i][id_t]^T
    (its entry contents are ignored, rows of -1 tokens untouched), then y as
    lora_expand computes it.  Arguments as for the two calls."""
    n, h = x.shape
    s, _, r = buf.shape
    _layer_checks("lora_shrink_expand", meta, n, x=x, lora_a=lora_a, lora_b=lora_b, bias=bias, buf=buf, y=y,
                  offset_start=offset_start)
    _need(len(lora_a) == s and len(lora_b) == s, LORA_ERR_SLICES, "lora_shrink_expand", "one weight per buf slice")
    widths = (ctypes.c_int * s)(*[int(t.shape[1]) for t in lora_b])
    biasptrs = None if bias is None else _ptr_array(bias)
    _check(_lib().lora_shrink_expand(x.data_ptr(), x.stride(0), n, h, _ptr_array(lora_a), _ptr_array(lora_b),
                                  biasptrs, widths, s, r, buf.data_ptr(), y.data_ptr(), y.stride(0),
                                  int(offset_start), int(bool(add_inputs)), ctypes.byref(meta.struct),
                                  float(scale), _stream(stream)), "lora_shrink_expand")


def lora_shrink_expand_noalloc(x, lora_a: Sequence, lora_b: Sequence, bias: Optional[Sequence], y,
                               meta: LoraMeta, scale: float, offset_start: int = 0, add_inputs: bool = True,
                               stream=None) -> None:
    """lora_shrink_expand without a buffer argument, for callers that cannot
    allocate: the fp32 buffer is the library's static device array (at most
    8388608 floats, S * N * r; larger calls raise LORA_ERR_SCRATCH)."""
    n, h = x.shape
    r = lora_a[0].shape[1]
    s = len(lora_a)
    where = "lora_shrink_expand_noalloc"
    _layer_checks(where, meta, n, x=x, lora_a=lora_a, lora_b=lora_b, bias=bias, y=y, offset_start=offset_start)
    _need(len(lora_b) == s, LORA_ERR_SLICES, where, "one lora_b entry per lora_a entry")
    _need(all(int(t.shape[2]) == r for t in lora_b) and all(int(t.shape[1]) == r for t in lora_a),
          LORA_ERR_SHAPE, where, "lora_a and lora_b must share the rank")
    widths = (ctypes.c_int * s)(*[int(t.shape[1]) for t in lora_b])
    biasptrs = None if bias is None else _ptr_array(bias)
    _check(_lib().lora_shrink_expand_noalloc(x.data_ptr(), x.stride(0), n, h, _ptr_array(lora_a),
                                             _ptr_array(lora_b), biasptrs, widths, s, r, y.data_ptr(), y.stride(0),
                                             int(offset_start), int(bool(add_inputs)), ctypes.byref(meta.struct),
                                             float(scale), _stream(stream)), where)


def lora_prepare_shrink_expand(mapping, x, lora_a: Sequence, lora_b: Sequence, bias: Optional[Sequence], buf, y,
                               meta: LoraMeta, scale: float, offset_start: int = 0, add_inputs: bool = True,
                               stream=None) -> None:
    """lora_prepare_meta(mapping) then lora_shrink_expand (buf written as a
    fresh buffer), in one call (one launch for small decode-like batches)."""
    import torch
    n = mapping.numel()
    _, h = x.shape
    s, _, r = buf.shape
    where = "lora_prepare_shrink_expand"
    if n:
        _dev(mapping, torch.int32, meta, where, "mapping")
        _need(mapping.is_contiguous(), LORA_ERR_SHAPE, where, "mapping must be contiguous")
    _need(n <= meta.max_num_tokens, LORA_ERR_NUM_TOKENS, where, "more tokens than the metadata holds")
    saved = meta.struct.num_tokens
    meta.struct.num_tokens = n          # the layer is checked against the batch about to be prepared
    try:
        _layer_checks(where, meta, n, x=x, lora_a=lora_a, lora_b=lora_b, bias=bias, buf=buf, y=y,
                      offset_start=offset_start)
    finally:
        meta.struct.num_tokens = saved
    _need(len(lora_a) == s and len(lora_b) == s, LORA_ERR_SLICES, where, "one weight per buf slice")
    widths = (ctypes.c_int * s)(*[int(t.shape[1]) for t in lora_b])
    biasptrs = None if bias is None else _ptr_array(bias)
    _check(_lib().lora_prepare_shrink_expand(mapping.data_ptr() if n else None, n, x.data_ptr(), x.stride(0), h,
                                          _ptr_array(lora_a), _ptr_array(lora_b), biasptrs, widths, s, r,
                                          buf.data_ptr(), y.data_ptr(), y.stride(0), int(offset_start),
                                          int(bool(add_inputs)), ctypes.byref(meta.struct), float(scale),
                                          _stream(stream)), "lora_prepare_shrink_expand")
