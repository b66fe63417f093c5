"""Run the HIP library and the CPU oracle on the same seeded inputs and compare.

Used by the GPU tests and by ``__graft_entry__.smoke()``.  The oracle's inputs
come from the seeded generator only (never from the HIP path); the HIP path's
outputs are compared element by element on every token (small cases) or on a
seeded sample of tokens (full sizes), and every token with id -1 is checked
bit for bit against the input.

Tolerances (derived from the arithmetic; the parity bar):
  shrink:  |buf_gpu - buf_ref| <= 1e-3 * |scale| * sum_k |x*a|  +  ulp_fp32(buf_ref)
  expand:  |y_gpu - y_ref| <= 2e-2 * (sum_j |buf*b| + |bias|)  +  ulp_bf16(y_ref)
           (+ sum_j delta_j*|b_j| when y_gpu was computed from the GPU's own
           shrink output, delta_j being the shrink tolerance of buf_j).
Metadata: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from _numeric import bits_to_f64

SHRINK_RTOL = 1e-3
EXPAND_RTOL = 2e-2
# Fill of the fp32 buffer handed to the one-launch calls: they write it as a
# fresh buffer ("=", add_lora_linear's zeroed buffer), so active rows must not
# depend on it and rows of -1 tokens must keep it bit for bit.
BUF_POISON = 12345.6789


def lib():
    import segmented_gather_lora_amd as sgl
    return sgl


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def ulp_bf16(b: np.ndarray) -> np.ndarray:
    a = (b.astype(np.int64) & 0x7FFF)
    a = np.minimum(a, 0x7F7E)
    return bits_to_f64(a + 1) - bits_to_f64(a)


# ------------------------------------------------------------------ metadata

def meta_numpy(meta, n: int) -> dict:
    v = {k: t.cpu().numpy().copy() for k, t in meta.views().items()}
    v["token_lora_mapping"] = v["token_lora_mapping"][:n]
    v["token_indices_sorted"] = v["token_indices_sorted"][:n]
    return v


def check_meta(meta, mapping: np.ndarray, max_loras: int, expect_status: int = 0) -> dict:
    n = mapping.size
    got = meta_numpy(meta, n)
    ref = oracle.prepare(mapping, max_loras)
    assert bool(got["no_lora_flag"][0]) == ref["no_lora"], "no-LoRA flag"
    assert np.array_equal(got["active_lora_ids"], ref["active_ids"]), "active_lora_ids"
    assert np.array_equal(got["num_tokens_per_lora"], ref["counts"]), "num_tokens_per_lora"
    assert np.array_equal(got["lora_token_start_loc"], ref["start_loc"]), "lora_token_start_loc"
    if not ref["no_lora"]:
        assert np.array_equal(got["token_indices_sorted"], ref["sorted"]), "token_indices_sorted"
        assert np.array_equal(got["token_lora_mapping"], ref["mapping"]), "token_lora_mapping"
    sgl = lib()
    want_status = sgl.LORA_ERR_ID_RANGE if ref["status"] else 0
    assert int(got["status"][0]) == want_status, "status"
    return got


# ------------------------------------------------------------------ shrink / expand

class DevLayer:
    def __init__(self, L: workloads.Layer, device="cuda"):
        self.spec = L.spec
        self.x = L.x.to(device)
        self.a = [t.to(device) for t in L.lora_a]
        self.b = [t.to(device) for t in L.lora_b]
        self.bias = None if L.bias is None else [t.to(device) for t in L.bias]
        self.y0 = L.y0.to(device)


def sample_tokens(mapping: np.ndarray, k: int, seed: int) -> np.ndarray:
    """Seeded sample: up to k tokens, spread over every id present (the first
    and last token of each segment included) plus random tokens."""
    rng = np.random.default_rng(seed)
    n = mapping.size
    if k >= n:
        return np.arange(n, dtype=np.int32)
    pick = set()
    for idv in np.unique(mapping):
        pos = np.nonzero(mapping == idv)[0]
        pick.add(int(pos[0]))
        pick.add(int(pos[-1]))
        if len(pick) >= k // 2:
            break
    rest = rng.choice(n, size=k, replace=False)
    for t in rest:
        if len(pick) >= k:
            break
        pick.add(int(t))
    return np.array(sorted(pick), dtype=np.int32)


def oracle_layer(L: workloads.Layer, mapping: np.ndarray, max_loras: int, tokens: np.ndarray,
                 add_inputs: bool, buf_in: np.ndarray | None = None, y_in: np.ndarray | None = None,
                 offset_start: int = 0, nthreads: int = 8):
    """The oracle on the sub-batch of `tokens` (each token's result depends
    only on its own row, so a sub-batch gives the same rows)."""
    sp = L.spec
    S, r = len(sp.slices), sp.rank
    msub = mapping[tokens]
    if sp.expand_only:
        # the layer's input is the expand input itself
        buf = np.ascontiguousarray(L.x.numpy()[:, tokens])
        bound = np.zeros(buf.shape, np.float64)
    else:
        xb = workloads.bf16_bits(L.x)[tokens]
        buf = np.zeros((S, tokens.size, r), np.float32)
        if buf_in is not None:
            buf = np.ascontiguousarray(buf_in[:, tokens])
        st, bound = oracle.shrink(xb, [workloads.bf16_bits(a) for a in L.lora_a], buf, msub, sp.scale,
                                  max_loras, with_bound=True, nthreads=nthreads)
        assert st == 0
    if y_in is None:
        y = np.ascontiguousarray(workloads.bf16_bits(L.y0)[tokens])
    else:
        y = np.ascontiguousarray(y_in[tokens])
    bias = None if L.bias is None else [workloads.bf16_bits(b) for b in L.bias]
    st, mag = oracle.expand(buf, [workloads.bf16_bits(b) for b in L.lora_b], bias, y, msub, max_loras,
                            offset_start=offset_start, add_inputs=add_inputs, with_mag=True,
                            nthreads=nthreads)
    assert st == 0
    return buf, y, bound, mag


def shrink_check(buf_gpu: np.ndarray, buf_ref: np.ndarray, bound: np.ndarray) -> float:
    err = np.abs(buf_gpu.astype(np.float64) - buf_ref.astype(np.float64))
    tol = SHRINK_RTOL * bound + np.spacing(np.abs(buf_ref)).astype(np.float64)
    ratio = float((err / tol).max()) if err.size else 0.0
    if ratio > 1.0:
        idx = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError("shrink parity: worst %s gpu=%r ref=%r bound=%r"
                             % (idx, buf_gpu[idx], buf_ref[idx], bound[idx]))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def propagated(L: workloads.Layer, msub: np.ndarray, buf_ref: np.ndarray, bound: np.ndarray) -> np.ndarray:
    """sum_j delta_j * |b_j| per output element, delta_j = shrink tolerance of buf_j."""
    sp = L.spec
    delta = SHRINK_RTOL * bound + np.spacing(np.abs(buf_ref)).astype(np.float64)
    out = np.zeros((msub.size, sum(sp.slices)))
    off = 0
    for i, w in enumerate(sp.slices):
        B = np.abs(bits_to_f64(workloads.bf16_bits(L.lora_b[i])))
        for m in np.unique(msub):
            if m < 0:
                continue
            P = np.nonzero(msub == m)[0]
            out[P, off:off + w] = delta[i][P] @ B[m].T
        off += w
    return out


def expand_check(y_gpu: np.ndarray, y_ref: np.ndarray, y0: np.ndarray, mag: np.ndarray, add_inputs: bool,
                 extra: np.ndarray | float = 0.0) -> dict:
    g = bits_to_f64(y_gpu)
    r = bits_to_f64(y_ref)
    base = mag - (np.abs(bits_to_f64(y0)) if add_inputs else 0.0)
    base = np.maximum(base, 0.0)
    tol = EXPAND_RTOL * base + extra + ulp_bf16(y_ref)
    err = np.abs(g - r)
    ratio = float((err / tol).max()) if err.size else 0.0
    if ratio > 1.0:
        idx = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError("expand parity: worst %s gpu=%r ref=%r base=%r extra=%r"
                             % (idx, g[idx], r[idx], base[idx],
                                extra[idx] if isinstance(extra, np.ndarray) else extra))
    big = np.abs(r) >= 1e-2 * np.maximum(mag, 1e-300)
    rel = float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0
    return dict(ratio=ratio, literal_rel=rel, exact_frac=float((y_gpu == y_ref).mean()) if err.size else 1.0)


def poison_meta(meta) -> None:
    """Overwrite every metadata array (not the fused counters) with garbage."""
    for k, v in meta.views().items():
        if k != "sync":
            v.fill_(-12345)


def run_and_check(wl: workloads.Workload, add_inputs: bool = True, sample: int | None = None,
                  seed: int = 0, offset_start: int = 0, ldy_extra: int = 0, fused: bool = False,
                  prep: bool = False, nthreads: int = 8) -> dict:
    """prepare + (shrink, expand) per layer on the GPU -- or the one
    lora_shrink_expand call per layer with `fused`, and with `prep` the first
    layer's call also prepares the batch (lora_prepare_shrink_expand, on
    poisoned metadata) -- with metadata, buffer and output compared with the
    oracle (all tokens, or a seeded sample)."""
    sgl = lib()
    mapping = wl.mapping.numpy()
    n, ml = mapping.size, wl.spec.max_loras
    meta = sgl.LoraMeta(ml, max(n, 1))
    mapping_dev = wl.mapping.to("cuda")
    if prep:
        fused = True
        poison_meta(meta)
    else:
        sgl.lora_prepare_meta(mapping_dev, meta)
        torch.cuda.synchronize()
        check_meta(meta, mapping, ml)
    # ids outside [-1, max_loras) are reported by prepare and count as -1
    mapping = np.where((mapping < -1) | (mapping >= ml), -1, mapping).astype(np.int32)
    tokens = np.arange(n, dtype=np.int32) if sample is None else sample_tokens(mapping, sample, seed)
    neg = mapping == -1
    stats = dict(shrink_ratio=0.0, expand_ratio=0.0, literal_rel=0.0)
    for L in wl.layers:
        sp = L.spec
        D = DevLayer(L)
        S, r, O = len(sp.slices), sp.rank, sum(sp.slices)
        if sp.expand_only:
            buf = D.x.clone()
        elif fused:
            buf = torch.full((S, n, r), BUF_POISON, dtype=torch.float32, device="cuda")
        else:
            buf = torch.zeros((S, n, r), dtype=torch.float32, device="cuda")
            sgl.lora_shrink(D.x, D.a, buf, meta, sp.scale)
        ldy = offset_start + O + ldy_extra
        y0full = torch.zeros((n, ldy), dtype=torch.bfloat16)
        y0full[:, offset_start:offset_start + O] = L.y0
        # distinct values outside the slice columns, which must stay untouched
        if ldy > O:
            fill = torch.arange(n * ldy, dtype=torch.float32).reshape(n, ldy).remainder(97).to(torch.bfloat16)
            y0full[:, :offset_start] = fill[:, :offset_start]
            y0full[:, offset_start + O:] = fill[:, offset_start + O:]
        y = y0full.to("cuda")
        if prep and not sp.expand_only:
            sgl.lora_prepare_shrink_expand(mapping_dev, D.x, D.a, D.b, D.bias, buf, y, meta, sp.scale,
                                           offset_start=offset_start, add_inputs=add_inputs)
            torch.cuda.synchronize()
            check_meta(meta, wl.mapping.numpy(), ml)
            prep = False
        elif fused and not sp.expand_only:
            sgl.lora_shrink_expand(D.x, D.a, D.b, D.bias, buf, y, meta, sp.scale, offset_start=offset_start,
                                   add_inputs=add_inputs)
        else:
            sgl.lora_expand(buf, D.b, D.bias, y, meta, offset_start=offset_start, add_inputs=add_inputs)
        torch.cuda.synchronize()
        if fused:
            check_sync_clear(meta, n)
        check_sk_clear(meta)
        buf_g = buf.cpu().numpy()
        y_g = bits(y)
        y0b = bits(y0full)
        # untouched: -1 rows everywhere, columns outside the slices everywhere
        if sp.expand_only:
            assert np.array_equal(buf_g, L.x.numpy()), "expand modified its input"
        else:
            fill = np.float32(BUF_POISON) if fused else np.float32(0.0)
            assert np.all(buf_g[:, neg, :] == fill), "shrink touched a -1 row"
        assert np.array_equal(y_g[neg], y0b[neg]), "expand touched a -1 row"
        assert np.array_equal(y_g[:, :offset_start], y0b[:, :offset_start])
        assert np.array_equal(y_g[:, offset_start + O:], y0b[:, offset_start + O:])
        # oracle on the sample
        buf_ref, y_ref, bound, mag = oracle_layer(L, mapping, ml, tokens, add_inputs, y_in=y0b,
                                                  offset_start=offset_start, nthreads=nthreads)
        # rows of -1 tokens were checked bit for bit above; a fresh buffer's
        # stay as they were, so the oracle's zero rows are not compared
        act = ~neg[tokens]
        sr = shrink_check(buf_g[:, tokens][:, act], buf_ref[:, act], bound[:, act])
        extra = propagated(L, mapping[tokens], buf_ref, bound)
        cols = slice(offset_start, offset_start + O)
        ex = expand_check(y_g[tokens][:, cols], y_ref[:, cols], y0b[tokens][:, cols], mag, add_inputs, extra)
        stats["shrink_ratio"] = max(stats["shrink_ratio"], sr)
        stats["expand_ratio"] = max(stats["expand_ratio"], ex["ratio"])
        stats["literal_rel"] = max(stats["literal_rel"], ex["literal_rel"])
    return stats


def sync_words(n: int, max_loras: int) -> int:
    """Counter words of the fused call for a batch of n tokens: 128 per
    16-token tile (ceil(min(n, 24576)/16) + min(slots, n) + 1 tiles)."""
    nn = min(n, 24576)
    return 128 * ((nn + 15) // 16 + min(max_loras + 1, nn) + 1)


def check_sync_clear(meta, n: int) -> None:
    """Every fused call leaves its counters and its accumulation area (after
    the counters of a region bound for max_num_tokens: 64 floats per token)
    at zero, and reports no timeout."""
    v = meta.views()
    off = meta.struct.sync - meta.region.data_ptr()
    words = meta.region[off:off + 4 * sync_words(n, meta.max_loras)].view(torch.int32).cpu().numpy()
    counters = words.reshape(-1, 128)[:, [0, 32] + list(range(64, 128))]
    assert np.all(counters == 0), "fused counters not reset: %s" % counters[np.any(counters != 0, axis=1)][:4]
    acc_off = off + 4 * sync_words(meta.max_num_tokens, meta.max_loras)
    acc = meta.region[acc_off:acc_off + 4 * 64 * min(n, 24576)].view(torch.int32).cpu().numpy()
    assert np.all(acc == 0), "accumulation area not cleared: %d nonzero words" % int((acc != 0).sum())
    assert int(v["status"][0]) in (0, lib().LORA_ERR_ID_RANGE), "status %d" % int(v["status"][0])


def check_sk_clear(meta) -> None:
    """The stream-K shrink's counters (1024 words after the LoRA-major part
    slots of a region bound for at least 1024 tokens) are zero after every
    launch, and no wait timed out."""
    N, ml = meta.max_num_tokens, meta.max_loras
    if N < 1024:
        return
    v = meta.views()
    off = meta.struct.sync - meta.region.data_ptr()
    words = sync_words(N, ml) + 64 * min(N, 24576) + 16 * 64 * min(N, 2048)
    c = meta.region[off + 4 * words:off + 4 * (words + 1024)].view(torch.int32).cpu().numpy()
    assert np.all(c == 0), "stream-K counters not reset: %d nonzero" % int((c != 0).sum())
    assert int(v["status"][0]) in (0, lib().LORA_ERR_ID_RANGE), "status %d" % int(v["status"][0])


def run_expand_only(wl: workloads.Workload, add_inputs: bool, seed: int = 1) -> dict:
    """lora_expand alone, from a synthetic fp32 buffer drawn by the generator."""
    sgl = lib()
    mapping = wl.mapping.numpy()
    n, ml = mapping.size, wl.spec.max_loras
    meta = sgl.LoraMeta(ml, max(n, 1))
    sgl.lora_prepare_meta(wl.mapping.to("cuda"), meta)
    out = {}
    for li, L in enumerate(wl.layers):
        sp = L.spec
        gen = torch.Generator().manual_seed(seed + li)
        bufc = workloads.make_buffer(gen, len(sp.slices), n, sp.rank, abs(sp.scale) * sp.sigma_w * sp.hidden ** 0.5)
        D = DevLayer(L)
        y = D.y0.clone()
        sgl.lora_expand(bufc.to("cuda"), D.b, D.bias, y, meta, add_inputs=add_inputs)
        torch.cuda.synchronize()
        y_g = bits(y)
        y0b = workloads.bf16_bits(L.y0)
        yr = y0b.copy()
        bias = None if L.bias is None else [workloads.bf16_bits(b) for b in L.bias]
        st, mag = oracle.expand(bufc.numpy(), [workloads.bf16_bits(b) for b in L.lora_b], bias, yr, mapping, ml,
                                add_inputs=add_inputs, with_mag=True, nthreads=8)
        assert st == 0
        neg = mapping == -1
        assert np.array_equal(y_g[neg], y0b[neg])
        out[li] = expand_check(y_g, yr, y0b, mag, add_inputs)
    return out
