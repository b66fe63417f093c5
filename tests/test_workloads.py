"""The seeded input generator: determinism and the recipe's structure."""
import numpy as np
import torch

import workloads


def test_deterministic():
    a, b = workloads.make_workload("tiny"), workloads.make_workload("tiny")
    assert torch.equal(a.mapping, b.mapping)
    assert torch.equal(a.layers[0].x.view(torch.int16), b.layers[0].x.view(torch.int16))
    c = workloads.make_workload("tiny", seed=99)
    assert not torch.equal(a.layers[0].x.view(torch.int16), c.layers[0].x.view(torch.int16))


def test_mapping_recipes():
    specs = workloads.WORKLOADS
    for name, spec in specs.items():
        g = torch.Generator().manual_seed(spec.seed)
        m = workloads.make_mapping(spec, g).numpy()
        assert m.dtype == np.int32 and m.size == spec.num_tokens
        assert m.min() >= -1 and m.max() < spec.max_loras
        if spec.neg_fraction:
            assert (m == -1).sum() == round(spec.neg_fraction * spec.num_tokens)
    g = torch.Generator().manual_seed(2)
    m = workloads.make_mapping(specs["prefill"], g).numpy()
    runs = m.reshape(16, 512)
    assert np.all(runs == runs[:, :1]) and not np.any(m == -1)
    g = torch.Generator().manual_seed(3)
    m = workloads.make_mapping(specs["zipf"], g).numpy()
    c = np.bincount(m[m >= 0], minlength=64)
    assert c[0] == c.max() and c[0] > 500          # id 0 is the head of the law
    g = torch.Generator().manual_seed(5)
    assert np.all(workloads.make_mapping(specs["large_nolora"], g).numpy() == -1)


def test_shapes_small_override():
    wl = workloads.make_workload("decode", num_tokens=40)
    L = wl.layers[0]
    assert L.x.shape == (40, 4096) and L.x.dtype == torch.bfloat16
    assert [a.shape for a in L.lora_a] == [(32, 16, 4096)] * 3
    assert [b.shape for b in L.lora_b] == [(32, 4096, 16), (32, 1024, 16), (32, 1024, 16)]
    assert L.y0.shape == (40, 6144) and L.bias is None
    wl = workloads.make_workload("prefill", num_tokens=64)
    assert [b.shape for b in wl.layers[0].bias] == [(8, 4096), (8, 1024), (8, 1024)]


def test_logits_and_embedding_shapes():
    wl = workloads.make_workload("logits", num_tokens=8)
    L = wl.layers[0]
    assert L.x.shape == (8, 4096) and [b.shape for b in L.lora_b] == [(32, 128256, 16)]
    assert L.y0.shape == (8, 128256)
    wl = workloads.make_workload("embedding", num_tokens=40)
    L = wl.layers[0]
    assert L.spec.expand_only and L.lora_a == []
    assert L.x.shape == (1, 40, 16) and L.x.dtype == torch.float32
    assert [b.shape for b in L.lora_b] == [(32, 4096, 16)] and L.y0.shape == (40, 4096)
