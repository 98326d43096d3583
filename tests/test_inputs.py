"""The seeded input generators: deterministic, correctly shaped and laid out."""

import numpy as np
import torch

from exact_tiled_attention_11_amd import inputs


def test_normal_is_deterministic_and_chunk_independent():
    a = inputs.normal((3, 1000), seed=5, dtype=torch.float32)
    b = inputs.normal((3, 1000), seed=5, dtype=torch.float32)
    assert torch.equal(a, b)
    assert not torch.equal(a, inputs.normal((3, 1000), seed=6, dtype=torch.float32))
    big = inputs.normal(((1 << 22) + 10,), seed=7, dtype=torch.float32)
    first = np.random.default_rng([7, 0]).standard_normal(1 << 22, dtype=np.float32)
    second = np.random.default_rng([7, 1]).standard_normal(10, dtype=np.float32)
    assert np.array_equal(big.numpy(), np.concatenate([first, second]))


def test_scale_applies_before_rounding():
    x = inputs.normal((4096,), seed=9, dtype=torch.float32, scale=30.0)
    y = inputs.normal((4096,), seed=9, dtype=torch.float32)
    assert torch.equal(x, y * 30.0)
    z = inputs.normal((4096,), seed=9, dtype=torch.bfloat16, scale=30.0)
    assert torch.equal(z, (y * 30.0).to(torch.bfloat16))


def test_paged_inputs_layout():
    lens = np.array([1, 16, 17, 100, 0])
    p = inputs.paged_decode_inputs(5, 8, 2, 64, lens, seed=3, max_pages=8)
    need = -(-lens // 16)
    assert p.block_table.shape == (5, 8) and p.block_table.dtype == torch.int32
    used = []
    for b in range(5):
        row = p.block_table[b].numpy()
        assert np.all(row[:need[b]] >= 0) and np.all(row[need[b]:] == -1)
        used.extend(row[:need[b]])
    assert len(set(used)) == len(used) == need.sum()
    assert p.k_pool.shape[0] == int(np.ceil(1.25 * need.sum()))
    unref = np.setdiff1d(np.arange(p.k_pool.shape[0]), used)
    assert torch.isnan(p.k_pool[torch.from_numpy(unref)]).all()
    assert not torch.isnan(p.k_pool[torch.from_numpy(np.array(used))]).any()
    assert torch.equal(p.seq_lens, torch.tensor(lens, dtype=torch.int32))
    c = inputs.paged_decode_inputs(5, 8, 2, 64, lens, seed=3, max_pages=8, contiguous=True)
    assert torch.equal(c.q, p.q)
    assert np.array_equal(c.block_table[3].numpy()[:need[3]],
                          np.arange(need[:3].sum(), need[:4].sum()))


def test_lengths_and_rows():
    L = inputs.uniform_lengths(64, 1024, 32768, seed=1)
    assert L.min() >= 1024 and L.max() <= 32768 and len(L) == 64
    r = inputs.sample_rows(256, 65536, seed=2)
    assert len(np.unique(r)) == 256 and r.min() >= 0 and r.max() < 65536
