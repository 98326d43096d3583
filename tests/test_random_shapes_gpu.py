"""A seeded sweep of random shapes through the dense and the paged forward
and the paged decode, each compared with the float64 oracle.

The shapes are drawn once, at import, from a fixed seed: head counts and
group sizes (powers of two and not, up to one KV head for 32 query heads),
head dims, query and key lengths that are and are not multiples
of the 64-key tile or of a wave's 32 rows (including fewer keys than queries,
fewer than one tile, and none at all), causal or not, 16-bit and fp32 inputs.
The sizes stay small enough for the oracle to finish in a second or two.

FA_RANDOM_SHAPES_SCALE=k (default 1) draws k times as many shapes from the
same seeds; the first draws are the default sweep's.
"""

import math
import os

import numpy as np
import pytest
import torch

from exact_tiled_attention_11_amd import inputs
import oracle
from parity_utils import (assert_f32, assert_lowp_acc, assert_lowp_out, assert_lse,
                          assert_rounded_from, np64)
from test_parity_gpu import gpu_decode, gpu_forward
from test_variants_gpu import gpu_forward_paged

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = inputs.TORCH_DTYPES


def say(*a):
    print(*a, flush=True)


def _draw_dense(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["bf16", "f16", "bf16", "f16", "f32"]))
        nq = int(rng.integers(1, 520))
        nk = [0, int(rng.integers(1, 64)), int(rng.integers(1, 700)), nq][
            int(rng.choice(4, p=[0.08, 0.17, 0.45, 0.30]))]
        cases.append((1 + int(rng.integers(0, 2)), hkv * g, hkv, nq, nk, d, dt,
                      bool(rng.integers(0, 2)), 1000 + i))
    return cases


def _draw_paged(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["bf16", "f16"]))
        nseq = int(rng.integers(1, 6))
        q_lens, kv_lens = [], []
        for _ in range(nseq):
            kv = [0, 1, int(rng.integers(1, 1500))][int(rng.choice(3, p=[0.08, 0.07, 0.85]))]
            q = [1, int(rng.integers(1, 400))][int(rng.choice(2, p=[0.35, 0.65]))]
            q_lens.append(q)
            kv_lens.append(max(kv, 0))
        cases.append((hkv * g, hkv, d, dt, q_lens, kv_lens, bool(rng.integers(0, 2)), 2000 + i))
    return cases


def _draw_decode(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["bf16", "f16"]))
        nseq = int(rng.integers(1, 9))
        lens = [[0, 1, int(rng.integers(1, 9000))][int(rng.choice(3, p=[0.05, 0.05, 0.9]))]
                for _ in range(nseq)]
        splits = int(rng.choice([0, 0, 1, int(rng.integers(2, 65))]))
        cases.append((hkv * g, hkv, d, dt, lens, splits, 3000 + i))
    return cases


def _draw_dense_large(n, seed):
    """Batches large enough to reach all three workgroup layouts (8, 4 and 2
    waves), with ragged query blocks and key tiles."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([2, 4, 8]))
        g = int(rng.choice([2, 3, 4, 6]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["bf16", "f16"]))
        nq = int(rng.integers(300, 1000))
        nk = [nq, int(rng.integers(1, 1300))][int(rng.choice(2, p=[0.6, 0.4]))]
        cases.append((int(rng.integers(1, 7)), hkv * g, hkv, nq, nk, d, dt,
                      bool(rng.integers(0, 2)), 5000 + i))
    return cases


def _draw_paged_decode_heavy(n, seed):
    """Ragged batches in which most sequences have one query row (computed
    by the decode kernel) beside a few longer ones (the tiled kernel)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 8]))
        g = int(rng.choice([1, 3, 4, 8, 16]))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["bf16", "f16"]))
        nseq = int(rng.integers(4, 12))
        q_lens = [1 if rng.random() < 0.75 else int(rng.integers(2, 300)) for _ in range(nseq)]
        kv_lens = [[0, 1, int(rng.integers(1, 5000))][int(rng.choice(3, p=[0.05, 0.05, 0.9]))]
                   for _ in range(nseq)]
        kv_lens = [max(k, q) for k, q in zip(kv_lens, q_lens)]
        cases.append((hkv * g, hkv, d, dt, q_lens, kv_lens, bool(rng.integers(0, 2)), 6000 + i))
    return cases


SCALE = max(1, int(os.environ.get("FA_RANDOM_SHAPES_SCALE", "1")))
DENSE = _draw_dense(24 * SCALE, 7321) + _draw_dense_large(10 * SCALE, 7324)
PAGED = _draw_paged(12 * SCALE, 7322) + _draw_paged_decode_heavy(8 * SCALE, 7325)
DECODE = _draw_decode(12 * SCALE, 7323)


@pytest.mark.parametrize("case", DENSE, ids=[
    f"b{c[0]}h{c[1]}/{c[2]}-q{c[3]}k{c[4]}-d{c[5]}-{c[6]}-{'c' if c[7] else 'n'}" for c in DENSE])
def test_forward_random_shape(case):
    B, H, Hkv, Nq, Nk, d, dt, causal, seed = case
    q, k, v = inputs.prefill_inputs(B, H, Hkv, Nq, Nk, d, TD[dt], seed=seed)
    say(f"random dense {case}: oracle")
    ro, rl = oracle.attention(q, k, v, 1 / math.sqrt(d), causal)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if dt == "f32":
        o, l = gpu_forward(qd, kd, vd, causal)
        assert_f32(f"dense {case}", np64(o), ro)
        assert_lse(f"dense {case}", np64(l), rl)
        return
    o32, l32 = gpu_forward(qd, kd, vd, causal, out_dtype=torch.float32)
    o16, l16 = gpu_forward(qd, kd, vd, causal)
    assert_lowp_acc(f"dense {case}", np64(o32), ro)
    assert_rounded_from(f"dense {case}", o16, o32)
    assert_lowp_out(f"dense {case}", o16, ro)
    assert_lse(f"dense {case}", np64(l32), rl)
    assert torch.equal(l16, l32)


@pytest.mark.parametrize("case", PAGED, ids=[
    f"h{c[0]}/{c[1]}-d{c[2]}-{c[3]}-b{len(c[4])}-{'c' if c[6] else 'n'}" for c in PAGED])
def test_forward_paged_random_shape(case):
    H, Hkv, d, dt, q_lens, kv_lens, causal, seed = case
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=seed, dtype=TD[dt])
    if ri.q.shape[0] == 0:
        pytest.skip("no query rows drawn")
    # token slots past each sequence's end hold NaN: they must never be used
    for b, L in enumerate(kv_lens):
        if L % 16:
            pg = int(ri.block_table[b, L // 16])
            ri.k_pool[pg, L % 16:] = float("nan")
            ri.v_pool[pg, L % 16:] = float("nan")
    say(f"random paged {case}: oracle")
    ro, rl = oracle.attention_ragged_paged(ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool,
                                           ri.block_table, ri.kv_lens, 1 / math.sqrt(d), causal)
    o32, l32 = gpu_forward_paged(ri, causal, torch.float32)
    o16, l16 = gpu_forward_paged(ri, causal)
    assert_lowp_acc(f"paged {case}", np64(o32), ro)
    assert_lse(f"paged {case}", np64(l32), rl)
    assert_rounded_from(f"paged {case}", o16, o32)
    assert torch.equal(l16, l32)


@pytest.mark.parametrize("case", DECODE, ids=[
    f"h{c[0]}/{c[1]}-d{c[2]}-{c[3]}-b{len(c[4])}-s{c[5]}" for c in DECODE])
def test_decode_random_shape(case):
    H, Hkv, d, dt, lens, splits, seed = case
    pi = inputs.paged_decode_inputs(len(lens), H, Hkv, d, lens, seed=seed, dtype=TD[dt])
    # token slots past each sequence's end hold NaN: they must never be used
    for b, L in enumerate(lens):
        if L % 16:
            pg = int(pi.block_table[b, L // 16])
            pi.k_pool[pg, L % 16:] = float("nan")
            pi.v_pool[pg, L % 16:] = float("nan")
    say(f"random decode {case}: oracle")
    ro, rl = oracle.decode_paged(pi.q, pi.k_pool, pi.v_pool, pi.block_table, pi.seq_lens,
                                 1 / math.sqrt(d))
    dev = dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
               t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))
    o32, l32 = gpu_decode(dev, splits, torch.float32)
    o16, l16 = gpu_decode(dev, splits)
    assert_lowp_acc(f"decode {case}", np64(o32), ro)
    assert_lse(f"decode {case}", np64(l32), rl)
    assert_rounded_from(f"decode {case}", o16, o32)
