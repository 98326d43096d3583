"""The paged decode's split partials go to a caller workspace and are merged
by the merge rule. The result must not depend on what the workspace held
before the call (zeros, all-ones bytes, random bytes, NaN, the leftovers of
another call of another shape), and repeat calls on one workspace give the
same bits; fixed split counts merge to the oracle's result.
"""

import math

import numpy as np
import pytest
import torch

from exact_tiled_attention_11_amd import inputs
import exact_tiled_attention_11_amd as fa
import oracle
from parity_utils import assert_lowp_acc, assert_lse, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def batch():
    lens = [1, 16, 17, 1024, 1025, 4096, 8999, 9000, 300, 5000, 2, 7777]
    B, H, Hkv, d = len(lens), 16, 4, 128
    pi = inputs.paged_decode_inputs(B, H, Hkv, d, lens, seed=5150, dtype=torch.bfloat16)
    dev = dict(q=pi.q.to(DEV), k=pi.k_pool.to(DEV), v=pi.v_pool.to(DEV),
               t=pi.block_table.to(DEV), s=pi.seq_lens.to(DEV))
    say(f"decode merge batch: lens {lens}, plan "
        f"{list(fa.decode_plan(lens, Hkv, pi.block_table.shape[1]))}; oracle")
    ro, rl = oracle.decode_paged(pi.q, pi.k_pool, pi.v_pool, pi.block_table, pi.seq_lens,
                                 1 / math.sqrt(d))
    need = fa.decode_workspace_size(B, H, Hkv, d, pi.block_table.shape[1])
    return dict(dev=dev, ro=ro, rl=rl, need=need, B=B, H=H, Hkv=Hkv, d=d)


def run(dev, ws, splits=0):
    o, l = fa.decode_paged(dev["q"], dev["k"], dev["v"], dev["t"], dev["s"], num_splits=splits,
                           out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    return o, l


def test_workspace_contents_do_not_matter(batch):
    dev, need = batch["dev"], batch["need"]
    assert fa.decode_max_splits(batch["B"], batch["Hkv"], dev["t"].shape[1]) > 1
    zero = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o0, l0 = run(dev, zero)
    assert_lowp_acc("decode merge", np64(o0), batch["ro"])
    assert_lse("decode merge", np64(l0), batch["rl"])
    g = torch.Generator(device="cpu").manual_seed(77)
    fills = {
        "ones": torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV),
        "random": torch.randint(0, 256, (need,), generator=g, dtype=torch.uint8).to(DEV),
        "nan": torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
        .view(torch.uint8),
    }
    for name, ws in fills.items():
        say(f"  workspace filled with {name}")
        o, l = run(dev, ws)
        assert torch.equal(o, o0) and torch.equal(l, l0), name
    # the same workspace after a call of another shape (3 sequences, 5 fixed
    # splits: its partials and counters sit at other offsets)
    other = {k: v[:3] if k in ("q", "t", "s") else v for k, v in dev.items()}
    shared = fills["random"]
    run(other, shared, splits=5)
    o, l = run(dev, shared)
    assert torch.equal(o, o0) and torch.equal(l, l0)


def test_repeat_calls_reuse_the_counters(batch):
    dev = batch["dev"]
    ws = torch.empty(batch["need"], dtype=torch.uint8, device=DEV)
    ref = run(dev, ws)
    for i in range(6):
        o, l = run(dev, ws, splits=0)
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), i


@pytest.mark.parametrize("splits", [2, 7, 64])
def test_fixed_splits_merge_in_launch(batch, splits):
    dev = batch["dev"]
    need = fa.decode_workspace_size(batch["B"], batch["H"], batch["Hkv"], batch["d"],
                                    dev["t"].shape[1], 0, splits)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    o, l = run(dev, ws, splits)
    assert_lowp_acc(f"decode merge s{splits}", np64(o), batch["ro"])
    assert_lse(f"decode merge s{splits}", np64(l), batch["rl"])
