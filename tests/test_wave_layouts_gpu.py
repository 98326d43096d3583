"""The dense 16-bit forward runs in workgroups of 8 waves (256 packed rows),
or, when that grid would have fewer workgroups than the chip has CUs, of 4
waves (128 rows), or of 2 waves (64 rows) when even the 4-wave grid would.
All three layouts are compared here with the float64 oracle on ragged shapes
on either side of the switches: tails of query blocks and key tiles, GQA
packing, bottom-right causal masks with Nq < Nk and Nq > Nk.
"""

import math

import numpy as np
import pytest
import torch

from exact_tiled_attention_11_amd import inputs
import oracle
from parity_utils import assert_lowp_acc, assert_lowp_out, assert_lse, assert_rounded_from, np64
from test_parity_gpu import gpu_forward
from test_variants_gpu import gpu_forward_paged

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = inputs.TORCH_DTYPES
CUS = 256


def waves_per_workgroup(B, Hkv, Nq, G, causal):
    """The host's rule: 8 waves unless that grid has fewer than 256 working
    workgroups (blocks of 32 rows per wave, causal blocks paired); then 4,
    or 2 when the 4-wave grid is short of 256 too and the 2-wave grid is not
    over 256."""
    def wgs(nw):
        nqb = -(-(Nq * G) // (nw * 32))
        return B * Hkv * ((nqb + 1) // 2 if causal else nqb)
    if wgs(8) >= CUS:
        return 8
    return 2 if wgs(4) < CUS and wgs(2) <= CUS else 4


# B, H, Hkv, Nq, Nk, d, dtype, causal
CASES = [
    (4, 32, 16, 1000, 1000, 128, "bf16", True),    # 256 units: 8 waves
    (2, 64, 16, 1000, 1000, 64, "f16", False),     # G = 4, 8 waves
    (5, 17, 17, 600, 600, 128, "bf16", True),      # 170 units of 8 waves: 4 waves
    (2, 32, 32, 1500, 1500, 128, "bf16", True),    # 192 units of 8 waves: 4 waves
    (1, 8, 8, 1000, 1000, 128, "f16", True),       # 16 / 32 / 64 units: 2 waves
    (1, 16, 4, 500, 700, 64, "bf16", False),       # G = 4, Nq < Nk, non-causal: 2 waves
    (1, 32, 32, 2048, 2048, 64, "bf16", False),    # exactly 256 units: 8 waves
    (8, 32, 8, 700, 1500, 128, "bf16", True),      # Nq < Nk, G = 4, 8 waves
    (2, 32, 8, 700, 1500, 64, "f16", True),        # the same, 4 waves
    (1, 32, 8, 700, 1500, 64, "f16", True),        # the same, 2 waves
    (8, 16, 16, 1100, 300, 128, "f16", True),      # Nq > Nk: first rows see no key, 8 waves
    (2, 16, 16, 1100, 300, 128, "bf16", True),     # the same, 4 waves
    (1, 16, 16, 1100, 300, 128, "f16", True),      # the same, 2 waves
    (3, 48, 16, 777, 777, 128, "bf16", False),     # G = 3, 8 waves
    (1, 48, 16, 777, 777, 128, "f16", False),      # G = 3, 4 waves
    # Causal blocks that end inside a query's group of heads (G does not
    # divide the block), where that query's last visible key opens a new key
    # tile: the block must stream that tile too.
    (8, 48, 8, 400, 422, 128, "bf16", True),       # G = 6, 8 waves
    (4, 48, 8, 400, 422, 128, "f16", True),        # G = 6, 4 waves
    (1, 48, 8, 400, 422, 64, "bf16", True),        # G = 6, 2 waves
    (16, 24, 8, 300, 343, 128, "f16", True),       # G = 3, 8 waves
    (8, 24, 8, 300, 343, 128, "bf16", True),       # G = 3, 4 waves
    (2, 24, 8, 300, 343, 128, "bf16", True),       # G = 3, 2 waves
]


def test_cases_cover_all_layouts():
    lay = [waves_per_workgroup(B, Hkv, Nq, H // Hkv, c) for B, H, Hkv, Nq, Nk, d, dt, c in CASES]
    assert lay == [8, 8, 4, 4, 2, 2, 8, 8, 4, 2, 8, 4, 2, 8, 4, 8, 4, 2, 8, 4, 2]


def block_tile_counts(Nq, Nk, G, BR):
    """Key tiles each causal query block streams: up to the last key the
    query of its last packed row sees (bottom-right causal mask)."""
    nrows, off = Nq * G, Nk - Nq
    out = []
    for qb in range(-(-nrows // BR)):
        last = min(Nk - 1, (min(qb * BR + BR, nrows) - 1) // G + off)
        out.append(last // 64 + 1 if last >= 0 else 0)
    return out


def test_block_tiles_reach_the_last_rows_query():
    # brute force: the last tile any row of the block sees
    for Nq, Nk, G in [(400, 422, 6), (300, 343, 3), (124, 18, 6), (77, 500, 5)]:
        for BR in (64, 128, 256):
            want = []
            for qb in range(-(-(Nq * G) // BR)):
                rows = range(qb * BR, min(qb * BR + BR, Nq * G))
                last = max(min(Nk - 1, r // G + Nk - Nq) for r in rows)
                want.append(last // 64 + 1 if last >= 0 else 0)
            assert block_tile_counts(Nq, Nk, G, BR) == want


@pytest.mark.parametrize("case", CASES, ids=[
    f"b{c[0]}h{c[1]}/{c[2]}-q{c[3]}k{c[4]}-d{c[5]}-{c[6]}-{'c' if c[7] else 'n'}" for c in CASES])
def test_forward_wave_layout(case):
    B, H, Hkv, Nq, Nk, d, dt, causal = case
    q, k, v = inputs.prefill_inputs(B, H, Hkv, Nq, Nk, d, TD[dt], seed=4100 + Nq + H)
    nw = waves_per_workgroup(B, Hkv, Nq, H // Hkv, causal)
    print(f"wave layout {case}: {nw} waves per workgroup; oracle", flush=True)
    ro, rl = oracle.attention(q, k, v, 1 / math.sqrt(d), causal)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o32, l32 = gpu_forward(qd, kd, vd, causal, out_dtype=torch.float32)
    o16, l16 = gpu_forward(qd, kd, vd, causal)
    assert_lowp_acc(f"layout {case}", np64(o32), ro)
    assert_rounded_from(f"layout {case}", o16, o32)
    assert_lowp_out(f"layout {case}", o16, ro)
    assert_lse(f"layout {case}", np64(l32), rl)
    assert torch.equal(l16, l32)
    if Nk < Nq and causal:   # rows before the first visible key: O = 0, LSE = -inf
        first = Nq - Nk
        assert torch.all(o32[:, :first] == 0)
        assert torch.all(torch.isneginf(l32[:, :, :first]))


@pytest.mark.parametrize("G", [3, 6])
def test_forward_paged_blocks_ending_inside_a_head_group(G):
    """Paged forward (8-wave blocks of 256 packed rows) on sequences whose
    causal blocks end inside a query's head group at a tile boundary."""
    H, Hkv, d = 8 * G, 8, 128
    q_lens, kv_lens = ([400, 300, 5], [422, 343, 700]) if G == 6 else ([300, 400, 9], [343, 422, 64])
    ri = inputs.ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed=4200 + G,
                                    dtype=torch.bfloat16)
    print(f"paged head-group boundary G={G}: oracle", flush=True)
    ro, rl = oracle.attention_ragged_paged(ri.q, ri.qo_indptr, ri.k_pool, ri.v_pool,
                                           ri.block_table, ri.kv_lens, 1 / math.sqrt(d), True)
    o32, l32 = gpu_forward_paged(ri, True, torch.float32)
    assert_lowp_acc(f"paged G={G}", np64(o32), ro)
    assert_lse(f"paged G={G}", np64(l32), rl)
