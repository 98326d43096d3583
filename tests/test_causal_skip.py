"""Causal tile skipping: how many (query block, key block) pairs are visited.

"FlashAttention and Optimized Kernels", section "It is exact", counts the block
pairs a causal kernel must compute at 2,048 tokens: 53 per cent with blocks of
128 and 52 per cent with blocks of 64; section "What it saves: the numbers"
counts 2,080 pairs at 8,192 tokens with blocks of 128. A pair is visited iff
the key block starts at or before the last key the query block can see
(blocks wholly above the diagonal are skipped); every other pair is skipped.

The same rule, at the forward kernel's own tile shape (waves of 32 query rows,
64-key tiles), predicts the number of matrix-core instructions the causal
prefill of 4 x 32 heads x 8192 tokens issues; the committed rocprofv3 counter
summary of that launch must agree with it.
"""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = os.path.join(ROOT, "profiles",
                       "fwd16_bf16_d128_causal__causal_prefill_bf16_b4_h32_n8192.md")


def tiles_visited(last_key: int, bk: int) -> int:
    """Key blocks of width bk holding at least one key <= last_key."""
    return last_key // bk + 1 if last_key >= 0 else 0


def visited_block_pairs(nq: int, nk: int, bq: int, bk: int) -> int:
    """Pairs (query block, key block) a causal pass visits; bottom-right
    alignment (query i sees keys j <= i + nk - nq)."""
    pairs = 0
    for q0 in range(0, nq, bq):
        last_row = min(q0 + bq, nq) - 1
        pairs += tiles_visited(min(nk - 1, last_row + nk - nq), bk)
    return pairs


def total_block_pairs(nq, nk, bq, bk):
    return -(-nq // bq) * -(-nk // bk)


@pytest.mark.parametrize("n,block,percent", [(2048, 128, 53), (2048, 64, 52)])
def test_visited_fraction_matches_the_pages(n, block, percent):
    v = visited_block_pairs(n, n, block, block)
    t = total_block_pairs(n, n, block, block)
    assert round(100 * v / t) == percent
    # closed form for square blocks: the lower triangle with its diagonal
    m = n // block
    assert v == m * (m + 1) // 2


def test_pair_count_at_8192_matches_the_pages():
    assert visited_block_pairs(8192, 8192, 128, 128) == 2080


def test_rectangular_and_bottom_right():
    # fewer queries than keys: the diagonal ends in the bottom-right corner
    assert visited_block_pairs(1, 1000, 64, 64) == 16          # the last query sees every key
    assert visited_block_pairs(64, 1000, 64, 64) == 16
    # more queries than keys: the first rows see nothing
    assert visited_block_pairs(300, 70, 64, 64) == 0 + 0 + 0 + 1 + 2
    assert visited_block_pairs(300, 10, 64, 64) == 0 + 0 + 0 + 0 + 1


def expected_mfma_instructions_causal_prefill(B=4, H=32, N=8192, rows_per_wave=32,
                                              waves=8, bk=64):
    """Matrix-core instructions of the 16-bit causal forward at d = 128 with
    one query head per KV head: every wave of a 256-row query block issues 32
    per visited 64-key tile (16 for the scores, 16 for P V) plus 16 for one
    score tile computed past its last visited tile (the software pipeline
    computes the scores of the following tile unconditionally)."""
    block = rows_per_wave * waves
    per_head = 0
    for q0 in range(0, N, block):
        for w in range(waves):
            last_row = q0 + w * rows_per_wave + rows_per_wave - 1
            per_head += 16 + 32 * tiles_visited(min(N - 1, last_row), bk)
    return per_head * B * H


def test_kernel_mfma_count_matches_the_profile():
    expect = expected_mfma_instructions_causal_prefill()
    # the visible work alone, one 32x32x16 instruction per 32768 FLOP
    visible = 4 * 128 * (8192 * 8193 // 2) * 4 * 32 // 32768
    assert 1.0 < expect / visible < 1.02
    text = open(PROFILE).read()
    m = re.search(r"\|\s*SQ_INSTS_MFMA\s*\|\s*([0-9.eE+]+)\s*\|", text)
    assert m, "SQ_INSTS_MFMA row missing from the profile summary"
    measured = float(m.group(1))
    assert abs(measured - expect) <= 5e-4 * expect, (measured, expect)
