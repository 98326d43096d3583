"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic. Values are N(0, 1) float32 from numpy's PCG64 stream,
multiplied by a query scale where a workload asks for it, then rounded to the
input dtype (round-to-nearest-even). Large tensors are drawn in fixed chunks of
2^22 elements, chunk i from default_rng([seed, i]), so the values depend only
on (seed, shape) and not on how many threads fill them.

Workloads (the shapes the pages' experiments and the target configurations
use) are listed in WORKLOADS.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, seed: int, dtype=torch.bfloat16, scale: float = 1.0) -> torch.Tensor:
    """CPU tensor of N(0,1)*scale values rounded to `dtype`."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=dtype)
    n_chunks = max(1, -(-n // _CHUNK))

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.default_rng([seed, i]).standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = torch.from_numpy(x).to(dtype)

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def prefill_inputs(B, H, Hkv, Nq, Nk, d, dtype, seed, q_scale=1.0):
    """q [B,Nq,H,d], k, v [B,Nk,Hkv,d] on the CPU."""
    q = normal((B, Nq, H, d), seed * 3 + 0, dtype, q_scale)
    k = normal((B, Nk, Hkv, d), seed * 3 + 1, dtype)
    v = normal((B, Nk, Hkv, d), seed * 3 + 2, dtype)
    return q, k, v


@dataclass
class PagedInputs:
    q: torch.Tensor             # [B, H, d]
    k_pool: torch.Tensor        # [P, page, Hkv, d]
    v_pool: torch.Tensor
    block_table: torch.Tensor   # [B, max_pages] int32, -1 past each sequence's pages
    seq_lens: torch.Tensor      # [B] int32
    referenced: np.ndarray = field(default=None)   # bool [P]: page used by some sequence


def paged_decode_inputs(B, H, Hkv, d, lens, seed, dtype=torch.bfloat16, page=16,
                        pool_factor=1.25, max_pages=None, unreferenced="nan",
                        contiguous=False):
    """Decode inputs over a shared page pool.

    lens: [B] sequence lengths. The pool holds ceil(pool_factor * pages used)
    pages; each sequence takes its pages from one random permutation of the
    pool (or consecutively when contiguous=True). Pages no sequence references
    are filled with NaN (unreferenced="nan") so that a stray read would show,
    or with N(0,1) values (unreferenced="normal").
    """
    lens = np.asarray(lens, dtype=np.int64)
    need = -(-lens // page)
    used = int(need.sum())
    n_pages = max(1, int(math.ceil(pool_factor * used)))
    rng = np.random.default_rng([seed, 1 << 20])
    order = np.arange(n_pages) if contiguous else rng.permutation(n_pages)
    if max_pages is None:
        max_pages = max(1, int(need.max()) if len(need) else 1)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = order[off:off + need[b]]
        off += need[b]
    referenced = np.zeros(n_pages, dtype=bool)
    referenced[order[:used]] = True
    q = normal((B, H, d), seed * 3 + 0, dtype)
    k_pool = normal((n_pages, page, Hkv, d), seed * 3 + 1, dtype)
    v_pool = normal((n_pages, page, Hkv, d), seed * 3 + 2, dtype)
    if unreferenced == "nan" and (~referenced).any():
        idx = torch.from_numpy(np.nonzero(~referenced)[0])
        k_pool[idx] = float("nan")
        v_pool[idx] = float("nan")
    return PagedInputs(q, k_pool, v_pool, torch.from_numpy(table),
                       torch.from_numpy(lens.astype(np.int32)), referenced)


@dataclass
class RaggedPagedInputs:
    q: torch.Tensor             # [total_q, H, d]
    qo_indptr: torch.Tensor     # [B + 1] int32
    k_pool: torch.Tensor        # [P, page, Hkv, d]
    v_pool: torch.Tensor
    block_table: torch.Tensor   # [B, max_pages] int32, -1 past each sequence's pages
    kv_lens: torch.Tensor       # [B] int32
    max_q_len: int


def ragged_paged_inputs(q_lens, kv_lens, H, Hkv, d, seed, dtype=torch.bfloat16, page=16,
                        pool_factor=1.25, unreferenced="nan", q_scale=1.0):
    """A ragged batch of queries (q_lens[b] rows for sequence b, concatenated)
    over a shared page pool holding kv_lens[b] tokens per sequence. Pages are
    taken from one random permutation of the pool; pages no sequence references
    hold NaN (unreferenced="nan") or N(0,1) values; token slots past a
    sequence's last token hold N(0,1) values."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv = paged_decode_inputs(len(q_lens), H, Hkv, d, kv_lens, seed, dtype, page, pool_factor,
                             None, unreferenced)
    indptr = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = normal((int(indptr[-1]), H, d), seed * 3 + 3, dtype, q_scale)
    return RaggedPagedInputs(q, torch.from_numpy(indptr), kv.k_pool, kv.v_pool, kv.block_table,
                             kv.seq_lens, int(q_lens.max()) if len(q_lens) else 0)


def uniform_lengths(B, lo, hi, seed):
    """B integers uniform in [lo, hi] (inclusive)."""
    return np.random.default_rng([seed, 1 << 21]).integers(lo, hi, size=B, endpoint=True)


def sample_rows(n_rows, N, seed):
    """n_rows distinct query positions in [0, N), sorted."""
    return np.sort(np.random.default_rng([seed, 1 << 22]).choice(N, size=n_rows, replace=False))


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    params: dict


WORKLOADS = {
    # One head, fp32, non-causal, 256 x 256, d = 64.
    "single_head_f32_n256": Workload("single_head_f32_n256", "prefill", dict(
        B=1, H=1, Hkv=1, N=256, d=64, dtypes=("f32",), causal=(False,), q_scales=(1.0,),
        seed=101)),
    # 12 heads, d = 64, 2048 tokens, causal and not, fp16 and fp32, Q and 30 Q.
    "mha12_d64_n2048": Workload("mha12_d64_n2048", "prefill", dict(
        B=1, H=12, Hkv=12, N=2048, d=64, dtypes=("f16", "f32"), causal=(False, True),
        q_scales=(1.0, 30.0), seed=102)),
    # Causal prefill, bf16, B = 4, 32 heads, 8192 tokens, d = 128.
    "causal_prefill_bf16_b4_h32_n8192": Workload("causal_prefill_bf16_b4_h32_n8192", "prefill", dict(
        B=4, H=32, Hkv=32, N=8192, d=128, dtypes=("bf16",), causal=(True,), q_scales=(1.0,),
        seed=103)),
    # Split-KV paged decode, bf16 GQA: 64 sequences, 32 query / 8 KV heads,
    # d = 128, 16-token pages, lengths uniform in [1024, 32768].
    "paged_decode_bf16_b64_h32_kv8": Workload("paged_decode_bf16_b64_h32_kv8", "decode", dict(
        B=64, H=32, Hkv=8, d=128, page=16, len_lo=1024, len_hi=32768, pool_factor=1.25,
        seed=104)),
    # Long-context causal prefill, bf16, 65536 tokens, 16 heads, d = 128, 30 Q;
    # checked on 256 sampled query rows plus every LSE value.
    "long_causal_prefill_bf16_n65536": Workload("long_causal_prefill_bf16_n65536", "prefill", dict(
        B=1, H=16, Hkv=16, N=65536, d=128, dtypes=("bf16",), causal=(True,), q_scales=(30.0,),
        sample_rows=256, seed=105)),
}

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
