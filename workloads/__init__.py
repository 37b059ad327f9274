"""Seeded synthetic inputs for paged GQA attention (decode and ragged prefill).

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no attention arithmetic: it only draws random numbers, rounds them to
bfloat16 bit patterns, builds block pools / block tables, and writes poison.

Every value the oracle and the GPU path consume comes from here, as raw bf16
bit patterns (uint16) plus int32 tables, so both sides see identical inputs.

Conventions (the cache layout of the RL.cu "Add Cuda Kernel" page, section
"include/kernels/attention.cuh", paged-decode launcher comment):
  q            [num_seqs, H_q, D]                 bf16 bits
  k/v_cache    [num_blocks, H_kv, block_size, D]   bf16 bits
  block_tables [num_seqs, max_blocks_per_seq]      int32, logical -> physical
  seq_lens     [num_seqs]                          int32, includes the new token
Prefill (AstrAI "CUDA Kernels" page, section "Q Scheduling and KV Addressing"):
  q/out        [total_q, H_q, D], cu_seqlens [num_seqs + 1] (the page's qo_indptr)

Draw order inside one case is fixed: lengths -> allocator -> q -> k pool ->
v pool -> poison.  Unused pool blocks and the slots of a sequence's last block
beyond its length are filled with poison (finite +-64), so a kernel that reads
them fails parity instead of passing silently.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import List, Optional, Sequence

import numpy as np

POISON = 64.0
_CHUNK = 1 << 22  # values per independently seeded chunk of random draws
_THREADS = min(16, os.cpu_count() or 1)


# --------------------------------------------------------------------------
# bf16 bit patterns
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite (normal draws and poison), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _chunk_seeds(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 2 ** 63 - 1, size=max(1, (n + _CHUNK - 1) // _CHUNK), dtype=np.int64)


def _parallel_chunks(n: int, seeds: np.ndarray, fill) -> np.ndarray:
    """Fill a uint16 array of n values chunk by chunk; chunk i uses child seed i.

    The result depends only on the seeds, not on the thread count."""
    out = np.empty(n, dtype=np.uint16)
    bounds = [(i, lo, min(n, lo + _CHUNK)) for i, lo in enumerate(range(0, n, _CHUNK))]

    def work(b):
        i, lo, hi = b
        fill(np.random.default_rng(int(seeds[i])), out[lo:hi])

    if len(bounds) <= 1:
        for b in bounds:
            work(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=_THREADS) as ex:
            list(ex.map(work, bounds))
    return out


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws rounded to bf16 bit patterns."""
    n = int(np.prod(shape))

    def fill(g, dst):
        dst[:] = f32_to_bf16_bits(g.standard_normal(dst.size, dtype=np.float32))

    return _parallel_chunks(n, _chunk_seeds(rng, n), fill).reshape(shape)


def _poison_bits(rng: np.random.Generator, n: int) -> np.ndarray:
    """Finite poison: +-POISON with random signs, as bf16 bit patterns."""
    pos, neg = f32_to_bf16_bits(np.array([POISON, -POISON], dtype=np.float32))

    def fill(g, dst):
        dst[:] = np.where(g.integers(0, 2, size=dst.size, dtype=np.uint8) == 1, pos, neg)

    return _parallel_chunks(n, _chunk_seeds(rng, n), fill)


# --------------------------------------------------------------------------
# cases
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PagedCase:
    """One synthetic paged-attention workload (decode or prefill)."""

    name: str
    q: np.ndarray             # uint16 bf16 bits, [S, H_q, D] (decode) / [total_q, H_q, D] (prefill)
    k_cache: np.ndarray       # uint16, [num_blocks, H_kv, bs, D]
    v_cache: np.ndarray       # uint16, [num_blocks, H_kv, bs, D]
    block_tables: np.ndarray  # int32, [S, max_blocks_per_seq]
    seq_lens: np.ndarray      # int32, [S]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: np.float32
    partition_size: int = 0
    cu_seqlens: Optional[np.ndarray] = None  # int32 [S+1], prefill only
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_q_len(self) -> int:
        if self.cu_seqlens is None:
            return 1
        return int(np.max(np.diff(self.cu_seqlens))) if self.num_seqs else 0

    @property
    def kv_tokens(self) -> int:
        return int(np.sum(self.seq_lens, dtype=np.int64))

    @property
    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of one pass: every valid token's K and V, all kv heads."""
        return self.kv_tokens * self.num_kv_heads * self.head_dim * 2 * 2


def _blocks_needed(lens: Sequence[int], bs: int) -> List[int]:
    return [(int(L) + bs - 1) // bs for L in lens]


def _alloc_shuffled(rng, lens, bs, pool_blocks):
    """Assign each sequence's blocks from one random permutation of the pool."""
    need = _blocks_needed(lens, bs)
    perm = rng.permutation(pool_blocks)
    tables, pos = [], 0
    for n in need:
        tables.append([int(b) for b in perm[pos:pos + n]])
        pos += n
    unused = [int(b) for b in perm[pos:]]
    return tables, unused


def _alloc_identity(lens, bs):
    need = _blocks_needed(lens, bs)
    tables, pos = [], 0
    for n in need:
        tables.append(list(range(pos, pos + n)))
        pos += n
    return tables, []


def _alloc_fragmented(rng, lens, bs, pool_blocks, rounds=8, fill=0.9,
                      phantom_median=1024.0, phantom_sigma=1.0, max_len=32768):
    """A LIFO free list aged by rounds of phantom allocations and random frees.

    Each round allocates phantom sequences (lognormal lengths) until about
    `fill` of the pool is in use, then frees a random half of the live phantoms.
    Finally all phantoms are freed and the real sequences are allocated from
    the resulting free list, so tables mix short contiguous runs with scatter.
    """
    free = list(range(pool_blocks - 1, -1, -1))  # pop() yields 0, 1, 2, ...
    live: List[List[int]] = []
    limit = int(fill * pool_blocks)
    for _ in range(rounds):
        while True:
            L = int(np.clip(round(rng.lognormal(math.log(phantom_median), phantom_sigma)), 1, max_len))
            n = (L + bs - 1) // bs
            if pool_blocks - len(free) + n > limit or n > len(free):
                break
            live.append([free.pop() for _ in range(n)])
        order = rng.permutation(len(live))
        keep = []
        for j, idx in enumerate(order):
            if j < len(live) // 2:
                free.extend(reversed(live[idx]))
            else:
                keep.append(live[idx])
        live = keep
    for idx in rng.permutation(len(live)):
        free.extend(reversed(live[idx]))
    live = []
    tables = []
    for n in _blocks_needed(lens, bs):
        if n > len(free):
            raise ValueError("fragmented pool too small for the real sequences")
        tables.append([free.pop() for _ in range(n)])
    used = set(b for t in tables for b in t)
    unused = [b for b in range(pool_blocks) if b not in used]
    return tables, unused


def build_case(name: str, seed: int, seq_lens: Sequence[int], num_q_heads: int,
               num_kv_heads: int, head_dim: int, block_size: int = 16,
               pool_factor: float = 1.25, pool_blocks: Optional[int] = None,
               layout: str = "shuffled", q_rows: Optional[int] = None,
               cu_seqlens: Optional[np.ndarray] = None, partition_size: int = 0,
               max_blocks_per_seq: Optional[int] = None,
               rng: Optional[np.random.Generator] = None,
               poison: bool = True) -> PagedCase:
    """Build a paged case. `rng` continues a generator whose lengths were already drawn."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = [int(L) for L in seq_lens]
    bs = block_size
    need = sum(_blocks_needed(lens, bs))
    if pool_blocks is None:
        pool_blocks = max(1, int(math.ceil(pool_factor * need)))
    if layout == "identity":
        tables, unused = _alloc_identity(lens, bs)
        pool_blocks = max(pool_blocks, need)
        unused = list(range(need, pool_blocks))
    elif layout == "shuffled":
        tables, unused = _alloc_shuffled(rng, lens, bs, pool_blocks)
    elif layout == "fragmented":
        tables, unused = _alloc_fragmented(rng, lens, bs, pool_blocks)
    else:
        raise ValueError(f"unknown layout {layout}")
    mbps = max([len(t) for t in tables] + [1])
    if max_blocks_per_seq is not None:
        mbps = max(mbps, int(max_blocks_per_seq))
    pad_block = unused[0] if unused else 0
    bt = np.full((len(lens), mbps), pad_block, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t

    rows = len(lens) if q_rows is None else int(q_rows)
    q = _normal_bf16(rng, (rows, num_q_heads, head_dim))
    kc = _normal_bf16(rng, (pool_blocks, num_kv_heads, bs, head_dim))
    vc = _normal_bf16(rng, (pool_blocks, num_kv_heads, bs, head_dim))

    if poison:
        for cache in (kc, vc):
            if unused:
                ub = np.asarray(unused, dtype=np.int64)
                cache[ub] = _poison_bits(rng, ub.size * num_kv_heads * bs * head_dim).reshape(
                    ub.size, num_kv_heads, bs, head_dim)
            for s, L in enumerate(lens):
                tail = L % bs
                if tail and tables[s]:
                    blk = tables[s][-1]
                    cache[blk, :, tail:, :] = _poison_bits(
                        rng, num_kv_heads * (bs - tail) * head_dim).reshape(
                        num_kv_heads, bs - tail, head_dim)

    return PagedCase(name=name, q=q, k_cache=kc, v_cache=vc, block_tables=bt,
                     seq_lens=np.asarray(lens, dtype=np.int32),
                     num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                     head_dim=head_dim, block_size=bs,
                     scale=np.float32(1.0 / math.sqrt(head_dim)),
                     partition_size=partition_size,
                     cu_seqlens=None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32),
                     seed=seed)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
def tiny_decode(seed: int = 1) -> PagedCase:
    """2 sequences of lengths 37 and 100, H_q=4, H_kv=1, D=64, 16 shuffled blocks."""
    return build_case("tiny_decode", seed, [37, 100], 4, 1, 64, pool_blocks=16,
                      layout="shuffled")


def llama3_8b_decode(seed: int = 2, num_seqs: int = 32) -> PagedCase:
    """Llama-3-8B-shaped decode: H_q=32, H_kv=8, D=128, lengths uniform in [512, 4096]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4096, size=num_seqs, endpoint=True)
    return build_case("llama3_8b_decode", seed, lens, 32, 8, 128, rng=rng)


def long_split_decode(seed: int = 3, seq_len: int = 100_000, num_seqs: int = 4) -> PagedCase:
    """4 sequences of 100,000 tokens, H_q=24, H_kv=4 (GQA 6), D=256, partitions of 512."""
    rng = np.random.default_rng(seed)
    lens = [seq_len] * num_seqs
    return build_case("long_split_decode", seed, lens, 24, 4, 256, rng=rng,
                      partition_size=512)


def large_ragged_decode(seed: int = 4, num_seqs: int = 256) -> PagedCase:
    """256 sequences, H_q=64, H_kv=8 (GQA 8), D=128, lognormal lengths, fragmented pool."""
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(rng.lognormal(math.log(1024.0), 1.0, size=num_seqs)), 1, 32768).astype(np.int64)
    return build_case("large_ragged_decode", seed, lens, 64, 8, 128, rng=rng,
                      layout="fragmented")


def ragged_prefill(seed: int = 5, num_seqs: int = 16) -> PagedCase:
    """16 sequences appending U[1,256] new rows after U[0,8192] cached tokens; H_q=32, H_kv=8, D=128."""
    rng = np.random.default_rng(seed)
    n_new = rng.integers(1, 256, size=num_seqs, endpoint=True)
    cached = rng.integers(0, 8192, size=num_seqs, endpoint=True)
    return prefill_case("ragged_prefill", seed, n_new, cached, 32, 8, 128, rng=rng)


def prefill_case(name: str, seed: int, n_new: Sequence[int], cached: Sequence[int],
                 num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int = 16,
                 layout: str = "shuffled", rng: Optional[np.random.Generator] = None,
                 pool_factor: float = 1.25) -> PagedCase:
    n_new = [int(n) for n in n_new]
    cached = [int(c) for c in cached]
    lens = [c + n for c, n in zip(cached, n_new)]
    cu = np.zeros(len(n_new) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n_new)
    return build_case(name, seed, lens, num_q_heads, num_kv_heads, head_dim,
                      block_size=block_size, layout=layout, q_rows=int(cu[-1]),
                      cu_seqlens=cu, rng=rng, pool_factor=pool_factor)


NAMED = {
    "tiny_decode": tiny_decode,
    "llama3_8b_decode": llama3_8b_decode,
    "long_split_decode": long_split_decode,
    "large_ragged_decode": large_ragged_decode,
    "ragged_prefill": ragged_prefill,
}


def num_partitions(max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    """Partition count covering the longest table row (shape arithmetic only)."""
    if partition_size <= 0:
        return 1
    return (max_blocks_per_seq * block_size + partition_size - 1) // partition_size
