"""The CPU oracle for paged GQA attention -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package.  The product library (`paged_kv_cache_34_amd`) never
imports it and shares no code with it.

`paged_attn_oracle.c` is plain fp64 C (OpenMP over independent outputs); this
module compiles it with gcc into `liboracle.so` next to the source and wraps it
with ctypes.  Inputs are the bf16 bit patterns and int32 tables produced by
`workloads`; outputs are float64 numpy arrays.

Definitions followed (details in the C source):
  decode      -- BI-V100 design page, section 1 "Problem Definition"; gather as
                 in the RL.cu page's paged decode kernel.
  partials    -- BI-V100 design page, section 2 ("attention_partial", Level 3),
                 with tmp_out stored normalized by its exp_sum.
  reduce      -- BI-V100 design page, section 2 "combine".
  prefill     -- AstrAI page, "Q Scheduling and KV Addressing" (qo_indptr rows),
                 causal rule of the RL.cu page's prefill kernel, end-aligned.
  tile_map    -- AstrAI page, "Q Scheduling and KV Addressing" worked example.
  kv_append   -- the cache write before decode/prefill (AstrAI page, backend
                 layer, which is responsible for writing and reading the KV
                 cache); new rows are the
                 last rows of each sequence, placed like the prefill rows.
  fp8         -- FP8 (OCP E4M3) KV cache with a per-position dequant scale (B200
                 page, "Stage D: FP8 Paged KV Gather" and "FP8 KV
                 Quantize/Dequant"): quantize_fp8, fp8_dequant, kv_append_fp8,
                 and decode / partials over the dequantized (fp64) cache.
  tokens      -- the AstrAI page's token-granular cache (decode with
                 page_size=1, kv_indptr + page indices): cache [num_slots, H_kv,
                 D], sequence s's token t in slot kv_indices[kv_indptr[s] + t].
  xpacked     -- the BI-V100 page's cache layouts (section 3 "Paged K/V
                 Gather"): K [num_blocks, H_kv, D/8, bs, 8], V [num_blocks,
                 H_kv, D, bs]; decode, partials and append over them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "paged_attn_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_c_int = ctypes.c_int


def compile_library(out_path: str = LIBRARY, mutant: int = 0) -> str:
    """Compile the oracle with gcc (portable flags: it runs on other hosts too)."""
    tmp = f"{out_path}.tmp{os.getpid()}"  # one per process: parallel builds do not collide
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
           f"-DORACLE_MUTANT={int(mutant)}", SOURCE, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def _needs_build(path: str) -> bool:
    return (not os.path.exists(path)) or os.path.getmtime(path) < os.path.getmtime(SOURCE)


class Oracle:
    """ctypes wrapper around one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and _needs_build(path):
            compile_library(path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_decode.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p] + [_c_int] * 6 + [
            ctypes.c_float, _f64p]
        lib.oracle_decode_partials.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p] + [_c_int] * 6 + [
            ctypes.c_float, _c_int, _c_int, _f64p, _f64p, _f64p]
        lib.oracle_reduce.argtypes = [_f64p, _f64p, _f64p, _i32p] + [_c_int] * 5 + [_f64p]
        lib.oracle_prefill.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p, _i32p] + [_c_int] * 7 + [
            ctypes.c_float, _f64p]
        _u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
        _f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
        lib.oracle_decode_f64kv.argtypes = [_u16p, _f64p, _f64p, _i32p, _i32p] + [_c_int] * 6 + [
            ctypes.c_float, _f64p]
        lib.oracle_decode_partials_f64kv.argtypes = [_u16p, _f64p, _f64p, _i32p, _i32p] + [_c_int] * 6 + [
            ctypes.c_float, _c_int, _c_int, _f64p, _f64p, _f64p]
        lib.oracle_kv_append.argtypes = [_u16p, _u16p, _i32p, _i32p, _i32p] + [_c_int] * 5 + [_u16p, _u16p]
        lib.oracle_kv_append_xpacked.argtypes = lib.oracle_kv_append.argtypes
        lib.oracle_decode_xpacked.argtypes = lib.oracle_decode.argtypes
        lib.oracle_decode_partials_xpacked.argtypes = lib.oracle_decode_partials.argtypes
        lib.oracle_decode_tokens.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p] + [_c_int] * 4 + [
            ctypes.c_float, _f64p]
        lib.oracle_decode_partials_tokens.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p] + [_c_int] * 4 + [
            ctypes.c_float, _c_int, _c_int, _f64p, _f64p, _f64p]
        lib.oracle_kv_append_fp8.argtypes = ([_u16p, _u16p, _i32p, _i32p, _i32p] + [_c_int] * 5 +
                                             [_u8p, _u8p, _f32p, _f32p])
        lib.oracle_quantize_fp8.argtypes = [_u16p, ctypes.c_long, _c_int, _u8p, _f32p]
        lib.oracle_fp8_dequant.argtypes = [_u8p, _f32p, ctypes.c_long, _c_int, _f64p]
        lib.oracle_e4m3_value.argtypes = [_c_int]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        for fn in ("oracle_decode", "oracle_decode_partials", "oracle_reduce", "oracle_prefill",
                   "oracle_mutant", "oracle_num_threads", "oracle_decode_f64kv",
                   "oracle_decode_partials_f64kv", "oracle_kv_append", "oracle_kv_append_fp8",
                   "oracle_quantize_fp8", "oracle_fp8_dequant", "oracle_kv_append_xpacked",
                   "oracle_decode_xpacked", "oracle_decode_partials_xpacked",
                   "oracle_decode_tokens", "oracle_decode_partials_tokens"):
            getattr(lib, fn).restype = ctypes.c_int
        self.lib = lib

    # ---- helpers -------------------------------------------------------
    @staticmethod
    def _c(a, dtype):
        return np.ascontiguousarray(a, dtype=dtype)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def mutant(self) -> int:
        return int(self.lib.oracle_mutant())

    # ---- O1 ------------------------------------------------------------
    def decode(self, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int,
               scale) -> np.ndarray:
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        kc = self._c(k_cache, np.uint16)
        bs = kc.shape[2]
        bt = self._c(block_tables, np.int32)
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.oracle_decode(q, kc, self._c(v_cache, np.uint16), bt,
                                    self._c(seq_lens, np.int32), S, Hq, num_kv_heads, D, bs,
                                    bt.shape[1], float(np.float32(scale)), out)
        if rc:
            raise ValueError(f"oracle_decode rejected the shapes (status {rc})")
        return out

    # ---- O2 ------------------------------------------------------------
    def decode_partials(self, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int,
                        scale, partition_size: int, max_num_partitions: Optional[int] = None
                        ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        kc = self._c(k_cache, np.uint16)
        bs = kc.shape[2]
        bt = self._c(block_tables, np.int32)
        if max_num_partitions is None:
            max_num_partitions = max(1, (bt.shape[1] * bs + partition_size - 1) // partition_size)
        NP = int(max_num_partitions)
        ml = np.full((S, Hq, NP), np.nan)
        es = np.full((S, Hq, NP), np.nan)
        to = np.full((S, Hq, NP, D), np.nan)
        rc = self.lib.oracle_decode_partials(q, kc, self._c(v_cache, np.uint16), bt,
                                             self._c(seq_lens, np.int32), S, Hq, num_kv_heads, D,
                                             bs, bt.shape[1], float(np.float32(scale)),
                                             int(partition_size), NP, ml, es, to)
        if rc:
            raise ValueError(f"oracle_decode_partials rejected the shapes (status {rc})")
        return ml, es, to

    # ---- O3 ------------------------------------------------------------
    def reduce(self, max_logits, exp_sums, tmp_out, seq_lens, partition_size: int) -> np.ndarray:
        ml = self._c(max_logits, np.float64)
        S, Hq, NP = ml.shape
        to = self._c(tmp_out, np.float64)
        D = to.shape[-1]
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.oracle_reduce(ml, self._c(exp_sums, np.float64), to,
                                    self._c(seq_lens, np.int32), S, Hq, D, int(partition_size),
                                    NP, out)
        if rc:
            raise ValueError(f"oracle_reduce rejected the shapes (status {rc})")
        return out

    # ---- O4 ------------------------------------------------------------
    def prefill(self, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens,
                num_kv_heads: int, scale) -> np.ndarray:
        q = self._c(q, np.uint16)
        total_q, Hq, D = q.shape
        kc = self._c(k_cache, np.uint16)
        bs = kc.shape[2]
        bt = self._c(block_tables, np.int32)
        sl = self._c(seq_lens, np.int32)
        out = np.empty((total_q, Hq, D), dtype=np.float64)
        rc = self.lib.oracle_prefill(q, kc, self._c(v_cache, np.uint16), bt, sl,
                                     self._c(cu_seqlens, np.int32), sl.shape[0], total_q, Hq,
                                     num_kv_heads, D, bs, bt.shape[1], float(np.float32(scale)), out)
        if rc:
            raise ValueError(f"oracle_prefill rejected the shapes (status {rc})")
        return out

    # ---- O1 / O2 over fp64 caches (dequantized FP8) ----------------------
    def decode_f64kv(self, q, k_values, v_values, block_tables, seq_lens, num_kv_heads: int,
                     scale) -> np.ndarray:
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        kc = self._c(k_values, np.float64)
        bt = self._c(block_tables, np.int32)
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.oracle_decode_f64kv(q, kc, self._c(v_values, np.float64), bt,
                                          self._c(seq_lens, np.int32), S, Hq, num_kv_heads, D,
                                          kc.shape[2], bt.shape[1], float(np.float32(scale)), out)
        if rc:
            raise ValueError(f"oracle_decode_f64kv rejected the shapes (status {rc})")
        return out

    def decode_partials_f64kv(self, q, k_values, v_values, block_tables, seq_lens,
                              num_kv_heads: int, scale, partition_size: int,
                              max_num_partitions: Optional[int] = None):
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        kc = self._c(k_values, np.float64)
        bs = kc.shape[2]
        bt = self._c(block_tables, np.int32)
        if max_num_partitions is None:
            max_num_partitions = max(1, (bt.shape[1] * bs + partition_size - 1) // partition_size)
        NP = int(max_num_partitions)
        ml = np.full((S, Hq, NP), np.nan)
        es = np.full((S, Hq, NP), np.nan)
        to = np.full((S, Hq, NP, D), np.nan)
        rc = self.lib.oracle_decode_partials_f64kv(q, kc, self._c(v_values, np.float64), bt,
                                                   self._c(seq_lens, np.int32), S, Hq, num_kv_heads,
                                                   D, bs, bt.shape[1], float(np.float32(scale)),
                                                   int(partition_size), NP, ml, es, to)
        if rc:
            raise ValueError(f"oracle_decode_partials_f64kv rejected the shapes (status {rc})")
        return ml, es, to

    # ---- O1 / O2 over the x-packed K / transposed V layouts -----------------
    def decode_xpacked(self, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int,
                       scale) -> np.ndarray:
        """k_cache [num_blocks, H_kv, D/8, bs, 8], v_cache [num_blocks, H_kv, D, bs] (bf16 bits)."""
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        kc = self._c(k_cache, np.uint16)
        bs = kc.shape[3]
        bt = self._c(block_tables, np.int32)
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.oracle_decode_xpacked(q, kc, self._c(v_cache, np.uint16), bt,
                                            self._c(seq_lens, np.int32), S, Hq, num_kv_heads, D, bs,
                                            bt.shape[1], float(np.float32(scale)), out)
        if rc:
            raise ValueError(f"oracle_decode_xpacked rejected the shapes (status {rc})")
        return out

    def decode_partials_xpacked(self, q, k_cache, v_cache, block_tables, seq_lens,
                                num_kv_heads: int, scale, partition_size: int,
                                max_num_partitions: Optional[int] = None):
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        kc = self._c(k_cache, np.uint16)
        bs = kc.shape[3]
        bt = self._c(block_tables, np.int32)
        if max_num_partitions is None:
            max_num_partitions = max(1, (bt.shape[1] * bs + partition_size - 1) // partition_size)
        NP = int(max_num_partitions)
        ml = np.full((S, Hq, NP), np.nan)
        es = np.full((S, Hq, NP), np.nan)
        to = np.full((S, Hq, NP, D), np.nan)
        rc = self.lib.oracle_decode_partials_xpacked(q, kc, self._c(v_cache, np.uint16), bt,
                                                     self._c(seq_lens, np.int32), S, Hq, num_kv_heads,
                                                     D, bs, bt.shape[1], float(np.float32(scale)),
                                                     int(partition_size), NP, ml, es, to)
        if rc:
            raise ValueError(f"oracle_decode_partials_xpacked rejected the shapes (status {rc})")
        return ml, es, to

    # ---- O1 / O2 over a token-granular cache (page_size 1, kv_indptr) -------
    def decode_tokens(self, q, k_cache, v_cache, kv_indptr, kv_indices, num_kv_heads: int,
                      scale) -> np.ndarray:
        """k_cache / v_cache [num_slots, H_kv, D] bf16 bits; sequence s's token t
        is slot kv_indices[kv_indptr[s] + t]."""
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        out = np.empty((S, Hq, D), dtype=np.float64)
        rc = self.lib.oracle_decode_tokens(q, self._c(k_cache, np.uint16), self._c(v_cache, np.uint16),
                                           self._c(kv_indptr, np.int32), self._c(kv_indices, np.int32),
                                           S, Hq, num_kv_heads, D, float(np.float32(scale)), out)
        if rc:
            raise ValueError(f"oracle_decode_tokens rejected the shapes (status {rc})")
        return out

    def decode_partials_tokens(self, q, k_cache, v_cache, kv_indptr, kv_indices, num_kv_heads: int,
                               scale, partition_size: int, max_num_partitions: int):
        q = self._c(q, np.uint16)
        S, Hq, D = q.shape
        NP = int(max_num_partitions)
        ml = np.full((S, Hq, NP), np.nan)
        es = np.full((S, Hq, NP), np.nan)
        to = np.full((S, Hq, NP, D), np.nan)
        rc = self.lib.oracle_decode_partials_tokens(q, self._c(k_cache, np.uint16),
                                                    self._c(v_cache, np.uint16),
                                                    self._c(kv_indptr, np.int32),
                                                    self._c(kv_indices, np.int32), S, Hq,
                                                    num_kv_heads, D, float(np.float32(scale)),
                                                    int(partition_size), NP, ml, es, to)
        if rc:
            raise ValueError(f"oracle_decode_partials_tokens rejected the shapes (status {rc})")
        return ml, es, to

    def kv_append_xpacked(self, k_new, v_new, block_tables, seq_lens, cu_seqlens, k_cache, v_cache):
        """Copies of the x-packed K / transposed V caches with the new rows written."""
        kn = self._c(k_new, np.uint16)
        kc = np.array(k_cache, dtype=np.uint16, copy=True, order="C")
        vc = np.array(v_cache, dtype=np.uint16, copy=True, order="C")
        bt = self._c(block_tables, np.int32)
        sl = self._c(seq_lens, np.int32)
        _, Hkv, D, bs = vc.shape
        rc = self.lib.oracle_kv_append_xpacked(kn, self._c(v_new, np.uint16), bt, sl,
                                               self._c(cu_seqlens, np.int32), sl.shape[0], Hkv, D, bs,
                                               bt.shape[1], kc, vc)
        if rc:
            raise ValueError(f"oracle_kv_append_xpacked rejected the inputs (status {rc})")
        return kc, vc

    # ---- KV append ---------------------------------------------------------
    def kv_append(self, k_new, v_new, block_tables, seq_lens, cu_seqlens, k_cache, v_cache):
        """Copies of the bf16 caches with the new rows written; inputs untouched."""
        kn = self._c(k_new, np.uint16)
        kc = np.array(k_cache, dtype=np.uint16, copy=True, order="C")
        vc = np.array(v_cache, dtype=np.uint16, copy=True, order="C")
        bt = self._c(block_tables, np.int32)
        sl = self._c(seq_lens, np.int32)
        _, Hkv, bs, D = kc.shape
        rc = self.lib.oracle_kv_append(kn, self._c(v_new, np.uint16), bt, sl,
                                       self._c(cu_seqlens, np.int32), sl.shape[0], Hkv, D, bs,
                                       bt.shape[1], kc, vc)
        if rc:
            raise ValueError(f"oracle_kv_append rejected the inputs (status {rc})")
        return kc, vc

    # ---- FP8 ---------------------------------------------------------------
    def e4m3_value(self, code: int) -> float:
        return float(self.lib.oracle_e4m3_value(int(code)))

    def quantize_fp8(self, x_bits):
        """Rows of bf16 bits [..., D] -> (E4M3 codes uint8 [..., D], scales float32 [...])."""
        x = self._c(x_bits, np.uint16)
        D = x.shape[-1]
        rows = x.size // D if D else 0
        codes = np.empty(x.shape, dtype=np.uint8)
        scales = np.empty(x.shape[:-1], dtype=np.float32)
        self.lib.oracle_quantize_fp8(x, rows, D, codes, scales)
        return codes, scales

    def fp8_dequant(self, codes, scales) -> np.ndarray:
        c = self._c(codes, np.uint8)
        sc = self._c(scales, np.float32)
        D = c.shape[-1]
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_fp8_dequant(c, sc, c.size // D if D else 0, D, out)
        return out

    def kv_append_fp8(self, k_new, v_new, block_tables, seq_lens, cu_seqlens, k_codes, v_codes,
                      k_scales, v_scales):
        """Copies of the FP8 caches (codes, scales) with the new rows quantized and written."""
        kc = np.array(k_codes, dtype=np.uint8, copy=True, order="C")
        vc = np.array(v_codes, dtype=np.uint8, copy=True, order="C")
        ks = np.array(k_scales, dtype=np.float32, copy=True, order="C")
        vs = np.array(v_scales, dtype=np.float32, copy=True, order="C")
        bt = self._c(block_tables, np.int32)
        sl = self._c(seq_lens, np.int32)
        _, Hkv, bs, D = kc.shape
        rc = self.lib.oracle_kv_append_fp8(self._c(k_new, np.uint16), self._c(v_new, np.uint16), bt,
                                           sl, self._c(cu_seqlens, np.int32), sl.shape[0], Hkv, D,
                                           bs, bt.shape[1], kc, vc, ks, vs)
        if rc:
            raise ValueError(f"oracle_kv_append_fp8 rejected the inputs (status {rc})")
        return kc, vc, ks, vs

    def decode_fp8(self, q, k_codes, v_codes, k_scales, v_scales, block_tables, seq_lens,
                   num_kv_heads: int, scale) -> np.ndarray:
        return self.decode_f64kv(q, self.fp8_dequant(k_codes, k_scales),
                                 self.fp8_dequant(v_codes, v_scales), block_tables, seq_lens,
                                 num_kv_heads, scale)

    def decode_partials_fp8(self, q, k_codes, v_codes, k_scales, v_scales, block_tables, seq_lens,
                            num_kv_heads: int, scale, partition_size: int,
                            max_num_partitions: Optional[int] = None):
        return self.decode_partials_f64kv(q, self.fp8_dequant(k_codes, k_scales),
                                          self.fp8_dequant(v_codes, v_scales), block_tables,
                                          seq_lens, num_kv_heads, scale, partition_size,
                                          max_num_partitions)

    # ---- case conveniences ----------------------------------------------
    def decode_case(self, case) -> np.ndarray:
        return self.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                           case.num_kv_heads, case.scale)

    def partials_case(self, case, partition_size: int, max_num_partitions: Optional[int] = None):
        return self.decode_partials(case.q, case.k_cache, case.v_cache, case.block_tables,
                                    case.seq_lens, case.num_kv_heads, case.scale,
                                    partition_size, max_num_partitions)

    def prefill_case(self, case) -> np.ndarray:
        return self.prefill(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                            case.cu_seqlens, case.num_kv_heads, case.scale)


def tile_map(qo_indptr: Sequence[int], tile_rows: int) -> Tuple[list, list]:
    """Q-tile work map of a packed ragged batch (AstrAI page, "Q Scheduling and
    KV Addressing"): tile k covers rows [index*tile_rows, ...) of request batch,
    for every request in order, one tile per started block of tile_rows rows."""
    to_batch, to_index = [], []
    for b in range(len(qo_indptr) - 1):
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        for i in range((n + tile_rows - 1) // tile_rows):
            to_batch.append(b)
            to_index.append(i)
    return to_batch, to_index


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The process-wide oracle (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
