"""Helpers for the GPU tests: moving synthetic cases to the device and the
comparison rules of the parity tests.

Tolerances (written here, used by every GPU test):
  * bf16 outputs vs the unrounded fp64 oracle: max-abs 1e-2; for |ref| >= 4 the
    bound is one bf16 ulp of ref instead (a half ulp there already exceeds
    1e-2, so 1e-2 would demand better than bf16 can represent).
  * fp32 partials vs the fp64 oracle: max_logits and tmp_out max-abs 1e-4,
    exp_sums relative 1e-4 (exp_sum grows with the partition size).
"""
from __future__ import annotations

import numpy as np

import workloads

OUT_TOL = 1e-2
PARTIAL_TOL = 1e-4


def torch():
    import torch as _t
    return _t


def bf16_dev(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(t.bfloat16).cuda()


def i32_dev(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bf16_host_f64(t) -> np.ndarray:
    bits = t.detach().cpu().contiguous().view(torch().int16).numpy().view(np.uint16)
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def bf16_bits_host(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch().int16).numpy().view(np.uint16).copy()


class Dev:
    """Device copies of one case's inputs."""

    def __init__(self, case):
        self.case = case
        self.q = bf16_dev(case.q)
        self.k = bf16_dev(case.k_cache)
        self.v = bf16_dev(case.v_cache)
        self.bt = i32_dev(case.block_tables)
        self.sl = i32_dev(case.seq_lens)
        self.cu = None if case.cu_seqlens is None else i32_dev(case.cu_seqlens)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7.0)


def assert_out_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    tol = np.where(np.abs(ref) >= 4.0, bf16_ulp(ref), OUT_TOL)
    bad = err > tol
    if np.any(bad):
        idx = np.unravel_index(int(np.argmax(err - tol)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at {idx}: "
                             f"gpu {gpu[idx]:.6f} ref {ref[idx]:.6f} (max-abs {err.max():.3e})")


def assert_partials_close(ml, es, to, ref_ml, ref_es, ref_to, seq_lens, partition_size, what: str):
    """Compare only partitions that exist (p < ceil(L / P))."""
    for s, L in enumerate(seq_lens):
        n = (int(L) + partition_size - 1) // partition_size
        if n == 0:
            continue
        e1 = np.max(np.abs(ml[s, :, :n] - ref_ml[s, :, :n]))
        e2 = np.max(np.abs(es[s, :, :n] - ref_es[s, :, :n]) / np.abs(ref_es[s, :, :n]))
        e3 = np.max(np.abs(to[s, :, :n] - ref_to[s, :, :n]))
        assert e1 <= PARTIAL_TOL, f"{what} seq {s}: max_logits max-abs {e1:.3e}"
        assert e2 <= PARTIAL_TOL, f"{what} seq {s}: exp_sums max-rel {e2:.3e}"
        assert e3 <= PARTIAL_TOL, f"{what} seq {s}: tmp_out max-abs {e3:.3e}"


def announce(msg: str):
    print(f"[gpu] {msg}", flush=True)
