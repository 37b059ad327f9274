"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each `pin_*` function takes an `oracle.Oracle` and raises AssertionError when
the oracle disagrees with something other than itself:
  * brute force in pure Python (math.fsum, fp64) over *contiguous* K/V that the
    test itself pages into a shuffled, poisoned block pool;
  * closed forms (one token returns its value exactly; equal keys or a zero
    query return the mean of V; one dominant key returns its value);
  * invariants (physical-block shuffles, V scaling, GQA = MHA with duplicated
    kv heads, split partials merged = unsplit, merge order);
  * textbook special cases of prefill (no cached context = square causal
    attention; one new row = decode);
  * the worked example the AstrAI page prints for its Q-tile work map, and the
    BI-V100 page's shape arithmetic.
`run_all(path)` evaluates every pin against the library at `path` and reports
which fail; the mutation test uses it on oracle builds with planted mistakes.
"""
from __future__ import annotations

import json
import math
import os
import sys
from typing import Callable, Dict, List

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from workloads import bf16_bits_to_f32, f32_to_bf16_bits  # noqa: E402

POISON_BITS = int(f32_to_bf16_bits(np.array([64.0], dtype=np.float32))[0])


# --------------------------------------------------------------------------
# test-owned paging of contiguous K/V (independent of workloads' allocators)
# --------------------------------------------------------------------------
def rand_bits(rng, shape, sd=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


def page_contiguous(kc_list, vc_list, bs, rng, extra_blocks=3, pad_cols=2):
    """Place each sequence's contiguous [L, H_kv, D] K/V into a shuffled block pool.

    Unused blocks and tail slots are poison; table padding points at poison."""
    Hkv, D = kc_list[0].shape[1], kc_list[0].shape[2]
    need = [(k.shape[0] + bs - 1) // bs for k in kc_list]
    pool = sum(need) + extra_blocks
    perm = [int(x) for x in rng.permutation(pool)]
    kcache = np.full((pool, Hkv, bs, D), POISON_BITS, dtype=np.uint16)
    vcache = np.full((pool, Hkv, bs, D), POISON_BITS, dtype=np.uint16)
    bt = np.full((len(kc_list), max(need) + pad_cols), perm[-1], dtype=np.int32)
    pos = 0
    for s, (kc, vc) in enumerate(zip(kc_list, vc_list)):
        for b in range(need[s]):
            phys = perm[pos]
            pos += 1
            bt[s, b] = phys
            rows = kc[b * bs:(b + 1) * bs]
            kcache[phys, :, :rows.shape[0], :] = np.transpose(rows, (1, 0, 2))
            vcache[phys, :, :rows.shape[0], :] = np.transpose(vc[b * bs:(b + 1) * bs], (1, 0, 2))
    return kcache, vcache, bt


def brute_attention(qrow, Kc, Vc, g, scale, upto):
    """softmax(scale * q . k_t) v_t over t < upto, pure Python fp64 with fsum."""
    D = len(qrow)
    z = [scale * math.fsum(qrow[d] * Kc[t][g][d] for d in range(D)) for t in range(upto)]
    m = max(z)
    e = [math.exp(x - m) for x in z]
    den = math.fsum(e)
    return [math.fsum(e[t] * Vc[t][g][d] for t in range(upto)) / den for d in range(D)], m, den


def _f(bits):
    return bf16_bits_to_f32(bits).astype(np.float64).tolist()


def _tiny_decode_problem(seed, Hq, Hkv, D, lens, bs=16):
    rng = np.random.default_rng(seed)
    kc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    vc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    q = rand_bits(rng, (len(lens), Hq, D))
    kcache, vcache, bt = page_contiguous(kc, vc, bs, rng)
    return q, kc, vc, kcache, vcache, bt, np.asarray(lens, dtype=np.int32)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max-abs {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# O1 decode
# --------------------------------------------------------------------------
def pin_decode_brute_force(orc):
    shapes = [(11, 4, 1, 16, [37, 100]), (12, 4, 2, 8, [1, 16, 17, 33]),
              (13, 6, 2, 32, [15, 48]), (14, 2, 2, 64, [70])]
    for seed, Hq, Hkv, D, lens in shapes:
        q, kc, vc, kcache, vcache, bt, sl = _tiny_decode_problem(seed, Hq, Hkv, D, lens)
        scale = np.float32(1.0 / math.sqrt(D))
        out = orc.decode(q, kcache, vcache, bt, sl, Hkv, scale)
        G = Hq // Hkv
        for s, L in enumerate(lens):
            K, V = _f(kc[s]), _f(vc[s])
            for h in range(Hq):
                ref, _, _ = brute_attention(_f(q[s, h]), K, V, h // G, float(scale), L)
                _close(out[s, h], ref, 1e-12, f"decode seed {seed} s{s} h{h}")


def pin_decode_tiny_config_library(orc):
    """The 2-sequence D=64 workload against numpy/scipy softmax on gathered rows."""
    from scipy.special import softmax
    case = workloads.tiny_decode()
    out = orc.decode_case(case)
    G = case.num_q_heads // case.num_kv_heads
    for s, L in enumerate(case.seq_lens):
        t = np.arange(L)
        phys = case.block_tables[s, t // case.block_size]
        for h in range(case.num_q_heads):
            K = bf16_bits_to_f32(case.k_cache[phys, h // G, t % case.block_size]).astype(np.float64)
            V = bf16_bits_to_f32(case.v_cache[phys, h // G, t % case.block_size]).astype(np.float64)
            qv = bf16_bits_to_f32(case.q[s, h]).astype(np.float64)
            p = softmax(float(case.scale) * (K @ qv))
            _close(out[s, h], p @ V, 1e-12, f"tiny config s{s} h{h}")


def pin_single_token_returns_value(orc):
    rng = np.random.default_rng(21)
    Hq, Hkv, D = 6, 2, 32
    lens = [1, 1, 1]
    kc = [rand_bits(rng, (1, Hkv, D)) for _ in lens]
    vc = [rand_bits(rng, (1, Hkv, D)) for _ in lens]
    q = rand_bits(rng, (3, Hq, D))
    kcache, vcache, bt = page_contiguous(kc, vc, 16, rng)
    out = orc.decode(q, kcache, vcache, bt, np.ones(3, np.int32), Hkv, np.float32(0.17))
    for s in range(3):
        for h in range(Hq):
            exact = bf16_bits_to_f32(vc[s][0, h // 3]).astype(np.float64)
            assert np.array_equal(out[s, h], exact), f"seq_len 1 must return V exactly (s{s} h{h})"


def pin_equal_keys_give_mean(orc):
    rng = np.random.default_rng(22)
    Hq, Hkv, D = 4, 2, 16
    lens = [5, 31, 40]
    kc = []
    for L in lens:
        one = rand_bits(rng, (1, Hkv, D))
        kc.append(np.repeat(one, L, axis=0))
    vc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    q = rand_bits(rng, (3, Hq, D))
    kcache, vcache, bt = page_contiguous(kc, vc, 16, rng)
    out = orc.decode(q, kcache, vcache, bt, np.asarray(lens, np.int32), Hkv, np.float32(0.25))
    for s, L in enumerate(lens):
        V = bf16_bits_to_f32(vc[s]).astype(np.float64)
        for h in range(Hq):
            mean = [math.fsum(V[t, h // 2, d] for t in range(L)) / L for d in range(D)]
            _close(out[s, h], mean, 1e-13, f"equal keys s{s} h{h}")


def pin_zero_query_gives_mean(orc):
    rng = np.random.default_rng(23)
    Hq, Hkv, D = 4, 4, 16
    lens = [3, 18, 64]
    kc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    vc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    q = np.zeros((3, Hq, D), dtype=np.uint16)
    kcache, vcache, bt = page_contiguous(kc, vc, 16, rng)
    out = orc.decode(q, kcache, vcache, bt, np.asarray(lens, np.int32), Hkv, np.float32(0.25))
    for s, L in enumerate(lens):
        V = bf16_bits_to_f32(vc[s]).astype(np.float64)
        for h in range(Hq):
            mean = [math.fsum(V[t, h, d] for t in range(L)) / L for d in range(D)]
            _close(out[s, h], mean, 1e-13, f"zero query s{s} h{h}")


def pin_dominant_key(orc):
    rng = np.random.default_rng(24)
    D, L, hot = 16, 29, 11
    K = np.zeros((L, 1, D), np.float32)
    K[hot, 0, 0] = 16.0
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 16.0
    kb = f32_to_bf16_bits(K)
    vb = rand_bits(rng, (L, 1, D))
    kcache, vcache, bt = page_contiguous([kb], [vb], 16, rng)
    out = orc.decode(f32_to_bf16_bits(q), kcache, vcache, bt, np.asarray([L], np.int32), 1,
                     np.float32(0.125))
    # score of the hot key is 32, all others 0: its weight is 1 - (L-1) e^-32 / (1 + ...)
    _close(out[0, 0], bf16_bits_to_f32(vb[hot, 0]).astype(np.float64), 1e-11, "dominant key")


def pin_block_shuffle_invariance(orc):
    case = workloads.build_case("shuffle", 31, [45, 16, 77, 1], 8, 2, 32, layout="shuffled")
    out = orc.decode_case(case)
    rng = np.random.default_rng(32)
    perm = rng.permutation(case.num_blocks)        # new physical index of every block
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    k2 = case.k_cache[inv]
    v2 = case.v_cache[inv]
    bt2 = perm[case.block_tables].astype(np.int32)
    out2 = orc.decode(case.q, k2, v2, bt2, case.seq_lens, case.num_kv_heads, case.scale)
    assert np.array_equal(out, out2), "physical block shuffle changed the output"


def pin_value_scaling(orc):
    case = workloads.build_case("vscale", 33, [20, 50], 4, 2, 16)
    out = orc.decode_case(case)
    v2 = f32_to_bf16_bits(bf16_bits_to_f32(case.v_cache) * np.float32(2.0))
    out2 = orc.decode(case.q, case.k_cache, v2, case.block_tables, case.seq_lens,
                      case.num_kv_heads, case.scale)
    assert np.array_equal(out2, 2.0 * out), "V * 2 must give out * 2 exactly"


def pin_gqa_equals_mha_with_duplicated_heads(orc):
    case = workloads.build_case("gqa", 34, [23, 64, 5], 6, 2, 16)
    out = orc.decode_case(case)
    G = 3
    k_mha = np.repeat(case.k_cache, G, axis=1)  # kv head j of MHA = kv head j // G
    v_mha = np.repeat(case.v_cache, G, axis=1)
    out2 = orc.decode(case.q, k_mha, v_mha, case.block_tables, case.seq_lens, 6, case.scale)
    assert np.array_equal(out, out2), "GQA must equal MHA over duplicated kv heads"


# --------------------------------------------------------------------------
# O2 / O3 partials and merge
# --------------------------------------------------------------------------
def pin_partials_brute_force(orc):
    seed, Hq, Hkv, D, lens = 41, 4, 2, 8, [16, 47, 50]
    q, kc, vc, kcache, vcache, bt, sl = _tiny_decode_problem(seed, Hq, Hkv, D, lens)
    scale = np.float32(0.3)
    P = 16
    ml, es, to = orc.decode_partials(q, kcache, vcache, bt, sl, Hkv, scale, P)
    for s, L in enumerate(lens):
        K, V = _f(kc[s]), _f(vc[s])
        for h in range(Hq):
            for p in range((L + P - 1) // P):
                t0, t1 = p * P, min(L, (p + 1) * P)
                o, m, den = brute_attention(_f(q[s, h]), K[t0:t1], V[t0:t1], h // 2, float(scale),
                                            t1 - t0)
                _close(ml[s, h, p], m, 1e-13, "partial max")
                _close(es[s, h, p], den, 1e-12, "partial exp_sum")
                _close(to[s, h, p], o, 1e-12, "partial out")
            for p in range((L + P - 1) // P, ml.shape[2]):
                assert np.isnan(ml[s, h, p]), "partitions past the sequence must stay unwritten"


def pin_split_equals_unsplit(orc):
    for P, lens in ((16, [1, 15, 16, 17, 100]), (48, [47, 48, 49, 200]), (512, [511, 512, 513, 1500])):
        case = workloads.build_case(f"split{P}", 42 + P, lens, 6, 2, 16)
        ref = orc.decode_case(case)
        ml, es, to = orc.partials_case(case, P)
        out = orc.reduce(ml, es, to, case.seq_lens, P)
        _close(out, ref, 1e-12, f"merged partials P={P}")


def pin_merge_order_invariance(orc):
    case = workloads.build_case("order", 45, [300, 129], 4, 4, 16)
    P = 32
    ml, es, to = orc.partials_case(case, P)
    ref = orc.reduce(ml, es, to, case.seq_lens, P)
    rng = np.random.default_rng(46)
    for s, L in enumerate(case.seq_lens):
        n = (int(L) + P - 1) // P
        perm = rng.permutation(n)
        ml[s, :, :n] = ml[s][:, perm]
        es[s, :, :n] = es[s][:, perm]
        to[s, :, :n] = to[s][:, perm, :]
    out = orc.reduce(ml, es, to, case.seq_lens, P)
    _close(out, ref, 1e-14, "merge order")


def pin_shape_arithmetic(orc):
    g = json.load(open(os.path.join(HERE, "golden", "shape_arithmetic_biv100.json")))
    assert g["seq_len"] // g["block_size"] == g["blocks"]
    n = workloads.num_partitions(g["blocks"], g["block_size"], g["partition_size"])
    assert n == g["partitions_exact"], n
    assert abs(n - g["partitions_page_rounded"]) <= 5
    assert 4 + 4 + 4 * g["head_dim"] == g["partial_record_bytes"]


# --------------------------------------------------------------------------
# O4 prefill
# --------------------------------------------------------------------------
def _prefill_problem(seed, Hq, Hkv, D, n_new, cached, bs=16):
    rng = np.random.default_rng(seed)
    lens = [c + n for c, n in zip(cached, n_new)]
    kc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    vc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(n_new)
    q = rand_bits(rng, (int(cu[-1]), Hq, D))
    kcache, vcache, bt = page_contiguous(kc, vc, bs, rng)
    return q, kc, vc, kcache, vcache, bt, np.asarray(lens, np.int32), cu


def pin_prefill_square_causal(orc):
    """No cached context: every sequence is textbook causal self-attention."""
    Hq, Hkv, D = 4, 2, 8
    n_new = [5, 1, 19]
    q, kc, vc, kcache, vcache, bt, sl, cu = _prefill_problem(51, Hq, Hkv, D, n_new, [0, 0, 0])
    scale = np.float32(1.0 / math.sqrt(D))
    out = orc.prefill(q, kcache, vcache, bt, sl, cu, Hkv, scale)
    for s, n in enumerate(n_new):
        K, V = _f(kc[s]), _f(vc[s])
        for i in range(n):
            for h in range(Hq):
                ref, _, _ = brute_attention(_f(q[cu[s] + i, h]), K, V, h // 2, float(scale), i + 1)
                _close(out[cu[s] + i, h], ref, 1e-12, f"square causal s{s} row{i} h{h}")


def pin_prefill_with_cache_brute_force(orc):
    Hq, Hkv, D = 2, 1, 8
    n_new, cached = [3, 7, 1], [13, 0, 30]
    q, kc, vc, kcache, vcache, bt, sl, cu = _prefill_problem(52, Hq, Hkv, D, n_new, cached)
    scale = np.float32(0.4)
    out = orc.prefill(q, kcache, vcache, bt, sl, cu, Hkv, scale)
    for s, (n, c) in enumerate(zip(n_new, cached)):
        K, V = _f(kc[s]), _f(vc[s])
        for j in range(n):
            for h in range(Hq):
                ref, _, _ = brute_attention(_f(q[cu[s] + j, h]), K, V, 0, float(scale), c + j + 1)
                _close(out[cu[s] + j, h], ref, 1e-12, f"cached prefill s{s} row{j}")


def pin_prefill_one_row_is_decode(orc):
    case = workloads.prefill_case("onerow", 53, [1, 1, 1, 1], [0, 16, 40, 99], 4, 2, 16)
    out = orc.prefill_case(case)
    ref = orc.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                     case.num_kv_heads, case.scale)
    assert np.array_equal(out, ref), "one new row per sequence must equal decode"


def pin_tile_map_golden(orc):
    import oracle as oracle_pkg
    g = json.load(open(os.path.join(HERE, "golden", "tile_map_astrai.json")))
    indptr = [0] + list(np.cumsum(g["q_lens"]))
    assert indptr == g["qo_indptr"]
    b, i = oracle_pkg.tile_map(g["qo_indptr"], g["tile_rows"])
    assert b == g["q_tile_to_batch"] and i == g["q_tile_to_index"], (b, i)


# --------------------------------------------------------------------------
# KV append (the cache write before decode / prefill)
# --------------------------------------------------------------------------
def _append_problem(seed, Hkv, D, lens, n_new, bs=16):
    """Contiguous K/V for every sequence, paged by the test; the last n_new[s]
    rows of sequence s are the rows to append."""
    rng = np.random.default_rng(seed)
    kc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    vc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    kcache, vcache, bt = page_contiguous(kc, vc, bs, rng)
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(n_new)
    k_new = np.concatenate([kc[s][L - n:] for s, (L, n) in enumerate(zip(lens, n_new))])
    v_new = np.concatenate([vc[s][L - n:] for s, (L, n) in enumerate(zip(lens, n_new))])
    return kc, vc, kcache, vcache, bt, np.asarray(lens, np.int32), cu, k_new, v_new


def _slots_of_new_rows(bt, lens, n_new, bs):
    """(block, slot) of every appended position, from the test's own paging."""
    out = []
    for s, (L, n) in enumerate(zip(lens, n_new)):
        for t in range(L - n, L):
            out.append((int(bt[s, t // bs]), t % bs))
    return out


def pin_kv_append_refills_erased_rows(orc):
    """Erase the last rows of each sequence from a paged cache, append them back
    from the contiguous rows: the cache must come back bit for bit (rows of
    sequences with nothing to append, and every other slot, untouched)."""
    lens, n_new, bs = [37, 16, 1, 70, 5], [5, 16, 1, 0, 3], 16
    kc, vc, kcache, vcache, bt, sl, cu, k_new, v_new = _append_problem(61, 2, 8, lens, n_new)
    k_er, v_er = kcache.copy(), vcache.copy()
    for b, t in _slots_of_new_rows(bt, lens, n_new, bs):
        k_er[b, :, t] = 0x7FC0  # NaN bits: any row left unwritten shows
        v_er[b, :, t] = 0x7FC0
    k2, v2 = orc.kv_append(k_new, v_new, bt, sl, cu, k_er, v_er)
    assert np.array_equal(k2, kcache) and np.array_equal(v2, vcache), "append did not restore the cache"
    b, t = _slots_of_new_rows(bt, lens, n_new, bs)[0]
    assert k_er[b, 0, t, 0] == 0x7FC0, "the input caches must not be modified in place"


# --------------------------------------------------------------------------
# FP8 (OCP E4M3) KV cache
# --------------------------------------------------------------------------
def _e4m3_half_ulp(y):
    """Half the E4M3 spacing at magnitude y (spacing 2^-9 below 2^-6, else 2^(e-3))."""
    if y < 2.0 ** -6:
        return 2.0 ** -10
    return 2.0 ** (math.floor(math.log2(y)) - 4)


def pin_e4m3_values_match_the_specification(orc):
    g = json.load(open(os.path.join(HERE, "golden", "e4m3_ocp_facts.json")))
    for code, v in g["values"].items():
        got = orc.e4m3_value(int(code, 16))
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (code, got, v)
    for code in g["nan_codes"]:
        assert math.isnan(orc.e4m3_value(int(code, 16))), code
    pos = [orc.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:])), "magnitudes must increase with the code"
    assert sum(1 for v in pos if v > 0) == g["finite_positive_codes"]
    assert max(pos) == g["max_finite"]
    for c in range(0x7F):
        assert orc.e4m3_value(c | 0x80) == -orc.e4m3_value(c)


def pin_fp8_quantize_ties_to_even(orc):
    """Rows whose largest magnitude is 448 get scale 1, so each x / scale is x
    itself: exact midpoints between neighbouring codes must take the even code."""
    x = np.array([[448.0, 1.0625, 1.1875, 1.5 * 2 ** -9, 2.0 ** -10, 432.0, 1.078125, -1.0625]],
                 dtype=np.float32)
    codes, scales = orc.quantize_fp8(f32_to_bf16_bits(x))
    assert scales[0] == 1.0, scales
    want = [0x7E, 0x38, 0x3A, 0x02, 0x00, 0x7E, 0x39, 0xB8]
    assert codes[0].tolist() == want, [hex(c) for c in codes[0]]


def pin_fp8_quantize_round_trip(orc):
    """Rows made of E4M3 values times 2^k with one entry at +-448 * 2^k: the
    scale is 2^k exactly and every code comes back unchanged."""
    rng = np.random.default_rng(62)
    for k in (-8, 0, 3):
        codes0 = rng.integers(0, 0x7F, size=(6, 32)).astype(np.uint8)
        codes0 |= (rng.integers(0, 2, size=codes0.shape) * 0x80).astype(np.uint8)
        codes0[:, 5] = 0x7E | (codes0[:, 5] & 0x80)
        vals = np.array([[orc.e4m3_value(int(c)) * 2.0 ** k for c in row] for row in codes0],
                        dtype=np.float32)
        bits = f32_to_bf16_bits(vals)
        assert np.array_equal(bf16_bits_to_f32(bits), vals), "test values must be bf16-exact"
        codes, scales = orc.quantize_fp8(bits)
        assert np.all(scales == np.float32(2.0 ** k)), scales
        # +-0 keep their sign bit; every other code is reproduced exactly
        assert np.array_equal(codes, codes0), np.argwhere(codes != codes0)[:4]


def pin_fp8_quantize_error_bound(orc):
    """Random rows: each dequantized value is within half an E4M3 spacing (of
    x / scale, times the scale) of x, and the row maximum maps to +-448."""
    rng = np.random.default_rng(63)
    x = (rng.standard_normal((40, 64)) * np.exp(rng.uniform(-6, 6, size=(40, 1)))).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    xv = bf16_bits_to_f32(bits).astype(np.float64)
    codes, scales = orc.quantize_fp8(bits)
    deq = orc.fp8_dequant(codes, scales)
    for r in range(x.shape[0]):
        s = float(scales[r])
        amax = float(np.max(np.abs(xv[r])))
        assert abs(s - amax / 448.0) <= amax / 448.0 * 2.0 ** -23
        j = int(np.argmax(np.abs(xv[r])))
        assert codes[r, j] & 0x7F == 0x7E
        for d in range(x.shape[1]):
            y = abs(xv[r, d]) / s
            bound = _e4m3_half_ulp(y) * s * (1 + 1e-6) + amax * 2.0 ** -22
            assert abs(deq[r, d] - xv[r, d]) <= bound, (r, d, deq[r, d], xv[r, d])


def pin_fp8_quantize_zero_row(orc):
    x = np.zeros((2, 16), np.float32)
    x[1] = -0.0
    codes, scales = orc.quantize_fp8(f32_to_bf16_bits(x))
    assert scales.tolist() == [0.0, 0.0]
    assert codes[0].tolist() == [0] * 16 and codes[1].tolist() == [0x80] * 16


def _pow2_fp8_cache(rng, shape):
    """FP8 codes with power-of-two scales: every dequantized value is bf16-exact."""
    codes = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=shape) * 0x80).astype(np.uint8)
    scales = (2.0 ** rng.integers(-9, -3, size=shape[:-1])).astype(np.float32)
    return codes, scales


def pin_fp8_decode_equals_bf16_decode_when_exact(orc):
    """With power-of-two scales the dequantized cache is exactly a bf16 cache:
    the FP8 decode (and its partials) must equal the bf16 decode bit for bit."""
    rng = np.random.default_rng(64)
    Hq, Hkv, D, bs = 8, 2, 16, 16
    lens = np.array([1, 40, 100], np.int32)
    nb = 20
    kq, ks = _pow2_fp8_cache(rng, (nb, Hkv, bs, D))
    vq, vs = _pow2_fp8_cache(rng, (nb, Hkv, bs, D))
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.stack([perm[:7], perm[7:14], perm[13:20]])
    q = rand_bits(rng, (3, Hq, D))
    kd, vd = orc.fp8_dequant(kq, ks), orc.fp8_dequant(vq, vs)
    kb, vb = f32_to_bf16_bits(kd.astype(np.float32)), f32_to_bf16_bits(vd.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(kb).astype(np.float64), kd)
    scale = np.float32(0.25)
    got = orc.decode_fp8(q, kq, vq, ks, vs, bt, lens, Hkv, scale)
    ref = orc.decode(q, kb, vb, bt, lens, Hkv, scale)
    assert np.array_equal(got, ref)
    gp = orc.decode_partials_fp8(q, kq, vq, ks, vs, bt, lens, Hkv, scale, 32)
    rp = orc.decode_partials(q, kb, vb, bt, lens, Hkv, scale, 32)
    for a, b in zip(gp, rp):
        assert np.array_equal(np.nan_to_num(a), np.nan_to_num(b))


def pin_fp8_decode_single_token(orc):
    """One cached token: the output is that token's dequantized value row."""
    rng = np.random.default_rng(65)
    kq, ks = _pow2_fp8_cache(rng, (3, 1, 16, 32))
    vq = rng.integers(0, 0x7F, size=(3, 1, 16, 32)).astype(np.uint8)
    vs = np.array([[[0.013] * 16]] * 3, np.float32)
    bt = np.array([[2], [0]], np.int32)
    q = rand_bits(rng, (2, 4, 32))
    out = orc.decode_fp8(q, kq, vq, ks, vs, bt, np.array([1, 1], np.int32), 1, np.float32(0.2))
    deq = orc.fp8_dequant(vq, vs)
    for s, blk in enumerate((2, 0)):
        for h in range(4):
            assert np.array_equal(out[s, h], deq[blk, 0, 0]), (s, h)


def pin_fp8_kv_append_refills_erased_rows(orc):
    """FP8 append of the last rows of each sequence equals those rows quantized
    one by one and paged by the test, bit for bit (codes and scales)."""
    lens, n_new, bs = [37, 16, 1, 70], [5, 16, 1, 0], 16
    Hkv, D = 2, 16
    kc, vc, kcache, vcache, bt, sl, cu, k_new, v_new = _append_problem(66, Hkv, D, lens, n_new)
    nb = kcache.shape[0]
    k8 = np.full((nb, Hkv, bs, D), 0x7F, np.uint8)
    v8 = np.full((nb, Hkv, bs, D), 0x7F, np.uint8)
    ksc = np.full((nb, Hkv, bs), np.nan, np.float32)
    vsc = np.full((nb, Hkv, bs), np.nan, np.float32)
    k2, v2, ks2, vs2 = orc.kv_append_fp8(k_new, v_new, bt, sl, cu, k8, v8, ksc, vsc)
    ek, ev, eks, evs = k8.copy(), v8.copy(), ksc.copy(), vsc.copy()
    row = 0
    for s, (L, n) in enumerate(zip(lens, n_new)):
        for t in range(L - n, L):
            b, slot = int(bt[s, t // bs]), t % bs
            for g in range(Hkv):
                c, sc = orc.quantize_fp8(k_new[row, g][None])
                ek[b, g, slot], eks[b, g, slot] = c[0], sc[0]
                c, sc = orc.quantize_fp8(v_new[row, g][None])
                ev[b, g, slot], evs[b, g, slot] = c[0], sc[0]
            row += 1
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert np.array_equal(ks2, eks, equal_nan=True) and np.array_equal(vs2, evs, equal_nan=True)


# --------------------------------------------------------------------------
# the BI-V100 page's cache layouts: x-packed K, transposed V
# --------------------------------------------------------------------------
def to_xpacked(kcache, vcache, x=8):
    """Row-major [blocks, H, bs, D] caches -> K [blocks, H, D/x, bs, x] and
    V [blocks, H, D, bs], by reshaping and transposing (the test's own layout
    conversion, independent of the oracle's address arithmetic)."""
    nb, H, bs, D = kcache.shape
    k = np.ascontiguousarray(kcache.reshape(nb, H, bs, D // x, x).transpose(0, 1, 3, 2, 4))
    v = np.ascontiguousarray(vcache.transpose(0, 1, 3, 2))
    return k, v


def pin_xpacked_decode_brute_force(orc):
    for seed, Hq, Hkv, D, lens in [(71, 4, 2, 16, [1, 16, 17, 40]), (72, 6, 2, 32, [70, 9])]:
        q, kc, vc, kcache, vcache, bt, sl = _tiny_decode_problem(seed, Hq, Hkv, D, lens)
        kx, vx = to_xpacked(kcache, vcache)
        scale = np.float32(1.0 / math.sqrt(D))
        out = orc.decode_xpacked(q, kx, vx, bt, sl, Hkv, scale)
        G = Hq // Hkv
        for s, L in enumerate(lens):
            K, V = _f(kc[s]), _f(vc[s])
            for h in range(Hq):
                ref, _, _ = brute_attention(_f(q[s, h]), K, V, h // G, float(scale), L)
                _close(out[s, h], ref, 1e-12, f"x-packed decode seed {seed} s{s} h{h}")


def pin_xpacked_equals_row_major(orc):
    """The same cache in both layouts gives bit-identical outputs and partials."""
    case = workloads.build_case("xpack", 73, [1, 33, 130, 512], 8, 2, 64)
    kx, vx = to_xpacked(case.k_cache, case.v_cache)
    a = orc.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, 2, case.scale)
    b = orc.decode_xpacked(case.q, kx, vx, case.block_tables, case.seq_lens, 2, case.scale)
    assert np.array_equal(a, b)
    pa_ = orc.decode_partials(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, 2,
                              case.scale, 64)
    pb_ = orc.decode_partials_xpacked(case.q, kx, vx, case.block_tables, case.seq_lens, 2, case.scale, 64)
    for u, w in zip(pa_, pb_):
        assert np.array_equal(np.nan_to_num(u), np.nan_to_num(w))


def pin_xpacked_append_refills_erased_rows(orc):
    lens, n_new, bs = [37, 16, 1, 70], [5, 16, 1, 0], 16
    kc, vc, kcache, vcache, bt, sl, cu, k_new, v_new = _append_problem(74, 2, 16, lens, n_new)
    kx, vx = to_xpacked(kcache, vcache)
    k_er, v_er = kcache.copy(), vcache.copy()
    for b, t in _slots_of_new_rows(bt, lens, n_new, bs):
        k_er[b, :, t] = 0x7FC0
        v_er[b, :, t] = 0x7FC0
    kex, vex = to_xpacked(k_er, v_er)
    k2, v2 = orc.kv_append_xpacked(k_new, v_new, bt, sl, cu, kex, vex)
    assert np.array_equal(k2, kx) and np.array_equal(v2, vx), "x-packed append did not restore the cache"


# --------------------------------------------------------------------------
# token-granular cache (page_size 1, kv_indptr + kv_indices)
# --------------------------------------------------------------------------
def _tokens_problem(seed, Hq, Hkv, D, lens, extra=7):
    """Contiguous K/V per sequence scattered by the test into a shuffled
    [num_slots, H_kv, D] slot pool (unused slots hold poison)."""
    rng = np.random.default_rng(seed)
    kc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    vc = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    q = rand_bits(rng, (len(lens), Hq, D))
    total = sum(lens)
    slots = total + extra
    perm = rng.permutation(slots).astype(np.int32)
    kpool = np.full((slots, Hkv, D), POISON_BITS, np.uint16)
    vpool = np.full((slots, Hkv, D), POISON_BITS, np.uint16)
    indptr = np.zeros(len(lens) + 1, np.int32)
    indptr[1:] = np.cumsum(lens)
    indices = perm[:total].copy()
    for s, L in enumerate(lens):
        idx = indices[indptr[s]:indptr[s + 1]]
        kpool[idx] = kc[s]
        vpool[idx] = vc[s]
    return q, kc, vc, kpool, vpool, indptr, indices


def pin_tokens_decode_brute_force(orc):
    for seed, Hq, Hkv, D, lens in [(81, 4, 2, 16, [1, 5, 17, 40]), (82, 6, 3, 32, [70, 0, 9])]:
        q, kc, vc, kpool, vpool, indptr, indices = _tokens_problem(seed, Hq, Hkv, D, lens)
        scale = np.float32(1.0 / math.sqrt(D))
        out = orc.decode_tokens(q, kpool, vpool, indptr, indices, Hkv, scale)
        G = Hq // Hkv
        for s, L in enumerate(lens):
            if L == 0:
                assert np.all(out[s] == 0.0)
                continue
            K, V = _f(kc[s]), _f(vc[s])
            for h in range(Hq):
                ref, _, _ = brute_attention(_f(q[s, h]), K, V, h // G, float(scale), L)
                _close(out[s, h], ref, 1e-12, f"token-granular decode seed {seed} s{s} h{h}")


def pin_tokens_equals_block_size_one(orc):
    """A token-granular cache is a block cache with one-token blocks whose
    table rows are the index lists: outputs and partials agree bit for bit."""
    lens = [33, 1, 130, 64]
    q, kc, vc, kpool, vpool, indptr, indices = _tokens_problem(83, 8, 2, 32, lens)
    bt = np.zeros((len(lens), max(lens)), np.int32)
    for s, L in enumerate(lens):
        bt[s, :L] = indices[indptr[s]:indptr[s + 1]]
    sl = np.asarray(lens, np.int32)
    kb, vb = kpool[:, :, None, :], vpool[:, :, None, :]
    scale = np.float32(0.2)
    assert np.array_equal(orc.decode_tokens(q, kpool, vpool, indptr, indices, 2, scale),
                          orc.decode(q, kb, vb, bt, sl, 2, scale))
    a = orc.decode_partials_tokens(q, kpool, vpool, indptr, indices, 2, scale, 32, 5)
    b = orc.decode_partials(q, kb, vb, bt, sl, 2, scale, 32, 5)
    for u, w in zip(a, b):
        assert np.array_equal(np.nan_to_num(u), np.nan_to_num(w))


PINS: Dict[str, Callable] = {name: fn for name, fn in sorted(globals().items())
                             if name.startswith("pin_") and callable(fn)}


def run_all(path: str) -> List[str]:
    """Evaluate every pin on the oracle library at `path`; return failing pin names."""
    import oracle as oracle_pkg
    orc = oracle_pkg.Oracle(path)
    failed = []
    for name, fn in PINS.items():
        try:
            fn(orc)
        except AssertionError as e:
            failed.append(f"{name}: {str(e)[:120]}")
        except Exception as e:  # a crash inside a pin also rejects the oracle library under test
            failed.append(f"{name}: {type(e).__name__} {str(e)[:120]}")
    return failed


if __name__ == "__main__":
    fails = run_all(sys.argv[1])
    print(json.dumps({"failed": fails}))
