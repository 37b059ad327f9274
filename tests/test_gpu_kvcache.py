"""GPU parity of the KV cache writes (bf16 append, FP8 quantize-and-append) and
of decode over an FP8 cache, against the CPU oracle, through the C ABI.
Needs an MI355X.  Cache writes are integer work and compare bit for bit;
decode outputs use the bf16 tolerances of the other decode tests."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_cache_34_amd as pa
import workloads
from tests.gpu_util import (Dev, announce, assert_out_close, assert_partials_close, bf16_dev,
                            bf16_host_f64, i32_dev, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def u8_dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def f32_dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def append_problem(name, seed, lens, n_new, Hkv, D, layout="shuffled"):
    """A paged case whose last n_new[s] rows of sequence s are to be appended
    (taken from a fresh seeded draw), plus cu_seqlens over the new rows."""
    case = workloads.build_case(name, seed, lens, Hkv, Hkv, D, layout=layout)
    rng = np.random.default_rng(seed + 1000)
    total = int(sum(n_new))
    k_new = workloads.f32_to_bf16_bits(rng.standard_normal((total, Hkv, D)).astype(np.float32))
    v_new = workloads.f32_to_bf16_bits(rng.standard_normal((total, Hkv, D)).astype(np.float32))
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(n_new)
    return case, k_new, v_new, cu


APPEND_CASES = [
    ("decode step", [37, 100, 16, 1, 4096], [1, 1, 1, 1, 1], 8, 128),
    ("ragged prefill rows", [300, 17, 64, 1000], [300, 5, 0, 129], 8, 128),
    ("head dim 64", [33, 90], [33, 20], 2, 64),
    ("head dim 256", [513, 48], [9, 48], 4, 256),
    ("one kv head", [70, 1], [70, 1], 1, 128),
]


@pytest.mark.parametrize("what,lens,n_new,Hkv,D", APPEND_CASES)
def test_kv_append_bf16_bit_exact(orc, what, lens, n_new, Hkv, D):
    t = torch()
    case, k_new, v_new, cu = append_problem("append", 501, lens, n_new, Hkv, D)
    ref_k, ref_v = orc.kv_append(k_new, v_new, case.block_tables, case.seq_lens, cu,
                                 case.k_cache, case.v_cache)
    dev = Dev(case)
    announce(f"kv append bf16: {what}")
    pa.paged_attn_kv_append(bf16_dev(k_new), bf16_dev(v_new), dev.bt, dev.sl, i32_dev(cu),
                            int(max(n_new)), dev.k, dev.v)
    t.cuda.synchronize()
    got_k = dev.k.cpu().view(t.int16).numpy().view(np.uint16)
    got_v = dev.v.cpu().view(t.int16).numpy().view(np.uint16)
    assert np.array_equal(got_k, ref_k) and np.array_equal(got_v, ref_v)


def fp8_empty(num_blocks, Hkv, D):
    """An FP8 cache of NaN codes and NaN scales: anything not written shows."""
    codes = np.full((num_blocks, Hkv, 16, D), 0x7F, np.uint8)
    scales = np.full((num_blocks, Hkv, 16), np.nan, np.float32)
    return codes, scales


def crafted_rows(Hkv, D):
    """New rows with exact E4M3 ties after scaling (largest magnitude 448, so
    scale 1), a zero row, a negative-zero row and a wide dynamic range."""
    rows = np.zeros((4, Hkv, D), np.float32)
    ties = [448.0, 1.0625, 1.1875, 1.5 * 2 ** -9, 2.0 ** -10, 432.0, -1.0625, 3.0 * 2 ** -10]
    rows[0, :, :len(ties)] = ties
    rows[1] = 0.0
    rows[2] = -0.0
    rows[3] = np.exp2(np.linspace(-20, 10, D))[None, :] * np.where(np.arange(D) % 2, -1, 1)
    return workloads.f32_to_bf16_bits(rows)


@pytest.mark.parametrize("what,lens,n_new,Hkv,D", APPEND_CASES)
def test_kv_append_fp8_bit_exact(orc, what, lens, n_new, Hkv, D):
    t = torch()
    case, k_new, v_new, cu = append_problem("append8", 502, lens, n_new, Hkv, D)
    if n_new[0] >= 4:  # plant the crafted rows among the first sequence's new rows
        k_new[:4] = crafted_rows(Hkv, D)
        v_new[:4] = crafted_rows(Hkv, D)[::-1]
    codes, scales = fp8_empty(case.num_blocks, Hkv, D)
    rk, rv, rks, rvs = orc.kv_append_fp8(k_new, v_new, case.block_tables, case.seq_lens, cu,
                                         codes, codes, scales, scales)
    kc, vc, ks, vs = u8_dev(codes), u8_dev(codes), f32_dev(scales), f32_dev(scales)
    announce(f"kv append fp8: {what}")
    pa.paged_attn_kv_append_fp8(bf16_dev(k_new), bf16_dev(v_new), i32_dev(case.block_tables),
                                i32_dev(case.seq_lens), i32_dev(cu), int(max(n_new)), kc, vc, ks, vs)
    t.cuda.synchronize()
    for got, ref, name in ((kc, rk, "k codes"), (vc, rv, "v codes")):
        g = got.cpu().numpy()
        bad = np.argwhere(g != ref)
        assert bad.size == 0, f"{name}: {len(bad)} differ, first at {bad[0]}: {g[tuple(bad[0])]:#x} vs {ref[tuple(bad[0])]:#x}"
    for got, ref, name in ((ks, rks, "k scales"), (vs, rvs, "v scales")):
        g = got.cpu().numpy()
        assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), name


def quantized_case(orc, case, P=0, nan_tails=True):
    """The case's bf16 cache quantized row by row with the oracle; slots past
    each sequence's end and unused blocks get NaN codes and NaN scales."""
    kq, ks = orc.quantize_fp8(case.k_cache)
    vq, vs = orc.quantize_fp8(case.v_cache)
    if nan_tails:
        used = np.zeros((case.num_blocks, 16), bool)
        for s, L in enumerate(case.seq_lens):
            for tok in range(int(L)):
                used[case.block_tables[s, tok // 16], tok % 16] = True
        for a in (kq, vq):  # [blocks, H_kv, 16, D] -> [blocks, 16, H_kv, D]
            a.transpose(0, 2, 1, 3)[~used] = 0x7F
        for a in (ks, vs):  # [blocks, H_kv, 16] -> [blocks, 16, H_kv]
            a.transpose(0, 2, 1)[~used] = np.nan
    return kq, vq, ks, vs


DECODE_CASES = [
    ("tiny", lambda: workloads.tiny_decode(), (0, 16, 48)),
    ("edges G=4 D=128", lambda: workloads.build_case("fp8edges", 511, [1, 15, 16, 17, 511, 512, 513, 2000], 8, 2, 128), (0, 32, 512)),
    ("G=6 D=256", lambda: workloads.build_case("fp8d256", 512, [1, 100, 1030], 12, 2, 256), (0, 256)),
    ("G=1 D=64", lambda: workloads.build_case("fp8d64", 513, [3, 64, 700], 2, 2, 64), (0, 64)),
    ("G=8 D=128", lambda: workloads.build_case("fp8g8", 514, [900, 40], 16, 2, 128), (0, 512)),
    ("llama3-8b shape", lambda: workloads.llama3_8b_decode(), (512,)),
]


@pytest.mark.parametrize("what,make,partitions", DECODE_CASES)
def test_decode_fp8_parity(orc, what, make, partitions):
    t = torch()
    case = make()
    kq, vq, ks, vs = quantized_case(orc, case)
    kd, vd = orc.fp8_dequant(kq, ks), orc.fp8_dequant(vq, vs)
    ref = orc.decode_f64kv(case.q, kd, vd, case.block_tables, case.seq_lens, case.num_kv_heads,
                           case.scale)
    q, bt, sl = bf16_dev(case.q), i32_dev(case.block_tables), i32_dev(case.seq_lens)
    kc, vc, ksd, vsd = u8_dev(kq), u8_dev(vq), f32_dev(ks), f32_dev(vs)
    for P in partitions:
        announce(f"fp8 decode {what}: P={P} S={case.num_seqs} Hq={case.num_q_heads} "
                 f"Hkv={case.num_kv_heads} D={case.head_dim}")
        out = t.empty_like(q)
        if P == 0:
            pa.paged_attn_decode_fp8(q, kc, vc, ksd, vsd, bt, sl, float(case.scale), 0, out=out)
            t.cuda.synchronize()
            assert_out_close(bf16_host_f64(out), ref, f"fp8 {what} single pass")
            continue
        npart = pa.paged_attn_num_partitions(case.max_blocks_per_seq, 16, P)
        ws = pa.DecodeWorkspace(case.num_seqs, case.num_q_heads, case.head_dim, npart, "cuda", num_kv_heads=case.num_kv_heads)
        for b in (ws.max_logits, ws.exp_sums, ws.tmp_out):
            b.fill_(float("nan"))
        pa.paged_attn_decode_fp8(q, kc, vc, ksd, vsd, bt, sl, float(case.scale), P,
                                 max_logits=ws.max_logits, exp_sums=ws.exp_sums, tmp_out=ws.tmp_out,
                                 max_num_partitions=npart)
        pa.paged_attn_decode_reduce(ws.max_logits, ws.exp_sums, ws.tmp_out, sl, P, out)
        t.cuda.synchronize()
        rml, res, rto = orc.decode_partials_f64kv(case.q, kd, vd, case.block_tables, case.seq_lens,
                                                  case.num_kv_heads, case.scale, P, npart)
        assert_partials_close(ws.max_logits.cpu().numpy().astype(np.float64),
                              ws.exp_sums.cpu().numpy().astype(np.float64),
                              ws.tmp_out.cpu().numpy().astype(np.float64), rml, res, rto,
                              case.seq_lens, P, f"fp8 {what} P={P}")
        assert_out_close(bf16_host_f64(out), ref, f"fp8 {what} merged P={P}")


def test_fp8_decode_block_shuffle_is_bit_identical(orc):
    t = torch()
    case = workloads.build_case("fp8shuffle", 515, [45, 16, 777, 1], 8, 2, 128)
    kq, vq, ks, vs = quantized_case(orc, case, nan_tails=False)
    rng = np.random.default_rng(516)
    perm = rng.permutation(case.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    outs = []
    for k_, v_, ks_, vs_, bt_ in ((kq, vq, ks, vs, case.block_tables),
                                  (kq[inv], vq[inv], ks[inv], vs[inv], perm[case.block_tables])):
        out = t.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=t.bfloat16, device="cuda")
        pa.paged_attn_decode_fp8(bf16_dev(case.q), u8_dev(k_), u8_dev(v_), f32_dev(ks_), f32_dev(vs_),
                                 i32_dev(bt_.astype(np.int32)), i32_dev(case.seq_lens), float(case.scale),
                                 0, out=out)
        t.cuda.synchronize()
        outs.append(out.cpu().view(t.int16).numpy())
    announce("fp8 shuffle invariance")
    assert np.array_equal(outs[0], outs[1])


def test_append_fp8_then_decode_fp8(orc):
    """The pipeline a decode step runs: the new token of every sequence is
    quantized into the FP8 cache on the GPU, then decode reads the cache."""
    t = torch()
    case = workloads.build_case("fp8pipe", 517, [200, 33, 1, 1500], 16, 4, 128)
    kq, vq, ks, vs = quantized_case(orc, case, nan_tails=False)
    rng = np.random.default_rng(518)
    S, Hkv, D = case.num_seqs, case.num_kv_heads, case.head_dim
    k_new = workloads.f32_to_bf16_bits(rng.standard_normal((S, Hkv, D)).astype(np.float32))
    v_new = workloads.f32_to_bf16_bits(rng.standard_normal((S, Hkv, D)).astype(np.float32))
    cu = np.arange(S + 1, dtype=np.int32)
    rk, rv, rks, rvs = orc.kv_append_fp8(k_new, v_new, case.block_tables, case.seq_lens, cu,
                                         kq, vq, ks, vs)
    ref = orc.decode_fp8(case.q, rk, rv, rks, rvs, case.block_tables, case.seq_lens, Hkv, case.scale)
    kc, vc, ksd, vsd = u8_dev(kq), u8_dev(vq), f32_dev(ks), f32_dev(vs)
    bt, sl = i32_dev(case.block_tables), i32_dev(case.seq_lens)
    announce("fp8 append then decode")
    pa.paged_attn_kv_append_fp8(bf16_dev(k_new), bf16_dev(v_new), bt, sl, i32_dev(cu), 1, kc, vc,
                                ksd, vsd)
    out = t.empty((S, case.num_q_heads, D), dtype=t.bfloat16, device="cuda")
    pa.paged_attn_decode_fp8(bf16_dev(case.q), kc, vc, ksd, vsd, bt, sl, float(case.scale), 0, out=out)
    t.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), rk) and np.array_equal(vsd.cpu().numpy(), rvs)
    assert_out_close(bf16_host_f64(out), ref, "fp8 pipeline")


# ---- the BI-V100 page's layouts: x-packed K, transposed V ------------------
from tests.oracle_pins import to_xpacked  # noqa: E402


@pytest.mark.parametrize("what,lens,n_new,Hkv,D", APPEND_CASES)
def test_kv_append_xpacked_bit_exact(orc, what, lens, n_new, Hkv, D):
    t = torch()
    case, k_new, v_new, cu = append_problem("appendx", 503, lens, n_new, Hkv, D)
    kx, vx = to_xpacked(case.k_cache, case.v_cache)
    ref_k, ref_v = orc.kv_append_xpacked(k_new, v_new, case.block_tables, case.seq_lens, cu, kx, vx)
    kd, vd = bf16_dev(kx), bf16_dev(vx)
    announce(f"kv append x-packed: {what}")
    pa.paged_attn_kv_append_xpacked(bf16_dev(k_new), bf16_dev(v_new), i32_dev(case.block_tables),
                                    i32_dev(case.seq_lens), i32_dev(cu), int(max(n_new)), kd, vd)
    t.cuda.synchronize()
    assert np.array_equal(kd.cpu().view(t.int16).numpy().view(np.uint16), ref_k)
    assert np.array_equal(vd.cpu().view(t.int16).numpy().view(np.uint16), ref_v)


XP_CASES = [
    ("tiny", lambda: workloads.tiny_decode(), (0, 16, 48)),
    ("edges G=4 D=128", lambda: workloads.build_case("xpedges", 521, [1, 15, 16, 17, 511, 512, 513, 2000], 8, 2, 128), (0, 32, 512)),
    ("G=6 D=256", lambda: workloads.build_case("xpd256", 522, [1, 100, 1030], 12, 2, 256), (0, 256)),
    ("G=1 D=64", lambda: workloads.build_case("xpd64", 523, [3, 64, 700], 2, 2, 64), (0, 64)),
    ("G=16 D=128", lambda: workloads.build_case("xpg16", 524, [900, 40, 1], 16, 1, 128), (0, 512)),
    ("llama3-8b shape", lambda: workloads.llama3_8b_decode(), (512,)),
]


def run_decode_layouts(case, P):
    """Decode (P = 0) or partials + merge through both layouts; returns
    (row-major out, x-packed out, x-packed partials or None)."""
    t = torch()
    kx, vx = to_xpacked(case.k_cache, case.v_cache)
    q, bt, sl = bf16_dev(case.q), i32_dev(case.block_tables), i32_dev(case.seq_lens)
    k, v, kxd, vxd = bf16_dev(case.k_cache), bf16_dev(case.v_cache), bf16_dev(kx), bf16_dev(vx)
    outs, parts = [], None
    for xp in (False, True):
        out = t.empty_like(q)
        fn = pa.paged_attn_decode_xpacked if xp else pa.paged_attn_decode
        kk, vv = (kxd, vxd) if xp else (k, v)
        if P == 0:
            fn(q, kk, vv, bt, sl, float(case.scale), 0, out=out)
        else:
            npart = pa.paged_attn_num_partitions(case.max_blocks_per_seq, 16, P)
            ws = pa.DecodeWorkspace(case.num_seqs, case.num_q_heads, case.head_dim, npart, "cuda", num_kv_heads=case.num_kv_heads)
            for b in (ws.max_logits, ws.exp_sums, ws.tmp_out):
                b.fill_(float("nan"))
            fn(q, kk, vv, bt, sl, float(case.scale), P, max_logits=ws.max_logits, exp_sums=ws.exp_sums,
               tmp_out=ws.tmp_out, max_num_partitions=npart)
            pa.paged_attn_decode_reduce(ws.max_logits, ws.exp_sums, ws.tmp_out, sl, P, out)
            if xp:
                parts = tuple(b.cpu().numpy().astype(np.float64) for b in (ws.max_logits, ws.exp_sums, ws.tmp_out))
        t.cuda.synchronize()
        outs.append(out)
    return outs[0], outs[1], parts, kx, vx


@pytest.mark.parametrize("what,make,partitions", XP_CASES)
def test_decode_xpacked_parity(orc, what, make, partitions):
    t = torch()
    case = make()
    ref = None
    for P in partitions:
        announce(f"x-packed decode {what}: P={P} S={case.num_seqs} Hq={case.num_q_heads} "
                 f"Hkv={case.num_kv_heads} D={case.head_dim}")
        o_rm, o_xp, parts, kx, vx = run_decode_layouts(case, P)
        if ref is None:
            ref = orc.decode_xpacked(case.q, kx, vx, case.block_tables, case.seq_lens, case.num_kv_heads,
                                     case.scale)
        assert_out_close(bf16_host_f64(o_xp), ref, f"x-packed {what} P={P}")
        # the same operands reach the same MFMAs in both layouts
        assert np.array_equal(o_rm.cpu().view(t.int16).numpy(), o_xp.cpu().view(t.int16).numpy()), \
            f"x-packed {what} P={P}: not bit-identical to the row-major layout"
        if parts is not None:
            rml, res, rto = orc.decode_partials_xpacked(case.q, kx, vx, case.block_tables, case.seq_lens,
                                                        case.num_kv_heads, case.scale, P, parts[0].shape[2])
            assert_partials_close(*parts, rml, res, rto, case.seq_lens, P, f"x-packed {what} P={P}")


def test_decode_xpacked_nan_in_unused_slots(orc):
    """Slots past a sequence's end may hold NaN in either layout."""
    t = torch()
    case = workloads.build_case("xpnan", 525, [5, 16, 33, 100], 8, 2, 128)
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    for s, L in enumerate(case.seq_lens):
        nb = (int(L) + 15) // 16
        if L % 16:
            b = case.block_tables[s, nb - 1]
            kc[b, :, L % 16:] = 0x7FC0
            vc[b, :, L % 16:] = 0x7FC0
    case2 = workloads.PagedCase(**{**case.__dict__, "k_cache": kc, "v_cache": vc})
    ref = orc.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, 2, case.scale)
    announce("x-packed decode with NaN tails")
    for P in (0, 32):
        _, o_xp, _, _, _ = run_decode_layouts(case2, P)
        assert_out_close(bf16_host_f64(o_xp), ref, f"x-packed NaN tails P={P}")


# ---- the AstrAI page's token-granular cache (page size 1, kv_indptr) -------
def tokens_case(seed, lens, Hq, Hkv, D, extra=50):
    """A [num_slots, H_kv, D] pool with each sequence's tokens in random slots
    (unused slots hold NaN), kv_indptr and kv_indices, and bf16 N(0,1) data."""
    rng = np.random.default_rng(seed)
    total = int(sum(lens))
    slots = total + extra
    pool_k = workloads.f32_to_bf16_bits(rng.standard_normal((slots, Hkv, D)).astype(np.float32))
    pool_v = workloads.f32_to_bf16_bits(rng.standard_normal((slots, Hkv, D)).astype(np.float32))
    perm = rng.permutation(slots).astype(np.int32)
    indptr = np.zeros(len(lens) + 1, np.int32)
    indptr[1:] = np.cumsum(lens)
    indices = perm[:total].copy()
    unused = perm[total:]
    pool_k[unused] = 0x7FC0
    pool_v[unused] = 0x7FC0
    q = workloads.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
    return q, pool_k, pool_v, indptr, indices, np.float32(1.0 / math.sqrt(D))


TOK_CASES = [
    ("edges G=4 D=128", [1, 15, 16, 17, 511, 512, 513, 2000], 8, 2, 128, (0, 32, 512)),
    ("G=6 D=256", [1, 100, 1030], 12, 2, 256, (0, 256)),
    ("G=1 D=64, a zero length", [3, 0, 64, 700], 2, 2, 64, (0, 64)),
    ("G=8 D=128, many chunks", [5000, 40], 16, 2, 128, (0, 1024)),
    # enough items that persistent workgroups take several each (the next
    # item's slot ids and first rows are fetched before an item's epilogue)
    ("G=4 D=128, several items per workgroup",
     [int(x) for x in np.random.default_rng(77).integers(200, 900, size=48)], 8, 2, 128, (32, 64)),
]


@pytest.mark.parametrize("what,lens,Hq,Hkv,D,partitions", TOK_CASES)
def test_decode_tokens_parity(orc, what, lens, Hq, Hkv, D, partitions):
    t = torch()
    q, kp, vp, indptr, indices, scale = tokens_case(531, lens, Hq, Hkv, D)
    ref = orc.decode_tokens(q, kp, vp, indptr, indices, Hkv, scale)
    qd, kd, vd = bf16_dev(q), bf16_dev(kp), bf16_dev(vp)
    ipd, ixd = i32_dev(indptr), i32_dev(indices if indices.size else np.zeros(1, np.int32))
    max_kv = max(max(lens), 1)
    for P in partitions:
        announce(f"token-granular decode {what}: P={P} S={len(lens)} Hq={Hq} Hkv={Hkv} D={D}")
        out = t.full_like(qd, float("nan"))
        if P == 0:
            pa.paged_attn_decode_tokens(qd, kd, vd, ipd, ixd, max_kv, float(scale), 0, out=out)
            t.cuda.synchronize()
            assert_out_close(bf16_host_f64(out), ref, f"tokens {what} single pass")
            continue
        npart = pa.paged_attn_num_partitions((max_kv + 15) // 16, 16, P)
        ws = pa.DecodeWorkspace(len(lens), Hq, D, npart, "cuda", num_kv_heads=Hkv)
        for b in (ws.max_logits, ws.exp_sums, ws.tmp_out):
            b.fill_(float("nan"))
        pa.paged_attn_decode_tokens(qd, kd, vd, ipd, ixd, max_kv, float(scale), P,
                                    max_logits=ws.max_logits, exp_sums=ws.exp_sums, tmp_out=ws.tmp_out,
                                    max_num_partitions=npart)
        pa.paged_attn_decode_reduce_indptr(ws.max_logits, ws.exp_sums, ws.tmp_out, ipd, P, out)
        t.cuda.synchronize()
        rml, res, rto = orc.decode_partials_tokens(q, kp, vp, indptr, indices, Hkv, scale, P, npart)
        assert_partials_close(ws.max_logits.cpu().numpy().astype(np.float64),
                              ws.exp_sums.cpu().numpy().astype(np.float64),
                              ws.tmp_out.cpu().numpy().astype(np.float64), rml, res, rto,
                              np.diff(indptr), P, f"tokens {what} P={P}")
        assert_out_close(bf16_host_f64(out), ref, f"tokens {what} merged P={P}")


def test_decode_tokens_equals_block_cache_one_kv_head():
    """With one kv head a block cache [blocks, 1, 16, D] is the slot pool
    [blocks * 16, 1, D]: the token-granular decode over slot ids
    16 * block + slot equals the block decode bit for bit."""
    t = torch()
    case = workloads.build_case("tokblk", 532, [1, 40, 300, 1100], 8, 1, 128)
    dev = Dev(case)
    idx, indptr = [], [0]
    for s, L in enumerate(case.seq_lens):
        for tok in range(int(L)):
            idx.append(int(case.block_tables[s, tok // 16]) * 16 + tok % 16)
        indptr.append(len(idx))
    nb = case.num_blocks
    kp = dev.k.view(nb * 16, 1, case.head_dim)
    vp = dev.v.view(nb * 16, 1, case.head_dim)
    announce("token-granular decode vs block decode, one kv head")
    for P in (0, 256):
        a, b = t.empty_like(dev.q), t.empty_like(dev.q)
        if P == 0:
            pa.paged_attn_decode(dev.q, dev.k, dev.v, dev.bt, dev.sl, float(case.scale), 0, out=a)
            pa.paged_attn_decode_tokens(dev.q, kp, vp, i32_dev(np.array(indptr, np.int32)),
                                        i32_dev(np.array(idx, np.int32)), int(case.seq_lens.max()),
                                        float(case.scale), 0, out=b)
        else:
            npart = pa.paged_attn_num_partitions(case.max_blocks_per_seq, 16, P)
            w1 = pa.DecodeWorkspace(case.num_seqs, case.num_q_heads, case.head_dim, npart, "cuda", num_kv_heads=case.num_kv_heads)
            w2 = pa.DecodeWorkspace(case.num_seqs, case.num_q_heads, case.head_dim, npart, "cuda", num_kv_heads=case.num_kv_heads)
            pa.paged_attn_decode(dev.q, dev.k, dev.v, dev.bt, dev.sl, float(case.scale), P,
                                 max_logits=w1.max_logits, exp_sums=w1.exp_sums, tmp_out=w1.tmp_out,
                                 max_num_partitions=npart)
            pa.paged_attn_decode_reduce(w1.max_logits, w1.exp_sums, w1.tmp_out, dev.sl, P, a)
            ipd = i32_dev(np.array(indptr, np.int32))
            pa.paged_attn_decode_tokens(dev.q, kp, vp, ipd, i32_dev(np.array(idx, np.int32)),
                                        case.max_blocks_per_seq * 16, float(case.scale), P,
                                        max_logits=w2.max_logits, exp_sums=w2.exp_sums, tmp_out=w2.tmp_out,
                                        max_num_partitions=npart)
            pa.paged_attn_decode_reduce_indptr(w2.max_logits, w2.exp_sums, w2.tmp_out, ipd, P, b)
        t.cuda.synchronize()
        assert np.array_equal(a.cpu().view(t.int16).numpy(), b.cpu().view(t.int16).numpy()), f"P={P}"
