"""GPU closed forms that hold bit for bit, through every decode path.

  * A sequence of one token returns that token's V row exactly: its score is
    the running max, its weight is exp(0) = 1 and its exp-sum 1, so nothing
    rounds.  Checked through the single pass, split-KV partials + merge, the
    fused merge and the FP8 cache (power-of-two dequant scales, so the
    dequantized row is bf16-exact).
  * Doubling V doubles the output exactly (every step is linear in V and a
    power-of-two scaling commutes with fp32 and bf16 rounding), through
    split-KV + merge and the fused merge as well as the single pass.

These are the survey's GPU pins (the oracle's own pins of the same forms are
in tests/oracle_pins.py); the RL.cu "Add Cuda Kernel" page's test section
checks fixed small cases against a reference the same way.  Expected values
come from the oracle, which is exact for these forms."""
import numpy as np
import pytest

import oracle
import paged_kv_cache_34_amd as pa
import workloads
from tests.gpu_util import (Dev, announce, assert_out_close, bf16_bits_host, bf16_dev, bf16_host_f64,
                            i32_dev, torch)

pytestmark = pytest.mark.gpu

# one-token sequences among longer ones (the longer ones make the partition
# schedule and the merge non-trivial); rows of the one-token ones must be exact
LENS = [1, 1, 37, 1, 600, 1]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def one_token_rows(case):
    return [s for s, L in enumerate(case.seq_lens) if L == 1]


def decode_all_paths(dev, P):
    """(name, bf16 output) for the single pass, split + merge and fused paths."""
    t = torch()
    c = dev.case
    outs = []
    out = t.full_like(dev.q, float("nan"))
    pa.paged_attn_decode(dev.q, dev.k, dev.v, dev.bt, dev.sl, float(c.scale), 0, out=out)
    outs.append(("single pass", out))
    npart = pa.paged_attn_num_partitions(c.max_blocks_per_seq, c.block_size, P)
    ws = pa.DecodeWorkspace(c.num_seqs, c.num_q_heads, c.head_dim, npart, "cuda",
                            num_kv_heads=c.num_kv_heads)
    for b in (ws.max_logits, ws.exp_sums, ws.tmp_out):
        b.fill_(float("nan"))
    out = t.full_like(dev.q, float("nan"))
    pa.paged_attn_decode(dev.q, dev.k, dev.v, dev.bt, dev.sl, float(c.scale), P,
                         max_logits=ws.max_logits, exp_sums=ws.exp_sums, tmp_out=ws.tmp_out,
                         max_num_partitions=npart)
    pa.paged_attn_decode_reduce(ws.max_logits, ws.exp_sums, ws.tmp_out, dev.sl, P, out)
    outs.append((f"split P={P} + merge", out))
    out = t.full_like(dev.q, float("nan"))
    pa.paged_attn_decode_fused(dev.q, dev.k, dev.v, dev.bt, dev.sl, float(c.scale), P, out,
                               ws.max_logits, ws.exp_sums, ws.tmp_out, ws.counters)
    outs.append((f"fused P={P}", out))
    t.cuda.synchronize()
    return outs


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_one_token_returns_v_exactly(orc, D, G):
    case = workloads.build_case(f"one_token_D{D}_G{G}", 700 + D + G, LENS, 2 * G, 2, D)
    ref = orc.decode_case(case)
    rows = one_token_rows(case)
    # the oracle's own closed form: the row is V of the one token, exactly
    for s in rows:
        g = np.arange(case.num_q_heads) // G
        v0 = workloads.bf16_bits_to_f32(case.v_cache[case.block_tables[s, 0], g, 0, :]).astype(np.float64)
        assert np.array_equal(ref[s], v0)
    dev = Dev(case)
    for P in (16, 512):
        announce(f"one-token rows bit-exact: D={D} G={G} P={P}")
        for name, out in decode_all_paths(dev, P):
            got = bf16_host_f64(out)
            assert np.array_equal(got[rows], ref[rows]), f"{name}: one-token rows differ from V"
            others = [s for s in range(case.num_seqs) if s not in rows]
            assert_out_close(got[others], ref[others], f"{name}: longer rows")


@pytest.mark.parametrize("D,G", [(128, 4), (256, 6)])
def test_one_token_returns_v_exactly_fp8(orc, D, G):
    """FP8 cache with power-of-two scales: the one token's dequantized V row
    (E4M3 value times 2^k) is a bf16 value, returned exactly."""
    t = torch()
    case = workloads.build_case(f"one_token_fp8_D{D}", 720 + D, LENS, 2 * G, 2, D)
    rng = np.random.default_rng(721 + D)
    shape = (case.num_blocks, case.num_kv_heads, 16, D)
    codes = [rng.integers(0, 256, size=shape).astype(np.uint8) for _ in range(2)]
    for c in codes:  # no NaN codes (0x7F / 0xFF) among the cached values
        c[(c & 0x7F) == 0x7F] = 0x7E
    scales = [np.exp2(rng.integers(-6, 3, size=shape[:3])).astype(np.float32) for _ in range(2)]
    kd, vd = orc.fp8_dequant(codes[0], scales[0]), orc.fp8_dequant(codes[1], scales[1])
    ref = orc.decode_f64kv(case.q, kd, vd, case.block_tables, case.seq_lens, case.num_kv_heads,
                           case.scale)
    rows = one_token_rows(case)
    q, bt, sl = bf16_dev(case.q), i32_dev(case.block_tables), i32_dev(case.seq_lens)
    kc, vc = (t.from_numpy(c).cuda() for c in codes)
    ks, vs = (t.from_numpy(s).cuda() for s in scales)
    for P in (0, 16):
        announce(f"fp8 one-token rows bit-exact: D={D} G={G} P={P}")
        out = t.full_like(q, float("nan"))
        if P == 0:
            pa.paged_attn_decode_fp8(q, kc, vc, ks, vs, bt, sl, float(case.scale), 0, out=out)
        else:
            npart = pa.paged_attn_num_partitions(case.max_blocks_per_seq, 16, P)
            ws = pa.DecodeWorkspace(case.num_seqs, case.num_q_heads, D, npart, "cuda",
                                    num_kv_heads=case.num_kv_heads)
            pa.paged_attn_decode_fp8(q, kc, vc, ks, vs, bt, sl, float(case.scale), P,
                                     max_logits=ws.max_logits, exp_sums=ws.exp_sums,
                                     tmp_out=ws.tmp_out, max_num_partitions=npart)
            pa.paged_attn_decode_reduce(ws.max_logits, ws.exp_sums, ws.tmp_out, sl, P, out)
        t.cuda.synchronize()
        got = bf16_host_f64(out)
        assert np.array_equal(got[rows], ref[rows]), f"fp8 P={P}: one-token rows differ from V"
        others = [s for s in range(case.num_seqs) if s not in rows]
        assert_out_close(got[others], ref[others], f"fp8 P={P}: longer rows")


@pytest.mark.parametrize("P", [16, 48, 512])
def test_value_doubling_is_exact_all_paths(P):
    case = workloads.build_case("vdouble", 730, [100, 37, 1, 2000, 513], 8, 2, 128)
    v2 = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(case.v_cache) * np.float32(2.0))
    case2 = workloads.PagedCase(**{**case.__dict__, "v_cache": v2})
    announce(f"value doubling, every path, P={P}")
    a = decode_all_paths(Dev(case), P)
    b = decode_all_paths(Dev(case2), P)
    for (name, o1), (_, o2) in zip(a, b):
        x1, x2 = bf16_host_f64(o1), bf16_host_f64(o2)
        assert np.all(np.isfinite(x1)), name
        assert np.array_equal(x2, 2.0 * x1), f"{name}: doubled V does not double the output exactly"
    # and the three paths agree with each other bit for bit on the one-token row
    assert np.array_equal(bf16_bits_host(a[0][1])[2], bf16_bits_host(a[2][1])[2])
