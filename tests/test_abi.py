"""The C ABI on the CPU: the library loads, exports every declared symbol, and
its host-side helpers and argument validation behave as documented.  No call
here reaches a kernel launch (every validation case fails before it)."""
import ctypes
import json
import os

import pytest

import paged_kv_cache_34_amd as pa

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIBRARY):
        from paged_kv_cache_34_amd import build
        build.build()
    return pa.library()


def test_exports_every_declared_symbol(lib):
    names = pa.declared_functions()
    assert set(names) == {
        "paged_attn_decode", "paged_attn_decode_fused", "paged_attn_decode_reduce",
        "paged_attn_prefill_ragged", "paged_attn_prefill_ragged_split",
        "paged_attn_prefill_chunk_size", "paged_attn_prefill_workspace_size",
        "paged_attn_num_partitions", "paged_attn_choose_partition_size",
        "paged_attn_prefill_tile_map", "paged_attn_status_string", "paged_attn_decode_fp8",
        "paged_attn_kv_append", "paged_attn_kv_append_fp8", "paged_attn_decode_xpacked",
        "paged_attn_kv_append_xpacked", "paged_attn_decode_tokens",
        "paged_attn_decode_reduce_indptr", "paged_attn_read_probe",
        "paged_attn_decode_fused_noalloc", "paged_attn_gather_probe"}
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert pa.status_string(0) == "ok"
    for code in range(1, 8):
        assert pa.status_string(code) not in ("ok", "unknown status")
    assert pa.status_string(99) == "unknown status"


def test_num_partitions(lib):
    g = json.load(open(os.path.join(HERE, "golden", "shape_arithmetic_biv100.json")))
    assert pa.paged_attn_num_partitions(g["blocks"], g["block_size"], g["partition_size"]) == g["partitions_exact"]
    assert pa.paged_attn_num_partitions(7, 16, 0) == 1
    assert pa.paged_attn_num_partitions(7, 16, 16) == 7
    assert pa.paged_attn_num_partitions(7, 16, 48) == 3
    assert pa.paged_attn_num_partitions(0, 16, 16) == -1
    assert pa.paged_attn_num_partitions(4, 16, -16) == -1


def test_tile_map_matches_printed_example(lib):
    g = json.load(open(os.path.join(HERE, "golden", "tile_map_astrai.json")))
    b, i = pa.paged_attn_prefill_tile_map(g["qo_indptr"], g["tile_rows"])
    assert b == g["q_tile_to_batch"] and i == g["q_tile_to_index"]


def test_tile_map_edge_cases(lib):
    assert pa.paged_attn_prefill_tile_map([0, 0, 0], 64) == ([], [])
    assert pa.paged_attn_prefill_tile_map([0, 64, 65], 64) == ([0, 1], [0, 0])
    with pytest.raises(ValueError):
        pa.paged_attn_prefill_tile_map([0, 5, 3], 64)


def test_choose_partition_size(lib):
    # small batch, long context: split-KV with a power of two >= 256
    p = pa.paged_attn_choose_partition_size(4, 4, 100_000, 400_000)
    assert p >= 256 and p & (p - 1) == 0
    # tiny problem with few (sequence, kv head) pairs: still split, never below 512
    assert pa.paged_attn_choose_partition_size(2, 1, 100, 137) == 512
    # the Llama-3-8B-shaped batch and the long-context batch use 512; the large ragged one 1024
    assert pa.paged_attn_choose_partition_size(32, 8, 4096, 72260) == 512
    assert pa.paged_attn_choose_partition_size(4, 4, 100_000, 400_000) == 512
    assert pa.paged_attn_choose_partition_size(256, 8, 32768, 449037) == 1024
    # enough (sequence, kv head) pairs with short contexts: single pass
    assert pa.paged_attn_choose_partition_size(4096, 8, 128, 4096 * 128) == 0
    assert pa.paged_attn_choose_partition_size(0, 8, 128) == 0


# ---- validation: every case below returns before any launch ----------------
NULL = None
FAKE = 0x10000  # 16-byte aligned non-null address, never dereferenced on these paths


def decode_call(lib, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=4, Hkv=1, D=64, bs=16, nb=16,
                mbps=7, scale=0.125, P=0, out=FAKE, ml=FAKE, es=FAKE, to=FAKE, NP=1)
    args.update(over)
    return lib.paged_attn_decode(args["q"], args["k"], args["v"], args["bt"], args["sl"], args["S"],
                                 args["Hq"], args["Hkv"], args["D"], args["bs"], args["nb"],
                                 args["mbps"], args["scale"], args["P"], args["out"], args["ml"],
                                 args["es"], args["to"], args["NP"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(k=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(bt=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(sl=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(out=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(P=16, to=NULL, NP=7), pa.PA_ERR_NULL_POINTER),
    (dict(Hq=6, Hkv=4), pa.PA_ERR_BAD_SHAPE),
    (dict(Hq=0), pa.PA_ERR_BAD_SHAPE),
    (dict(S=-1), pa.PA_ERR_BAD_SHAPE),
    (dict(nb=0), pa.PA_ERR_BAD_SHAPE),
    (dict(P=24, NP=5), pa.PA_ERR_BAD_SHAPE),
    (dict(P=-16), pa.PA_ERR_BAD_SHAPE),
    (dict(P=16, NP=6), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(D=512), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=32), pa.PA_ERR_UNSUPPORTED),
    (dict(Hq=34, Hkv=2), pa.PA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), pa.PA_ERR_ALIGNMENT),
    (dict(out=FAKE + 2), pa.PA_ERR_ALIGNMENT),
    (dict(scale=0.0), pa.PA_ERR_BAD_VALUE),
    (dict(scale=-0.125), pa.PA_ERR_BAD_VALUE),
    (dict(scale=float("inf")), pa.PA_ERR_BAD_VALUE),
    (dict(scale=float("nan")), pa.PA_ERR_BAD_VALUE),
    (dict(S=0), pa.PA_OK),
])
def test_decode_validation(lib, over, status):
    assert decode_call(lib, **over) == status


@pytest.mark.parametrize("over,status", [
    (dict(ml=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(P=0), pa.PA_ERR_BAD_SHAPE),
    (dict(P=20), pa.PA_ERR_BAD_SHAPE),
    (dict(NP=0), pa.PA_ERR_BAD_SHAPE),
    (dict(D=80), pa.PA_ERR_UNSUPPORTED),
    (dict(to=FAKE + 4), pa.PA_ERR_ALIGNMENT),
    (dict(S=0), pa.PA_OK),
])
def test_reduce_validation(lib, over, status):
    a = dict(ml=FAKE, es=FAKE, to=FAKE, sl=FAKE, S=2, Hq=4, D=64, P=16, NP=7, out=FAKE)
    a.update(over)
    st = lib.paged_attn_decode_reduce(a["ml"], a["es"], a["to"], a["sl"], a["S"], a["Hq"], a["D"],
                                      a["P"], a["NP"], a["out"], None)
    assert st == status


@pytest.mark.parametrize("over,status", [
    (dict(cu=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(out=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(total_q=-1), pa.PA_ERR_BAD_SHAPE),
    (dict(max_q=9, total_q=8), pa.PA_ERR_BAD_SHAPE),
    (dict(Hq=8, Hkv=3), pa.PA_ERR_BAD_SHAPE),
    (dict(D=48), pa.PA_ERR_UNSUPPORTED),
    (dict(out=FAKE + 6), pa.PA_ERR_ALIGNMENT),
    (dict(scale=-1.0), pa.PA_ERR_BAD_VALUE),
    (dict(scale=float("nan")), pa.PA_ERR_BAD_VALUE),
    (dict(total_q=0, max_q=0), pa.PA_OK),
    (dict(S=0), pa.PA_OK),
])
def test_prefill_validation(lib, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, S=2, total_q=8, max_q=4, Hq=4, Hkv=1,
             D=64, bs=16, nb=16, mbps=7, scale=0.125, out=FAKE)
    a.update(over)
    st = lib.paged_attn_prefill_ragged(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["cu"], a["S"],
                                       a["total_q"], a["max_q"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                       a["nb"], a["mbps"], a["scale"], a["out"], None)
    assert st == status


@pytest.mark.parametrize("over,status", [
    (dict(cnt=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(out=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(ml=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(P=0), pa.PA_ERR_BAD_SHAPE),
    (dict(P=16, NP=6), pa.PA_ERR_BAD_SHAPE),
    (dict(D=32), pa.PA_ERR_UNSUPPORTED),
    (dict(out=FAKE + 2), pa.PA_ERR_ALIGNMENT),
    (dict(scale=0.0), pa.PA_ERR_BAD_VALUE),
    (dict(S=0), pa.PA_OK),
])
def test_fused_decode_validation(lib, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=4, Hkv=1, D=64, bs=16, nb=16,
             mbps=7, scale=0.125, P=16, out=FAKE, ml=FAKE, es=FAKE, to=FAKE, NP=7, cnt=FAKE)
    a.update(over)
    st = lib.paged_attn_decode_fused(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["S"], a["Hq"],
                                     a["Hkv"], a["D"], a["bs"], a["nb"], a["mbps"], a["scale"],
                                     a["P"], a["out"], a["ml"], a["es"], a["to"], a["NP"], a["cnt"],
                                     None)
    assert st == status


def split_call(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, S=2, total_q=300, max_q=200, Hq=32,
             Hkv=8, D=128, bs=16, nb=1024, mbps=500, scale=0.125, chunk=256, ws=FAKE,
             wsb=1 << 40, out=FAKE)
    a.update(over)
    return lib.paged_attn_prefill_ragged_split(
        a["q"], a["k"], a["v"], a["bt"], a["sl"], a["cu"], a["S"], a["total_q"], a["max_q"], a["Hq"],
        a["Hkv"], a["D"], a["bs"], a["nb"], a["mbps"], a["scale"], a["chunk"], a["ws"], a["wsb"],
        a["out"], None)


@pytest.mark.parametrize("over,status", [
    (dict(cu=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(out=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(ws=NULL, S=0), pa.PA_OK),
    (dict(scale=0.0), pa.PA_ERR_BAD_VALUE),
    (dict(chunk=-32), pa.PA_ERR_BAD_SHAPE),
    (dict(chunk=48), pa.PA_ERR_BAD_SHAPE),
    (dict(chunk=96), pa.PA_ERR_BAD_SHAPE),
    (dict(chunk=8192 + 64), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(out=FAKE + 2), pa.PA_ERR_ALIGNMENT),
    (dict(max_q=301), pa.PA_ERR_BAD_SHAPE),
    (dict(S=0), pa.PA_OK),
    (dict(total_q=0, max_q=0), pa.PA_OK),
])
def test_prefill_split_validation(lib, over, status):
    assert split_call(lib, **over) == status


def test_prefill_split_workspace_checks(lib):
    # a chunk that splits needs a workspace of the documented size
    need = pa.paged_attn_prefill_workspace_size(300, 32, 128, 500, 16, 256)
    assert split_call(lib, ws=NULL) == pa.PA_ERR_NULL_POINTER
    assert split_call(lib, ws=FAKE + 8) == pa.PA_ERR_ALIGNMENT
    assert split_call(lib, wsb=need - 1) == pa.PA_ERR_BAD_SHAPE


def test_prefill_workspace_size_formula(lib):
    def ru(x):
        return (x + 255) // 256 * 256
    for total_q, hq, d, mbps, chunk in [(300, 32, 128, 500, 256), (1, 1, 64, 1, 32),
                                        (1815, 32, 128, 525, 1536), (7, 12, 256, 100, 8192)]:
        splits = -(-mbps * 16 // chunk)
        recs = total_q * hq * splits
        assert pa.paged_attn_prefill_workspace_size(total_q, hq, d, mbps, 16, chunk) == \
            256 + 2 * ru(recs * 4) + ru(recs * d * 4)
    assert pa.paged_attn_prefill_workspace_size(10, 4, 64, 10, 16, 0) == -1
    assert pa.paged_attn_prefill_workspace_size(10, 0, 64, 10, 16, 64) == -1


def test_prefill_chunk_size_heuristic(lib):
    # Without a GPU the device has 256 CUs in this formula: chunk =
    # ceil((ceil(total_q / (256 / G)) + S) * H_kv * L_max * 5 / (13 * 256)), rounded
    # up to 256, clamped to [512, 8192]; 0 when it covers L_max or the pairs overflow.
    # ragged prefill shape: 16 sequences, 1815 rows, G = 4, L_max = 525 * 16:
    # 45 * 8 * 8400 * 5 / 3328 = 4543.3 -> 4608
    assert pa.paged_attn_prefill_chunk_size(16, 1815, 32, 8, 525, 16) == 4608
    # one sequence, 64 new rows after a 100k context: 2 * 8 * 100000 * 5 / 3328
    # = 2403.8 -> 2560, many chunks for 8 workgroups
    assert pa.paged_attn_prefill_chunk_size(1, 64, 32, 8, 6250, 16) == 2560
    # short contexts: one chunk would cover them, so single pass
    assert pa.paged_attn_prefill_chunk_size(4, 100, 32, 8, 8, 16) == 0
    # more than 1024 (sequence, query tile) pairs: single pass
    assert pa.paged_attn_prefill_chunk_size(2000, 4000, 32, 8, 100, 16) == 0
    assert pa.paged_attn_prefill_chunk_size(0, 10, 32, 8, 100, 16) == 0
    # more than 128 query heads: single pass
    assert pa.paged_attn_prefill_chunk_size(2, 100, 256, 16, 1000, 16) == 0


@pytest.mark.parametrize("over,status", [
    (dict(ks=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(vs=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(q=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(ks=FAKE + 4), pa.PA_ERR_ALIGNMENT),
    (dict(vs=FAKE + 8), pa.PA_ERR_ALIGNMENT),
    (dict(k=FAKE + 1), pa.PA_ERR_ALIGNMENT),
    (dict(P=24, NP=5), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), pa.PA_ERR_BAD_VALUE),
    (dict(S=0), pa.PA_OK),
])
def test_decode_fp8_validation(lib, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=4, Hkv=1, D=64,
             bs=16, nb=16, mbps=7, scale=0.125, P=0, out=FAKE, ml=FAKE, es=FAKE, to=FAKE, NP=1)
    a.update(over)
    st = lib.paged_attn_decode_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["sl"], a["S"],
                                   a["Hq"], a["Hkv"], a["D"], a["bs"], a["nb"], a["mbps"], a["scale"],
                                   a["P"], a["out"], a["ml"], a["es"], a["to"], a["NP"], None)
    assert st == status


def append_call(lib, fp8, **over):
    a = dict(kn=FAKE, vn=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, S=3, T=40, maxn=20, Hkv=8, D=128, bs=16,
             nb=64, mbps=9, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE)
    a.update(over)
    common = (a["kn"], a["vn"], a["bt"], a["sl"], a["cu"], a["S"], a["T"], a["maxn"], a["Hkv"],
              a["D"], a["bs"], a["nb"], a["mbps"], a["kc"], a["vc"])
    if fp8:
        return lib.paged_attn_kv_append_fp8(*common, a["ks"], a["vs"], None)
    return lib.paged_attn_kv_append(*common, None)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("over,status", [
    (dict(kn=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(cu=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(vc=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(S=-1), pa.PA_ERR_BAD_SHAPE),
    (dict(T=-1), pa.PA_ERR_BAD_SHAPE),
    (dict(Hkv=0), pa.PA_ERR_BAD_SHAPE),
    (dict(maxn=41), pa.PA_ERR_BAD_SHAPE),
    (dict(D=80), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=8), pa.PA_ERR_UNSUPPORTED),
    (dict(kn=FAKE + 2), pa.PA_ERR_ALIGNMENT),
    (dict(vc=FAKE + 8), pa.PA_ERR_ALIGNMENT),
    (dict(S=0), pa.PA_OK),
    (dict(T=0, maxn=0), pa.PA_OK),
])
def test_kv_append_validation(lib, fp8, over, status):
    assert append_call(lib, fp8, **over) == status


def test_kv_append_fp8_needs_scales(lib):
    assert append_call(lib, True, ks=NULL) == pa.PA_ERR_NULL_POINTER
    assert append_call(lib, True, vs=FAKE + 4) == pa.PA_ERR_ALIGNMENT
    # the bf16 form takes no scales: its validation never looks at them
    assert append_call(lib, False, maxn=41, ks=NULL, vs=NULL) == pa.PA_ERR_BAD_SHAPE


@pytest.mark.parametrize("over,status", [
    (dict(q=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(P=16, to=NULL, NP=7), pa.PA_ERR_NULL_POINTER),
    (dict(Hq=6, Hkv=4), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(k=FAKE + 8), pa.PA_ERR_ALIGNMENT),
    (dict(scale=-1.0), pa.PA_ERR_BAD_VALUE),
    (dict(S=0), pa.PA_OK),
])
def test_decode_xpacked_validation(lib, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=4, Hkv=1, D=64, bs=16, nb=16,
             mbps=7, scale=0.125, P=0, out=FAKE, ml=FAKE, es=FAKE, to=FAKE, NP=1)
    a.update(over)
    st = lib.paged_attn_decode_xpacked(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["S"], a["Hq"],
                                       a["Hkv"], a["D"], a["bs"], a["nb"], a["mbps"], a["scale"],
                                       a["P"], a["out"], a["ml"], a["es"], a["to"], a["NP"], None)
    assert st == status


@pytest.mark.parametrize("over,status", [
    (dict(kn=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(maxn=41), pa.PA_ERR_BAD_SHAPE),
    (dict(D=80), pa.PA_ERR_UNSUPPORTED),
    (dict(vc=FAKE + 8), pa.PA_ERR_ALIGNMENT),
    (dict(S=0), pa.PA_OK),
])
def test_kv_append_xpacked_validation(lib, over, status):
    a = dict(kn=FAKE, vn=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, S=3, T=40, maxn=20, Hkv=8, D=128, bs=16,
             nb=64, mbps=9, kc=FAKE, vc=FAKE)
    a.update(over)
    st = lib.paged_attn_kv_append_xpacked(a["kn"], a["vn"], a["bt"], a["sl"], a["cu"], a["S"], a["T"],
                                          a["maxn"], a["Hkv"], a["D"], a["bs"], a["nb"], a["mbps"],
                                          a["kc"], a["vc"], None)
    assert st == status


@pytest.mark.parametrize("over,status", [
    (dict(ip=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(ix=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(q=NULL), pa.PA_ERR_NULL_POINTER),
    (dict(maxkv=0), pa.PA_ERR_BAD_SHAPE),
    (dict(slots=0), pa.PA_ERR_BAD_SHAPE),
    (dict(P=32, NP=3), pa.PA_ERR_BAD_SHAPE),   # ceil(100 / 16) tiles of 16 -> 4 partitions of 32
    (dict(Hq=6, Hkv=4), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(k=FAKE + 2), pa.PA_ERR_ALIGNMENT),
    (dict(scale=0.0), pa.PA_ERR_BAD_VALUE),
    (dict(S=0), pa.PA_OK),
])
def test_decode_tokens_validation(lib, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ip=FAKE, ix=FAKE, S=2, Hq=4, Hkv=1, D=64, slots=300, maxkv=100,
             scale=0.125, P=0, out=FAKE, ml=FAKE, es=FAKE, to=FAKE, NP=1)
    a.update(over)
    st = lib.paged_attn_decode_tokens(a["q"], a["k"], a["v"], a["ip"], a["ix"], a["S"], a["Hq"],
                                      a["Hkv"], a["D"], a["slots"], a["maxkv"], a["scale"], a["P"],
                                      a["out"], a["ml"], a["es"], a["to"], a["NP"], None)
    assert st == status


def test_reduce_indptr_validation(lib):
    st = lib.paged_attn_decode_reduce_indptr(FAKE, FAKE, FAKE, None, 2, 4, 64, 16, 7, FAKE, None)
    assert st == pa.PA_ERR_NULL_POINTER
    st = lib.paged_attn_decode_reduce_indptr(FAKE, FAKE, FAKE, FAKE, 2, 4, 80, 16, 7, FAKE, None)
    assert st == pa.PA_ERR_UNSUPPORTED
    assert lib.paged_attn_decode_reduce_indptr(FAKE, FAKE, FAKE, FAKE, 0, 4, 64, 16, 7, FAKE, None) == pa.PA_OK


@pytest.mark.parametrize("buf,nbytes,part,nwg,status", [
    (NULL, 1024, FAKE, 8, pa.PA_ERR_NULL_POINTER),
    (FAKE, 1024, NULL, 8, pa.PA_ERR_NULL_POINTER),
    (FAKE, 0, FAKE, 8, pa.PA_ERR_BAD_SHAPE),
    (FAKE, -16, FAKE, 8, pa.PA_ERR_BAD_SHAPE),
    (FAKE, 1000, FAKE, 8, pa.PA_ERR_BAD_SHAPE),    # not a multiple of 16 bytes
    (FAKE, 1024, FAKE, 0, pa.PA_ERR_BAD_SHAPE),
    (FAKE + 8, 1024, FAKE, 8, pa.PA_ERR_ALIGNMENT),
])
def test_read_probe_validation(lib, buf, nbytes, part, nwg, status):
    assert lib.paged_attn_read_probe(buf, nbytes, part, nwg, None) == status


def test_decode_workspace_needs_kv_heads():
    """The fused merge indexes its counters by (sequence, kv head): a workspace
    must know the kv head count (no default that would size them for one)."""
    with pytest.raises(TypeError):
        pa.DecodeWorkspace(4, 8, 64, 2, "cpu")
    with pytest.raises(ValueError):
        pa.DecodeWorkspace(4, 8, 64, 2, "cpu", num_kv_heads=3)
    ws = pa.DecodeWorkspace(4, 8, 64, 2, "cpu", num_kv_heads=2)
    assert ws.counters.numel() == 8 and tuple(ws.tmp_out.shape) == (4, 8, 2, 64)


def _decode_tensors(S=4, Hq=8, Hkv=2, D=64, NP=3, nb=20, mb=3):
    import torch
    return dict(q=torch.zeros((S, Hq, D), dtype=torch.bfloat16),
                k=torch.zeros((nb, Hkv, 16, D), dtype=torch.bfloat16),
                v=torch.zeros((nb, Hkv, 16, D), dtype=torch.bfloat16),
                bt=torch.zeros((S, mb), dtype=torch.int32), sl=torch.ones(S, dtype=torch.int32),
                out=torch.zeros((S, Hq, D), dtype=torch.bfloat16),
                ml=torch.zeros((S, Hq, NP), dtype=torch.float32),
                es=torch.zeros((S, Hq, NP), dtype=torch.float32),
                to=torch.zeros((S, Hq, NP, D), dtype=torch.float32),
                ctr=torch.zeros(S * Hkv, dtype=torch.int32))


@pytest.mark.parametrize("bad", ["counters", "max_logits", "exp_sums", "tmp_out", "out", "seq_lens",
                                 "block_tables"])
def test_fused_binding_checks_buffer_sizes(lib, bad):
    """Every buffer of the fused entry point is checked against the sizes the
    library will use, before the call (host tensors: nothing reaches a GPU)."""
    import torch
    t = _decode_tensors()
    S, Hq, Hkv, D, NP = 4, 8, 2, 64, 3
    if bad == "counters":
        t["ctr"] = torch.zeros(S * Hkv - 1, dtype=torch.int32)
    elif bad == "max_logits":
        t["ml"] = torch.zeros((S, Hq, NP - 1), dtype=torch.float32)
    elif bad == "exp_sums":
        t["es"] = torch.zeros((S, Hq - 1, NP), dtype=torch.float32)
    elif bad == "tmp_out":
        t["to"] = torch.zeros((S, Hq, NP, D // 2), dtype=torch.float32)
    elif bad == "out":
        t["out"] = torch.zeros((S - 1, Hq, D), dtype=torch.bfloat16)
    elif bad == "seq_lens":
        t["sl"] = torch.ones(S - 1, dtype=torch.int32)
    else:
        t["bt"] = torch.zeros((S - 1, 3), dtype=torch.int32)
    with pytest.raises(ValueError):
        pa.paged_attn_decode_fused(t["q"], t["k"], t["v"], t["bt"], t["sl"], 0.125, 16, t["out"],
                                   t["ml"], t["es"], t["to"], t["ctr"])


@pytest.mark.parametrize("bad", ["max_logits", "tmp_out", "out"])
def test_decode_binding_checks_partial_shapes(lib, bad):
    import torch
    t = _decode_tensors()
    if bad == "max_logits":
        t["ml"] = torch.zeros((4, 8, 2), dtype=torch.float32)
    elif bad == "tmp_out":
        t["to"] = torch.zeros((4, 8, 3, 32), dtype=torch.float32)
    else:
        t["out"] = torch.zeros((4, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.paged_attn_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], 0.125, 16, out=t["out"],
                             max_logits=t["ml"], exp_sums=t["es"], tmp_out=t["to"])
    with pytest.raises(ValueError):
        pa.paged_attn_decode_reduce(t["ml"], t["es"], t["to"], t["sl"], 16, t["out"])


def _noalloc_call(lib, S, Hq, Hkv, D, mbps, P, ptr=16):
    return lib.paged_attn_decode_fused_noalloc(ptr, ptr, ptr, ptr, ptr, S, Hq, Hkv, D, 16, 8, mbps,
                                               0.125, P, ptr, None)


@pytest.mark.parametrize("S,Hq,Hkv,D,mbps,P,why", [
    (32, 32, 8, 128, 3000, 16, "records of 3000 partitions x 1024 rows exceed 64 MiB"),
    (256, 64, 8, 128, 2048, 1024, "the large ragged batch at P = 1024 (272 MB of records)"),
    (32769, 2, 2, 64, 1, 16, "more (sequence, kv head) pairs than counters"),
])
def test_noalloc_rejects_problems_beyond_its_scratch(lib, S, Hq, Hkv, D, mbps, P, why):
    """Rejected on the host before anything touches a device (dummy pointers)."""
    assert _noalloc_call(lib, S, Hq, Hkv, D, mbps, P) == pa.PA_ERR_SCRATCH_LIMIT, why


@pytest.mark.parametrize("over,status", [
    (dict(P=0), pa.PA_ERR_BAD_SHAPE), (dict(P=24), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED), (dict(ptr=8), pa.PA_ERR_ALIGNMENT),
])
def test_noalloc_validation(lib, over, status):
    a = dict(S=4, Hq=8, Hkv=2, D=64, mbps=3, P=16, ptr=16)
    a.update(over)
    assert _noalloc_call(lib, **a) == status


@pytest.mark.parametrize("over,status", [
    (dict(k=None), pa.PA_ERR_NULL_POINTER), (dict(pref=None), pa.PA_ERR_NULL_POINTER),
    (dict(S=0), pa.PA_ERR_BAD_SHAPE), (dict(nwg=0), pa.PA_ERR_BAD_SHAPE), (dict(whole=3), pa.PA_ERR_BAD_SHAPE),
    (dict(whole=-1), pa.PA_ERR_BAD_SHAPE),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED), (dict(bs=32), pa.PA_ERR_UNSUPPORTED), (dict(S=1025), pa.PA_ERR_UNSUPPORTED),
    (dict(k=8), pa.PA_ERR_ALIGNMENT),
])
def test_gather_probe_validation(lib, over, status):
    a = dict(k=16, v=16, bt=16, pref=16, S=4, hkv=2, D=64, bs=16, mbps=3, whole=0, part=16, nwg=4)
    a.update(over)
    assert lib.paged_attn_gather_probe(a["k"], a["v"], a["bt"], a["pref"], a["S"], a["hkv"], a["D"], a["bs"],
                                       a["mbps"], a["whole"], a["part"], a["nwg"], None) == status
