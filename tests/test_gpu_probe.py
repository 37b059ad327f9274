"""GPU check of the HBM read-stream probe through the C ABI: the XOR of the
per-workgroup words must equal the XOR of every 32-bit word of the buffer
(integer work, compared exactly), for ragged sizes and several grids.
Needs an MI355X."""
import numpy as np
import pytest

import paged_kv_cache_34_amd as pa
from tests.gpu_util import announce, torch

pytestmark = pytest.mark.gpu


def host_xor(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.view(np.uint32)))


@pytest.mark.parametrize("n_words,nwg", [
    (4, 1),                  # one 16-byte word, one workgroup
    (4 * 1001, 3),           # fewer words than lanes in the grid
    (4 * 1_000_003, 37),     # ragged against the unrolled stride
    (4 * 1_000_003, 2048),
    (1 << 24, 8192),         # 64 MiB, the unrolled loop and no tail
])
def test_read_probe_xor(n_words, nwg):
    t = torch()
    announce(f"read probe: {n_words * 4} bytes, {nwg} workgroups")
    rng = np.random.default_rng(n_words + nwg)
    host = rng.integers(0, 2 ** 32, size=n_words, dtype=np.uint64).astype(np.uint32)
    buf = t.from_numpy(host.view(np.int32)).cuda()
    partial = t.full((nwg,), -1, dtype=t.int32, device="cuda")
    pa.paged_attn_read_probe(buf, partial)
    t.cuda.synchronize()
    got = host_xor(partial.cpu().numpy())
    assert got == host_xor(host)


def test_read_probe_status_through_binding():
    t = torch()
    buf = t.zeros(5, dtype=t.int32, device="cuda")   # 20 bytes: not a multiple of 16
    partial = t.zeros(4, dtype=t.int32, device="cuda")
    with pytest.raises(pa.PagedAttnError):
        pa.paged_attn_read_probe(buf, partial)


def used_tiles_xor(case) -> int:
    """XOR of every 32-bit word of the K and V tiles of the blocks each
    sequence uses (ceil(L / 16) logical blocks, all kv heads), on the host."""
    acc = 0
    for s, L in enumerate(case.seq_lens):
        nb = (int(L) + 15) // 16
        for blk in case.block_tables[s, :nb]:
            for pool in (case.k_cache, case.v_cache):
                acc ^= host_xor(np.ascontiguousarray(pool[int(blk)]).view(np.uint32).ravel())
    return acc


@pytest.mark.parametrize("lens,hkv,D,nwg", [
    ([1, 37, 100], 1, 64, 1),
    ([16, 17, 511, 2000], 2, 128, 3),
    ([700, 1, 4096, 33], 8, 128, 64),
    ([300, 1000], 4, 256, 512),
    ([5] * 40, 3, 64, 7),            # odd kv head count: a piece straddles K and V
])
@pytest.mark.parametrize("whole", [0, 1, 2])
def test_gather_probe_xor(lens, hkv, D, nwg, whole):
    import workloads
    t = torch()
    case = workloads.build_case("gather_probe", 900 + D + hkv, lens, hkv, hkv, D)
    announce(f"gather probe: lens={lens} H_kv={hkv} D={D} grid={nwg} whole_blocks={whole}")
    pref = np.zeros(len(lens) + 1, np.int32)
    pref[1:] = np.cumsum([(int(L) + 15) // 16 for L in case.seq_lens])
    k = t.from_numpy(case.k_cache.view(np.int16)).view(t.bfloat16).cuda()
    v = t.from_numpy(case.v_cache.view(np.int16)).view(t.bfloat16).cuda()
    partial = t.full((nwg,), -1, dtype=t.int32, device="cuda")
    pa.paged_attn_gather_probe(k, v, t.from_numpy(case.block_tables).cuda(), t.from_numpy(pref).cuda(),
                               whole, partial)
    t.cuda.synchronize()
    assert host_xor(partial.cpu().numpy()) == used_tiles_xor(case)
