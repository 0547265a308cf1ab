"""The memory-ceiling probes against plain torch results: the mix probe's
output is exact (XOR of its source planes), and the read and gather probes
leave their sink untouched for a key their data does not produce."""
import pytest
import torch

import paged_kv_cache_270_amd as pkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 32 * 1024 + 48, (3 << 20) + 16 * 7, 64 << 20])
@pytest.mark.parametrize("rpw", [1, 2])
@pytest.mark.parametrize("wg", [0, 1, 7])
def test_mix_probe_writes_the_xor_of_its_planes(nbytes, rpw, wg):
    g = torch.Generator(device="cuda").manual_seed(nbytes + rpw)
    src = torch.randint(-2**31, 2**31 - 1, (rpw * nbytes // 4,), dtype=torch.int32,
                        device="cuda", generator=g)
    dst = torch.full((nbytes // 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    guard = torch.zeros(1024, dtype=torch.int32, device="cuda")   # allocated after dst
    pkv.pkv_hbm_mix_probe(src, dst, rpw, workgroups=wg)
    torch.cuda.synchronize()
    want = src[: nbytes // 4].clone()
    if rpw == 2:
        want ^= src[nbytes // 4:]
    assert torch.equal(dst, want)
    assert not guard.any()


def test_read_probe_reads_without_writing():
    buf = torch.randint(0, 255, ((8 << 20) + 16 * 5,), dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    for wg in (0, 1, 5, 4096):
        pkv.pkv_hbm_read_probe(buf, sink, workgroups=wg)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]


def test_gather_probe_reads_without_writing():
    lay = pkv.CacheLayout(64, 2, pkv.PKV_FP8_E4M3FN)
    tb = pkv.pkv_pool_bytes(lay)
    k = torch.randint(0, 255, (tb,), dtype=torch.uint8, device="cuda")
    v = torch.randint(0, 255, (tb,), dtype=torch.uint8, device="cuda")
    tables = torch.randint(0, 64, (3, 20), dtype=torch.int32, device="cuda")
    lens = torch.tensor([0, 17, 320], dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    pkv.pkv_tile_gather_probe(k, v, tables, lens, 320, lay, sink)
    torch.cuda.synchronize()
    assert sink.item() == 9
