"""GPU tile selector vs the oracle: bitmaps and counts bit for bit.

The cases cover the selector's own paths and degenerate inputs: equal scores everywhere (the order is
then the tile index alone, and the boundary bucket is too large for the in-LDS candidate list, so
the radix passes rescan all tiles), a handful of distinct norm values (ties across the boundary), all
scores zero, every tile and no tile chosen, exactly one tile, the chunk offset, and the largest tile
grid the entry point accepts (1024 x 4096).
"""
import numpy as np
import pytest
import torch

from oracle import selection as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _norms(kind, shape, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "const":
        return torch.full(shape, 1.0)
    if kind == "zero":
        return torch.zeros(shape)
    if kind == "levels":
        return torch.randint(0, 4, shape, generator=g).float()
    return torch.rand(shape, generator=g) * 200.0


CASES = {
    #              B  Hq Hkv  Lq      Lk      causal num  den   norms
    "ties_rescan": (1, 2, 1, 32768, 32768, False, 5, 100, "const"),
    "ties_chunk_offset": (1, 4, 1, 2048, 131072, True, 5, 100, "const"),
    "few_values_gqa": (2, 4, 2, 4096, 4096, True, 17, 100, "levels"),
    "all_zero_scores": (1, 2, 2, 1024, 1024, True, 5, 100, "zero"),
    "every_tile": (1, 2, 1, 2048, 4096, True, 100, 100, "rand"),
    "no_tile": (1, 2, 1, 2048, 4096, True, 0, 100, "rand"),
    "one_tile": (1, 2, 1, 1024, 1024, False, 1, 1000, "rand"),
    "largest_grid": (1, 1, 1, 131072, 524288, True, 5, 100, "rand"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_select_bit_exact(fa4, name):
    B, Hq, Hkv, Lq, Lk, causal, num, den, kind = CASES[name]
    qn = _norms(kind, (B, Hq, Lq), 11)
    kn = _norms(kind, (B, Hkv, Lk), 12)
    bm, cnt = fa4.select_tiles(qn.cuda(), kn.cuda(), causal, num, den)
    torch.cuda.synchronize()
    ref_bm, ref_cnt = S.select_tiles(qn.numpy(), kn.numpy(), Lq, Lk, causal, num, den)
    got = bm.cpu().numpy()
    assert np.array_equal(cnt.cpu().numpy(), ref_cnt), name
    assert np.array_equal(got.sum(axis=(2, 3)), ref_cnt), name
    mism = int((got != ref_bm).sum())
    assert mism == 0, f"{name}: {mism} tiles differ"
