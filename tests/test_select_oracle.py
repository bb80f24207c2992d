"""Pins of the oracle's tile selection: brute-force sort, order properties, the tile counts of the workloads."""
import os

import numpy as np

import bruteforce as bf
from oracle import selection as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_valid_tile_counts_and_k_match_fixture():
    for line in open(os.path.join(GOLDEN, "selection_counts.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        Lq, Lk, nvalid, ksel = (int(v) for v in line.split())
        valid = S.valid_tiles(Lq, Lk, True)
        assert int(valid.sum()) == nvalid
        qn = np.ones((1, 1, Lq), np.float32)
        kn = np.ones((1, 1, Lk), np.float32)
        if Lq * Lk <= 4096 * 4096:
            bm, cnt = S.select_tiles(qn, kn, Lq, Lk, True)
            assert int(cnt[0, 0]) == ksel and int(bm.sum()) == ksel


def test_selection_vs_python_sort():
    rng = np.random.default_rng(0)
    for causal, Lq, Lk in [(True, 1024, 1024), (False, 512, 768), (True, 512, 1536)]:
        B, Hq, Hkv = 1, 4, 2
        qn = rng.exponential(100, (B, Hq, Lq)).astype(np.float32)
        kn = rng.exponential(100, (B, Hkv, Lk)).astype(np.float32)
        # force exact ties in scores
        qn[0, 1, :] = 5.0
        kn[0, 0, :] = 7.0
        bm, cnt = S.select_tiles(qn, kn, Lq, Lk, causal, num=5, den=100)
        valid = S.valid_tiles(Lq, Lk, causal)
        nvalid = int(valid.sum())
        k = -(-5 * nvalid // 100)
        for h in range(Hq):
            a = S.tile_max(qn[0, h])
            b = S.tile_max(kn[0, h // 2])
            ref = bf.select_by_sort([float(v) for v in a], [float(v) for v in b],
                                    lambda i, j: bool(valid[i, j]), k)
            got = np.nonzero(bm[0, h].reshape(-1))[0].tolist()
            assert got == ref
            assert cnt[0, h] == k


def test_selected_scores_dominate_and_ties_break_low():
    rng = np.random.default_rng(1)
    Lq = Lk = 2048
    qn = rng.integers(1, 4, (1, 1, Lq)).astype(np.float32)
    kn = rng.integers(1, 4, (1, 1, Lk)).astype(np.float32)
    bm, cnt = S.select_tiles(qn, kn, Lq, Lk, True, num=5, den=100)
    a = S.tile_max(qn[0, 0])
    b = S.tile_max(kn[0, 0])
    score = (a[:, None] * b[None, :]).astype(np.float32)
    valid = S.valid_tiles(Lq, Lk, True)
    sel = bm[0, 0].astype(bool)
    assert not np.any(sel & ~valid)
    lo = score[sel].min()
    assert np.all(score[valid & ~sel] <= lo)
    # among tiles tied at the boundary score, the selected ones have the lowest linear indices
    lin = np.arange(score.size).reshape(score.shape)
    tied = valid & (score == lo)
    assert lin[tied & sel].max() < lin[tied & ~sel].min() if np.any(tied & ~sel) else True


def test_zero_fraction_and_all():
    qn = np.ones((1, 2, 512), np.float32)
    kn = np.ones((1, 1, 512), np.float32)
    bm, cnt = S.select_tiles(qn, kn, 512, 512, True, num=0, den=100)
    assert bm.sum() == 0
    bm, cnt = S.select_tiles(qn, kn, 512, 512, True, num=100, den=100)
    assert np.array_equal(bm[0, 0].astype(bool), S.valid_tiles(512, 512, True))
