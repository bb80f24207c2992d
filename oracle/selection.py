"""Tile-importance selection of the oracle (ThriftAttention-style).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module. Shares no code with the GPU path.

Source: "ThriftAttention: selective mixed precision for long-context FP4
attention" (ai-feeds.com paper summary), Method step 2 and the Limitations
section: query-key tiles (e.g. 128x128) get a cheap importance score built from
norms, and only the top ~5% of tiles are computed in high precision.

Readings taken here: the score of tile (i, j) is the product of the largest
squared query-row norm in q-tile i and the largest squared key-row norm in
k-tile j, rounded to float32 (a monotone function of the product of the row
norms, so it ranks tiles identically); only tiles holding at least one
unmasked (query, key) pair are candidates; the count per (batch, query head)
is k = ceil(num * N_valid / den) (num/den = 5/100); equal scores are broken
by the lower linear tile index i * n_k + j.
"""
import numpy as np

TILE = 128


def tile_max(norm2, tile=TILE):
    """[..., L] -> [..., L/tile]: the maximum of each run of `tile` rows."""
    n = np.asarray(norm2, dtype=np.float32)
    L = n.shape[-1]
    assert L % tile == 0
    return n.reshape(n.shape[:-1] + (L // tile, tile)).max(axis=-1)


def valid_tiles(Lq, Lk, causal, tile=TILE):
    """[nq, nk] bool: tile (i, j) holds an unmasked pair. Query i sits at key position Lk-Lq+i."""
    nq, nk = Lq // tile, Lk // tile
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    off = Lk - Lq
    return tile * j <= off + tile * i + tile - 1


def select_tiles(q_norm2, k_norm2, Lq, Lk, causal, num=5, den=100, tile=TILE):
    """Bitmap [B, Hq, nq, nk] uint8 and counts [B, Hq] of the tiles computed in bf16.

    q_norm2: [B, Hq, Lq] float32 squared row norms; k_norm2: [B, Hkv, Lk].
    Query head h reads key head h // (Hq // Hkv).
    """
    qn = np.asarray(q_norm2, dtype=np.float32)
    kn = np.asarray(k_norm2, dtype=np.float32)
    B, Hq, _ = qn.shape
    Hkv = kn.shape[1]
    group = Hq // Hkv
    a = tile_max(qn, tile)                # [B, Hq, nq]
    b = tile_max(kn, tile)                # [B, Hkv, nk]
    nq, nk = a.shape[-1], b.shape[-1]
    valid = valid_tiles(Lq, Lk, causal, tile)
    n_valid = int(valid.sum())
    k = -(-num * n_valid // den)         # ceil
    bitmap = np.zeros((B, Hq, nq, nk), dtype=np.uint8)
    counts = np.zeros((B, Hq), dtype=np.int32)
    lin = (np.arange(nq)[:, None] * nk + np.arange(nk)[None, :])
    for bb in range(B):
        for h in range(Hq):
            score = (a[bb, h][:, None] * b[bb, h // group][None, :]).astype(np.float32)
            s = score[valid].astype(np.float64)
            idx = lin[valid]
            order = np.lexsort((idx, -s))   # primary: score descending; secondary: index ascending
            chosen = idx[order[:k]]
            flat = bitmap[bb, h].reshape(-1)
            flat[chosen] = 1
            counts[bb, h] = len(chosen)
    return bitmap, counts
