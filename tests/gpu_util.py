"""Helpers for the GPU parity tests.

The tolerance check lives with the oracle (oracle/tolerance.py); host <-> device
copies live in the package (onnx_matmul_family_amd/hostdev.py).  For Gemm with
alpha != 1 or a beta*C term, a test may take t as |alpha| t + |beta C| (the same
bound applied to each term of the sum); the five workloads are checked with the
plain t.
"""
import numpy as np

from onnx_matmul_family_amd.hostdev import dev, host_f32, host_f64  # noqa: F401
from oracle.tolerance import TOL, check_close  # noqa: F401


def sample_indices(total, n, seed):
    rng = np.random.default_rng(seed)
    if total <= n:
        return np.arange(total, dtype=np.int64)
    s = rng.choice(total, size=n, replace=False).astype(np.int64)
    # always include the first and last elements (tile corners and the ragged tail)
    return np.unique(np.concatenate([s, [0, total - 1]]))


def routing_from_workspace(ws, M, S, G):
    """The grouped routing's result as the grouped kernels read it from the
    workspace: (tile table rows (group, first sorted pair, rows), sorted pair
    ids).  Offsets as the library lays the workspace out: a 64-byte header
    (tile count, invalid count), counts and cursors (int32 x G each), the tile
    table at the next 256-byte boundary (room for P/128 + G + 1 entries of 4
    int32), the sorted pair ids at the 256-byte boundary after it."""
    P = M * S
    off_tiles = (64 + 8 * G + 255) // 256 * 256
    cap = P // 128 + G + 1
    off_sorted = (off_tiles + 16 * cap + 255) // 256 * 256
    w = ws.cpu().numpy()
    hdr = w[:8].view(np.int32)
    ntiles = int(hdr[0])
    assert 0 < ntiles <= cap
    tiles = w[off_tiles:off_tiles + 16 * ntiles].view(np.int32).reshape(ntiles, 4)[:, :3]
    sorted_ids = w[off_sorted:off_sorted + 4 * P].view(np.int32)
    return int(hdr[1]), tiles, sorted_ids


def check_routing(idx, tiles, sorted_ids, G, BM):
    """The routing is a counting sort of the pairs by group cut into BM-row
    tiles (every index valid): tile count, permutation, group runs, tile bounds."""
    idx = np.asarray(idx).reshape(-1)
    counts = np.bincount(idx, minlength=G)
    assert len(tiles) == int(((counts + BM - 1) // BM).sum())
    assert np.array_equal(np.sort(sorted_ids), np.arange(idx.size))
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    for g in range(G):
        assert np.all(idx[sorted_ids[starts[g]:starts[g] + counts[g]]] == g), g
    for ti, (g, start, rows) in enumerate(tiles):
        assert 1 <= rows <= BM and starts[g] <= start and start + rows <= starts[g] + counts[g], (ti, g, start, rows)
    assert int(tiles[:, 2].sum()) == idx.size


def tile_row_pairs(tiles, sorted_ids, per_tile, BM):
    """Pairs whose whole output rows a test compares: per_tile rows of every
    routed tile, at slots (j * BM / per_tile + 11 * tile) % BM, which walk every
    row slot of a tile over a launch of enough tiles."""
    pairs = set()
    for ti, (g, start, rows) in enumerate(tiles):
        for j in range(per_tile):
            slot = (j * (BM // per_tile) + 11 * ti) % BM
            if slot < rows:
                pairs.add(int(sorted_ids[start + slot]))
    return np.array(sorted(pairs), dtype=np.int64)
