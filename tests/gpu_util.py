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


def routing_from_workspace(ws, M, S, G, BM=256):
    """The grouped routing's result as the grouped kernels read it from the
    workspace: (invalid count, tile table rows (group, first sorted pair,
    rows), sorted pair ids, raw table (group, first pair, end of the group's
    pairs, run)).  Offsets as the library lays the workspace out: a 64-byte
    header (tile count, invalid count), counts and cursors (int32 x G each),
    the tile table at the next 256-byte boundary (room for P/128 + G + 1
    entries of 4 int32), the sorted pair ids at the 256-byte boundary after
    it.  BM is the tile height the call routed for."""
    P = M * S
    off_tiles = (64 + 8 * G + 255) // 256 * 256
    cap = P // 128 + G + 1
    off_sorted = (off_tiles + 16 * cap + 255) // 256 * 256
    w = ws.cpu().numpy()
    hdr = w[:8].view(np.int32)
    ntiles = int(hdr[0])
    assert 0 < ntiles <= cap
    raw = w[off_tiles:off_tiles + 16 * ntiles].view(np.int32).reshape(ntiles, 4).copy()
    tiles = np.stack([raw[:, 0], raw[:, 1], np.minimum(BM, raw[:, 2] - raw[:, 1])], axis=1)
    sorted_ids = w[off_sorted:off_sorted + 4 * P].view(np.int32)
    return int(hdr[1]), tiles, sorted_ids, raw


def check_routing(idx, tiles, sorted_ids, G, BM, raw=None):
    """The routing is a counting sort of the pairs by group cut into BM-row
    tiles (every index valid): tile count, permutation, group runs, tile bounds.
    With the raw table: each entry's group end, and the walk runs (first row
    tile, height) cover each group's row tiles exactly, in order: one run for
    a group of at most 12 row tiles, runs of at most 8 rows otherwise."""
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
    if raw is None:
        return
    ntile = (counts + BM - 1) // BM
    first = np.concatenate([[0], np.cumsum(ntile)[:-1]])
    for g in range(G):
        if ntile[g] == 0:
            continue
        ent = raw[first[g]:first[g] + ntile[g]]
        assert np.all(ent[:, 2] == starts[g] + counts[g]), g
        t = first[g]
        while t < first[g] + ntile[g]:
            c0, h = int(raw[t, 3]) >> 4, (int(raw[t, 3]) & 15) + 1
            assert c0 == t and t + h <= first[g] + ntile[g], (g, t, c0, h)
            assert np.all(raw[t:t + h, 3] == raw[t, 3]), (g, t)
            assert h == ntile[g] if ntile[g] <= 12 else h <= 8, (g, h, ntile[g])
            t += h


def run_heights(raw):
    """{group: [row tiles of each walk run, in order]} from the raw tile table."""
    runs = {}
    for t, e in enumerate(raw):
        if (int(e[3]) >> 4) == t:
            runs.setdefault(int(e[0]), []).append((int(e[3]) & 15) + 1)
    return runs


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
