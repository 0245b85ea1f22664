"""Host check of the grouped GEMM's work mapping (grouped_gemm.hip,
gemm_work): the grid's workgroups, dealt to 8 XCDs round robin, cover every
(route block, 128-row weight tile) of a layer exactly once, and the block a
workgroup derives from its expert's segment (start = segment start + i *
block_m for the expert's i-th block) is the one route preparation wrote.
The mapping is restated here in numpy, vectorised over the grid; the route
blocks come from the oracle's route preparation of each layer workload's
routing, at every block size the GEMM takes."""
import numpy as np
import pytest

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O

XCD, CHUNK = 8, 8


def _map(rp, L, N, BM):
    nb = rp["num_blocks"]
    be = rp["block_expert"][:nb].astype(np.int64)
    bs = rp["block_start"][:nb].astype(np.int64)
    off = rp["expert_offsets"].astype(np.int64)
    n_tiles = N // 128
    grid = (rp["max_blocks"] + XCD - 1) // XCD * n_tiles * XCD
    b = np.arange(grid, dtype=np.int64)
    x, slot = b % XCD, b // XCD
    lo, hi = nb * x // XCD, nb * (x + 1) // XCD
    live = slot < (hi - lo) * n_tiles
    x, slot, lo, hi = x[live], slot[live], lo[live], hi[live]
    gq = lo + slot // n_tiles
    eg = be[gq]
    off_e, end_e = off[eg], off[eg + 1]
    ig = (bs[gq] - off_e) // BM
    nbe = (end_e - off_e + BM - 1) // BM
    cq = ig // CHUNK * CHUNK
    c0 = np.maximum(gq - ig + cq, lo)
    c1 = np.minimum(gq - ig + np.minimum(cq + CHUNK, nbe), hi)
    r = slot - (c0 - lo) * n_tiles
    span = c1 - c0
    nt, blk = r // span, c0 + r % span
    start = off_e + (ig + blk - gq) * BM
    ln = np.minimum(BM, end_e - start)
    return nb, n_tiles, nt, blk, eg, start, ln, be, bs


@pytest.mark.parametrize("case", ["tiny", "decode_m16", "decode_m32", "small_m128", "small_m512", "large_m2048"])
@pytest.mark.parametrize("BM", [16, 32, 64])
def test_gemm_work_covers_each_block_tile_once(case, BM):
    c = synth.LAYER_CASES[case]
    ids = synth.routing_for(c, 0)
    ids = np.asarray(ids[0] if isinstance(ids, tuple) else ids, np.int32)
    rp = O.route_prepare(ids, 0, c.E, BM)
    for N in (2 * c.I, c.H):
        nb, n_tiles, nt, blk, eg, start, ln, be, bs = _map(rp, c.E, N, BM)
        assert ((nt >= 0) & (nt < n_tiles)).all()
        assert ((blk >= 0) & (blk < nb)).all()
        assert (be[blk] == eg).all() and (bs[blk] == start).all()
        assert ((ln >= 1) & (ln <= BM)).all()
        seen = np.zeros(nb * n_tiles, np.int64)
        np.add.at(seen, blk * n_tiles + nt, 1)
        assert (seen == 1).all(), f"{case} BM={BM} N={N}: some (block, tile) not covered exactly once"
