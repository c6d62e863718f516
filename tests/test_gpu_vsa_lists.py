"""GPU parity of the VSA 128-token block lists and the pooled tile means
("[perf] FastH3 two-Spark: gather packed FP4 inputs before head projections",
block_lists.py and kv_pool.py) against the oracle: bit-exact (marked gpu)."""
import numpy as np
import pytest

import oracle
import synth
import synth.workloads as wl
from parity_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check_lists(lib, mask, valid, tile):
    idx, counts, kv, quad = lib.vsa_tile_mask_to_block_lists(dev(mask.astype(np.uint8)), dev(valid), tile)
    torch.cuda.synchronize()
    r_idx, r_counts, r_kv, r_quad = oracle.block_lists(mask, valid, tile, quadrants=tile == 64)
    assert np.array_equal(counts.cpu().numpy(), r_counts)
    assert np.array_equal(kv.cpu().numpy(), r_kv)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    if tile == 64:
        assert np.array_equal(quad.cpu().numpy(), r_quad)
    return r_counts


@pytest.mark.parametrize("B,H,T,tile,density", [(1, 2, 10, 64, 0.3), (2, 3, 9, 64, 0.5),   # odd half count
                                                (1, 2, 7, 128, 0.4), (1, 1, 130, 64, 0.1),  # more than 64 blocks
                                                (1, 1, 1024, 64, 0.02), (1, 2, 512, 128, 0.05),  # the largest
                                                (1, 1, 3, 64, 0.0)])                            # empty mask
def test_block_lists_bit_exact(lib, B, H, T, tile, density):
    say(f"block lists B{B} H{H} T{T} tile{tile} density {density}")
    rng = np.random.default_rng(T + tile)
    mask = rng.random((B, H, T, T)) < density
    valid = np.full(T, tile, np.int32)
    valid[-1] = tile // 2 + 3            # a partial last tile
    if T > 3:
        valid[1] = 0                     # an empty tile
    _check_lists(lib, mask, valid, tile)


def test_block_lists_of_the_vsa_selection(lib):
    """The lists of the video workload's own top-64 selection (576 tiles of 64
    tokens, dense prefix query tiles 0-1 attending everywhere)."""
    w = wl.VSA
    q, k, _ = wl.vsa_inputs(w)
    sel = lib.vsa_block_select(dev(q), dev(k), w["topk"], block=w["block"]).cpu().numpy()
    nb = sel.shape[2]
    mask = np.zeros((w["B"], w["H"], nb, nb), bool)
    b, h, i = np.meshgrid(np.arange(w["B"]), np.arange(w["H"]), np.arange(nb), indexing="ij")
    mask[b[..., None], h[..., None], i[..., None], sel] = True
    mask[:, :, : w["dense_prefix"]] = True
    say(f"block lists of the VSA selection: {nb} tiles, {int(mask.sum())} selected pairs")
    counts = _check_lists(lib, mask, np.full(nb, 64, np.int32), 64)
    assert counts.max() <= 288 and counts[:, :, 0].min() == 288   # the dense first query block lists all


@pytest.mark.parametrize("B,H,L", [(1, 2, 64 * 20 + 37), (2, 3, 64), (1, 1, 5), (1, 8, 36864)])
def test_tile_means_bit_exact(lib, B, H, L):
    say(f"tile means B{B} H{H} L{L}")
    v = synth.normal_f16(14, synth.TID_V, (B, H, L, 128))
    got = lib.vsa_tile_means(dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.tile_means(v, 64))
