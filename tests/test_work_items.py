"""Host replay of every launcher's work-item decode (CPU only): for the five
workload shapes, the extra workloads and every GPU test shape, each decoded
(batch, head, query tile, segment), key range and partial-state row stays
inside the tensors and the workspace, the block -> item map is a bijection,
and the segments of each query tile cover its keys exactly as the merge
reads them."""
import pytest

import work_items

DENSE = [(1, 8, 36864, 36864, 128), (1, 56, 15360, 29678, 128), (1, 2, 256, 256, 128), (2, 3, 300, 1000, 128),
         (1, 2, 129, 65, 256), (1, 2, 200, 100, 128), (1, 1, 130, 321, 128), (1, 2, 600, 4100, 128),
         (1, 1, 1, 1, 128), (1, 4, 200, 200, 128)]
CAUSAL = [(1, 6, 1, 256, 8000, 8000, 128000), (1, 6, 1, 256, 8000, 8000, 256000),
          (1, 6, 1, 256, 256, 200, 4096), (1, 6, 1, 256, 128, 128, 160), (1, 4, 2, 128, 192, 150, 2400),
          (1, 2, 1, 256, 64, 64, 16480), (1, 3, 1, 128, 64, 40, 9024), (2, 4, 2, 256, 128, 90, 3072),
          (1, 6, 1, 256, 128, 100, 2048), (1, 4, 2, 128, 192, 150, 1056), (1, 6, 1, 256, 128, 70, 2048),
          (2, 4, 2, 128, 128, 100, 640), (1, 6, 1, 256, 8192, 8192, 262144), (1, 6, 1, 256, 64, 1, 32)]
DECODE = [(1, 6, 1, 256, 16, 16, 256000), (1, 6, 1, 256, 16, 16, 4096), (1, 6, 1, 256, 5, 3, 2080),
          (1, 4, 2, 128, 1, 1, 1024), (1, 8, 1, 128, 16, 16, 8192), (1, 4, 2, 128, 2, 2, 16416),
          (2, 6, 1, 256, 16, 16, 1056), (1, 6, 1, 256, 1, 1, 262144), (1, 1, 1, 128, 1, 1, 32),
          # one-wave workgroups (at most 32 packed rows), up to 1024 segments
          (1, 6, 1, 256, 1, 1, 256000), (1, 6, 1, 256, 5, 5, 256000), (1, 8, 1, 128, 4, 4, 262144),
          (2, 4, 2, 256, 3, 2, 40000), (1, 6, 1, 256, 1, 1, 65536), (1, 6, 1, 256, 6, 6, 100000),
          (1, 6, 1, 256, 1, 1, 131072), (1, 6, 1, 256, 5, 4, 32768), (1, 6, 1, 256, 4, 4, 8192),
          (1, 2, 1, 128, 16, 16, 65536), (1, 8, 2, 128, 4, 3, 32800),
          (1, 6, 1, 256, 8, 8, 8192), (1, 4, 1, 256, 16, 11, 32992), (1, 6, 1, 256, 11, 9, 20000),
          (1, 6, 1, 256, 16, 16, 1056), (2, 8, 2, 256, 12, 10, 4128), (2, 4, 2, 256, 3, 3, 2080)]
BLOCKS = [(1, 8, 36864, 128, 64, 64, 2), (1, 2, 2048, 128, 64, 8, 2), (1, 2, 1280, 128, 64, 20, 0),
          (1, 2, 1024, 128, 64, 3, 16), (1, 2, 64 * 30 + 37, 128, 64, 7, 2), (1, 2, 64 * 6 + 1, 128, 64, 7, 7),
          (2, 3, 64 * 12 + 5, 128, 64, 5, 1), (1, 1, 50, 128, 64, 1, 1), (1, 8, 36864, 128, 64, 116, 2)]


@pytest.mark.parametrize("shape", DENSE)
def test_dense_items(shape):
    assert work_items.check("dense", *shape).startswith("OK")


# dense shapes whose items leave a partial last round of at most half the
# slots: the whole rounds, then the rest with each item's keys split in halves
DENSE_TAIL = [(1, 8, 36864, 36864, 128), (1, 56, 15360, 29678, 128), (1, 4, 16640, 200, 128),
              (1, 4, 16640, 130, 128), (1, 4, 16640, 65, 128), (1, 4, 16640, 4100, 128)]


@pytest.mark.parametrize("shape", DENSE_TAIL)
def test_dense_tail_items(shape):
    assert work_items.check("dense_tail", *shape).startswith("OK")


def test_dense_tail_split_applies_only_after_whole_rounds():
    # fewer items than one round, a full last round, and a rest past half a
    # round all keep the single launch
    for shape in [(1, 2, 600, 4100, 128), (1, 8, 32768, 32768, 128), (1, 6, 16640, 4100, 128),
                  (1, 4, 16640, 64, 128)]:
        rc, out = work_items.run("dense_tail", *shape)
        assert rc == 1 and "no split" in out, (shape, out)


@pytest.mark.parametrize("shape", CAUSAL)
def test_causal_items(shape):
    assert work_items.check("causal", *shape).startswith("OK")


@pytest.mark.parametrize("shape", DECODE)
def test_decode_items(shape):
    assert work_items.check("decode", *shape).startswith("OK")


@pytest.mark.parametrize("shape", BLOCKS)
def test_block_list_items(shape):
    assert work_items.check("blocks", *shape).startswith("OK")


def test_replay_catches_a_decode_that_runs_past_the_tensors():
    """The checks fire on the class of launcher/kernel mismatch that once
    faulted the GPU: causal work items decoded with the dense decode give
    batch indices past the tensors' ends."""
    rc, out = work_items.run("causal", 1, 6, 1, 256, 8000, 8000, 128000, decode_as="dense")
    assert rc == 1 and "batch out of range" in out, out
    rc, out = work_items.run("decode", 1, 6, 1, 256, 16, 16, 256000, decode_as="causal")
    assert rc == 1, out
    its = work_items.items("causal", 1, 6, 1, 256, 8000, 8000, 128000)
    assert len(its) == 756 and max(i["b"] for i in its) == 0
    assert sorted({i["seg"] for i in its}) == [0, 1]
