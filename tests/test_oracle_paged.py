"""Paged latent caches: the oracle's page gather against the packed layout it
must reproduce (brute force over ragged lengths and page sizes), and the
generator's page placement (every reached page distinct, unreached rows
garbage)."""
import numpy as np
import pytest

from oracle import dspark as O
from synth import gen


@pytest.mark.parametrize("page_size", [32, 64, 256])
def test_gather_pages_recovers_packed(page_size):
    lens = [0, 37, 300, 64, 1]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    packed = [gen.normal((int(off[-1]), 12), 5, 40 + l) for l in range(2)]
    pc = gen.paged_layout(packed, off, page_size, seed=11)
    for l in range(2):
        got = O.gather_pages(pc.pools[l], pc.table, lens, page_size)
        assert got.shape == packed[l].shape
        assert np.array_equal(got, packed[l])


def test_paged_layout_pages_distinct_and_garbage_elsewhere():
    lens = [100, 5]
    off = np.array([0, 100, 105], np.int32)
    packed = [gen.normal((105, 8), 3, 9)]
    pc = gen.paged_layout(packed, off, 32, seed=2)
    used = [int(pc.table[0, p]) for p in range(4)] + [int(pc.table[1, 0])]
    assert len(set(used)) == len(used)
    # the tail of sequence 0's last page (rows 100..127) is not its data
    tail = pc.pools[0][pc.table[0, 3], 4:]
    assert not np.any(np.all(np.isin(tail, packed[0]), axis=1))
    # bf16 storage keeps the bits
    pb = gen.paged_layout([gen.to_bf16_bits(packed[0])], off, 64, seed=2)
    assert pb.pools[0].dtype == np.uint16
    assert np.array_equal(O.gather_pages(pb.pools[0], pb.table, lens, 64), gen.to_bf16_bits(packed[0]))
