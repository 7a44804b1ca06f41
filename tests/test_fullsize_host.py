"""Host checks of the every-element full-size comparison's chunking (no GPU):
the chunks tile [0, d) exactly, no chunk exceeds its target, and every cut
lies on a block boundary of the tensor it falls in (so the oracle's block
partials of a tensor, computed chunk by chunk, are those of the whole
tensor)."""
import pytest

from synth import workloads as wls
from tests.fullsize_check import BLOCK, column_chunks


@pytest.mark.parametrize("wl", wls.ALL, ids=lambda w: w.name)
@pytest.mark.parametrize("target", [1 << 16, 1 << 22])
def test_column_chunks_tile_on_block_boundaries(wl, target):
    off = wl.offsets
    chunks = column_chunks(wl, target)
    assert chunks[0][0] == 0 and chunks[-1][1] == wl.d
    seen = {}
    for k, (j0, j1, pieces) in enumerate(chunks):
        if k:
            assert j0 == chunks[k - 1][1]
        assert 0 < j1 - j0 <= target
        assert pieces[0][1] == j0 and pieces[-1][2] == j1
        for p, (T, a, b) in enumerate(pieces):
            if p:
                assert a == pieces[p - 1][2]
            assert off[T] <= a < b <= off[T + 1]
            assert (a - off[T]) % BLOCK == 0
            assert T not in seen or seen[T] == a
            seen[T] = b
    assert all(seen[T] == off[T + 1] for T in range(wl.n_tensors))
