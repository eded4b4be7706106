"""Host logic of the static mode schedule (no GPU): validation and the
owner/consumer graph it derives."""
import pytest

from fp4_compressed_sparse_csa2_amd.schedule import FULL, REINDEX, REUSE, Layer, Schedule


def test_pattern_and_owners():
    s = Schedule.pattern(9, 8192, 2048, period=4)
    assert [l.mode for l in s.layers] == [FULL, REINDEX, REUSE, REUSE, REUSE,
                                          REINDEX, REUSE, REUSE, REUSE]
    assert s.index_owner == [0, 1, 1, 1, 1, 5, 5, 5, 5]
    assert s.pool_owner == [None, 0, None, None, None, 0, None, None, None]
    assert s.selecting_layers() == [0, 1, 5]


def test_explicit_sources():
    s = Schedule([Layer(FULL, 4096), Layer(REUSE), Layer(REINDEX, 1024), Layer(REUSE, source=0),
                  Layer(FULL, 2048), Layer(REINDEX, 512, source=0), Layer(REUSE, source=2)])
    assert s.index_owner == [0, 0, 2, 0, 4, 5, 2]
    assert s.pool_owner == [None, None, 0, None, None, 0, None]


@pytest.mark.parametrize("layers", [
    [],
    [Layer(REUSE)],                                     # no owner yet
    [Layer(REINDEX, 16)],
    [Layer(FULL, 0)],                                   # empty pool
    [Layer(FULL, 64), Layer(REINDEX, 128)],             # Top-K' beyond the pool
    [Layer(FULL, 64), Layer(REUSE), Layer(REUSE, source=1)],   # reuse of a Reuse layer
    [Layer(FULL, 64), Layer(REINDEX, 8, source=1)],     # source after / not Full
    [Layer(FULL, 64), Layer("sliding", 8)],
])
def test_invalid_schedules(layers):
    with pytest.raises(ValueError):
        Schedule(layers)
