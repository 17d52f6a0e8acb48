"""Host-side tests of the rolling latent cache (mla_ring_*) and the cache
byte counts; no GPU work.

The ring is checked against a plain simulation: a list of cached chunk ids
where sinks never leave and the oldest window chunk leaves when a new chunk
is committed to a full window, with slots handed out first-free.
"""

import itertools

import pytest

mla = pytest.importorskip("latent_kv_cache_chunk_amd.mla",
                          reason="libmla_hip.so not built (python -m latent_kv_cache_chunk_amd.build)")


class SimRing:
    def __init__(self, sink, window):
        self.sink, self.window = sink, window
        self.slots = [None] * (sink + window + 1)    # chunk id per chunk slot
        self.k = 0
        self.slots[0] = 0

    def current(self):
        return self.slots.index(self.k)

    def live(self):
        return sum(s is not None for s in self.slots)

    def commit(self):
        self.k += 1
        window = sorted(j for j in self.slots if j is not None and j >= self.sink)
        if len(window) > self.window:                # window full: the oldest window chunk leaves
            self.slots[self.slots.index(window[0])] = None
        self.slots[self.slots.index(None)] = self.k  # first free slot


@pytest.mark.parametrize("sink,window", list(itertools.product([0, 1, 2], [0, 1, 3, 6])))
def test_ring_matches_simulation(sink, window):
    C = 5
    ring = mla.Ring(C, sink, window)
    sim = SimRing(sink, window)
    assert ring.capacity == (sink + window + 1) * C
    for _ in range(3 * (sink + window + 2)):
        off, n_k = ring.current()
        assert off == sim.current() * C
        assert n_k == sim.live() * C
        # the live slots are exactly [0, n_k): contiguous, so attention needs no gather
        assert all(s is not None for s in sim.slots[: n_k // C])
        assert ring.slot_chunks() == [-1 if s is None else s for s in sim.slots]
        ring.commit()
        sim.commit()
        assert ring.committed == sim.k


def test_ring_keeps_sinks_and_recent_window():
    ring = mla.Ring(48, 1, 6)
    for _ in range(30):
        ring.commit()
    chunks = sorted(ring.slot_chunks())
    assert chunks == [0] + list(range(24, 31))      # sink 0, the six latest committed, current 30
    assert ring.current()[1] == ring.capacity


def test_ring_validation():
    with pytest.raises(ValueError):
        mla.Ring(0, 1, 1)
    with pytest.raises(ValueError):
        mla.Ring(4, -1, 1)
    with pytest.raises(ValueError):
        mla.Ring(1 << 30, 2, 2)   # capacity beyond int32


def test_cache_bytes_match_the_pages_footprint():
    # 224 latent scalars per token against 2 x 12 x 128 = 3072 for dense K and V (92.7% less)
    d = mla.Dims(batch=2)
    import torch
    lat = mla.cache_bytes(d, torch.bfloat16, 86400)
    dense = mla.dense_kv_bytes(d, torch.bfloat16, 86400)
    assert lat == 2 * 86400 * 224 * 2
    assert dense == 2 * 86400 * 3072 * 2
    assert round(1 - lat / dense, 3) == 0.927
    assert mla.cache_bytes(d, torch.float32, 10) == 2 * 10 * 224 * 4


@pytest.mark.parametrize("stop", [0, 1, 3, 9])
def test_ring_state_round_trip(stop):
    """A ring rebuilt from a saved state hands out the same slots and key
    counts as the original from that point on (checkpoint and resume)."""
    a = mla.Ring(7, 1, 3)
    for _ in range(stop):
        a.commit()
    b = mla.Ring.from_state(a.state())
    for _ in range(12):
        assert a.current() == b.current() and a.slot_chunks() == b.slot_chunks() and a.state() == b.state()
        a.commit()
        b.commit()
