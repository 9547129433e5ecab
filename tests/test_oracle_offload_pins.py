"""Pins of the oracle's host-offload pool ([MemDecay] §III-E tiered
extension: offload before dropping, recover when relevant again; [LRFU-fig]:
a block's state survives its eviction).  The slot arithmetic is fixed by
hand on small traces."""
import pytest

import oracle as orc


def test_ring_order_reuse_and_release_by_hand():
    p = orc.HostOffloadPool(3)
    # one selection evicts blocks 5 and 2 of sequence 0 and block 7 of sequence 1:
    # ranked (0, 2), (0, 5), (1, 7) into slots 0, 1, 2
    p.offload([(0, 5), (1, 7), (0, 2)])
    assert [p.slot(k) for k in [(0, 2), (0, 5), (1, 7)]] == [0, 1, 2]
    assert p.ring == 0
    # the next eviction reuses slot 0: block (0, 2) loses its copy
    p.offload([(0, 9)])
    assert p.slot((0, 9)) == 0 and p.slot((0, 2)) == -1 and p.ring == 1
    # re-admission releases the slot
    p.readmit((0, 5))
    assert p.slot((0, 5)) == -1 and p.slots[1] is None
    # (0, 3) and (1, 1) take slots 1 and 2; (1, 7) loses slot 2
    p.offload([(1, 1), (0, 3)])
    assert p.slot((0, 3)) == 1 and p.slot((1, 1)) == 2 and p.slot((1, 7)) == -1
    assert p.where == {(0, 9): 0, (0, 3): 1, (1, 1): 2}
    with pytest.raises(KeyError):
        p.readmit((1, 7))


def test_overflow_within_one_selection_keeps_the_last():
    p = orc.HostOffloadPool(2)
    p.offload([(1, 0)])  # ring at 1
    p.offload([(0, 4), (0, 1), (1, 3), (0, 8), (1, 2)])
    # ranked (0,1) (0,4) (0,8) (1,2) (1,3): the last two take slots 1 and 0
    assert p.where == {(1, 2): 1, (1, 3): 0}
    assert p.ring == 1


def test_pool_holds_the_latest_evictions_not_readmitted():
    """Against a plain model: the last `capacity` offloaded keys in order,
    minus those re-admitted after their last offload."""
    import random
    rnd = random.Random(3)
    C = 5
    p = orc.HostOffloadPool(C)
    log = []            # offloaded keys in pool order
    resident = set()    # keys currently re-admitted (not in the pool)
    for step in range(200):
        ev = rnd.sample([(s, j) for s in range(3) for j in range(12)], rnd.randint(0, 7))
        ev = [k for k in ev if k not in p.where]  # a block in the pool is not resident: not evictable
        order = sorted(ev)
        p.offload(ev)
        log.extend(order)
        for k in order:
            resident.discard(k)
        if p.where and rnd.random() < 0.3:
            k = rnd.choice(sorted(p.where))
            p.readmit(k)
            resident.add(k)
        latest = log[-C:]
        want = {k for i, k in enumerate(latest) if k not in resident and k not in latest[i + 1:]}
        assert set(p.where) == want, step


def test_dropped_evictions_do_not_advance_the_ring():
    """Evictions below the score threshold are dropped before the pool sees
    them: the ring advances only by the offloaded ones."""
    p = orc.HostOffloadPool(4)
    scores = {(0, 1): 0.5, (0, 2): 0.01, (1, 5): 0.3, (1, 6): 0.002}
    keep = [k for k, v in scores.items() if v >= 0.1]
    p.offload(keep)
    assert p.where == {(0, 1): 0, (1, 5): 1} and p.ring == 2
