"""The grid barrier's protocol (fused compress and decompress-sum-compress),
modelled step by step on the CPU with random interleavings of the workgroups'
atomic steps across many calls of varying grid size.

The model follows the protocol described in the kernel source: leaf lines of
16 workgroups with running counts that advance by exactly 16 per call (each
workgroup adds 1 to its leaf at its start, the first of a partial leaf also
the missing arrivals, workgroup 0 advances every leaf the grid does not use),
so each workgroup's own add yields the call number c; then each workgroup
stores (c + 1, its max) into its own slot and polls the slots of the grid
until all carry epoch c + 1.  Epochs are the low bits of c + 1 (32 in the
kernel), and workgroup 0 writes the call's epoch into every slot beyond the
grid, so no slot can hold a stale value equal to the current epoch however
the grid sizes vary; the model checks this with 2-bit epochs, and that
without the refresh the same model catches the stale slot.  It checks that
every workgroup leaves with the true maximum, that no wait is endless, and
that calls in which some workgroups gave up (bounded waits) leave the state
right for the next call.  Host logic only: it does not run the kernel.
"""
import random

import pytest

LEAF, LEAVES = 16, 64
SLOTS = LEAF * LEAVES


def run_calls(seed, calls, spin_limits=(None,), epoch_bits=32, refresh=True, grids=None):
    """spin_limits: per call, a bound on the poll rounds drawn from this list
    (None: unbounded).  A workgroup that reaches it gives up (NaN, here None)
    and sets timed_out; it has counted itself and stored its slot.  grids:
    the grid size of each call (default: drawn at random)."""
    rnd = random.Random(seed)
    count = [0] * LEAVES
    slots = {}                                   # workgroup -> (epoch, max)
    timed_out = False
    mask = (1 << epoch_bits) - 1
    for i in range(calls):
        G = grids[i] if grids else rnd.choice([1, 2, 15, 16, 17, 100, 255, 256, 512, 1000, 1024])
        nleaves = (G + LEAF - 1) // LEAF
        vals = [rnd.randint(0, 10 ** 6) for _ in range(G)]
        limit = rnd.choice(spin_limits)

        def workgroup(b):
            nonlocal timed_out
            l = b // LEAF
            in_leaf = min(LEAF, G - l * LEAF)
            inc = 1 + ((LEAF - in_leaf) if b % LEAF == 0 else 0)
            count[l] += inc                                          # atomic add
            call = (count[l] - 1) // LEAF
            yield
            if b == 0:
                for j in range(nleaves, LEAVES):                     # unused leaves
                    count[j] += LEAF
                    yield
            yield                                                    # loads, rotation
            epoch = (call + 1) & mask
            slots[b] = (epoch, vals[b])                              # 64-bit store
            yield
            if b == 0 and refresh:
                for j in range(G, SLOTS):                            # slots beyond the grid
                    slots[j] = (epoch, 0)
                    if j % 64 == 63:
                        yield
            rounds = 0
            while True:
                seen = []
                for j in range(G):                                   # one load per slot
                    seen.append(slots.get(j, (0, 0)))
                    if j % 64 == 63:
                        yield
                if all(e == epoch for e, _ in seen):
                    return max(v for _, v in seen)
                rounds += 1
                assert rounds < 10 ** 5, "endless wait"
                if limit is not None and rounds >= limit:
                    timed_out = True
                    return None
                yield

        live = {b: workgroup(b) for b in range(G)}
        got = {}
        while live:
            b = rnd.choice(list(live))
            try:
                next(live[b])
            except StopIteration as e:
                got[b] = e.value
                del live[b]
        assert all(v is None or v == max(vals) for v in got.values())
        if limit is None:
            assert all(v is not None for v in got.values())
        assert all(c % LEAF == 0 for c in count)                    # every leaf in step
        assert len(set(count)) == 1
    return timed_out


def test_barrier_protocol_random_interleavings():
    for seed in range(3):
        assert not run_calls(seed, 30)


def test_barrier_survives_workgroups_that_give_up():
    """Calls whose waits are bounded (some workgroups give up) interleaved with
    unbounded ones: the unbounded calls still all get the true maximum, so a
    timeout leaves the barrier state consistent for the next call."""
    gave_up = False
    for seed in range(3, 6):
        gave_up |= run_calls(seed, 30, spin_limits=(None, 1, 2, 8))
    assert gave_up


def test_narrow_epochs_with_refreshed_slots():
    """2-bit epochs (the kernel's are 32-bit): the refresh of the slots beyond
    the grid keeps every slot at the last call's epoch, so random grid sizes,
    and a large grid after several small ones, never meet a stale slot."""
    for seed in range(6, 8):
        assert not run_calls(seed, 20, epoch_bits=2)
    for seed in range(9, 12):
        assert not run_calls(seed, 5, epoch_bits=2, grids=[1024, 1, 2, 1, 1024])


def test_stale_slot_is_caught_without_the_refresh():
    """The model detects the failure the refresh prevents: with 2-bit epochs, a
    large grid 4 calls after another large grid (the same epoch) finds its
    slots at the current epoch before their owners write them, and some
    workgroup leaves with a stale maximum."""
    with pytest.raises(AssertionError):
        for seed in range(9, 12):
            run_calls(seed, 5, epoch_bits=2, refresh=False, grids=[1024, 1, 2, 1, 1024])
