"""The grid barrier's protocol (fused compress and decompress-sum-compress),
modelled step by step on the CPU with random interleavings of the workgroups'
atomic steps across many calls of varying grid size.

The model follows the protocol described in the kernel source (leaf lines of
16 workgroups with running counts that advance by exactly 16 per call, a root
count that advances by 64, padding for partial and unused leaves, leaf maxima
taken by atomic exchange, release words (call + 1, max)); it checks that every
workgroup leaves the barrier with the true maximum and that no wait is
endless.  Host logic only: it does not run the kernel.
"""
import random

LEAF, LEAVES = 16, 64


def run_calls(seed, calls, spin_limits=(None,)):
    """spin_limits: per call, a bound on the polls is drawn from this list
    (None: unbounded).  A workgroup that reaches the bound gives up (NaN, here
    None) and sets timed_out; it has arrived, so the others still complete."""
    rnd = random.Random(seed)
    timed_out = False
    leaf = [{"count": 0, "max": 0, "rel": 0} for _ in range(LEAVES)]
    root = {"count": 0}
    for _ in range(calls):
        G = rnd.choice([1, 2, 15, 16, 17, 100, 255, 256, 512, 1000, 1024])
        nleaves = (G + LEAF - 1) // LEAF
        vals = [rnd.randint(0, 10 ** 6) for _ in range(G)]
        limit = rnd.choice(spin_limits)

        def workgroup(b):
            l = b // LEAF
            in_leaf = min(LEAF, G - l * LEAF)
            lf = leaf[l]
            lf["max"] = max(lf["max"], vals[b])                      # atomic max, waited for
            yield
            inc = 1 + ((LEAF - in_leaf) if b % LEAF == 0 else 0)
            lf["count"] += inc                                       # atomic add
            a = lf["count"]
            yield
            call = (a - 1) // LEAF
            last = False
            if a % LEAF == 0:
                rinc = 1 + ((LEAVES - nleaves) if l == 0 else 0)
                root["count"] += rinc
                last = root["count"] % LEAVES == 0
                yield
            want = (call + 1) & 0xFFFFFFFF
            if last:
                mx = 0
                for k in range(LEAVES):
                    if k < nleaves:
                        mx = max(mx, leaf[k]["max"])                 # atomic exchange with 0
                        leaf[k]["max"] = 0
                    else:
                        leaf[k]["count"] = (call + 1) * LEAF
                    yield
                for k in range(LEAVES):
                    leaf[k]["rel"] = (want << 32) | mx
                    yield
                return mx
            spins = 0
            while (leaf[l]["rel"] >> 32) != want:
                spins += 1
                assert spins < 10 ** 6, "endless wait"
                if limit is not None and spins >= limit:
                    nonlocal timed_out
                    timed_out = True
                    return None
                yield
            return leaf[l]["rel"] & 0xFFFFFFFF

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
        assert sum(v is not None for v in got.values()) >= 1      # the completing workgroup
        if limit is None:
            assert all(v is not None for v in got.values())
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
