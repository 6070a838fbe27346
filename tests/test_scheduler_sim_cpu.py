"""A randomised CPU model of the engine's device scheduler protocol.

Every workgroup runs the stage list of a step in order. A stage that depends
on stage d waits until the arrival counters of d show every workgroup done
with d in this epoch: workgroup w increments counter stripe w % 32, so stripe
i must reach epoch * (number of workgroups in stripe i), compared modulo 2^32
as (int32)(seen - target) >= 0. A resident launch starts step e + 1 once the
counters of the last stage show step e complete. The model interleaves the
workgroups at random, starts the epoch just below 2^32 so the counters wrap,
and checks at every passed wait that
  * every workgroup really has finished the awaited stage of this epoch
    (safety: a wait never passes early, also across the wrap), and
  * no stripe of the awaited stage is ahead of this epoch's target (the
    counters cannot be pushed past a waiter's target by the next epoch),
and that the run never deadlocks. The stage dependencies are the planner's
(pdm_describe_plan) for the tiny and ragged models. Pure Python: no GPU."""
import random

import pytest

from synth import configs

STRIPES = 32
MASK = (1 << 32) - 1


def _i32(v):
    v &= MASK
    return v - (1 << 32) if v >= (1 << 31) else v


def _stripe_count(G, i):
    return (G - i + STRIPES - 1) // STRIPES


def simulate(waits, G, epochs, epoch0, seed, skip=None):
    """waits[s]: the stage stage s waits for (-1 none). Returns the number of
    passed waits; raises AssertionError on a protocol violation."""
    rnd = random.Random(seed)
    n = len(waits)
    # counters as epochs epoch0 - 1, epoch0 - 2, ... completed left them (modulo 2^32)
    counters = [[((epoch0 - 1) * _stripe_count(G, i)) & MASK for i in range(STRIPES)] for _ in range(n)]
    done = [[epoch0 - 1] * G for _ in range(n)]   # last epoch each workgroup finished stage s
    pc = [(epoch0, 0)] * G                         # (epoch, next stage) of every workgroup
    passed = 0
    end = epoch0 + epochs
    live = set(range(G))
    stalls = 0
    while live:
        w = rnd.choice(sorted(live))
        e, s = pc[w]
        # the stage this step of workgroup w must wait for
        dep, dep_epoch = waits[s], e
        if s == 0 and e != epoch0:
            dep, dep_epoch = n - 1, e - 1       # resident: step e waits for step e - 1
        ok = True
        if dep >= 0:
            for i in range(min(STRIPES, G)):
                target = (dep_epoch * _stripe_count(G, i)) & MASK
                if _i32(counters[dep][i] - target) < 0:
                    ok = False
                    break
        if not ok:
            stalls += 1
            assert stalls < 1_000_000, "deadlock"
            continue
        stalls = 0
        if dep >= 0:
            passed += 1
            assert all(done[dep][v] >= dep_epoch for v in range(G)), (dep, dep_epoch, w)
            for i in range(min(STRIPES, G)):
                target = (dep_epoch * _stripe_count(G, i)) & MASK
                assert counters[dep][i] == target, (dep, i)   # nobody is ahead of this epoch
        # run stage s of epoch e, then signal
        done[s][w] = e
        if skip != (s, w):
            counters[s][w % STRIPES] = (counters[s][w % STRIPES] + 1) & MASK
        if s + 1 < n:
            pc[w] = (e, s + 1)
        elif e + 1 < end:
            pc[w] = (e + 1, 0)
        else:
            live.discard(w)
    return passed


def _plan_waits(name):
    from persistent_decode_megakernel_amd import describe_plan, _lib as L
    import os
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    cfg = configs.get(name)
    return [s["wait"] for s in describe_plan(cfg, cfg.prompt_len + 8)]


@pytest.mark.parametrize("name,G", [("tiny", 40), ("ragged", 67), ("tiny_fp4", 256)])
def test_protocol_is_safe_under_random_interleavings(name, G):
    waits = _plan_waits(name)
    assert waits[0] == -1 and all(-1 <= d < s for s, d in enumerate(waits))
    for seed in range(3):
        # epochs wrap through 2^32 within the run
        epoch0 = (1 << 32) - 2
        assert simulate(waits, G, epochs=4, epoch0=epoch0, seed=seed) > 0


def test_model_catches_a_missing_signal():
    """A workgroup that skips one signal leaves the waiters of that stage stuck:
    the model reports a deadlock instead of letting a wait pass."""
    waits = [-1, 0, 1, 2]
    with pytest.raises(AssertionError, match="deadlock"):
        simulate(waits, 40, epochs=2, epoch0=5, seed=1, skip=(1, 7))


def test_model_catches_a_wrong_stripe_target():
    """With the target computed without the per-stripe workgroup count (one
    count for every stripe), waits pass before all workgroups are done."""
    global _stripe_count
    saved = _stripe_count
    try:
        _stripe_count = lambda G, i: 1  # noqa: E731
        with pytest.raises(AssertionError):
            simulate([-1, 0, 1], 70, epochs=2, epoch0=3, seed=2)
    finally:
        _stripe_count = saved
