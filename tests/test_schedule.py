"""The streamed step's schedule as data (mt_schedule), proven race-free on
the CPU for every schedule and flag that changes it, with planted mistakes
to show the proof catches each kind of missing wait.  The plan comes from
the same code that issues the step: a dry run records what it would enqueue
and the waits it would place, and issues nothing."""
import copy
import ctypes
import itertools

import pytest

import datagen
import host_memory_layer_amd as mt
from tests.hazards import ADAM, COMPUTE, FETCH, OFFLOAD, POISON, check_hazards, use_order

TINY = datagen.PRESETS["tiny"]
SMALL = datagen.ModelShape("small-bf16", 4, 256, 2, 128, 512, 1000, 2, 128)
# compute-bound against the host link: offloads are held behind the next prefetch
LONG = datagen.ModelShape("long-ctx", 3, 256, 2, 128, 512, 1000, 1, 65536)

MODES = ("streamed", "serialized", "single_slot")
FLAG_SETS = (0, mt.MT_FLAG_POISON, mt.MT_FLAG_SDMA_QUEUES, mt.MT_FLAG_DUPLEX_LINK,
             mt.MT_FLAG_POISON | mt.MT_FLAG_SDMA_QUEUES)


def plan(shape, mode="streamed", flags=0, **kw):
    return mt.schedule(mt.make_config(shape, mode, flags=flags, **kw))


def expected_uses(L):
    """The pages' sweep: forward over the embedding, every layer and the head
    (which runs its backward on the same pass), then the layers backward and
    the embedding last."""
    fwd = [(u, u) for u in range(L + 2)]
    bwd = [(L + 2 + i, L - i) for i in range(L)] + [(2 * L + 2, 0)]
    return fwd + bwd


@pytest.mark.parametrize("shape", [TINY, SMALL, LONG], ids=lambda s: s.name)
@pytest.mark.parametrize("mode,flags", list(itertools.product(MODES, FLAG_SETS)))
def test_every_schedule_is_race_free(shape, mode, flags):
    ops = plan(shape, mode, flags)
    L = shape.n_layers
    assert check_hazards(ops, L + 2) == []
    assert use_order(ops) == expected_uses(L)
    n_fetch = sum(o["kind"] == FETCH for o in ops)
    # every block once for the forward, every layer again for its backward
    # but the top one, which stays in its slot from the forward (with one
    # slot the head has taken it, so it is fetched too); the embedding's
    # backward reads no weights
    assert n_fetch == (2 * L + 2 if mode == "single_slot" else 2 * L + 1)
    assert sum(o["kind"] == POISON for o in ops) == (n_fetch if flags & mt.MT_FLAG_POISON else 0)
    assert sum(o["kind"] == OFFLOAD for o in ops) == L + 2


def test_token_passes_and_micro_batches_keep_the_schedule():
    base = plan(SMALL)
    assert plan(SMALL.replace(batch=4), token_chunk=256) == plan(SMALL.replace(batch=4))
    assert plan(SMALL, micro_batches=3) == base
    assert check_hazards(base, SMALL.n_layers + 2) == []


def test_offloads_yield_the_link_only_when_compute_bound():
    """At a long context a layer's backward takes longer than moving its
    weights and gradients, so each offload waits for the next prefetch's
    copy (a link-only ordering); prefetches never wait for offloads."""
    ops = plan(LONG)
    linked = [o for o in ops if o["kind"] == OFFLOAD and o["link"]]
    # one offload held behind each prefetch of the backward sweep (of layers
    # n_layers-1 .. 1): the head's, then each layer's but the last two
    assert len(linked) == LONG.n_layers - 1
    for o in linked:
        assert all(ops[f]["kind"] == FETCH for f in o["link"])
    for o in ops:
        if o["kind"] == FETCH:
            assert all(ops[w]["kind"] != OFFLOAD for w in o["waits"])
    assert not any(o["link"] for o in plan(LONG, flags=mt.MT_FLAG_DUPLEX_LINK))
    assert not any(o["link"] for o in plan(SMALL))


def _drop(ops, victim, dropped):
    ops = copy.deepcopy(ops)
    ops[victim]["waits"] = [w for w in ops[victim]["waits"] if w != dropped]
    return ops


def _find(ops, kind, pred=lambda o: True):
    return [i for i, o in enumerate(ops) if o["kind"] == kind and pred(o)]


@pytest.mark.parametrize("flags", [0, mt.MT_FLAG_POISON])
def test_planted_missing_waits_are_caught(flags):
    """Remove one wait at a time from the streamed plan: each kind of missing
    wait is reported."""
    ops = plan(SMALL, "streamed", flags)
    n = SMALL.n_layers + 2
    assert check_hazards(ops, n) == []
    cases = []
    for c in _find(ops, COMPUTE, lambda o: o["wslot"] >= 0):
        for w in ops[c]["waits"]:
            if ops[w]["kind"] == FETCH:
                cases.append(("compute before its weights arrive", c, w))
            if ops[w]["kind"] == OFFLOAD:
                cases.append(("compute overwrites a gradient slot being offloaded", c, w))
    for f in _find(ops, FETCH):
        for w in ops[f]["waits"]:
            cases.append(("prefetch overwrites a slot still being read", f, w))
    for o in _find(ops, OFFLOAD):
        for w in ops[o]["waits"]:
            cases.append(("offload before the gradient is written", o, w))
    for a in _find(ops, ADAM):
        for w in ops[a]["waits"]:
            cases.append(("Adam before the gradient lands", a, w))
    kinds = {k for k, _, _ in cases}
    assert len(kinds) == 5, kinds
    for what, victim, dropped in cases:
        found = check_hazards(_drop(ops, victim, dropped), n)
        assert found, (what, victim, dropped)


def test_a_swapped_slot_is_caught():
    ops = plan(SMALL)
    bad = copy.deepcopy(ops)
    c = _find(bad, COMPUTE, lambda o: o["use"] == 3)[0]
    bad[c]["wslot"] ^= 1
    assert check_hazards(bad, SMALL.n_layers + 2)
    bad = copy.deepcopy(ops)
    o = _find(bad, OFFLOAD, lambda o: o["use"] == SMALL.n_layers + 3)[0]
    bad[o]["gslot"] ^= 1
    assert check_hazards(bad, SMALL.n_layers + 2)


def test_schedule_errors():
    with pytest.raises(mt.MtError):
        plan(SMALL, "resident")
    cfg = mt.make_config(SMALL)
    cfg.n_layers = 0
    with pytest.raises(mt.MtError):
        mt.schedule(cfg)
    assert mt.lib().mt_schedule(ctypes.byref(mt.make_config(SMALL)), None, -1) == mt.MT_E_INVALID
