"""Hazard proof for a streamed step's schedule (mt_schedule), on the CPU.

The schedule is a list of operations in issue order.  Each runs on a lane:
the prefetch, compute and offload lanes execute their operations in issue
order, and host Adam updates are unordered among themselves.  An operation
starts once every operation it waits for has finished.  From these two
rules alone this module builds the happens-before relation and proves the
data discipline of the double-buffered pipeline of the MegaTrain pages
([Methodik]: the next block's weights stream into the free buffer while the
current block computes, and gradients stream out behind the compute).

Resources and their rules:

* weight slot s: written by FETCH (and POISON), read by COMPUTE.  The last
  write ordered before a read must be the FETCH of the block the read
  computes, and every other write to the slot must be ordered before that
  FETCH or after the read.
* gradient slot g: written by COMPUTE, read by OFFLOAD.  The offload of a
  use reads what that use's compute wrote; every other compute writing the
  slot is ordered before that compute or after the offload.
* host region G of block j: written by the one OFFLOAD of j in the step,
  read by ADAM(j).  Host region W of block j: read by every FETCH of j,
  written by ADAM(j), which must come after all of them.

Orderings the schedule marks as link-only (an offload held back behind a
prefetch so that the prefetch has the host link to itself) carry no data:
the proof does not use them, so it holds with or without them.

The module shares nothing with the library: it reads the exported plan only.
"""
from __future__ import annotations

FETCH, POISON, COMPUTE, OFFLOAD, ADAM, END = range(6)
ORDERED_LANES = (0, 1, 2)
NAMES = ("FETCH", "POISON", "COMPUTE", "OFFLOAD", "ADAM", "END")


def happens_before(ops):
    """hb[i]: bit set of the operations that finish before operation i starts."""
    hb = []
    last = {}
    for i, o in enumerate(ops):
        preds = list(o["waits"])
        if o["lane"] in ORDERED_LANES and o["lane"] in last:
            preds.append(last[o["lane"]])
        m = 0
        for p in preds:
            if not 0 <= p < i:
                raise ValueError(f"operation {i} waits for {p}, not an earlier operation")
            m |= hb[p] | (1 << p)
        hb.append(m)
        if o["lane"] in ORDERED_LANES:
            last[o["lane"]] = i
    return hb


def _desc(ops, i):
    o = ops[i]
    return f"#{i} {NAMES[o['kind']]}(use {o['use']}, block {o['block']})"


def check_hazards(ops, n_blocks):
    """List of hazards (empty: the schedule is proven race-free)."""
    hb = happens_before(ops)

    def before(a, b):
        return (hb[b] >> a) & 1 == 1

    bad = []
    idx = lambda kind: [i for i, o in enumerate(ops) if o["kind"] == kind]
    fetches, computes, offloads, adams = idx(FETCH), idx(COMPUTE), idx(OFFLOAD), idx(ADAM)

    def sees(read, writes, ok_writer, what):
        prior = [w for w in writes if before(w, read)]
        for w in writes:
            if w not in prior and not before(read, w):
                bad.append(f"{what}: {_desc(ops, w)} may overlap {_desc(ops, read)}")
        if not prior:
            bad.append(f"{what}: {_desc(ops, read)} has no write before it")
            return
        latest = [w for w in prior if all(v == w or before(v, w) for v in prior)]
        if len(latest) != 1:
            bad.append(f"{what}: writes before {_desc(ops, read)} are unordered")
        elif not ok_writer(latest[0]):
            bad.append(f"{what}: {_desc(ops, read)} sees {_desc(ops, latest[0])}")

    # weight slots
    for c in computes:
        s = ops[c]["wslot"]
        if s < 0:
            continue
        writes = [i for i in fetches + idx(POISON) if ops[i]["wslot"] == s]
        sees(c, writes, lambda w: ops[w]["kind"] == FETCH and ops[w]["block"] == ops[c]["block"],
             f"weight slot {s}")
    # gradient slots
    for o in offloads:
        g = ops[o]["gslot"]
        writes = [i for i in computes if ops[i]["gslot"] == g]
        sees(o, writes, lambda w: ops[w]["use"] == ops[o]["use"], f"gradient slot {g}")
    # host G and W of each block
    for j in range(n_blocks):
        offs = [i for i in offloads if ops[i]["block"] == j]
        ads = [i for i in adams if ops[i]["block"] == j]
        if len(offs) != 1 or len(ads) != 1:
            bad.append(f"block {j}: {len(offs)} offloads and {len(ads)} Adam updates in the step")
            continue
        if not before(offs[0], ads[0]):
            bad.append(f"host G of block {j}: {_desc(ops, ads[0])} may read before {_desc(ops, offs[0])}")
        for f in fetches:
            if ops[f]["block"] == j and not before(f, ads[0]):
                bad.append(f"host W of block {j}: {_desc(ops, ads[0])} may write during {_desc(ops, f)}")
    # the step's end follows every device operation
    ends = idx(END)
    if len(ends) != 1:
        bad.append(f"{len(ends)} END operations")
    else:
        for i, o in enumerate(ops):
            if o["lane"] in ORDERED_LANES and i != ends[0] and not before(i, ends[0]):
                bad.append(f"{_desc(ops, i)} may still run after the step's end")
    return bad


def use_order(ops):
    """(use, block) of the compute operations in issue order."""
    return [(o["use"], o["block"]) for o in ops if o["kind"] == COMPUTE]
