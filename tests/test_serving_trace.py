"""The serving-loop event trace on the allocator model alone (CPU): no step's
appends run out of blocks or past a table, and the trace admits, forks, frees,
copies on write and recycles blocks as often as the GPU loop test relies on."""

import numpy as np
import pytest

import workloads as W
from oracle import AllocatorModel
from tests.serving_trace import CASES, next_events


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_trace_keeps_room_and_covers_the_path(case):
    name, hq, hkv, d, bs, nb, M, steps, seed, max_prompt, chunk = case
    rng = np.random.default_rng(seed)
    model = AllocatorModel(nb, bs, M, W.free_order(nb, seed))
    live, next_id = [], 0
    seen = {"admit": 0, "fork": 0, "free": 0, "cow": 0, "recycled": 0}
    ever_held = set()
    for _ in range(steps):
        events, next_id = next_events(rng, model, live, next_id, max_prompt)
        for ev in events:
            if ev[0] == "free":
                model.free_seq(ev[1])
                live.remove(ev[1])
            elif ev[0] == "fork":
                model.fork(ev[1], ev[2])
                live.append(ev[2])
            else:
                model.add_seq(ev[1], ev[2])
                fresh = set(model.seq_blocks(ev[1]))
                seen["recycled"] += len(fresh & ever_held)
                ever_held |= fresh
                live.append(ev[1])
            seen[ev[0]] += 1
        assert model.num_free() >= len(live)
        for s in live:
            before = set(model.seq_blocks(s))
            _, src, _ = model.append_slot(s)          # raises if out of blocks
            seen["cow"] += src >= 0
            fresh = set(model.seq_blocks(s)) - before
            seen["recycled"] += len(fresh & ever_held)
            ever_held |= fresh
        # Every running sequence's blocks are distinct unless shared by a fork.
        refs = {}
        for s in live:
            for b in set(model.seq_blocks(s)):
                refs[b] = refs.get(b, 0) + 1
        assert all(model.refcount(b) == n for b, n in refs.items())
    assert seen["admit"] >= 10 and seen["fork"] >= 5 and seen["free"] >= 10, seen
    assert seen["cow"] >= 5 and seen["recycled"] >= 20, seen
