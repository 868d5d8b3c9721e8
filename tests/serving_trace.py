"""Seeded event trace of a small serving loop over the paged cache.

Continuous batching as the pages describe it ("vLLM core architecture ...",
section 3; "Deep dive into the nano-vLLM inference engine architecture ...",
section "Continuous batching and memory management working together"):
requests are admitted with their prompt, every running request gains one token
a step, finished requests free their blocks for later admissions, and a forked
request shares its parent's blocks until one of them writes into a shared,
partly filled block (copy-on-write).

``next_events`` decides what happens before a step from a numpy generator and
the allocator state the oracle side keeps (``AllocatorModel``); it computes
nothing the path computes, so both sides replay the same events in order.
"""

# Loop configurations: name, q heads, KV heads, head_dim, block, pool blocks,
# blocks per sequence, steps, seed, longest prompt, prefill chunk (not a
# multiple of the block, so chunks end inside blocks).
CASES = [
    ("gqa_bs16", 8, 2, 128, 16, 64, 16, 48, 11, 90, 40),
    ("mha_bs8_d64", 4, 4, 64, 8, 96, 32, 48, 12, 60, 20),
]


def next_events(rng, model, live, next_id, max_prompt, p_admit=0.45, p_fork=0.2, p_free=0.15):
    """Events of one step, in the order they are to be applied:
    ``("free", seq)``, ``("fork", parent, child)``, ``("admit", seq, tokens)``.

    ``live`` lists the running sequences in admission order.  Room is kept so
    that the step's appends cannot run out of blocks: every running sequence
    may need one block (a fresh one, or the target of a copy), so at least that
    many stay free, and a sequence whose table is full is finished first.
    Returns (events, next unused sequence id)."""
    events = []
    bs, M = model.block_size, model.max_blocks_per_seq
    free_blocks = model.num_free()
    # Blocks held by each running sequence, as the step's events leave them
    # (an admitted sequence holds fresh blocks, named here by placeholders).
    held = {s: list(model.seq_blocks(s)) for s in live}
    length = {s: model.seq_len(s) for s in live}
    running = list(live)

    def finish(seq):
        nonlocal free_blocks
        events.append(("free", seq))
        running.remove(seq)
        mine = held.pop(seq)
        others = {b for s in running for b in held[s]}
        free_blocks += sum(1 for b in set(mine) if b not in others)

    for seq in list(running):
        if length[seq] + 1 > M * bs:
            finish(seq)
    if len(running) > 1 and rng.random() < p_free:
        finish(running[int(rng.integers(len(running)))])
    if running and rng.random() < p_fork:
        parent = running[int(rng.integers(len(running)))]
        child = next_id
        next_id += 1
        events.append(("fork", parent, child))
        held[child] = list(held[parent])
        length[child] = length[parent]
        running.append(child)
    if not running or rng.random() < p_admit:
        n = int(rng.integers(1, max_prompt + 1))
        need = -(-n // bs)
        while running and free_blocks - need < len(running) + 1:
            finish(running[0])
        if free_blocks - need >= len(running) + 1:
            seq = next_id
            next_id += 1
            events.append(("admit", seq, n))
            held[seq] = [("new", seq, j) for j in range(need)]
            length[seq] = n
            free_blocks -= need
            running.append(seq)
    while running and free_blocks < len(running):
        finish(running[0])
    return events, next_id
