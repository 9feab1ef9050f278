"""KV-cache memory under continuous batching: static reservation against paged blocks.

The pages contrast two ways of holding each request's KV cache ("vLLM — PagedAttention
and Continuous Batching", §2.1-2.3 and §3; "vLLM and PagedAttention", §2 "The
Problem with the Traditional KV Cache"; "How vLLM Works?", sections 02-04):

* static: one contiguous region per request, sized for the most tokens it may
  reach, reserved at admission; the part it never fills is wasted (internal
  fragmentation) and, with regions of different sizes, free space splits into
  holes a new request may not fit (external fragmentation);
* paged: fixed 16-token blocks taken one at a time as the request grows, so only
  the last block of a sequence can be partly empty.

``simulate`` runs the same request stream through both under iteration-level
(continuous) batching: each iteration admits waiting requests in arrival order
while their memory fits, gives every running request one new token, and
releases the finished ones.  Paged admission needs the prompt's blocks plus
``headroom`` free blocks per running request (room to grow before the next
admission); when a growing request still finds no free block, the most recently
admitted request is preempted (its blocks are released and it waits again at
the head of the queue, its tokens so far to be recomputed as its prompt).  The
paged side runs on the library's C++ allocator.

No model is run: lengths are drawn, and memory is counted in token slots.
"""

import numpy as np

from .allocator import BlockAllocator

BLOCK = 16


def static_waste(reserved, used):
    """Slots reserved but never filled by one request."""
    return int(reserved) - int(used)


def paged_waste(used, block_size=BLOCK):
    """Slots of a request's blocks not filled: at most block_size - 1 (its last block)."""
    return -(-int(used) // block_size) * block_size - int(used)


def draw_requests(rng, n, prompt_lo, prompt_hi, mean_output, max_new):
    """``n`` requests arriving one per iteration: prompt uniform in [lo, hi]
    (inclusive), output length geometric with the given mean, capped at max_new."""
    prompts = rng.integers(prompt_lo, prompt_hi + 1, size=n)
    outputs = np.minimum(rng.geometric(1.0 / mean_output, size=n), max_new)
    return [(int(i), int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outputs))]


class _StaticArena:
    """First-fit contiguous reservations in an arena of ``slots`` token slots."""

    def __init__(self, slots):
        self.slots = slots
        self.used = {}                      # request -> (start, size)

    def _holes(self):
        pos = 0
        for start, size in sorted(self.used.values()):
            if start > pos:
                yield pos, start - pos
            pos = start + size
        if pos < self.slots:
            yield pos, self.slots - pos

    def reserve(self, req, size):
        for start, length in self._holes():
            if length >= size:
                self.used[req] = (start, size)
                return True
        return False

    def free_slots(self):
        return self.slots - sum(s for _, s in self.used.values())

    def release(self, req):
        del self.used[req]


def simulate(requests, memory_slots, max_new, policy, headroom=1.0, max_iters=100_000):
    """Run ``requests`` [(id, prompt_len, output_len)] through one policy.

    policy "static": each request reserves prompt + max_new slots at admission.
    policy "paged": 16-token blocks from the C++ allocator, one at a time.
    Returns per-run means: running requests per iteration, the fraction of held
    memory not filled (waste), memory filled, preemptions, and the largest
    per-request waste seen (paged: under one block).
    """
    queue = list(requests)
    running = {}                            # id -> [prompt_len, output_len, generated]
    order = []                              # admission order (paged preemption picks the newest)
    arena = _StaticArena(memory_slots) if policy == "static" else None
    alloc = BlockAllocator(memory_slots // BLOCK, BLOCK) if policy == "paged" else None
    conc, waste_frac, filled, preempt, worst = [], [], [], 0, 0
    it = 0
    while (queue or running) and it < max_iters:
        it += 1
        # admit in arrival order while memory fits
        while queue:
            rid, p, o = queue[0]
            if policy == "static":
                ok = arena.reserve(rid, p + max_new)
            else:
                ok = alloc.num_free() >= -(-p // BLOCK) + headroom * len(running)
                if ok:
                    alloc.add_seq(rid)
                    alloc.append(rid, p)
            if not ok:
                break
            queue.pop(0)
            running[rid] = [p, o, 0]
            order.append(rid)
        if not running:
            break
        # one new token for every running request
        if policy == "paged":
            for rid in list(order):
                if rid not in running:
                    continue
                while True:
                    try:
                        alloc.append(rid, 1)
                        break
                    except MemoryError:
                        victim = order[-1]     # the newest running request is recomputed later:
                        order.pop()            # its tokens so far become its prompt
                        p, o, g = running.pop(victim)
                        alloc.free_seq(victim)
                        queue.insert(0, (victim, p + g, o - g))
                        preempt += 1
                        if victim == rid:
                            break
        for rid in list(running):
            if policy == "static" or rid in order:
                running[rid][2] += 1
        # account, then release the finished
        used = sum(p + g for p, _, g in running.values())
        if policy == "static":
            held = sum(s for _, s in arena.used.values())
            worst = max([worst] + [static_waste(p + max_new, p + g) for p, _, g in running.values()])
        else:
            held = sum(-(-(p + g) // BLOCK) * BLOCK for p, _, g in running.values())
            worst = max([worst] + [paged_waste(p + g) for p, _, g in running.values()])
        conc.append(len(running))
        waste_frac.append(1.0 - used / held if held else 0.0)
        filled.append(used / memory_slots)
        for rid in [r for r, (p, o, g) in running.items() if g >= o]:
            del running[rid]
            if policy == "static":
                arena.release(rid)
            else:
                order.remove(rid)
                alloc.free_seq(rid)
    if alloc is not None:
        alloc.close()
    return {"policy": policy, "iterations": it, "mean_running": float(np.mean(conc)),
            "mean_waste_fraction": float(np.mean(waste_frac)), "mean_memory_filled": float(np.mean(filled)),
            "preemptions": preempt, "max_waste_per_request": int(worst)}
