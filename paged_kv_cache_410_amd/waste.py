"""KV-cache memory waste: contiguous max-length reservation vs paged blocks.

Reproduces the mechanism behind the pages' memory figures on synthetic
request streams (no traces, no model):

  * "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn), section 1:
    engines that cannot predict a request's length reserve contiguous room for
    the maximum (e.g. 2,048 tokens); what the request does not use is idle
    (internal fragmentation, the reservation), and variable-sized contiguous
    regions leave holes that new requests cannot use (external
    fragmentation). Section 2: paged KV blocks are taken one at a time as
    tokens arrive, so a sequence wastes at most the unused tail of its last
    block. Section 3: waste drops from about 80% to under 4%, and servers can
    run two to four times as many requests at once.
  * "vLLM & PagedAttention" (completesystemdesign.dev), section 01: with one
    contiguous max-length buffer per request only 20-38% of KV memory holds
    useful tokens.

Model (one decode step per tick; one new token per running request):
  requests arrive all at once and are admitted first come, first served;
  a request needs its prompt cached at admission and one more slot per
  generated token; it finishes at its final length and frees its memory.
  contiguous  admission reserves max_len slots in one region of a linear
              arena (first fit among the holes); a request never needs more.
  contiguous, per request: the same with each request's own declared bound
              (prompt + its generation limit) reserved instead of max_len; the
              regions then differ in size and leave holes.
  paged       admission takes the prompt's blocks (plus the first generated
              token's) from the library's block manager; each generated token
              that starts a block takes one more; when none is free, the most
              recently admitted running request is preempted (its blocks
              freed, the request queued again at the front, restarting).
Reported per policy, averaged over the ticks with at least one running
request: the fraction of allocated KV slots holding tokens, the waste split
into reservation slack (contiguous), last-block slack (paged) and the share of
free memory unusable for the next request (external fragmentation), plus mean
concurrency, preemptions and ticks to drain the stream.

    python -m paged_kv_cache_410_amd.waste [--requests 2000] [--slots 262144]
"""

import argparse
import json
import math
from dataclasses import dataclass

import numpy as np


@dataclass
class Request:
    prompt: int
    final: int        # prompt + generated tokens at completion
    bound: int = 0    # prompt + the request's own generation limit (>= final)


def lognormal_requests(n, seed, median=500.0, sigma=0.7, lo=16, hi=2048, out_frac=(0.1, 0.6)):
    """Final lengths lognormal (the 13B-shape mix), a U(out_frac) share generated;
    each request's declared bound is its prompt plus up to twice what it
    actually generates, capped at `hi`."""
    rng = np.random.default_rng(seed)
    final = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, n))), lo, hi).astype(int)
    share = rng.uniform(out_frac[0], out_frac[1], n)
    prompt = np.maximum(1, np.rint(final * (1.0 - share)).astype(int))
    prompt = np.minimum(prompt, final)
    slack = rng.uniform(1.0, 2.0, n)
    bound = np.minimum(hi, np.maximum(final, np.rint(prompt + (final - prompt) * slack))).astype(int)
    return [Request(int(p), int(f), int(b)) for p, f, b in zip(prompt, final, bound)]


def snapshot_waste(lengths, max_len, block_size):
    """Idle KV slots held by live sequences of the given lengths: under a
    contiguous max_len reservation each, and under paged blocks."""
    contiguous = sum(max_len - n for n in lengths)
    paged = sum(block_size * -(-n // block_size) - n for n in lengths)
    return contiguous, paged


class ContiguousArena:
    """First-fit allocator of fixed-size regions in [0, slots): the prior design."""

    def __init__(self, slots):
        self.slots = slots
        self.holes = [(0, slots)]          # sorted (start, length)

    def alloc(self, n):
        for i, (start, length) in enumerate(self.holes):
            if length >= n:
                if length == n:
                    self.holes.pop(i)
                else:
                    self.holes[i] = (start + n, length - n)
                return start
        return None

    def free(self, start, n):
        self.holes.append((start, n))
        self.holes.sort()
        merged = []
        for s, ln in self.holes:
            if merged and merged[-1][0] + merged[-1][1] == s:
                merged[-1] = (merged[-1][0], merged[-1][1] + ln)
            else:
                merged.append((s, ln))
        self.holes = merged

    def free_slots(self):
        return sum(ln for _, ln in self.holes)

    def largest_hole(self):
        return max((ln for _, ln in self.holes), default=0)


def simulate_contiguous(reqs, slots, max_len, per_request=False):
    """Contiguous reservations: max_len each, or (per_request) each request's
    own declared bound, whose varying sizes leave holes in the arena."""
    arena = ContiguousArena(slots)
    queue = list(range(len(reqs)))
    running = {}                                 # id -> (start, reserved, length)
    acc = dict(ticks=0, busy=0, used=0.0, alloc=0.0, reserve=0.0, ext=0.0, conc=0.0)
    size = (lambda r: r.bound) if per_request else (lambda r: max_len)
    while queue or running:
        while queue:                                       # admit FCFS
            i = queue[0]
            if reqs[i].final > size(reqs[i]):
                raise ValueError("a request longer than its reservation")
            start = arena.alloc(size(reqs[i]))
            if start is None:
                break
            queue.pop(0)
            running[i] = (start, size(reqs[i]), reqs[i].prompt)
        if running:
            used = sum(ln for _, _, ln in running.values())
            alloc = sum(rs for _, rs, _ in running.values())
            free = arena.free_slots()
            acc["busy"] += 1
            acc["used"] += used / alloc
            acc["alloc"] += alloc / slots
            acc["reserve"] += (alloc - used) / alloc
            # free memory the next request in line cannot use (no hole fits it)
            blocked = queue and arena.largest_hole() < size(reqs[queue[0]])
            acc["ext"] += (free / slots) if blocked else 0.0
            acc["conc"] += len(running)
        acc["ticks"] += 1
        for i in list(running):                            # one decode step
            start, rs, ln = running[i]
            ln += 1
            if ln >= reqs[i].final:
                arena.free(start, rs)
                del running[i]
            else:
                running[i] = (start, rs, ln)
    b = max(acc["busy"], 1)
    return dict(policy="contiguous_per_request" if per_request else "contiguous", max_len=max_len,
                slots=slots, ticks=acc["ticks"],
                useful_fraction=acc["used"] / b, reservation_waste=acc["reserve"] / b,
                last_block_waste=0.0, unusable_free_fraction=acc["ext"] / b,
                mean_running=acc["conc"] / b, preemptions=0)


def simulate_paged(reqs, slots, block_size, manager_factory):
    nb = slots // block_size
    bm = manager_factory(nb, block_size)
    queue = list(range(len(reqs)))
    running = {}                                 # id -> seq
    order = []                                   # admission order of running ids
    preempt = 0
    acc = dict(ticks=0, busy=0, used=0.0, last=0.0, ext=0.0, conc=0.0)

    def admit(i):
        # the prompt plus the first generated token must fit now
        need = -(-(reqs[i].prompt + 1) // block_size)
        if need > bm.num_free():
            return False
        sid = bm.add_seq()
        bm.append(sid, reqs[i].prompt)
        running[i] = sid
        order.append(i)
        return True

    while queue or running:
        while queue and admit(queue[0]):
            queue.pop(0)
        if running:
            used = sum(bm.seq_len(s) for s in running.values())
            blocks = nb - bm.num_free()
            acc["busy"] += 1
            acc["used"] += used / (blocks * block_size)
            acc["last"] += (blocks * block_size - used) / (blocks * block_size)
            acc["conc"] += len(running)
        acc["ticks"] += 1
        for i in list(order):                              # one decode step
            if i not in running:
                continue
            sid = running[i]
            # a token that starts a block needs a free one: preempt the newest
            while bm.seq_len(sid) % block_size == 0 and bm.num_free() == 0:
                victim = order.pop()
                bm.free_seq(running.pop(victim))
                queue.insert(0, victim)
                preempt += 1
                if victim == i:
                    break
            if i not in running:
                continue
            bm.append(sid, 1)
            if bm.seq_len(sid) >= reqs[i].final:
                bm.free_seq(sid)
                del running[i]
                order.remove(i)
    b = max(acc["busy"], 1)
    return dict(policy="paged", block_size=block_size, slots=slots, ticks=acc["ticks"],
                useful_fraction=acc["used"] / b, reservation_waste=0.0,
                last_block_waste=acc["last"] / b, unusable_free_fraction=0.0,
                mean_running=acc["conc"] / b, preemptions=preempt)


def compare(reqs, slots, max_len=2048, block_size=16, manager_factory=None):
    if manager_factory is None:
        from . import BlockManager
        manager_factory = BlockManager
    c = simulate_contiguous(reqs, slots, max_len)
    v = simulate_contiguous(reqs, slots, max_len, per_request=True)
    p = simulate_paged(reqs, slots, block_size, manager_factory)
    return dict(contiguous=c, contiguous_per_request=v, paged=p,
                concurrency_gain=p["mean_running"] / max(c["mean_running"], 1e-9),
                concurrency_gain_vs_per_request=p["mean_running"] / max(v["mean_running"], 1e-9),
                drain_speedup=c["ticks"] / max(p["ticks"], 1))


def main():
    ap = argparse.ArgumentParser(description="KV memory waste: contiguous reservation vs paged")
    ap.add_argument("--requests", type=int, default=2000)
    ap.add_argument("--slots", type=int, default=262144, help="KV token slots of the budget")
    ap.add_argument("--max-len", type=int, default=2048)
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--seed", type=int, default=8)
    args = ap.parse_args()
    reqs = lognormal_requests(args.requests, args.seed, hi=args.max_len)
    print(json.dumps(compare(reqs, args.slots, args.max_len, args.block_size)))


if __name__ == "__main__":
    main()
