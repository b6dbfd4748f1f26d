"""The KV memory-waste simulator (paged_kv_cache_410_amd.waste), CPU only.

Pinned to the pages' worked example (tests/golden/page_facts.json: a
2,048-token reservation that stops at 150 tokens leaves 1,898 slots idle;
"Why OS Virtual Memory Paging Saved LLM Inference", a8q9.cn, section 1), to
hand-traced accounting on tiny streams, and to the first-fit arena's
behaviour; the pages' qualitative claims (waste under 4% with paging, two to
four times as many requests at once; same page, section 3) are checked as
outcomes on a synthetic stream (waste under 4% holds; the concurrency gain on
this length mix is about 2x, so the test asks only for a clear multiple).
"""

import json
import os

import pytest

import oracle
from paged_kv_cache_410_amd import BlockManager
from paged_kv_cache_410_amd import waste

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def test_pages_internal_fragmentation_example():
    facts = json.load(open(GOLDEN))["internal_fragmentation_example"]
    contiguous, paged = waste.snapshot_waste([facts["used_tokens"]], facts["reserved_tokens"], 16)
    assert contiguous == facts["idle_slots_contiguous"]           # 1898
    assert paged == facts["derived_paged"]["idle_slots"]          # 10 (10 blocks, 160 slots)


def test_arena_first_fit_and_merging():
    a = waste.ContiguousArena(100)
    assert a.alloc(30) == 0 and a.alloc(30) == 30 and a.alloc(30) == 60
    assert a.alloc(20) is None and a.largest_hole() == 10
    a.free(30, 30)
    assert a.alloc(40) is None                 # 30 + 10 free, but not contiguous
    assert a.free_slots() == 40 and a.largest_hole() == 30
    a.free(60, 30)                             # merges with [30, 60) and [90, 100)
    assert a.holes == [(30, 70)]
    assert a.alloc(25) == 30


def test_tiny_stream_by_hand():
    reqs = [waste.Request(prompt=1, final=3, bound=3)]
    c = waste.simulate_contiguous(reqs, slots=64, max_len=8)
    # ticks with the request running: lengths 1 then 2 of 8 reserved slots
    assert c["ticks"] == 2 and c["useful_fraction"] == pytest.approx((1 / 8 + 2 / 8) / 2)
    v = waste.simulate_contiguous(reqs, slots=64, max_len=8, per_request=True)
    assert v["useful_fraction"] == pytest.approx((1 / 3 + 2 / 3) / 2)
    p = waste.simulate_paged(reqs, slots=64, block_size=4, manager_factory=BlockManager)
    # one 4-slot block holding 1, then 2 tokens
    assert p["ticks"] == 2 and p["useful_fraction"] == pytest.approx((1 / 4 + 2 / 4) / 2)
    for r in (c, v):
        assert r["useful_fraction"] + r["reservation_waste"] == pytest.approx(1.0)
    assert p["useful_fraction"] + p["last_block_waste"] == pytest.approx(1.0)


def test_paged_preempts_the_newest_when_blocks_run_out():
    # 2 blocks of 4: two requests each need a second block at their 5th token
    reqs = [waste.Request(4, 8, 8), waste.Request(4, 8, 8)]
    p = waste.simulate_paged(reqs, slots=12, block_size=4, manager_factory=BlockManager)
    assert p["preemptions"] >= 1
    assert p["ticks"] > 4                        # the preempted one restarts afterwards


def test_native_and_oracle_managers_agree():
    reqs = waste.lognormal_requests(200, seed=3, hi=1024)
    a = waste.simulate_paged(reqs, 16384, 16, BlockManager)
    b = waste.simulate_paged(reqs, 16384, 16, oracle.BlockManager)
    assert a == b


def test_pages_claims_hold_on_a_synthetic_stream():
    reqs = waste.lognormal_requests(400, seed=8)
    r = waste.compare(reqs, slots=65536)
    assert r["paged"]["last_block_waste"] < 0.04                   # "under 4%"
    assert r["contiguous"]["reservation_waste"] > 0.5
    # the pages report 2-4x on their workloads; this length mix gives about 1.9x here
    # (2.0x on the 2000-request default stream), a measured outcome, not a bound
    assert r["concurrency_gain"] >= 1.5
    assert r["contiguous_per_request"]["unusable_free_fraction"] > 0.0   # holes appear
