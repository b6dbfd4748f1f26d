"""GPU: the precondition checks (pa_check_slots, pa_check_pairs, pa_check_tables)
count exactly the violations planted in otherwise valid inputs, and none in
the workloads' own step inputs."""

import numpy as np
import pytest
import torch

from paged_kv_cache_410_amd.workloads import Spec

from gpu_cases import Step, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def i32(x):
    return torch.tensor(x, dtype=torch.int32, device="cuda")


def test_check_slots(pa):
    say("[check slots]")
    # duplicates of 5 and of 9 (twice) after their first use; negatives are exempt
    assert pa.check_slots(i32([5, 9, -1, 5, -1, 9, 9, 3])) == 3
    assert pa.check_slots(i32([-1, -1, -1])) == 0
    assert pa.check_slots(i32([7])) == 0
    assert pa.check_slots(torch.empty(0, dtype=torch.int32, device="cuda")) == 0
    rng = np.random.default_rng(3)
    slots = rng.permutation(200000)[:20000].astype(np.int32)   # distinct, several waves
    assert pa.check_slots(i32(slots)) == 0
    where = 2 * rng.choice(np.arange(1, 10000), 7, replace=False)   # even: sources stay intact
    planted = slots.copy()
    planted[where] = slots[where - 1]                           # 7 repeats of a neighbour
    assert pa.check_slots(i32(planted)) == 7


def test_check_pairs(pa):
    say("[check pairs]")
    assert pa.check_pairs(i32([[1, 2], [3, 4], [5, 2]]), 10) == 1      # destination 2 twice
    assert pa.check_pairs(i32([[1, 2], [2, 3]]), 10) == 1              # 2 written and read
    assert pa.check_pairs(i32([[4, 4]]), 10) == 1                      # a block onto itself
    assert pa.check_pairs(i32([[1, 2], [50, 2], [3, -1]]), 10) == 0    # skipped pairs exempt
    assert pa.check_pairs(i32([[1, 2], [3, 4], [5, 6]]), 10) == 0
    assert pa.check_pairs(torch.empty(0, 2, dtype=torch.int32, device="cuda"), 10) == 0


def test_check_tables(pa):
    say("[check tables]")
    NB, MB = 20, 4
    bt = np.full((5, MB), -1, np.int32)
    bt[0, :2] = [3, 7]
    bt[1, :1] = [4]
    bt[2, :4] = [0, 1, 2, 5]
    bt[3, :1] = [9]
    cl = np.array([20, 16, 64, 1, 0], np.int32)
    assert pa.check_tables(i32(bt), i32(cl), NB, 64) == 0
    b2, c2 = bt.copy(), cl.copy()
    b2[0, 1] = NB + 5          # used entry outside the pool
    b2[1, 3] = 99              # unused entry (past ceil(16 / 16)): not a violation
    c2[3] = -1                 # negative length
    c2[4] = MB * 16 + 1        # past the table
    assert pa.check_tables(i32(b2), i32(c2), NB, 1000) == 3
    assert pa.check_tables(i32(bt), i32(cl), NB, 32) == 1   # 64 > max_ctx


@pytest.mark.parametrize("name,spec", [
    ("cow", Spec("cow", "bf16", 8, 4, 4, 128, seed=21, lengths=("cow",),
                 cow=dict(prompts=2, samples=4, prompt_len=96, r_max=15, tail_lo=1,
                          tail_hi=40))),
    ("chunk", Spec("chunk", "bf16", 4, 16, 2, 128, seed=31, lengths=("uniform", 1, 2000),
                   chunk=("uniform", 1, 20))),
])
def test_workload_inputs_pass_the_checks(pa, name, spec):
    say(f"[check workload] {name}")
    st = Step(spec, oracle_full=False)
    slots = pa.slot_mapping(st.block_tables, st.step_pos, seq_ids=st.step_seq)
    assert pa.check_slots(slots) == 0
    assert pa.check_pairs(st.pairs, st.tb.NB) == 0
    assert pa.check_tables(st.block_tables, st.context_lens, st.tb.NB, st.max_ctx) == 0
