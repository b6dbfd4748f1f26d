"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: whole-pool bit-exact cache bookkeeping, and every attention
output row against the fp64 oracle.

Paging only moves where each token's K/V rows live, so the result must be the
attention of the sequence's whole history wherever its blocks sit ("Can OS
paging techniques reduce LLM serving memory waste?", mechanism paragraph;
"Why OS Virtual Memory Paging Saved LLM Inference", section 2). That is
checked on every (query row, head) of every decode workload. The 512-token
chunk workloads (about 6e11 products for the whole step at head_dim 128) are
checked on every row and head of their 4 longest and 4 shortest sequences.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_410_amd import workloads

from gpu_cases import TOL, Step, host_bits, record_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def bench_partition(pa, spec, rows, max_ctx):
    if spec.partition:
        return spec.partition
    return pa.default_partition(rows, spec.Hq, spec.Hkv, spec.D, max_ctx)


def run_step(pa, name):
    """The benchmark's step on the workload's seeded inputs: copies, the fused
    slot mapping + cache write, then attention at the benchmark's partition.
    Returns the Step and the attention output; the bookkeeping is checked."""
    spec = workloads.CONFIGS[name]
    say(f"[full config] {name}: building inputs")
    st = Step(spec, values_device="cuda", oracle_full=False)
    part = bench_partition(pa, spec, st.q.shape[0], st.max_ctx)
    say(f"[full config] {name}: NB={st.tb.NB} MB={st.tb.MB} T={len(st.tb.slots)} "
        f"pairs={len(st.tb.pairs)} partition={part}")
    # the generated step respects the preconditions the kernels take on trust
    assert pa.check_tables(st.block_tables, st.context_lens, st.tb.NB, st.max_ctx) == 0
    assert pa.check_pairs(st.pairs, st.tb.NB) == 0
    slots = st.run_cache_ops(pa, fused=True)     # the launches bench.py times
    assert pa.check_slots(slots) == 0
    out = st.multi(pa, partition=part) if spec.chunk else st.decode(pa, partition=part)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), st.tb.slots)
    assert np.array_equal(host_bits(st.k_cache), st.k_after)
    assert np.array_equal(host_bits(st.v_cache), st.v_after)
    return st, out


@pytest.mark.parametrize("name", ["7b", "13b", "gqa", "gqa_d64", "gqa_f32", "cow", "prefix",
                                  "13b_verify4", "gqa_short"])
def test_full_config_whole_output(pa, name):
    st, out = run_step(pa, name)
    say(f"    oracle over the whole output {tuple(out.shape)}")
    expect = st.oracle_decode()
    got = out.float().cpu().numpy().astype(np.float64)
    assert got.shape == expect.shape
    err = float(np.max(np.abs(got - expect)))
    say(f"    whole-output max abs err {err:.3e} (tol {TOL[st.spec.dtype]})")
    record_parity(f"{name} (pa_decode/pa_multi_query, {got.shape[0]}x{got.shape[1]} rows)", err,
                  TOL[st.spec.dtype])
    assert err <= TOL[st.spec.dtype]


@pytest.mark.parametrize("name", ["gqa_chunk512", "gqa_chunk512_d64"])
def test_full_config_chunk512_longest_and_shortest(pa, name):
    st, out = run_step(pa, name)
    cl = st.tb.context_lens
    qs = st.tb.query_start
    order = np.argsort(cl, kind="stable")
    seqs = sorted(set(order[:4].tolist()) | set(order[-4:].tolist()))
    Hq = st.spec.Hq
    rows = [r for s in seqs for r in range(int(qs[s]), int(qs[s + 1]))]
    pairs = [(r, h) for r in rows for h in range(Hq)]
    say(f"    oracle over sequences {seqs} (contexts {cl[seqs].tolist()}): "
        f"{len(rows)} rows x {Hq} heads")
    expect = st.oracle_decode(pairs=pairs)
    got = out.float().cpu().numpy().astype(np.float64)
    got = got[np.asarray(rows)].reshape(len(rows) * Hq, -1)
    err = float(np.max(np.abs(got - expect)))
    say(f"    max abs err {err:.3e} (tol {TOL[st.spec.dtype]})")
    record_parity(f"{name} (pa_multi_query, every row of 8 of 16 sequences)", err,
                  TOL[st.spec.dtype])
    assert err <= TOL[st.spec.dtype]
    # the rest of the rows: finite, and (a convex combination of N(0,1) bf16
    # V rows) inside the range of the pool's values
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    assert np.abs(o).max() <= 8.0
