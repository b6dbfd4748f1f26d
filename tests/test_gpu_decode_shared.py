"""GPU parity of pa_decode_shared: decode attention that reads each group's
shared blocks once for all the group's sequences, then each sequence's own
tokens, and merges the two partials.

Outputs must lie within max-abs 2e-3 (fp32) / 1.5e-2 (bf16) of the fp64 oracle
on the same inputs, as pa_decode's do. Unused pool slots are poisoned with NaN,
so a read past a context or outside the shared part would show.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_cases import TOL, Step, max_abs_err, oracle_view, record_parity, say
from test_gpu_parity import SMALL
from paged_kv_cache_410_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def groups_of(pa, st, max_group=None):
    G = st.spec.Hq // st.spec.Hkv
    mg = max_group or 16 // G
    gs, sh = pa.shared_groups(st.tb.block_tables, st.tb.context_lens, mg)
    return gs, sh, mg


def run_shared(pa, st, gs, sh, mg, partition, context_lens=None):
    cl = st.context_lens if context_lens is None else context_lens
    return pa.decode_shared(st.q, st.k_cache, st.v_cache, st.block_tables, cl,
                            torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda(),
                            st.spec.scale, st.max_ctx, mg, int(sh.max()), partition=partition)


@pytest.mark.parametrize("name", ["cow_small", "cow_gqa", "prefix_small", "mha_bf16", "gqa8",
                                  "long_mha", "cow_small_d64", "cow_gqa_d64", "prefix_small_d64",
                                  "mha_bf16_d64", "cow_small_f32", "cow_gqa_f32",
                                  "prefix_small_f32_d64", "gqa_f32", "mha_f32_d128"])
@pytest.mark.parametrize("partition", [0, 16, 48, 512])
def test_decode_shared_matches_oracle(pa, name, partition):
    spec = SMALL[name]
    st = Step(spec, poison=True)
    st.run_cache_ops(pa)
    gs, sh, mg = groups_of(pa, st)
    say(f"[decode_shared] {name} partition={partition} groups={len(gs) - 1} "
        f"shared={sorted(set(sh.tolist()))}")
    out = run_shared(pa, st, gs, sh, mg, partition)
    ref = st.decode(pa, partition=partition or None)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o)), "NaN-poisoned unused slots leaked into the output"
    err = max_abs_err(out, st.expect)
    say(f"    max abs err {err:.3e} (tol {TOL[spec.dtype]})")
    assert err <= TOL[spec.dtype]
    assert float((out.float() - ref.float()).abs().max()) <= TOL[spec.dtype]


@pytest.mark.parametrize("max_group", [1, 2, 3])
def test_decode_shared_smaller_groups(pa, max_group):
    st = Step(SMALL["cow_small"], poison=True)
    st.run_cache_ops(pa)
    gs, sh, mg = groups_of(pa, st, max_group)
    assert np.diff(gs).max() <= max_group
    out = run_shared(pa, st, gs, sh, mg, 32)
    torch.cuda.synchronize()
    assert max_abs_err(out, st.expect) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["cow_small", "cow_small_f32", "cow_gqa_f32"])
def test_decode_shared_empty_tails_and_contexts(pa, name):
    """A sequence whose whole context is shared (empty own part), and an empty
    sequence in a group of its own."""
    st = Step(SMALL[name], poison=True, oracle_full=False)
    st.run_cache_ops(pa)
    gs, sh, mg = groups_of(pa, st)
    cl = st.tb.context_lens.copy()
    members = [s for s in range(st.spec.B) if sh[s] > 0]
    cl[members[1]] = sh[members[1]]          # nothing of its own
    # a last, empty sequence alone: make the last group's last member a singleton
    last = st.spec.B - 1
    gs2 = np.concatenate([gs[:-1], [last, st.spec.B]]).astype(np.int32)
    sh2 = sh.copy()
    sh2[last] = 0
    cl[last] = 0
    expect = oracle.decode(oracle_view(st.q_bits), oracle_view(st.k_after),
                           oracle_view(st.v_after), st.tb.block_tables, cl, st.spec.scale)
    out = run_shared(pa, st, gs2, sh2, mg, 16, context_lens=torch.from_numpy(cl).cuda())
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.count_nonzero(o[last]) == 0
    assert np.all(np.isfinite(o))
    assert float(np.max(np.abs(o - expect))) <= TOL[st.spec.dtype]


@pytest.mark.parametrize("name", ["cow_small", "cow_small_f32", "cow_gqa_f32"])
def test_decode_shared_bad_shared_length_poisons_only_its_row(pa, name):
    st = Step(SMALL[name], oracle_full=False)
    st.run_cache_ops(pa)
    gs, sh, mg = groups_of(pa, st)
    good = run_shared(pa, st, gs, sh, mg, 0).float().cpu()
    s_bad = int(gs[0]) + 1                   # a member that is not its group's first
    bad = sh.copy()
    bad[s_bad] = 8                           # not a multiple of the block size
    out = run_shared(pa, st, gs, bad, mg, 0).float().cpu()
    assert torch.isnan(out[s_bad]).all()
    keep = [s for s in range(st.spec.B) if s != s_bad]
    assert torch.equal(out[keep], good[keep])


@pytest.mark.parametrize("name", ["cow", "prefix", "cow_gqa8"])
def test_decode_shared_full_config_whole_output(pa, name):
    """Full-size sharing workloads in the launch configuration the benchmark
    times (its groups, shared-part partition and cache flags): every output
    row against the oracle."""
    spec = workloads.CONFIGS[name]
    st = Step(spec, values_device="cuda", oracle_full=False)
    st.run_cache_ops(pa, fused=True)
    plan = pa.shared_plan(st.tb.block_tables, st.tb.context_lens, spec.Hq, spec.Hkv, 16)
    assert plan is not None
    gs, sh = plan["group_start"], plan["seq_shared"]
    say(f"[decode_shared full config] {name}: groups={len(gs) - 1} "
        f"shared={sorted(set(sh.tolist()))} partition={plan['partition']} "
        f"groups_overlap={plan['groups_overlap']} shared_kv={plan['shared_kv']}")
    gs_d, sh_d = torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda()
    assert pa.check_groups(gs_d, sh_d, st.block_tables, st.context_lens,
                           plan["max_group"]) == 0
    out = pa.decode_shared(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens, gs_d,
                           sh_d, spec.scale, st.max_ctx, plan["max_group"], plan["max_shared"],
                           partition=plan["partition"], shared_kv=plan["shared_kv"],
                           groups_overlap=plan["groups_overlap"])
    torch.cuda.synchronize()
    expect = st.oracle_decode()
    got = out.float().cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - expect)))
    say(f"    whole-output max abs err {err:.3e} (tol {TOL[spec.dtype]})")
    record_parity(f"{name} (pa_decode_shared, {got.shape[0]}x{got.shape[1]} rows)", err,
                  TOL[spec.dtype])
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("name", ["cow_small", "prefix_small", "cow_gqa", "cow_gqa_d64",
                                  "cow_gqa_f32"])
def test_decode_shared_cache_flags_give_identical_bits(pa, name):
    """PA_KV_SHARED and PA_KV_SHARED_GROUPS change how tiles are cached, never
    the result."""
    st = Step(SMALL[name], oracle_full=False)
    st.run_cache_ops(pa)
    gs, sh, mg = groups_of(pa, st)
    args = (st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
            torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda(), st.spec.scale,
            st.max_ctx, mg, int(sh.max()))
    outs = [pa.decode_shared(*args, partition=16, shared_kv=a, groups_overlap=b)
            for a in (False, True) for b in (False, True)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_check_groups_counts_violations(pa):
    """pa_check_groups: zero on the planner's groups; one per planted fault."""
    for name in ("cow_small", "prefix_small", "cow_gqa", "mha_bf16"):
        st = Step(SMALL[name], oracle_full=False)
        gs, sh, mg = groups_of(pa, st)
        assert pa.check_groups(torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda(),
                               st.block_tables, st.context_lens, mg) == 0, name
    st = Step(SMALL["cow_small"], oracle_full=False)
    gs, sh, mg = groups_of(pa, st)
    a = int(gs[0])
    cases = []
    bt = st.tb.block_tables.copy()
    bt[a + 1, 0] = bt[a + 1, 0] + 1            # a member's shared entry differs
    cases.append((gs, sh, bt, st.tb.context_lens, mg))
    sh2 = sh.copy()
    sh2[a + 2] -= 16                           # a member's shared length differs
    cases.append((gs, sh2, st.tb.block_tables, st.tb.context_lens, mg))
    cases.append((gs, sh, st.tb.block_tables, st.tb.context_lens, 2))   # groups too large
    cl = st.tb.context_lens.copy()
    cl[a + 3] = int(sh[a]) - 1                 # shared part beyond a member's context
    cases.append((gs, sh, st.tb.block_tables, cl, mg))
    expect = [1, 1, len(gs) - 1, 1]
    for (g_, s_, b_, c_, m_), e in zip(cases, expect):
        n = pa.check_groups(torch.from_numpy(np.ascontiguousarray(g_)).cuda(),
                            torch.from_numpy(np.ascontiguousarray(s_)).cuda(),
                            torch.from_numpy(np.ascontiguousarray(b_)).cuda(),
                            torch.from_numpy(np.ascontiguousarray(c_)).cuda(), m_)
        assert n == e, (n, e)


def fork_tree_batch(seed, Hq, Hkv, NB=600, D=128, dtype="bf16"):
    """Sequences of a random fork tree (roots, children, grandchildren), built
    with the oracle's block manager, in the order they were made: sharing of
    leading blocks at many depths, private tails of random length."""
    rng = np.random.default_rng(seed)
    bm = oracle.blockmgr.BlockManager(NB, 16, list(rng.permutation(NB)))
    seqs = []
    for _ in range(int(rng.integers(1, 4))):
        root = bm.add_seq()
        bm.append(root, int(rng.integers(1, 200)))
        family = [root]
        for _ in range(int(rng.integers(0, 6))):
            parent = family[int(rng.integers(0, len(family)))]
            child = bm.fork(parent)
            bm.append(child, int(rng.integers(0, 60)))
            family.append(child)
        for sq in family:                 # the root may also grow after its forks
            if rng.random() < 0.3:
                bm.append(sq, int(rng.integers(1, 30)))
        seqs += family
    if rng.random() < 0.5:
        seqs = [seqs[i] for i in rng.permutation(len(seqs))]   # interleaved families
    MB = max(len(bm.tables[s]) for s in seqs) + 1
    bt = np.full((len(seqs), MB), -1, np.int32)
    for i, s in enumerate(seqs):
        bt[i, :len(bm.tables[s])] = bm.tables[s]
    cl = np.array([bm.seq_len(s) for s in seqs], np.int32)
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.randn(NB, Hkv, 16, D, generator=g).to(dt)
    v = torch.randn(NB, Hkv, 16, D, generator=g).to(dt)
    q = torch.randn(len(seqs), Hq, D, generator=g).to(dt)
    return q, k, v, bt, cl


def host_view(t):
    """A pool or query tensor as the oracle takes it: bf16 as raw uint16
    bits, fp32 as values."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
@pytest.mark.parametrize("seed", list(range(8)))
def test_decode_shared_random_fork_trees(pa, seed, dtype, D):
    Hq, Hkv = (8, 8) if seed % 2 == 0 else (8, 2)
    q, k, v, bt, cl = fork_tree_batch(seed, Hq, Hkv, D=D, dtype=dtype)
    B = len(cl)
    expect = oracle.decode(host_view(q), host_view(k), host_view(v), bt, cl, 1 / np.sqrt(D))
    G = Hq // Hkv
    dev = torch.device("cuda")
    args = [t.to(dev) for t in (q, k, v)] + [torch.from_numpy(bt).to(dev),
                                              torch.from_numpy(cl).to(dev)]
    for max_group, partition in ((16 // G, 0), (2, 32), (3, 16)):
        gs, sh = pa.shared_groups(bt, cl, max_group)
        gs_d, sh_d = torch.from_numpy(gs).to(dev), torch.from_numpy(sh).to(dev)
        assert pa.check_groups(gs_d, sh_d, args[3], args[4], max_group) == 0
        out = pa.decode_shared(*args, gs_d, sh_d, 1 / np.sqrt(D), int(cl.max()), max_group,
                               int(sh.max()), partition=partition, shared_kv=True,
                               groups_overlap=True)
        torch.cuda.synchronize()
        err = max_abs_err(out, expect)
        say(f"[decode_shared fork tree] {dtype} D{D} seed={seed} B={B} groups={len(gs) - 1} "
            f"shared={sorted(set(sh.tolist()))[:6]} max_group={max_group} err={err:.2e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed", [11, 12, 13])
@pytest.mark.parametrize("max_group", [3, 4, 8])
def test_decode_shared_groups_past_one_tile(pa, seed, max_group, dtype):
    """Groups whose members x query heads exceed 16 columns per kv head (8
    query heads per kv head: 24, 32 and 64 columns) run their shared part on
    the chunk kernel in bf16, on one fp32 matrix-core workgroup per 16-column
    tile in fp32."""
    q, k, v, bt, cl = fork_tree_batch(seed, 16, 2, dtype=dtype)
    expect = oracle.decode(host_view(q), host_view(k), host_view(v), bt, cl, 1 / np.sqrt(128))
    dev = torch.device("cuda")
    gs, sh = pa.shared_groups(bt, cl, max_group)
    args = [t.to(dev) for t in (q, k, v)] + [torch.from_numpy(bt).to(dev),
                                              torch.from_numpy(cl).to(dev)]
    for partition in (0, 48, None):
        out = pa.decode_shared(*args, torch.from_numpy(gs).to(dev), torch.from_numpy(sh).to(dev),
                               1 / np.sqrt(128), int(cl.max()), max_group, int(sh.max()),
                               partition=partition)
        torch.cuda.synchronize()
        err = max_abs_err(out, expect)
        say(f"[decode_shared wide groups] {dtype} seed={seed} max_group={max_group} "
            f"sizes={np.diff(gs).tolist()} partition={partition} err={err:.2e}")
        assert np.all(np.isfinite(out.float().cpu().numpy()))
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,D", [(32, 128), (48, 64)])
@pytest.mark.parametrize("seed", [31, 32])
def test_decode_shared_more_than_16_heads_per_kv_head(pa, seed, Hq, D, dtype):
    """One kv head for 32 or 48 query heads (multi-query attention): the
    group pass takes 2 or 3 column tiles per member; the tail pass takes the
    vector kernel in bf16 and 2 or 3 fp32 matrix-core tiles in fp32."""
    q, k, v, bt, cl = fork_tree_batch(seed, Hq, 1, D=D, dtype=dtype)
    expect = oracle.decode(host_view(q), host_view(k), host_view(v), bt, cl, 1 / np.sqrt(D))
    dev = torch.device("cuda")
    args = [t.to(dev) for t in (q, k, v)] + [torch.from_numpy(bt).to(dev),
                                              torch.from_numpy(cl).to(dev)]
    for max_group, partition in ((1, 0), (3, 32), (4, None)):
        gs, sh = pa.shared_groups(bt, cl, max_group)
        out = pa.decode_shared(*args, torch.from_numpy(gs).to(dev), torch.from_numpy(sh).to(dev),
                               1 / np.sqrt(D), int(cl.max()), max_group, int(sh.max()),
                               partition=partition)
        torch.cuda.synchronize()
        err = max_abs_err(out, expect)
        say(f"[decode_shared {Hq}/1 heads] {dtype} D{D} seed={seed} max_group={max_group} "
            f"partition={partition} err={err:.2e}")
        assert np.all(np.isfinite(out.float().cpu().numpy()))
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,Hkv", [("bf16", 8), ("f32", 8), ("f32", 2)])
def test_decode_shared_malformed_groups_stay_in_bounds(pa, dtype, Hkv):
    """Group bounds outside the batch: the call completes (every read stays
    inside its buffer), and the rows of the intact groups are those of a
    well-formed call; the affected members' rows are undefined."""
    q, k, v, bt, cl = fork_tree_batch(5, 8, Hkv, dtype=dtype)
    gs, sh = pa.shared_groups(bt, cl, 4)
    assert len(gs) - 1 >= 3
    dev = torch.device("cuda")
    args = [t.to(dev) for t in (q, k, v)] + [torch.from_numpy(bt).to(dev),
                                              torch.from_numpy(cl).to(dev)]
    B = len(cl)
    ws_bytes = pa.decode_shared_workspace_bytes(B, 8, 128, int(sh.max()), 0)

    def run(g):
        ws = torch.full((max(ws_bytes, 4) // 4,), float("nan"), device=dev)
        return pa.decode_shared(*args, torch.from_numpy(g).to(dev), torch.from_numpy(sh).to(dev),
                                1 / np.sqrt(128), int(cl.max()), 4, int(sh.max()), partition=0,
                                workspace=ws.view(torch.uint8)).float().cpu()

    good = run(gs)
    bad_gs = gs.copy()
    bad_gs[1] = B + 5                         # groups 0 and 1 out of the batch
    out = run(bad_gs)
    torch.cuda.synchronize()
    intact = np.arange(int(gs[2]), B)
    assert torch.equal(out[intact], good[intact])


@pytest.mark.parametrize("name", ["cow_small", "prefix_small", "cow_gqa", "prefix_small_d64",
                                  "cow_gqa_f32", "prefix_small_f32_d64"])
def test_decode_shared_permutation_invariant_and_deterministic(pa, name):
    """The blocks relabelled by a random permutation of the pool (pools and
    tables alike) give bitwise the same outputs, as does a second run:
    nothing in the arithmetic order depends on physical block ids."""
    st = Step(SMALL[name], oracle_full=False)
    st.run_cache_ops(pa)
    gs, sh, mg = groups_of(pa, st)
    out1 = run_shared(pa, st, gs, sh, mg, 32)
    out2 = run_shared(pa, st, gs, sh, mg, 32)
    rng = np.random.default_rng(5)
    perm = rng.permutation(st.tb.NB)               # old block b -> new block perm[b]
    inv = np.argsort(perm)
    bt = st.tb.block_tables.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    idx = torch.from_numpy(inv).cuda()
    k2, v2 = st.k_cache[idx].contiguous(), st.v_cache[idx].contiguous()
    out3 = pa.decode_shared(st.q, k2, v2, torch.from_numpy(bt).cuda(), st.context_lens,
                            torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda(),
                            st.spec.scale, st.max_ctx, mg, int(sh.max()), partition=32)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
