"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Cache bookkeeping (slot mapping, copy-on-write block copies, the cache write)
must be bit-exact over the whole pool; attention outputs must lie within
max-abs 2e-3 (fp32 I/O) or 1.5e-2 (bf16 I/O) of the fp64 oracle.
"""

import numpy as np
import pytest
import torch

from oracle import cache_ops
from paged_kv_cache_410_amd.workloads import Spec

from gpu_cases import TOL, Step, host_bits, max_abs_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


# Small workloads: several 16-token tiles, ragged tails, the edge cases.
SMALL = {
    "tiny": Spec("tiny", "f32", 4, 8, 8, 64, seed=0, lengths=("fixed", [1, 17, 100, 250]),
                 pool_blocks=64),
    "mha_bf16": Spec("mha_bf16", "bf16", 6, 4, 4, 128, seed=10, lengths=("uniform", 1, 700)),
    "mha_bf16_d64": Spec("mha_bf16_d64", "bf16", 5, 3, 3, 64, seed=11, lengths=("uniform", 1, 400)),
    "mha_f32_d128": Spec("mha_f32_d128", "f32", 4, 2, 2, 128, seed=12, lengths=("uniform", 1, 300)),
    "gqa_f32": Spec("gqa_f32", "f32", 3, 8, 2, 64, seed=13, lengths=("uniform", 1, 300)),
    "gqa8": Spec("gqa8", "bf16", 3, 16, 2, 128, seed=14, lengths=("uniform", 1, 3000)),
    "gqa2": Spec("gqa2", "bf16", 4, 4, 2, 128, seed=15, lengths=("uniform", 1, 600)),
    "gqa3": Spec("gqa3", "bf16", 3, 6, 2, 128, seed=16, lengths=("uniform", 1, 600)),
    "gqa16": Spec("gqa16", "bf16", 2, 16, 1, 128, seed=17, lengths=("uniform", 1, 900)),
    "gqa32": Spec("gqa32", "bf16", 2, 32, 1, 128, seed=18, lengths=("uniform", 1, 500)),
    "gqa_bf16_d64": Spec("gqa_bf16_d64", "bf16", 3, 8, 2, 64, seed=19, lengths=("uniform", 1, 300)),
    "exact_blocks": Spec("exact_blocks", "bf16", 4, 2, 2, 128, seed=20,
                         lengths=("fixed", [16, 32, 48, 512])),
    # unsplit contexts longer than one 64-block id chunk per wave (8 waves x 64 x 16 tokens)
    "long_mha": Spec("long_mha", "bf16", 2, 2, 2, 128, seed=23, lengths=("fixed", [9000, 20000])),
    "long_f32": Spec("long_f32", "f32", 2, 2, 2, 64, seed=24, lengths=("fixed", [8200, 17000])),
    "long_gqa": Spec("long_gqa", "bf16", 2, 16, 2, 128, seed=25, lengths=("fixed", [2100, 5000])),
    # more (sequence, head) items than 8 per compute unit: the unsplit vector
    # kernel with 8-wave workgroups, the 13B-shape batch's kernel
    "many_items": Spec("many_items", "bf16", 64, 40, 40, 128, seed=27,
                       lengths=("uniform", 1, 160)),
    "cow_small": Spec("cow_small", "bf16", 8, 4, 4, 128, seed=21, lengths=("cow",),
                      cow=dict(prompts=2, samples=4, prompt_len=96, r_max=15, tail_lo=1,
                               tail_hi=40)),
    "prefix_small": Spec("prefix_small", "bf16", 6, 4, 2, 128, seed=26, lengths=("prefix",),
                         prefix=dict(shared=80, tail_lo=1, tail_hi=40, vocab=50)),
    "cow_gqa": Spec("cow_gqa", "bf16", 6, 8, 2, 128, seed=22, lengths=("cow",),
                    cow=dict(prompts=2, samples=3, prompt_len=64, r_max=15, tail_lo=1,
                             tail_hi=30)),
    # the sharing workloads at head_dim 64, and 32 heads per kv head there
    # (two column tiles: the chunk kernel with 128-byte rows)
    "cow_small_d64": Spec("cow_small_d64", "bf16", 8, 4, 4, 64, seed=50, lengths=("cow",),
                          cow=dict(prompts=2, samples=4, prompt_len=96, r_max=15, tail_lo=1,
                                   tail_hi=40)),
    "prefix_small_d64": Spec("prefix_small_d64", "bf16", 6, 4, 2, 64, seed=51,
                             lengths=("prefix",),
                             prefix=dict(shared=80, tail_lo=1, tail_hi=40, vocab=50)),
    "cow_gqa_d64": Spec("cow_gqa_d64", "bf16", 6, 8, 2, 64, seed=52, lengths=("cow",),
                        cow=dict(prompts=2, samples=3, prompt_len=64, r_max=15, tail_lo=1,
                                 tail_hi=30)),
    "gqa32_d64": Spec("gqa32_d64", "bf16", 2, 32, 1, 64, seed=53, lengths=("uniform", 1, 500)),
    # the sharing workloads in fp32: one query head per kv head (the vector
    # kernel's tail pass), 4 and 2 heads per kv head (the fp32 matrix-core
    # kernel's group and tail passes)
    "cow_small_f32": Spec("cow_small_f32", "f32", 8, 4, 4, 128, seed=54, lengths=("cow",),
                          cow=dict(prompts=2, samples=4, prompt_len=96, r_max=15, tail_lo=1,
                                   tail_hi=40)),
    "cow_gqa_f32": Spec("cow_gqa_f32", "f32", 6, 8, 2, 128, seed=55, lengths=("cow",),
                        cow=dict(prompts=2, samples=3, prompt_len=64, r_max=15, tail_lo=1,
                                 tail_hi=30)),
    "prefix_small_f32_d64": Spec("prefix_small_f32_d64", "f32", 6, 4, 2, 64, seed=56,
                                 lengths=("prefix",),
                                 prefix=dict(shared=80, tail_lo=1, tail_hi=40, vocab=50)),
    # fp32 grouped heads on the matrix cores (v_mfma_f32_16x16x4_f32): 8 heads
    # per kv head; a full 16-column tile at head_dim 64; two tiles per kv head
    # (32 heads); unsplit rows longer than one 64-block id chunk per wave
    "gqa8_f32": Spec("gqa8_f32", "f32", 6, 16, 2, 128, seed=42, lengths=("uniform", 1, 1500)),
    "gqa16_f32_d64": Spec("gqa16_f32_d64", "f32", 2, 16, 1, 64, seed=43,
                          lengths=("uniform", 1, 700)),
    "gqa32_f32": Spec("gqa32_f32", "f32", 2, 32, 1, 128, seed=44, lengths=("uniform", 1, 500)),
    "long_gqa_f32": Spec("long_gqa_f32", "f32", 2, 8, 2, 128, seed=45,
                         lengths=("fixed", [2100, 9000])),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("fused", [False, True])
def test_cache_ops_bit_exact(pa, name, fused):
    say(f"[cache ops] {name} fused={fused}")
    st = Step(SMALL[name], oracle_full=False)
    slots = st.run_cache_ops(pa, fused=fused)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), st.tb.slots)
    assert np.array_equal(host_bits(st.k_cache), st.k_after)
    assert np.array_equal(host_bits(st.v_cache), st.v_after)


def test_append_kv_without_slot_output(pa):
    say("[append_kv] no slot output")
    st = Step(SMALL["cow_gqa"], oracle_full=False)
    assert st.run_cache_ops(pa, fused=True, want_slots=False) is None
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(st.k_cache), st.k_after)
    assert np.array_equal(host_bits(st.v_cache), st.v_after)


def test_append_kv_edge_cases(pa):
    # positions and tables that give no slot (-1) or a slot past the pool: the
    # slot output matches the oracle's slot mapping, and nothing is written for
    # them. Entries 2^28 + 1 and (2^31 - 16) / 16 + 1 would overflow an int32
    # slot number: no slot. (2^31 - 16) / 16 itself is a valid slot number
    # past the pool: reported, not written.
    say("[append_kv] edges")
    NB, Hkv, D = 6, 2, 64
    big = (2**31 - 1 - 15) // 16
    bt_h = np.array([[5, -1, 7], [2, 3, 4], [2**28 + 1, big, big + 1]], np.int32)
    pos_h = np.array([0, 17, 47, 48, -1, 33, 20, 40, 3, 20, 40, 5], np.int32)
    seq_h = np.array([0, 0, 1, 1, 1, 3, 1, 0, 2, 2, 2, -1], np.int32)
    bt = torch.from_numpy(bt_h).to("cuda")
    pos = torch.from_numpy(pos_h).to("cuda")
    seq = torch.from_numpy(seq_h).to("cuda")
    T = pos.shape[0]
    gen = torch.Generator().manual_seed(5)
    k_new = torch.randn(T, Hkv, D, generator=gen).to("cuda")
    v_new = torch.randn(T, Hkv, D, generator=gen).to("cuda")
    k = torch.zeros(NB, Hkv, 16, D, device="cuda")
    v = torch.zeros_like(k)
    slots = torch.empty(T, dtype=torch.int32, device="cuda")
    pa.append_kv(k_new, v_new, k, v, bt, pos, seq_ids=seq, slots_out=slots)
    expect = cache_ops.slot_mapping(bt_h, pos_h, 16, seq_ids=seq_h)
    assert expect.tolist() == [80, -1, 4 * 16 + 15, -1, -1, -1, 3 * 16 + 4, 7 * 16 + 8,
                               -1, big * 16 + 4, -1, -1]
    assert slots.cpu().numpy().tolist() == expect.tolist()
    assert pa.slot_mapping(bt, pos, seq_ids=seq).cpu().numpy().tolist() == expect.tolist()
    kk = np.zeros((NB, Hkv, 16, D), np.float32)
    vv = np.zeros_like(kk)
    inside = np.where(expect < NB * 16, expect, -1)   # slots past the pool: not written
    cache_ops.write_kv(kk, vv, k_new.cpu().numpy(), v_new.cpu().numpy(), inside)
    assert np.array_equal(host_bits(k), kk.view(np.uint32))
    assert np.array_equal(host_bits(v), vv.view(np.uint32))


def test_copy_blocks_alone_bit_exact(pa):
    say("[copy_blocks] cow_small")
    st = Step(SMALL["cow_small"], oracle_full=False)
    assert len(st.tb.pairs) > 0
    pa.copy_blocks(st.k_cache, st.v_cache, st.pairs)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(st.k_cache), st.k_copied)
    assert np.array_equal(host_bits(st.v_cache), st.v_copied)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("partition", [None, 0, 16, 64, 256, 512, 1024])
def test_decode_matches_oracle(pa, name, partition):
    spec = SMALL[name]
    say(f"[decode] {name} partition={partition}")
    st = Step(spec, poison=True)
    st.run_cache_ops(pa)
    out = st.decode(pa, partition=partition)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o)), "NaN-poisoned unused slots leaked into the output"
    err = max_abs_err(out, st.expect)
    say(f"    max abs err {err:.3e} (tol {TOL[spec.dtype]})")
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("name", ["mha_bf16", "gqa8", "tiny", "cow_small", "prefix_small",
                                  "gqa8_f32"])
def test_cache_policy_gives_identical_bits(pa, name):
    """Streaming and cached tile loads (PA_KV_SHARED) move the same bits."""
    say(f"[cache policy] {name}")
    st = Step(SMALL[name], oracle_full=False)
    st.run_cache_ops(pa)
    for part in (0, 64):
        a = st.decode(pa, partition=part, shared_kv=False)
        b = st.decode(pa, partition=part, shared_kv=True)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), part


def test_decode_deterministic_and_permutation_invariant(pa):
    """Same inputs twice -> same bits; physical blocks moved elsewhere (tables
    remapped) -> same bits: the arithmetic order never depends on block ids."""
    say("[decode invariance] gqa8 / mha_bf16 / gqa8_f32")
    for name, part in (("mha_bf16", 64), ("gqa8", 512), ("gqa8", 0), ("gqa8_f32", 64),
                       ("gqa8_f32", 0)):
        st = Step(SMALL[name], oracle_full=False)
        st.run_cache_ops(pa)
        a = st.decode(pa, partition=part).clone()
        b = st.decode(pa, partition=part).clone()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        NB = st.tb.NB
        perm = torch.from_numpy(np.random.default_rng(5).permutation(NB)).to(torch.int64).cuda()
        k2 = torch.empty_like(st.k_cache)
        v2 = torch.empty_like(st.v_cache)
        k2[perm] = st.k_cache
        v2[perm] = st.v_cache
        bt = st.block_tables.to(torch.int64)
        bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32).contiguous()
        c = pa.decode(st.q, k2, v2, bt2, st.context_lens, st.spec.scale, st.max_ctx, partition=part)
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("name", ["cow_small", "prefix_small"])
def test_decode_shared_blocks_equal_private_copies(pa, name):
    """Blocks shared by forks (copy-on-write) or across requests (prefix
    cache) give the bits that private copies of them give."""
    say(f"[decode shared vs private] {name}")
    st = Step(SMALL[name], oracle_full=False)
    st.run_cache_ops(pa)
    shared = st.decode(pa, partition=32).clone()
    bt = st.tb.block_tables.copy()
    k2 = [st.k_cache]
    v2 = [st.v_cache]
    nxt = st.tb.NB
    extra = []
    for s in range(bt.shape[0]):
        for j in range(bt.shape[1]):
            b = bt[s, j]
            if b >= 0 and (st.tb.block_tables == b).sum() > 1:
                extra.append(int(b))
                bt[s, j] = nxt
                nxt += 1
    assert extra
    idx = torch.tensor(extra, device="cuda")
    k2 = torch.cat([st.k_cache, st.k_cache[idx]]).contiguous()
    v2 = torch.cat([st.v_cache, st.v_cache[idx]]).contiguous()
    private = pa.decode(st.q, k2, v2, torch.from_numpy(bt).cuda(), st.context_lens,
                        st.spec.scale, st.max_ctx, partition=32)
    assert torch.equal(shared.view(torch.int16), private.view(torch.int16))


@pytest.mark.parametrize("name", ["mha_bf16", "gqa8_f32"])
def test_decode_bad_entries_give_nan_rows_only(pa, name):
    """A context beyond max_ctx or a block id outside the pool poisons only its
    own sequence's rows (NaN), reads nothing out of bounds, and leaves the other
    rows as they were."""
    say(f"[decode bad entries] {name}")
    st = Step(SMALL[name])
    st.run_cache_ops(pa)
    good = {part: st.decode(pa, partition=part).float().cpu() for part in (0, 64)}
    bt = st.block_tables.clone()
    bt[1, 0] = st.tb.NB + 5                  # out of range
    bt[3, 0] = -7                            # negative
    cl = st.context_lens.clone()
    cl[4] = st.max_ctx + 1                   # beyond the host bound
    for part in (0, 64):
        out = pa.decode(st.q, st.k_cache, st.v_cache, bt, cl, st.spec.scale, st.max_ctx,
                        partition=part).float().cpu()
        for s in (1, 3, 4):
            if int(st.tb.context_lens[s]) > 0 or s == 4:
                assert torch.isnan(out[s]).all(), (s, part)
        for s in (0, 2, 5):   # the intact sequences keep their bits
            assert torch.equal(out[s], good[part][s]), (s, part)


def test_decode_empty_context_gives_zeros(pa):
    say("[decode empty context]")
    st = Step(SMALL["mha_bf16"], oracle_full=False)
    st.run_cache_ops(pa)
    cl = st.context_lens.clone()
    cl[2] = 0
    for part in (0, 64):
        out = pa.decode(st.q, st.k_cache, st.v_cache, st.block_tables, cl, st.spec.scale,
                        st.max_ctx, partition=part)
        assert torch.count_nonzero(out[2].float()) == 0


def test_slot_mapping_edge_cases(pa):
    say("[slot mapping edges]")
    big = (2**31 - 1 - 15) // 16
    bt_h = np.array([[5, -1, 7], [2, 3, 4], [2**28 + 1, big, big + 1]], np.int32)
    pos_h = np.array([0, 17, 47, 48, -1, 33, 0, 31, 32, 15], np.int32)
    seq_h = np.array([0, 0, 1, 1, 1, 3, 2, 2, 2, -4], np.int32)
    got = pa.slot_mapping(torch.from_numpy(bt_h).to("cuda"), torch.from_numpy(pos_h).to("cuda"),
                          seq_ids=torch.from_numpy(seq_h).to("cuda")).cpu().numpy()
    expect = cache_ops.slot_mapping(bt_h, pos_h, 16, seq_ids=seq_h)
    assert expect.tolist() == [80, -1, 4 * 16 + 15, -1, -1, -1, -1, 2**31 - 1, -1, -1]
    assert got.tolist() == expect.tolist()


@pytest.mark.parametrize("name,partition", [("gqa8", 64), ("mha_bf16", 0), ("cow_small", 128)])
def test_step_graph_replays_match_eager(pa, name, partition):
    # The step (copies, fused slot mapping + write, attention with its merge)
    # captured once as a HIP graph. Each replay starts from the pools the
    # first step saw (restored by eager copies between replays) and must give
    # the eager step's output bits, slots and pools. A repeated copy-on-write
    # step would not reproduce the pools: the last sharer writes into the
    # shared block, and the next copy carries its tail into the other copies,
    # in slots past their contexts.
    say(f"[graph replay] {name} partition={partition}")
    st = Step(SMALL[name], oracle_full=False)
    rows = st.q.shape[0]
    ws = torch.empty(max(1, pa.decode_workspace_bytes(rows, st.spec.Hq, st.spec.D, st.max_ctx,
                                                      partition)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q)
    slots = torch.empty(st.step_pos.shape[0], dtype=torch.int32, device="cuda")
    shared = pa.shares_blocks(st.tb.block_tables)
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()

    def step():
        if len(st.tb.pairs):
            pa.copy_blocks(st.k_cache, st.v_cache, st.pairs)
        pa.append_kv(st.k_new, st.v_new, st.k_cache, st.v_cache, st.block_tables, st.step_pos,
                     seq_ids=st.step_seq, slots_out=slots)
        pa.decode(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens, st.spec.scale,
                  st.max_ctx, partition=partition, out=out, workspace=ws, shared_kv=shared)

    def check(what):
        assert np.array_equal(slots.cpu().numpy(), st.tb.slots), what
        assert np.array_equal(host_bits(st.k_cache), st.k_after), what
        assert np.array_equal(host_bits(st.v_cache), st.v_after), what

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        st.k_cache.copy_(k0)
        st.v_cache.copy_(v0)
        out.fill_(float("nan"))
        slots.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        check(f"replay {i}")
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("f32", 1, 1, 64), ("bf16", 8, 1, 128)])
def test_decode_at_the_batch_limit(pa, dtype, Hq, Hkv, D):
    # 65535 sequences (the largest batch the ABI takes: one grid row each),
    # short ragged contexts including empty ones, blocks scattered over a
    # shuffled pool; every output row against the oracle.
    say(f"[batch limit] {dtype} Hq={Hq} Hkv={Hkv} D={D}")
    import oracle
    B = 65535
    rng = np.random.default_rng(41)
    cl = rng.integers(0, 41, B).astype(np.int32)
    nblk = (cl + 15) // 16
    NB = int(nblk.sum()) + 7
    MB = int(nblk.max())
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((B, MB), -1, np.int32)
    start = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    for j in range(MB):
        has = nblk > j
        bt[has, j] = perm[start[has] + j]
    if dtype == "f32":
        mk = lambda *s: rng.standard_normal(s, dtype=np.float32)  # noqa: E731
        tdt = torch.float32
    else:
        mk = lambda *s: (rng.standard_normal(s, dtype=np.float32).view(np.uint32) >> 16  # noqa: E731
                         ).astype(np.uint16) & np.uint16(0xFF7F)     # finite bf16 bits
        tdt = torch.bfloat16
    q, k, v = mk(B, Hq, D), mk(NB, Hkv, 16, D), mk(NB, Hkv, 16, D)
    dev = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16  # noqa: E731
                     else torch.from_numpy(a)).to("cuda")
    scale = 1.0 / np.sqrt(D)
    for part in (0, 16):
        out = pa.decode(dev(q), dev(k), dev(v), torch.from_numpy(bt).to("cuda"),
                        torch.from_numpy(cl).to("cuda"), scale, int(cl.max()), partition=part)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        expect = oracle.decode(q, k, v, bt, cl, scale)
        assert np.all(got[cl == 0] == 0.0)
        assert max_abs_err(out, expect) <= TOL[dtype], part


def test_default_partition_policy(pa):
    """The library's split choice on this device: no split when the unsplit
    workgroups fill the GPU (at least 4 per compute unit), or the contexts
    are short: up to 512 tokens, or up to 2048 with grouped heads (the
    matrix-core kernels); else 512-token partitions."""
    say("[default partition]")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert pa.default_partition(cus // 2, 8, 8, 128, 32768) == 0       # enough workgroups
    assert pa.default_partition(4, 8, 8, 128, 512) == 0                # short contexts
    assert pa.default_partition(4, 40, 40, 128, 560) == 512            # one head per kv head
    assert pa.default_partition(128, 40, 8, 128, 2048) == 0            # grouped, short
    assert pa.default_partition(16, 32, 8, 64, 2048) == 0
    assert pa.default_partition(16, 32, 8, 128, 2049) == 512           # grouped, long
    assert pa.default_partition(16, 64, 8, 128, 32768) == 512
    assert pa.default_partition(cus // 2, 32, 8, 128, 8192) == 0       # grouped, 4 per CU
    assert pa.default_partition(cus // 2 - 1, 32, 8, 128, 8192) == 512
    assert pa.default_partition(cus // 8, 32, 32, 128, 8192) == 0      # 4 per CU
    assert pa.default_partition(cus // 16, 32, 32, 128, 8192) == 512
