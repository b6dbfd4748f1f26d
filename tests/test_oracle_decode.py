"""Pins for the fp64 decode oracle (oracle/pa_oracle.c), CPU only.

Each test ties the oracle to something other than itself: the textbook dense
definition, a library routine, a closed form, or an invariant the pages state
(blocks may live anywhere in physical memory and be shared, and attention
still comes out the same).
"""

import math

import numpy as np
import pytest
import torch

from oracle import blockmgr, cache_ops, dense

RNG_SEED = 1234


# ---------------------------------------------------------------- helpers
def bf16_bits(x):
    """float array -> raw bf16 bits (uint16), round to nearest even (via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(bits_or_f32):
    a = np.asarray(bits_or_f32)
    if a.dtype == np.uint16:
        return dense.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def contiguous_case(rng, lens, Hq, Hkv, D, dtype, bs=16):
    """Per-sequence dense K/V laid into a pool with the identity block table.

    Sequence s owns blocks off_s .. off_s + nb_s - 1 in order. Returns the
    paged inputs and the dense per-sequence K/V [Hkv, L, D] (as element bits).
    """
    B = len(lens)
    nbs = [max(1, -(-L // bs)) for L in lens]
    NB = sum(nbs)
    MB = max(nbs)
    conv = bf16_bits if dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    q = conv(rng.standard_normal((B, Hq, D)))
    kpool = conv(rng.standard_normal((NB, Hkv, bs, D)))
    vpool = conv(rng.standard_normal((NB, Hkv, bs, D)))
    bt = np.full((B, MB), -1, np.int32)
    dense_kv = []
    off = 0
    for s, L in enumerate(lens):
        nb = nbs[s]
        bt[s, :nb] = np.arange(off, off + nb)
        # [nb, Hkv, bs, D] -> [Hkv, nb*bs, D] -> first L rows
        Ks = kpool[off:off + nb].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :L]
        Vs = vpool[off:off + nb].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :L]
        dense_kv.append((Ks, Vs))
        off += nb
    return q, kpool, vpool, bt, np.asarray(lens, np.int32), dense_kv


def dense_reference(q, dense_kv, Hq, Hkv, scale):
    B = q.shape[0]
    D = q.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for s in range(B):
        Ks, Vs = dense_kv[s]
        for h in range(Hq):
            out[s, h] = dense.attention(widen(q[s, h]), widen(Ks[h // G]), widen(Vs[h // G]), np.float32(scale))
    return out


# ---------------------------------------------------------------- pins
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(8, 2, 2), (64, 8, 8), (128, 4, 2), (128, 8, 1), (64, 16, 2)])
def test_identity_table_equals_dense_numpy(oracle_mod, dtype, D, Hq, Hkv):
    rng = np.random.default_rng(RNG_SEED + D + Hq)
    lens = [1, 15, 16, 17, 40, 100]
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, lens, Hq, Hkv, D, dtype)
    scale = 1.0 / math.sqrt(D)
    got = oracle_mod.decode(q, kp, vp, bt, cl, scale)
    ref = dense_reference(q, dkv, Hq, Hkv, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_tiny_config_equals_torch_sdpa_f64(oracle_mod):
    """Tiny shape (4 seqs, 8 heads, D=64, contexts {1,17,100,250}) against
    torch's scaled_dot_product_attention in float64 on the CPU."""
    rng = np.random.default_rng(7)
    lens = [1, 17, 100, 250]
    H, D = 8, 64
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, lens, H, H, D, "f32")
    scale = 1.0 / math.sqrt(D)
    got = oracle_mod.decode(q, kp, vp, bt, cl, scale)
    for s, L in enumerate(lens):
        Ks, Vs = dkv[s]
        qt = torch.from_numpy(q[s].astype(np.float64)).reshape(1, H, 1, D)
        kt = torch.from_numpy(Ks.astype(np.float64)).reshape(1, H, L, D)
        vt = torch.from_numpy(Vs.astype(np.float64)).reshape(1, H, L, D)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=float(np.float32(scale))).reshape(H, D).numpy()
        assert np.max(np.abs(got[s] - ref)) <= 1e-12


def test_gqa_head_grouping_against_sdpa(oracle_mod):
    """Query head h reads kv head h // G: compare with SDPA on repeated kv heads."""
    rng = np.random.default_rng(11)
    lens = [33, 70]
    Hq, Hkv, D = 8, 2, 32
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, lens, Hq, Hkv, D, "f32")
    got = oracle_mod.decode(q, kp, vp, bt, cl, 0.25)
    for s, L in enumerate(lens):
        Ks, Vs = dkv[s]
        kt = torch.from_numpy(Ks.astype(np.float64)).repeat_interleave(Hq // Hkv, 0).reshape(1, Hq, L, D)
        vt = torch.from_numpy(Vs.astype(np.float64)).repeat_interleave(Hq // Hkv, 0).reshape(1, Hq, L, D)
        qt = torch.from_numpy(q[s].astype(np.float64)).reshape(1, Hq, 1, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.25).reshape(Hq, D).numpy()
        assert np.max(np.abs(got[s] - ref)) <= 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_permutation_invariance_bitwise(oracle_mod, dtype):
    """Moving every physical block elsewhere (and remapping the tables) leaves
    the output bit-for-bit unchanged: blocks may sit anywhere in memory."""
    rng = np.random.default_rng(21)
    lens = [5, 16, 31, 64, 129]
    q, kp, vp, bt, cl, _ = contiguous_case(rng, lens, 4, 4, 64, dtype)
    NB = kp.shape[0]
    extra = 9  # room to move blocks to ids the original never used
    perm = rng.permutation(NB + extra)[:NB]
    kp2 = np.full((NB + extra,) + kp.shape[1:], 0, kp.dtype)
    vp2 = np.full_like(kp2, 0)
    kp2[perm] = kp
    vp2[perm] = vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    a = oracle_mod.decode(q, kp, vp, bt, cl, 0.125)
    b = oracle_mod.decode(q, kp2, vp2, bt2, cl, 0.125)
    assert np.array_equal(a, b)


def test_cow_shared_equals_private_copies_bitwise(oracle_mod):
    """Samples that share prompt blocks (reference counted, copy-on-write)
    give the same outputs as samples each holding private copies."""
    rng = np.random.default_rng(31)
    bs, Hkv, D = 16, 2, 16
    NB = 64
    prompt_len = 37  # last prompt block partly filled -> copy-on-write
    samples = 4
    tails = [1, 3, 20, 2]
    bm = blockmgr.BlockManager(NB, bs, rng.permutation(NB))
    parent = bm.add_seq()
    prompt_slots, _ = bm.append(parent, prompt_len)
    seqs = [parent] + [bm.fork(parent) for _ in range(samples - 1)]
    kp = bf16_bits(rng.standard_normal((NB, Hkv, bs, D)))
    vp = bf16_bits(rng.standard_normal((NB, Hkv, bs, D)))
    all_pairs = []
    writes = []
    for i, sid in enumerate(seqs):
        slots, pairs = bm.append(sid, tails[i])
        all_pairs += pairs
        writes.append(slots)
    assert len(all_pairs) == samples - 1          # every writer but the last copies
    cache_ops.copy_blocks(kp, vp, all_pairs)
    T = sum(tails)
    kn = bf16_bits(rng.standard_normal((T, Hkv, D)))
    vn = bf16_bits(rng.standard_normal((T, Hkv, D)))
    cache_ops.write_kv(kp, vp, kn, vn, [s for w in writes for s in w])
    MB = max(len(bm.block_table(s)) for s in seqs)
    bt = np.asarray(bm.tables_array(seqs, MB), np.int32)
    cl = np.asarray([bm.seq_len(s) for s in seqs], np.int32)
    q = bf16_bits(rng.standard_normal((samples, 4, D)))
    shared = oracle_mod.decode(q, kp, vp, bt, cl, 0.25)

    # private version: give every sample its own copy of every shared block
    kp2 = np.concatenate([kp, np.zeros((samples * MB,) + kp.shape[1:], kp.dtype)])
    vp2 = np.concatenate([vp, np.zeros_like(kp2[NB:])])
    bt2 = bt.copy()
    nxt = NB
    for s in range(samples):
        for j in range(MB):
            b = bt[s, j]
            if b >= 0 and (bt == b).sum() > 1:
                kp2[nxt] = kp[b]
                vp2[nxt] = vp[b]
                bt2[s, j] = nxt
                nxt += 1
    assert nxt > NB  # the prompt's full blocks really were shared
    private = oracle_mod.decode(q, kp2, vp2, bt2, cl, 0.25)
    assert np.array_equal(shared, private)


def test_single_token_returns_its_value_exactly(oracle_mod):
    rng = np.random.default_rng(41)
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, [1, 1, 1], 4, 4, 64, "bf16")
    out = oracle_mod.decode(q, kp, vp, bt, cl, 0.3)
    for s in range(3):
        assert np.array_equal(out[s], widen(dkv[s][1][:, 0, :]))


def test_zero_query_or_equal_keys_gives_mean(oracle_mod):
    rng = np.random.default_rng(51)
    lens = [3, 17, 50]
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, lens, 2, 2, 16, "f32")
    out = oracle_mod.decode(np.zeros_like(q), kp, vp, bt, cl, 0.5)
    for s in range(3):
        assert np.max(np.abs(out[s] - widen(dkv[s][1]).mean(axis=1))) <= 1e-13
    # equal keys: every row of every block of K is the same vector
    kp_eq = np.broadcast_to(kp[0:1, :, 0:1, :], kp.shape).copy()
    out = oracle_mod.decode(q, kp_eq, vp, bt, cl, 0.5)
    for s in range(3):
        assert np.max(np.abs(out[s] - widen(dkv[s][1]).mean(axis=1))) <= 1e-13


def test_two_tokens_sigmoid_closed_form(oracle_mod):
    rng = np.random.default_rng(61)
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, [2], 1, 1, 8, "f32")
    scale = np.float32(0.7)
    out = oracle_mod.decode(q, kp, vp, bt, cl, scale)[0, 0]
    K, V = widen(dkv[0][0][0]), widen(dkv[0][1][0])
    x0 = float(scale) * float(widen(q[0, 0]) @ K[0])
    x1 = float(scale) * float(widen(q[0, 0]) @ K[1])
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))  # noqa: E731
    ref = sig(x0 - x1) * V[0] + sig(x1 - x0) * V[1]
    assert np.max(np.abs(out - ref)) <= 1e-14


def test_constant_values_and_affine_equivariance(oracle_mod):
    rng = np.random.default_rng(71)
    lens = [7, 40, 90]
    q, kp, vp, bt, cl, _ = contiguous_case(rng, lens, 2, 2, 32, "f32")
    c = np.float32(0.375)
    out = oracle_mod.decode(q, kp, np.full_like(vp, c), bt, cl, 0.2)
    assert np.max(np.abs(out - float(c))) <= 1e-14
    alpha, beta = np.float32(2.0), np.float32(-0.5)
    vp = (np.round(vp * 1024) / 1024).astype(np.float32)   # so alpha*v + beta is exact in fp32
    base = oracle_mod.decode(q, kp, vp, bt, cl, 0.2)
    aff = oracle_mod.decode(q, kp, (alpha * vp + beta).astype(np.float32), bt, cl, 0.2)
    assert np.max(np.abs(aff - (float(alpha) * base + float(beta)))) <= 1e-12


def test_split_context_lse_merge_equals_unsplit(oracle_mod):
    """Cutting the context into 32-token partitions, attending within each and
    merging with log-sum-exp weights equals attending over the whole."""
    rng = np.random.default_rng(81)
    L, D, P = 203, 16, 32
    q, kp, vp, bt, cl, dkv = contiguous_case(rng, [L], 1, 1, D, "f32")
    scale = np.float32(0.25)
    full = oracle_mod.decode(q, kp, vp, bt, cl, scale)[0, 0]
    qq = widen(q[0, 0])
    K, V = widen(dkv[0][0][0]), widen(dkv[0][1][0])
    outs, lses = [], []
    for start in range(0, L, P):
        n = min(P, L - start)
        # the partition as a sequence of its own: its blocks, its length
        sub_bt = bt[:, start // 16: start // 16 + (n + 15) // 16]
        o = oracle_mod.decode(q, kp, vp, np.ascontiguousarray(sub_bt), np.array([n], np.int32), scale)[0, 0]
        x = float(scale) * (K[start:start + n] @ qq)
        lses.append(x.max() + math.log(np.exp(x - x.max()).sum()))
        outs.append(o)
    M = max(lses)
    w = np.exp(np.asarray(lses) - M)
    merged = (w[:, None] * np.asarray(outs)).sum(0) / w.sum()
    assert np.max(np.abs(merged - full)) <= 1e-13 * max(1.0, np.abs(full).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_poison_in_unused_slots_and_entries(oracle_mod, dtype):
    """Slots past the context and table entries past the last block are never
    read: NaN there leaves every output finite and bit-identical."""
    rng = np.random.default_rng(91)
    lens = [1, 17, 33, 100]
    q, kp, vp, bt, cl, _ = contiguous_case(rng, lens, 2, 2, 32, dtype)
    clean = oracle_mod.decode(q, kp, vp, bt, cl, 0.2)
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32("nan")
    kp2, vp2 = kp.copy(), vp.copy()
    for s, L in enumerate(lens):
        nb = -(-L // 16)
        last = bt[s, nb - 1]
        kp2[last, :, L - (nb - 1) * 16:, :] = nan
        vp2[last, :, L - (nb - 1) * 16:, :] = nan
    bt2 = np.concatenate([bt, np.full((bt.shape[0], 3), -1, np.int32)], axis=1)
    poisoned = oracle_mod.decode(q, kp2, vp2, bt2, cl, 0.2)
    assert np.all(np.isfinite(poisoned))
    assert np.array_equal(clean, poisoned)


def test_empty_context_gives_zeros(oracle_mod):
    rng = np.random.default_rng(95)
    q, kp, vp, bt, cl, _ = contiguous_case(rng, [5, 9], 2, 2, 8, "f32")
    cl = np.array([0, 9], np.int32)
    out = oracle_mod.decode(q, kp, vp, bt, cl, 0.5)
    assert np.all(out[0] == 0.0)


def test_sampled_pairs_match_full(oracle_mod):
    rng = np.random.default_rng(97)
    q, kp, vp, bt, cl, _ = contiguous_case(rng, [20, 50, 3], 4, 2, 16, "bf16")
    full = oracle_mod.decode(q, kp, vp, bt, cl, 0.25)
    pairs = [(2, 3), (0, 0), (1, 2)]
    part = oracle_mod.decode(q, kp, vp, bt, cl, 0.25, pairs=pairs)
    for i, (s, h) in enumerate(pairs):
        assert np.array_equal(part[i], full[s, h])


def test_out_of_range_block_id_is_an_error(oracle_mod):
    rng = np.random.default_rng(99)
    q, kp, vp, bt, cl, _ = contiguous_case(rng, [20], 1, 1, 8, "f32")
    bt = bt.copy()
    bt[0, 1] = kp.shape[0]
    with pytest.raises(ValueError):
        oracle_mod.decode(q, kp, vp, bt, cl, 0.25)
