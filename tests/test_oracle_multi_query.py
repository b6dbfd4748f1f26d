"""Pins for the fp64 multi-query (causal chunk) oracle, CPU only.

Several new tokens per sequence, each attending to every position up to its
own: the look-back rule of "vLLM & PagedAttention" (completesystemdesign.dev),
section 01 (a new token looks back at all earlier tokens' keys and values),
applied to each token of a chunk; paging only moves rows ("Why OS Virtual
Memory Paging Saved LLM Inference", a8q9.cn, section 2). The oracle is tied to
the textbook causal attention written out densely, to torch's SDPA with an
explicit causal mask, to closed forms and to block-permutation invariance.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import dense

from test_oracle_decode import bf16_bits, contiguous_case, widen


def chunk_layout(rng, lens, max_new):
    """Random n_s in [0, min(max_new, ctx_s)] and the matching query_start."""
    n = [int(rng.integers(0, min(max_new, L) + 1)) for L in lens]
    qs = np.zeros(len(lens) + 1, np.int32)
    qs[1:] = np.cumsum(n)
    return n, qs


def dense_causal(qrows, K, V, first_pos, scale):
    """Textbook causal attention of a chunk: row i (position first_pos + i)
    sees K/V rows 0 .. first_pos + i. qrows [n, D]; K, V [L, D] in float64."""
    n = qrows.shape[0]
    x = float(scale) * (qrows @ K.T)                       # [n, L]
    pos = first_pos + np.arange(n)[:, None]
    allowed = np.arange(K.shape[0])[None, :] <= pos
    x = np.where(allowed, x, -np.inf)
    w = np.exp(x - x.max(axis=1, keepdims=True))
    return (w @ V) / w.sum(axis=1, keepdims=True)


def make_case(seed, lens, Hq, Hkv, D, dtype, max_new):
    rng = np.random.default_rng(seed)
    _, kpool, vpool, bt, cl, dense_kv = contiguous_case(rng, lens, Hq, Hkv, D, dtype)
    n, qs = chunk_layout(rng, lens, max_new)
    Tq = int(qs[-1])
    conv = bf16_bits if dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    q = conv(rng.standard_normal((Tq, Hq, D)))
    return q, kpool, vpool, bt, cl, qs, n, dense_kv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(8, 2, 2), (64, 4, 4), (128, 8, 2), (64, 8, 1)])
def test_identity_table_equals_dense_causal(oracle_mod, dtype, D, Hq, Hkv):
    lens = [1, 5, 16, 17, 40, 77]
    q, kp, vp, bt, cl, qs, n, dkv = make_case(7 + D + Hq, lens, Hq, Hkv, D, dtype, max_new=20)
    scale = 1.0 / np.sqrt(D)
    got = oracle.multi_query(q, kp, vp, bt, cl, qs, scale)
    G = Hq // Hkv
    for s, L in enumerate(lens):
        Ks, Vs = dkv[s]
        rows = slice(qs[s], qs[s + 1])
        for h in range(Hq):
            want = dense_causal(widen(q[rows, h]), widen(Ks[h // G]), widen(Vs[h // G]),
                                L - n[s], np.float32(scale))
            np.testing.assert_allclose(got[rows, h], want, rtol=0, atol=1e-12)


def test_against_torch_sdpa_with_causal_mask(oracle_mod):
    lens = [30, 64, 100]
    Hq = Hkv = 4
    D = 32
    q, kp, vp, bt, cl, qs, n, dkv = make_case(99, lens, Hq, Hkv, D, "f32", max_new=30)
    scale = 1.0 / np.sqrt(D)
    got = oracle.multi_query(q, kp, vp, bt, cl, qs, scale)
    for s, L in enumerate(lens):
        if n[s] == 0:
            continue
        Ks, Vs = dkv[s]
        rows = slice(qs[s], qs[s + 1])
        qt = torch.from_numpy(widen(q[rows]).transpose(1, 0, 2).copy())       # [H, n, D]
        kt = torch.from_numpy(widen(Ks))                                       # [H, L, D]
        vt = torch.from_numpy(widen(Vs))
        mask = torch.arange(L)[None, :] <= (L - n[s] + torch.arange(n[s]))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)))
        np.testing.assert_allclose(got[rows], ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_whole_prompt_chunk_is_causal_self_attention(oracle_mod):
    """A chunk covering the whole context (prefill from scratch): the first row
    sees only token 0, so it returns v_0 exactly; every row matches the dense
    causal form."""
    lens = [48, 9]
    Hq = Hkv = 2
    D = 16
    rng = np.random.default_rng(5)
    _, kp, vp, bt, cl, dkv = contiguous_case(rng, lens, Hq, Hkv, D, "f32")
    qs = np.array([0, 48, 57], np.int32)
    q = rng.standard_normal((57, Hq, D)).astype(np.float32)
    got = oracle.multi_query(q, kp, vp, bt, cl, qs, 0.25)
    for s, L in enumerate(lens):
        Ks, Vs = dkv[s]
        for h in range(Hq):
            assert np.array_equal(got[qs[s], h], widen(Vs[h][0]))
            want = dense_causal(widen(q[qs[s]:qs[s + 1], h]), widen(Ks[h]), widen(Vs[h]), 0,
                                np.float32(0.25))
            np.testing.assert_allclose(got[qs[s]:qs[s + 1], h], want, rtol=0, atol=1e-12)


def test_block_permutation_invariance_bitwise(oracle_mod):
    lens = [33, 70, 5]
    q, kp, vp, bt, cl, qs, n, _ = make_case(11, lens, 4, 2, 64, "bf16", max_new=12)
    base = oracle.multi_query(q, kp, vp, bt, cl, qs, 0.125)
    NB = kp.shape[0]
    perm = np.random.default_rng(3).permutation(NB)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], bt).astype(np.int32)
    again = oracle.multi_query(q, kp2, vp2, bt2, cl, qs, 0.125)
    assert np.array_equal(base, again)


def test_chunk_longer_than_context_is_an_error(oracle_mod):
    lens = [4]
    rng = np.random.default_rng(0)
    _, kp, vp, bt, cl, _ = contiguous_case(rng, lens, 1, 1, 8, "f32")
    q = np.zeros((5, 1, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.multi_query(q, kp, vp, bt, cl, np.array([0, 5], np.int32), 0.5)


def test_one_token_chunks_match_decode(oracle_mod):
    """Consistency with the decode entry point (same definition, n_s = 1)."""
    lens = [1, 17, 100]
    rng = np.random.default_rng(21)
    q, kp, vp, bt, cl, _ = contiguous_case(rng, lens, 4, 2, 64, "f32")
    qs = np.arange(len(lens) + 1, dtype=np.int32)
    a = oracle.multi_query(q, kp, vp, bt, cl, qs, 0.125)
    b = oracle.decode(q, kp, vp, bt, cl, 0.125)
    assert np.array_equal(a, b)


def test_sampled_pairs_match_full(oracle_mod):
    lens = [40, 90]
    q, kp, vp, bt, cl, qs, n, _ = make_case(17, lens, 4, 2, 64, "f32", max_new=10)
    full = oracle.multi_query(q, kp, vp, bt, cl, qs, 0.125)
    pairs = [(int(qs[-1]) - 1, 3), (0, 0), (int(qs[1]), 1)]
    part = oracle.multi_query(q, kp, vp, bt, cl, qs, 0.125, pairs=pairs)
    for i, (j, h) in enumerate(pairs):
        assert np.array_equal(part[i], full[j, h])
