"""Pin of the oracle's bf16 decoding against torch's own bfloat16 type, CPU only.

Both oracle paths that read bf16 bits (the C widening inside oracle.decode /
oracle.multi_query, and dense.bf16_bits_to_f64) are the same idea: a bf16
value is the top half of an IEEE binary32. Here every one of the 65,536 bit
patterns is decoded by torch's bfloat16 -> float64 conversion, which shares no
code with either, and the oracle must give the same values:

  * dense.bf16_bits_to_f64 on the raw patterns;
  * oracle.decode with a one-token context per sequence, whose output is that
    token's V row exactly (softmax over one logit is 1; 1 * v / 1 = v), with
    the patterns placed in V;
  * the same through oracle.multi_query (one new token per sequence);
  * the query and key operands through the two-token closed form
    out[0] = sigmoid(scale * q_d * k_d) with one-hot V rows.
"""

import numpy as np
import torch

import oracle
from oracle import dense

D = 128


def all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def torch_widen(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def test_torch_reference_is_a_real_decoder():
    # a few patterns whose values are known by hand, so the torch side is
    # itself pinned: 1.0, -2.0, the smallest denormal, the largest finite, inf
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x7F80, 0x8000], np.uint16)
    want = [1.0, -2.0, 2.0**-133, (2 - 2.0**-7) * 2.0**127, np.inf, -0.0]
    got = torch_widen(bits)
    assert got.tolist() == want
    assert np.signbit(got[5])


def test_dense_widening_matches_torch_on_every_pattern():
    bits = all_patterns()
    with np.errstate(invalid="ignore"):     # signalling NaN patterns are widened too
        got = dense.bf16_bits_to_f64(bits)
    want = torch_widen(bits)
    nan = np.isnan(want)
    assert nan.sum() == 2 * 127                      # exponent all ones, mantissa != 0
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))   # signed zeros


def one_token_case():
    """512 sequences of one token each; sequence i's V row holds patterns
    128 i .. 128 i + 127. Non-finite patterns are kept: 1 * v / 1 keeps them."""
    bits = all_patterns()
    B = bits.size // D
    NB = B
    q = np.full((B, 1, D), 0x3F80, np.uint16)            # 1.0
    k = np.zeros((NB, 1, 16, D), np.uint16)
    v = np.zeros((NB, 1, 16, D), np.uint16)
    v[:, 0, 0, :] = bits.reshape(B, D)
    perm = np.random.default_rng(7).permutation(NB)        # blocks anywhere in the pool
    kp, vp = np.empty_like(k), np.empty_like(v)
    kp[perm], vp[perm] = k, v
    bt = perm.astype(np.int32).reshape(B, 1)
    ctx = np.ones(B, np.int32)
    return bits, q, kp, vp, bt, ctx


def check_rows(out, bits):
    # values equal (a sum that starts at 0 turns -0 into +0, the same value)
    got = out.reshape(-1)
    want = torch_widen(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_one_token_returns_torch_widened_v():
    bits, q, k, v, bt, ctx = one_token_case()
    out = oracle.decode(q, k, v, bt, ctx, 1.0)
    check_rows(out, bits)


def test_multi_query_one_token_returns_torch_widened_v():
    bits, q, k, v, bt, ctx = one_token_case()
    qs = np.arange(q.shape[0] + 1, dtype=np.int32)
    out = oracle.multi_query(q, k, v, bt, ctx, qs, 1.0)
    check_rows(out, bits)


def test_query_and_key_widening_through_two_token_closed_form():
    # token 0: key = e_d; token 1: key = 0. V rows one-hot: v0 = e_0, v1 = e_1.
    # Logits: x0 = scale * q_d, x1 = 0, so out[0] = sigmoid(scale * q_d) and
    # out[1] = 1 - out[0]. q_d runs over every finite pattern whose logit
    # stays where the sigmoid is informative, and the same with the roles of
    # q and k swapped (q = e_d, k_0 = the pattern).
    bits = all_patterns()
    vals = torch_widen(bits)
    keep = np.isfinite(vals) & (np.abs(vals) < 30.0)
    bits, vals = bits[keep], vals[keep]
    n = bits.size
    one = np.uint16(0x3F80)
    scale = 0.75
    for pattern_in_q in (True, False):
        q = np.zeros((n, 1, D), np.uint16)
        k = np.zeros((n, 1, 16, D), np.uint16)
        v = np.zeros((n, 1, 16, D), np.uint16)
        d = np.arange(n) % D
        if pattern_in_q:
            q[np.arange(n), 0, d] = bits
            k[np.arange(n), 0, 0, d] = one
        else:
            q[np.arange(n), 0, d] = one
            k[np.arange(n), 0, 0, d] = bits
        v[:, 0, 0, 0] = one
        v[:, 0, 1, 1] = one
        bt = np.arange(n, dtype=np.int32).reshape(n, 1)
        ctx = np.full(n, 2, np.int32)
        out = oracle.decode(q, k, v, bt, ctx, scale)
        x = np.float64(np.float32(scale)) * vals
        want0 = 1.0 / (1.0 + np.exp(-x))
        np.testing.assert_allclose(out[:, 0, 0], want0, rtol=1e-14, atol=0)
        np.testing.assert_allclose(out[:, 0, 1], 1.0 - want0, rtol=0, atol=1e-15)
