"""GPU bit-exactness of the cache bookkeeping on payloads that float arithmetic
would change: quiet and signalling NaNs with payloads, infinities, signed
zeros and denormals, in bf16 and fp32.

The cache write puts each new token's K/V rows into the slot the block table
names, and a copy-on-write copy duplicates a block exactly ("Why OS Virtual
Memory Paging Saved LLM Inference" (a8q9.cn), section 2 "On-Demand
Allocation" and section 3 "Copy-on-Write for Prompt Sharing"). Both are moves
of bits, so the whole pool after pa_write_kv, pa_append_kv and pa_copy_blocks
must equal the oracle's numpy bit moves on the same inputs, every element.
"""

import numpy as np
import pytest
import torch

from oracle import cache_ops

from gpu_cases import host_bits, say

pytestmark = pytest.mark.gpu

SPECIAL = {
    # quiet NaNs with payloads, signalling NaNs, negative NaN, +-inf, -0, +0,
    # smallest and largest denormals of both signs, largest finite
    "bf16": [0x7FC1, 0x7F81, 0xFFC1, 0xFF81, 0x7FFF, 0x7F80, 0xFF80, 0x8000, 0x0000,
             0x0001, 0x8001, 0x007F, 0x807F, 0x7F7F],
    "f32": [0x7FC00001, 0x7F800001, 0xFFC00001, 0xFF800001, 0x7FFFFFFF, 0x7F800000,
            0xFF800000, 0x80000000, 0x00000000, 0x00000001, 0x80000001, 0x007FFFFF,
            0x807FFFFF, 0x7F7FFFFF],
}
BITS = {"bf16": (np.uint16, np.int16, torch.bfloat16), "f32": (np.uint32, np.int32, torch.float32)}


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def rand_bits(rng, dt, shape):
    """Uniform over every bit pattern (NaNs of every payload included), with the
    special patterns at the head of each row."""
    u, _, _ = BITS[dt]
    x = rng.integers(0, np.iinfo(u).max, size=shape, dtype=u, endpoint=True)
    sp = np.asarray(SPECIAL[dt], u)
    x[..., :sp.size] = sp
    return x


def to_dev(bits, dt):
    _, signed, tdt = BITS[dt]
    return torch.from_numpy(np.ascontiguousarray(bits).view(signed)).to("cuda").view(tdt)


def case(dt, D, seed):
    rng = np.random.default_rng(seed)
    NB, Hkv, T = 14, 3, 9
    kp = rand_bits(rng, dt, (NB, Hkv, 16, D))
    vp = rand_bits(rng, dt, (NB, Hkv, 16, D))
    kn = rand_bits(rng, dt, (T, Hkv, D))
    vn = rand_bits(rng, dt, (T, Hkv, D))
    # the specials land in different dims of different rows too
    kn[:, :, D // 2:D // 2 + len(SPECIAL[dt])] = np.asarray(SPECIAL[dt])[::-1]
    return rng, NB, Hkv, T, kp, vp, kn, vn


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_write_kv_special_payloads(pa, dt, D):
    say(f"[special payloads] write_kv {dt} D={D}")
    rng, NB, Hkv, T, kp, vp, kn, vn = case(dt, D, 31 + D)
    slots = rng.choice(NB * 16, T, replace=False).astype(np.int32)
    slots[2] = -1                                        # padding: skipped
    k, v = to_dev(kp, dt), to_dev(vp, dt)
    pa.write_kv(to_dev(kn, dt), to_dev(vn, dt), k, v, torch.from_numpy(slots).to("cuda"))
    ke, ve = kp.copy(), vp.copy()
    cache_ops.write_kv(ke, ve, kn, vn, slots)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(k), ke)
    assert np.array_equal(host_bits(v), ve)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_append_kv_special_payloads(pa, dt, D):
    say(f"[special payloads] append_kv {dt} D={D}")
    rng, NB, Hkv, T, kp, vp, kn, vn = case(dt, D, 41 + D)
    B, MB = 4, 4
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((B, MB), -1, np.int32)
    bt[:, :3] = perm[:12].reshape(B, 3)
    seq = rng.integers(0, B, T).astype(np.int32)
    # distinct (sequence, position) pairs inside the 3 filled entries, one
    # past them (entry -1: no slot) and one negative position
    pos = np.empty(T, np.int32)
    used = set()
    for i in range(T):
        while True:
            p = int(rng.integers(0, 48))
            if (int(seq[i]), p) not in used:
                used.add((int(seq[i]), p))
                pos[i] = p
                break
    pos[3] = 50
    pos[5] = -2
    expect = cache_ops.slot_mapping(bt, pos, 16, seq_ids=seq)
    assert expect[3] == -1 and expect[5] == -1 and len(set(expect[expect >= 0])) == (expect >= 0).sum()
    k, v = to_dev(kp, dt), to_dev(vp, dt)
    out = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    pa.append_kv(to_dev(kn, dt), to_dev(vn, dt), k, v, torch.from_numpy(bt).to("cuda"),
                 torch.from_numpy(pos).to("cuda"), seq_ids=torch.from_numpy(seq).to("cuda"),
                 slots_out=out)
    ke, ve = kp.copy(), vp.copy()
    cache_ops.write_kv(ke, ve, kn, vn, expect)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), expect)
    assert np.array_equal(host_bits(k), ke)
    assert np.array_equal(host_bits(v), ve)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_copy_blocks_special_payloads(pa, dt, D):
    say(f"[special payloads] copy_blocks {dt} D={D}")
    rng, NB, Hkv, T, kp, vp, kn, vn = case(dt, D, 51 + D)
    perm = rng.permutation(NB)
    src, dst = perm[:5], perm[5:10]                      # distinct; no dst is a src
    pairs = np.stack([src, dst], 1).astype(np.int32)
    k, v = to_dev(kp, dt), to_dev(vp, dt)
    pa.copy_blocks(k, v, torch.from_numpy(pairs).to("cuda"))
    ke, ve = kp.copy(), vp.copy()
    cache_ops.copy_blocks(ke, ve, pairs)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(k), ke)
    assert np.array_equal(host_bits(v), ve)
