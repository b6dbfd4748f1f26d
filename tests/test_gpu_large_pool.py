"""GPU parity on pools larger than 4 GiB: block ids whose byte offsets need
64 bits, in every kernel that addresses the pools.

Each pool is allocated whole on the device (over 5 GiB), but only the blocks
the tables name are filled, every other one among the pool's last 8192
blocks.
The oracle reads a compact copy of just those blocks under the same tables
with the ids renumbered: where a block sits does not change the result (the
permutation pin of the oracle), so its output is the expectation for the
large pool. Unused rows of each sequence's last block hold NaN. Cache writes,
the fused slot mapping and write, and block copies into high ids are compared
bit for bit with the oracle's bookkeeping on the compact copy.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_cases import TOL, max_abs_err, record_parity, say
from oracle import cache_ops

pytestmark = pytest.mark.gpu

POOL_BYTES = 5 << 30  # per pool
NAN = {"bf16": np.uint16(0x7FC0), "f32": np.uint32(0x7FC00000)}


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def _bits(rng, dtype, shape):
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32)
    return ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)


def _dev(bits, tdt):
    v = bits.view(np.int16) if bits.dtype == np.uint16 else bits.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(v)).to("cuda").view(tdt)


class LargePool:
    """A > 4 GiB pool pair with B sequences placed on high and low block ids,
    and the compact copy of the used blocks that the oracle reads."""

    def __init__(self, dtype, Hkv, D, lens, seed):
        self.dtype = dtype
        e = 4 if dtype == "f32" else 2
        self.tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        self.Hkv, self.D = Hkv, D
        block_bytes = Hkv * 16 * D * e
        self.NB = POOL_BYTES // block_bytes + 123
        assert (self.NB - 1) * block_bytes > 2**32
        rng = np.random.default_rng(seed)
        self.rng = rng
        self.cl = np.asarray(lens, np.int32)
        B = len(lens)
        nblk = (self.cl + 15) // 16
        n = int(nblk.sum()) + 8  # 8 spare blocks for the write and copy tests
        # compact block j -> pool id: even j among the last 8192 blocks (byte
        # offsets past 4 GiB), odd j anywhere below them
        self.ids = np.empty(n, np.int64)
        self.ids[0::2] = rng.choice(8192, (n + 1) // 2, replace=False) + (self.NB - 8192)
        self.ids[1::2] = rng.choice(self.NB - 8192, n // 2, replace=False)
        MB = int(nblk.max())
        self.bt_c = np.full((B, MB), -1, np.int32)  # compact ids
        j = 0
        for s in range(B):
            self.bt_c[s, :nblk[s]] = np.arange(j, j + nblk[s])
            j += nblk[s]
        self.spare = np.arange(j, n)
        self.bt = np.where(self.bt_c >= 0, self.ids[np.maximum(self.bt_c, 0)], -1).astype(np.int32)
        self.k_c = _bits(rng, dtype, (n, Hkv, 16, D))
        self.v_c = _bits(rng, dtype, (n, Hkv, 16, D))
        for s in range(B):  # rows past each context: NaN, never read
            last, used = self.bt_c[s, nblk[s] - 1], self.cl[s] - 16 * (nblk[s] - 1)
            self.k_c[last, :, used:, :] = NAN[dtype]
            self.v_c[last, :, used:, :] = NAN[dtype]
        self.k = torch.empty((self.NB, Hkv, 16, D), dtype=self.tdt, device="cuda")
        self.v = torch.empty((self.NB, Hkv, 16, D), dtype=self.tdt, device="cuda")
        self.ids_t = torch.from_numpy(self.ids).to("cuda")
        self.k[self.ids_t] = _dev(self.k_c, self.tdt)
        self.v[self.ids_t] = _dev(self.v_c, self.tdt)
        self.bt_t = torch.from_numpy(self.bt).to("cuda")
        self.cl_t = torch.from_numpy(self.cl).to("cuda")

    def gathered(self):
        """The used blocks' bits, back from the device, in compact order."""
        def back(t):
            g = t[self.ids_t].cpu().contiguous()
            return (g.view(torch.int16).numpy().view(np.uint16) if self.dtype == "bf16"
                    else g.view(torch.int32).numpy().view(np.uint32))
        return back(self.k), back(self.v)

    def to_compact_slot(self, slot):
        where = {int(b): j for j, b in enumerate(self.ids)}
        return np.asarray([where[int(s) // 16] * 16 + int(s) % 16 for s in slot], np.int32)


def _view(bits):
    return bits.view(np.float32) if bits.dtype == np.uint32 else bits


# bf16 grouped heads (matrix-core kernel, head_dim 128 and 64), one head per
# kv head (vector kernel) in bf16 and fp32, fp32 grouped heads (fp32
# matrix-core kernel)
CASES = [("bf16", 64, 8, 128), ("bf16", 64, 8, 64), ("bf16", 8, 8, 128), ("f32", 8, 8, 128),
         ("f32", 32, 8, 64)]


@pytest.mark.parametrize("dtype,Hq,Hkv,D", CASES)
def test_decode_on_a_pool_past_4_gib(pa, dtype, Hq, Hkv, D):
    say(f"[large pool decode] {dtype} Hq={Hq} Hkv={Hkv} D={D}")
    lp = LargePool(dtype, Hkv, D, [1, 16, 17, 300, 511, 700], seed=61)
    q_bits = _bits(lp.rng, dtype, (len(lp.cl), Hq, D))
    q = _dev(q_bits, lp.tdt)
    scale = 1.0 / np.sqrt(D)
    expect = oracle.decode(q_bits if dtype == "bf16" else q_bits.view(np.float32),
                           _view(lp.k_c), _view(lp.v_c), lp.bt_c, lp.cl, scale)
    for part in (0, 64, 512):
        out = pa.decode(q, lp.k, lp.v, lp.bt_t, lp.cl_t, scale, int(lp.cl.max()), partition=part)
        torch.cuda.synchronize()
        err = max_abs_err(out, expect)
        say(f"    partition {part}: max abs err {err:.3e}")
        record_parity(f"large pool {dtype} {Hq}/{Hkv} D{D} p{part}", err, TOL[dtype])
        assert np.all(np.isfinite(out.float().cpu().numpy()))
        assert err <= TOL[dtype], part
    del lp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_new", [2, 40])
def test_multi_query_on_a_pool_past_4_gib(pa, n_new):
    # 2 new tokens x 8 heads (one 16-column tile): the matrix-core decode
    # kernel; 40 x 8: the chunk kernel
    say(f"[large pool multi-query] n_new={n_new}")
    lp = LargePool("bf16", 8, 128, [40, 64, 300, 700], seed=62)
    B, Hq = len(lp.cl), 64
    n = np.minimum(n_new, lp.cl).astype(np.int32)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q_bits = _bits(lp.rng, "bf16", (int(qs[-1]), Hq, 128))
    scale = 1.0 / np.sqrt(128)
    expect = oracle.multi_query(q_bits, lp.k_c, lp.v_c, lp.bt_c, lp.cl, qs, scale)
    for part in (0, 128):
        out = pa.multi_query(_dev(q_bits, lp.tdt), lp.k, lp.v, lp.bt_t, lp.cl_t,
                             torch.from_numpy(qs).to("cuda"), scale, int(lp.cl.max()),
                             int(n.max()), partition=part)
        torch.cuda.synchronize()
        err = max_abs_err(out, expect)
        say(f"    partition {part}: max abs err {err:.3e}")
        assert err <= TOL["bf16"], part
    del lp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,Hkv,D", [("bf16", 8, 128), ("f32", 4, 64)])
def test_writes_and_copies_on_a_pool_past_4_gib(pa, dtype, Hkv, D):
    say(f"[large pool writes] {dtype} Hkv={Hkv} D={D}")
    lp = LargePool(dtype, Hkv, D, [5, 33, 200], seed=63)
    k_exp, v_exp = lp.k_c.copy(), lp.v_c.copy()

    # copy-on-write pairs between spare blocks: low to high, high to low,
    # high to high ids (even compact ids are the high ones)
    hi = [int(j) for j in lp.spare if j % 2 == 0]
    lo = [int(j) for j in lp.spare if j % 2 == 1]
    pairs_c = np.asarray([[lo[0], hi[0]], [hi[1], lo[1]], [hi[2], hi[3]]], np.int32)
    pairs = lp.ids[pairs_c].astype(np.int32)
    pa.copy_blocks(lp.k, lp.v, torch.from_numpy(pairs).to("cuda"))
    cache_ops.copy_blocks(k_exp, v_exp, pairs_c)

    # the fused slot mapping and write: each sequence's next position
    pos = lp.cl.copy()
    pos[pos % 16 == 0] -= 1  # stay inside the table's blocks
    T = len(pos)
    kn, vn = _bits(lp.rng, dtype, (T, Hkv, D)), _bits(lp.rng, dtype, (T, Hkv, D))
    slots = torch.empty(T, dtype=torch.int32, device="cuda")
    pa.append_kv(_dev(kn, lp.tdt), _dev(vn, lp.tdt), lp.k, lp.v, lp.bt_t,
                 torch.from_numpy(pos).to("cuda"), slots_out=slots)
    expect_slots = cache_ops.slot_mapping(lp.bt, pos, 16)
    assert slots.cpu().numpy().tolist() == expect_slots.tolist()
    assert int(expect_slots.max()) * Hkv * D * (4 if dtype == "f32" else 2) > 2**32
    cache_ops.write_kv(k_exp, v_exp, kn, vn, lp.to_compact_slot(expect_slots))

    # plain writes into the spare high and low blocks
    wslots_c = np.asarray([hi[3] * 16 + 0, hi[3] * 16 + 15, lo[2] * 16 + 9], np.int32)
    wslots = np.asarray([int(lp.ids[s // 16]) * 16 + s % 16 for s in wslots_c], np.int32)
    kw, vw = _bits(lp.rng, dtype, (3, Hkv, D)), _bits(lp.rng, dtype, (3, Hkv, D))
    pa.write_kv(_dev(kw, lp.tdt), _dev(vw, lp.tdt), lp.k, lp.v, torch.from_numpy(wslots).to("cuda"))
    cache_ops.write_kv(k_exp, v_exp, kw, vw, wslots_c)

    torch.cuda.synchronize()
    k_got, v_got = lp.gathered()
    assert np.array_equal(k_got, k_exp)
    assert np.array_equal(v_got, v_exp)
    del lp
    torch.cuda.empty_cache()
