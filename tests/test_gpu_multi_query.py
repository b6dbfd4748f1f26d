"""GPU parity for several new tokens per sequence (pa_multi_query): the HIP
library against the fp64 oracle on the same seeded inputs. Cache writes of the
chunk are bit-exact over the whole pool; outputs lie within max-abs 2e-3 (fp32
I/O) or 1.5e-2 (bf16 I/O).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_410_amd.workloads import Spec

import oracle
from gpu_cases import TOL, Step, host_bits, max_abs_err, oracle_view, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


CHUNKS = {
    # matrix-core path: 16 query rows of one head per tile (MHA), or rows x group heads
    "mq_mha": Spec("mq_mha", "bf16", 4, 4, 4, 128, seed=30, lengths=("uniform", 1, 700),
                   chunk=("uniform", 1, 40)),
    "mq_gqa8": Spec("mq_gqa8", "bf16", 3, 16, 2, 128, seed=31, lengths=("uniform", 1, 2000),
                    chunk=("uniform", 1, 20)),
    "mq_gqa3": Spec("mq_gqa3", "bf16", 3, 6, 2, 128, seed=32, lengths=("uniform", 1, 600),
                    chunk=("uniform", 1, 13)),
    "mq_gqa24": Spec("mq_gqa24", "bf16", 2, 24, 1, 128, seed=33, lengths=("uniform", 1, 500),
                     chunk=("uniform", 1, 5)),
    "mq_prefill": Spec("mq_prefill", "bf16", 2, 2, 2, 128, seed=34, lengths=("uniform", 100, 300),
                       chunk=("all",)),
    "mq_single": Spec("mq_single", "bf16", 5, 8, 2, 128, seed=35, lengths=("uniform", 1, 400),
                      chunk=("uniform", 1, 1)),
    # fp32 (the fp32 matrix-core kernel, one query head per kv head)
    "mq_f32": Spec("mq_f32", "f32", 3, 4, 4, 64, seed=36, lengths=("uniform", 1, 300),
                   chunk=("uniform", 1, 12)),
    # fp32 on the matrix cores: up to 48 (row, head) columns per kv head, so
    # one to three 16-column tiles
    "mq_f32_gqa": Spec("mq_f32_gqa", "f32", 3, 8, 2, 128, seed=46, lengths=("uniform", 1, 600),
                       chunk=("uniform", 1, 12)),
    # the same at head_dim 64: 20 to 36 columns, two or three tiles per kv head
    "mq_f32_gqa_d64": Spec("mq_f32_gqa_d64", "f32", 2, 8, 2, 64, seed=49,
                           lengths=("uniform", 40, 700), chunk=("uniform", 5, 9)),
    "mq_bf16_d64": Spec("mq_bf16_d64", "bf16", 3, 4, 2, 64, seed=37, lengths=("uniform", 1, 300),
                        chunk=("uniform", 1, 9)),
    # head_dim 64 past one tile: 160 to 320 columns per kv head, 10 to 20
    # tiles on the chunk kernel (128-byte rows, two tiles per wave)
    "mq_gqa8_d64": Spec("mq_gqa8_d64", "bf16", 2, 16, 2, 64, seed=48, lengths=("uniform", 100, 900),
                        chunk=("uniform", 20, 40)),
    # head_dim 64 on the matrix cores: at most 16 (row, head) columns per kv head
    "mq_bf16_d64_mfma": Spec("mq_bf16_d64_mfma", "bf16", 3, 8, 2, 64, seed=40,
                             lengths=("uniform", 1, 700), chunk=("uniform", 1, 4)),
    # unsplit rows longer than one 64-block id chunk per wave
    "mq_long": Spec("mq_long", "bf16", 2, 2, 2, 128, seed=38, lengths=("fixed", [9000, 3000]),
                    chunk=("uniform", 2, 6)),
    # one or two 16-column tiles per kv head: the matrix-core decode kernel,
    # and the chunk kernel's 4-wave shape with waves that only load
    "mq_gqa8_short": Spec("mq_gqa8_short", "bf16", 4, 16, 2, 128, seed=39,
                          lengths=("uniform", 1, 900), chunk=("uniform", 2, 4)),
}


@pytest.mark.parametrize("name", list(CHUNKS))
@pytest.mark.parametrize("partition", [None, 0, 16, 48, 64, 512])
def test_multi_query_matches_oracle(pa, name, partition):
    spec = CHUNKS[name]
    say(f"[multi-query] {name} partition={partition}")
    st = Step(spec, poison=True)
    slots = st.run_cache_ops(pa)
    out = st.multi(pa, partition=partition)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), st.tb.slots)
    assert np.array_equal(host_bits(st.k_cache), st.k_after)
    assert np.array_equal(host_bits(st.v_cache), st.v_after)
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o)), "NaN-poisoned unused slots leaked into the output"
    err = max_abs_err(out, st.expect)
    say(f"    rows={out.shape[0]} max_q={st.max_q} max abs err {err:.3e} (tol {TOL[spec.dtype]})")
    assert err <= TOL[spec.dtype]


def test_one_token_chunks_equal_decode_bitwise(pa):
    """n_s = 1 everywhere: the same kernels, the same arithmetic order as pa_decode."""
    say("[multi-query vs decode] mq_single")
    st = Step(CHUNKS["mq_single"], oracle_full=False)
    st.run_cache_ops(pa)
    for part in (0, 64):
        a = st.multi(pa, partition=part)
        b = st.decode(pa, partition=part)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), part


def test_bad_row_counts_poison_only_their_rows(pa):
    say("[multi-query bad rows] mq_mha")
    st = Step(CHUNKS["mq_mha"])
    st.run_cache_ops(pa)
    good = st.multi(pa, partition=64).float().cpu()
    qs = st.tb.query_start
    # sequence 1 claims one more row than its context holds
    cl = st.context_lens.clone()
    n1 = int(qs[2] - qs[1])
    cl[1] = n1 - 1
    out = pa.multi_query(st.q, st.k_cache, st.v_cache, st.block_tables, cl, st.query_start,
                         st.spec.scale, st.max_ctx, st.max_q, partition=64).float().cpu()
    assert torch.isnan(out[qs[1]:qs[2]]).all()
    keep = torch.ones(out.shape[0], dtype=torch.bool)
    keep[qs[1]:qs[2]] = False
    assert torch.equal(out[keep], good[keep])   # the intact rows keep their bits


@pytest.mark.parametrize("name", list(CHUNKS))
def test_chunk_append_kv_bit_exact(pa, name):
    # several tokens per sequence through the fused slot-mapping + write
    say(f"[chunk append_kv] {name}")
    st = Step(CHUNKS[name], oracle_full=False)
    slots = st.run_cache_ops(pa, fused=True)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), st.tb.slots)
    assert np.array_equal(host_bits(st.k_cache), st.k_after)
    assert np.array_equal(host_bits(st.v_cache), st.v_after)


@pytest.mark.parametrize("name", ["mq_gqa8", "mq_gqa8_short", "mq_single", "mq_f32",
                                  "mq_f32_gqa", "mq_bf16_d64"])
@pytest.mark.parametrize("scale_mul", [-1.0, 0.0])
def test_negative_and_zero_scale(pa, name, scale_mul):
    # A negative logit scale and a zero one through every multi-query kernel
    # (chunk, matrix-core decode in bf16 at head_dim 128 and 64, fp32
    # matrix-core), against the oracle at that scale.
    say(f"[scale x{scale_mul}] {name}")
    st = Step(CHUNKS[name], oracle_full=False)
    st.run_cache_ops(pa)
    scale = st.spec.scale * scale_mul
    out = pa.multi_query(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                         st.query_start, scale, st.max_ctx, st.max_q, partition=64)
    expect = oracle.multi_query(oracle_view(st.q_bits), oracle_view(st.k_after),
                                oracle_view(st.v_after), st.tb.block_tables, st.tb.context_lens,
                                st.tb.query_start, scale)
    err = max_abs_err(out, expect)
    say(f"    max abs err {err:.3e}")
    assert err <= TOL[st.spec.dtype]


@pytest.mark.parametrize("big_tile", [0, 1])
@pytest.mark.parametrize("partition", [None, 0, 64])
def test_two_tiles_per_wave_keep_their_own_max(pa, big_tile, partition):
    # 64 rows x 8 heads per kv head: 32 column tiles, so the chunk kernel's
    # waves hold two tiles each (tiles 2w and 2w + 1) and take both tiles'
    # column maxima from one shared lane exchange. One tile of each pair gets
    # queries 64x larger (exact in bf16), so its logits span hundreds of log2
    # units: a tile that took the other's max as its reference would overflow
    # to inf or underflow to an all-zero sum, while the right reference keeps
    # every probability in range.
    spec = Spec("mq_gqa8_wide", "bf16", 2, 16, 2, 128, seed=40, lengths=("uniform", 300, 1200),
                chunk=("uniform", 64, 64))
    say(f"[two tiles per wave] big tile {big_tile} partition={partition}")
    st = Step(spec, oracle_full=False)
    st.run_cache_ops(pa)
    G = spec.Hq // spec.Hkv
    bits = st.q_bits.copy()
    qs = st.tb.query_start
    for s in range(spec.B):
        for i in range(qs[s + 1] - qs[s]):
            if (i * G // 16) % 2 == big_tile:
                row = (bits[qs[s] + i].astype(np.uint32) << 16).view(np.float32) * np.float32(64.0)
                bits[qs[s] + i] = (row.view(np.uint32) >> 16).astype(np.uint16)
    q = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(st.q.device)
    out = pa.multi_query(q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                         st.query_start, st.spec.scale, st.max_ctx, st.max_q, partition=partition)
    expect = oracle.multi_query(oracle_view(bits), oracle_view(st.k_after), oracle_view(st.v_after),
                                st.tb.block_tables, st.tb.context_lens, st.tb.query_start,
                                st.spec.scale)
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    err = max_abs_err(out, expect)
    say(f"    max abs err {err:.3e}")
    assert err <= TOL[spec.dtype]


@pytest.mark.parametrize("name", ["mq_gqa8", "mq_gqa8_short", "mq_mha", "mq_single", "mq_long",
                                  "mq_f32_gqa", "mq_gqa8_d64"])
@pytest.mark.parametrize("partition", [0, 64])
def test_bad_block_ids_poison_only_their_rows(pa, name, partition):
    # A block id outside the pool, or negative, in a block every row of its
    # sequence attends to: that sequence's rows come out NaN, nothing is read
    # out of bounds, and every other row keeps its bits. The kernels cover
    # two tiles per wave (mq_gqa8), one tile per wave on 2 or 4 waves
    # (mq_gqa8_short, mq_mha), the matrix-core decode kernel (mq_single), and
    # an id in the second 64-block chunk of a long unsplit row (mq_long), and
    # the fp32 matrix-core kernel over several tiles (mq_f32_gqa), and the
    # head_dim-64 matrix-core kernel over many tiles (mq_gqa8_d64).
    say(f"[multi-query bad block ids] {name} partition={partition}")
    st = Step(CHUNKS[name], oracle_full=False)
    st.run_cache_ops(pa)
    good = st.multi(pa, partition=partition)
    bt = st.block_tables.clone()
    qs = st.tb.query_start
    B = st.spec.B
    j0 = 70 if name == "mq_long" else 0
    assert int(st.tb.context_lens[0]) > 16 * j0
    bt[0, j0] = st.tb.NB + 5
    bad = [0]
    if B >= 3:
        bt[2, 0] = -7
        bad.append(2)
    out = pa.multi_query(st.q, st.k_cache, st.v_cache, bt, st.context_lens, st.query_start,
                         st.spec.scale, st.max_ctx, st.max_q, partition=partition)
    torch.cuda.synchronize()
    o = out.float().cpu()
    for s in range(B):
        rows = slice(int(qs[s]), int(qs[s + 1]))
        if s in bad:
            assert torch.isnan(o[rows]).all(), s
        else:
            assert torch.equal(out[rows].view(torch.int16).cpu(), good[rows].view(torch.int16).cpu()), s
