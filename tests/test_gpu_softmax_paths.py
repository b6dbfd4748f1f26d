"""GPU parity on logits built to drive the online softmax's reference steps.

The kernels keep, per column, a reference max that moves only when a block's
logits pass it by more than a margin (and the chunk kernel skips the whole
reference step on pairs where no lane passes it). Random inputs move the
reference on the first blocks and rarely after. Here every query row's logits
are set to rise, or fall, by about 12 log2 units from one 16-token block to
the next (keys along the query's direction, scaled per block, with small
noise), so that rising contexts move the reference on every block and
falling ones never after the first. Every attention kernel is covered:
vector decode (one head per kv head), bf16 and fp32 matrix-core decode, and
the chunk kernel with one and with two column tiles per wave, unsplit and
split. Outputs against the fp64 oracle on the same bits.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_cases import TOL, max_abs_err, record_parity, say

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def _bits(x, dtype):
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "f32":
        return x.view(np.uint32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _dev(bits, dtype):
    v = bits.view(np.int16) if bits.dtype == np.uint16 else bits.view(np.int32)
    t = torch.from_numpy(np.ascontiguousarray(v)).to("cuda")
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _view(bits):
    return bits.view(np.float32) if bits.dtype == np.uint32 else bits


def build(dtype, Hq, Hkv, D, lens, n_new, direction, seed):
    """Pools, tables and queries whose logits step by about 12 log2 units per
    block along the context (direction +1: rising, -1: falling)."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    cl = np.asarray(lens, np.int32)
    B = len(lens)
    nblk = (cl + 15) // 16
    NB = int(nblk.sum()) + 5
    perm = rng.permutation(NB).astype(np.int32)
    MB = int(nblk.max())
    bt = np.full((B, MB), -1, np.int32)
    j = 0
    for s in range(B):
        bt[s, :nblk[s]] = perm[j:j + nblk[s]]
        j += nblk[s]
    # every query of kv head g points along one unit direction u_g
    u = rng.standard_normal((Hkv, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    n = np.minimum(n_new, cl).astype(np.int32) if n_new else np.ones(B, np.int32)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    Tq = int(qs[-1])
    q = np.zeros((Tq, Hq, D), np.float32)
    for h in range(Hq):
        q[:, h, :] = 4.0 * u[h // G] + 0.05 * rng.standard_normal((Tq, D))
    # key of token t: its block's step along u (logit = scale * 4 * c), so
    # consecutive blocks differ by ~12 / log2(e) in natural-log logits
    k = 0.3 * rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32)
    # V at half scale: the probabilities gather on a few tokens, so an
    # output row is close to one V row, and rows below 2 in size keep the
    # bf16 rounding of the output (half an ulp) under 0.004
    v = 0.5 * rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32)
    step = 12.0 / LOG2E / (scale * 4.0)
    for s in range(B):
        for i in range(nblk[s]):
            c = direction * step * (i - nblk[s] / 2)
            k[bt[s, i]] += c * u[:, None, :]
    return dict(q=_bits(q, dtype), k=_bits(k, dtype), v=_bits(v, dtype), bt=bt, cl=cl, qs=qs,
                n=n, scale=scale, multi=bool(n_new))


# (dtype, Hq, Hkv, D, new rows per sequence): the kernel each one reaches
CASES = [
    ("bf16", 8, 8, 128, 0),     # vector decode kernel
    ("f32", 8, 8, 64, 0),       # vector decode kernel, fp32
    ("bf16", 64, 8, 128, 0),    # bf16 matrix-core decode kernel
    ("bf16", 64, 8, 64, 0),     # the same at head_dim 64
    ("f32", 64, 8, 128, 0),     # fp32 matrix-core decode kernel
    ("bf16", 64, 8, 128, 6),    # chunk kernel, one tile per wave (3 tiles per kv head)
    ("bf16", 64, 8, 128, 40),   # chunk kernel, two tiles per wave (20 tiles)
    ("bf16", 64, 8, 64, 40),    # the same at head_dim 64
]


@pytest.mark.parametrize("direction", [1, -1], ids=["rising", "falling"])
@pytest.mark.parametrize("dtype,Hq,Hkv,D,n_new", CASES)
def test_softmax_reference_paths(pa, dtype, Hq, Hkv, D, n_new, direction):
    say(f"[softmax paths] {dtype} {Hq}/{Hkv} D{D} new={n_new} "
        f"{'rising' if direction > 0 else 'falling'}")
    c = build(dtype, Hq, Hkv, D, [50, 333, 700, 1024], n_new, direction, seed=70 + D + n_new)
    k_t, v_t = _dev(c["k"], dtype), _dev(c["v"], dtype)
    bt_t = torch.from_numpy(c["bt"]).to("cuda")
    cl_t = torch.from_numpy(c["cl"]).to("cuda")
    q_t = _dev(c["q"], dtype)
    if c["multi"]:
        expect = oracle.multi_query(_view(c["q"]), _view(c["k"]), _view(c["v"]), c["bt"], c["cl"],
                                    c["qs"], c["scale"])
    else:
        expect = oracle.decode(_view(c["q"]), _view(c["k"]), _view(c["v"]), c["bt"], c["cl"],
                               c["scale"])
    for part in (0, 128):
        if c["multi"]:
            out = pa.multi_query(q_t, k_t, v_t, bt_t, cl_t, torch.from_numpy(c["qs"]).to("cuda"),
                                 c["scale"], int(c["cl"].max()), int(c["n"].max()),
                                 partition=part)
        else:
            out = pa.decode(q_t, k_t, v_t, bt_t, cl_t, c["scale"], int(c["cl"].max()),
                            partition=part)
        torch.cuda.synchronize()
        err = max_abs_err(out, expect)
        say(f"    partition {part}: max abs err {err:.3e}")
        record_parity(f"softmax paths {dtype} {Hq}/{Hkv} D{D} new={n_new} "
                      f"{'rising' if direction > 0 else 'falling'} p{part}", err, TOL[dtype])
        assert np.all(np.isfinite(out.float().cpu().numpy()))
        assert err <= TOL[dtype], part
