"""Split-context partials of bf16 attention.

A partition's partial (running max m, sum l, unnormalised row o) travels to
the merge as an fp16 row z = o / c with (m + log2 c, l / c), c = l * 2^k: an
equivalent online-softmax state, with k chosen so that the row's largest |z|
lies in [2^14, 2^15). These cases scale V by powers of two far past fp16's
range both ways (exact in bf16, and the attention output scales by the same
power): 2^20 and 2^100 need k > 0 to stay finite, 2^-20 needs k < 0 to stay
out of fp16's subnormals (fixed spacing 2^-24, a 6% error on rows of size
2^-20). Every fp16 partial is covered: the vector kernel's (one query head
per kv head; head_dim 128 and 64), the matrix-core kernel's (grouped heads,
one tile per kv head), the chunk kernel's (several tiles per kv head: two
per workgroup up to two tiles per wave, head_dim 128 and 64) and the
shared-prefix group pass's on both (groups of one tile and wider). The output
divided by the power must match the oracle's unscaled output to the bf16
tolerance.
"""

import numpy as np
import pytest
import torch

from gpu_cases import TOL, Step, max_abs_err, say
from paged_kv_cache_410_amd.workloads import Spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


CASES = {
    "valu_d128": Spec("valu_d128", "bf16", 4, 4, 4, 128, seed=31, lengths=("uniform", 200, 1500)),
    "valu_d64": Spec("valu_d64", "bf16", 3, 3, 3, 64, seed=32, lengths=("uniform", 200, 1200)),
    "mfma_gqa8": Spec("mfma_gqa8", "bf16", 3, 16, 2, 128, seed=33, lengths=("uniform", 300, 3000)),
    "mfma_gqa8_d64": Spec("mfma_gqa8_d64", "bf16", 3, 16, 2, 64, seed=37,
                          lengths=("uniform", 300, 3000)),
    # head_dim 64, 3 to 5 rows x 8 heads: two or three tiles per kv head on
    # the chunk kernel (2- or 4-wave workgroups)
    "mfma_d64_tiles": Spec("mfma_d64_tiles", "bf16", 2, 16, 2, 64, seed=47,
                           lengths=("uniform", 300, 1200), chunk=("uniform", 3, 5)),
    # 8 rows x 8 heads: 4 column tiles, one per wave
    "chunk_tpw1": Spec("chunk_tpw1", "bf16", 2, 16, 2, 128, seed=34,
                       lengths=("uniform", 300, 1200), chunk=("uniform", 8, 8)),
    # 64 rows x 8 heads: 32 column tiles, two per wave
    "chunk_tpw2": Spec("chunk_tpw2", "bf16", 2, 16, 2, 128, seed=35,
                       lengths=("uniform", 300, 1200), chunk=("uniform", 64, 64)),
    # the same at head_dim 64, and 3 rows x 8 heads (two tiles, 2-wave workgroups)
    "chunk_tpw2_d64": Spec("chunk_tpw2_d64", "bf16", 2, 16, 2, 64, seed=38,
                           lengths=("uniform", 300, 1200), chunk=("uniform", 64, 64)),
    "chunk_2tiles": Spec("chunk_2tiles", "bf16", 3, 16, 2, 128, seed=39,
                         lengths=("uniform", 300, 1500), chunk=("uniform", 3, 4)),
}


def scaled_step(pa, spec, shift):
    """The step with every V value (pool and new tokens) times 2^shift."""
    st = Step(spec)
    st.v_cache.mul_(2.0 ** shift)
    st.v_new.mul_(2.0 ** shift)
    st.run_cache_ops(pa)
    return st


def check(out, st, shift):
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    err = max_abs_err(out.float() / 2.0 ** shift, st.expect)
    say(f"    max abs err (unscaled) {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("shift", [0, 20, 100, -20])
@pytest.mark.parametrize("partition", [64, 512])
def test_partials_past_fp16_range(pa, name, shift, partition):
    spec = CASES[name]
    say(f"[partials] {name} V x 2^{shift} partition={partition}")
    st = scaled_step(pa, spec, shift)
    out = st.multi(pa, partition=partition) if spec.chunk else st.decode(pa, partition=partition)
    torch.cuda.synchronize()
    check(out, st, shift)


@pytest.mark.parametrize("shift", [0, 20, 100, -20])
@pytest.mark.parametrize("partition", [0, 32])
@pytest.mark.parametrize("max_group", [4, 8])  # 16 columns (matrix-core kernel), 32 (chunk)
def test_shared_prefix_group_partials_past_fp16_range(pa, shift, partition, max_group):
    spec = Spec("cow_big", "bf16", 8, 8, 2, 128, seed=36, lengths=("cow",),
                cow=dict(prompts=2, samples=4, prompt_len=200, r_max=15, tail_lo=1, tail_hi=60))
    say(f"[partials] shared prefix V x 2^{shift} partition={partition} max_group={max_group}")
    st = scaled_step(pa, spec, shift)
    gs, sh = pa.shared_groups(st.tb.block_tables, st.tb.context_lens, max_group)
    assert sh.max() > 0
    out = pa.decode_shared(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                           torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda(),
                           spec.scale, st.max_ctx, max_group, int(sh.max()),
                           partition=partition)
    torch.cuda.synchronize()
    check(out, st, shift)
