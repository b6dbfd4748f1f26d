"""pa_decode_noalloc: pa_decode with the library's own per-GPU scratch area in
place of a caller's workspace, for callers that cannot allocate.

Through the C ABI (the binding only marshals arguments), its output must be
bit-identical to pa_decode's with a workspace on the same inputs (the same
kernels run), on calls in a row whose second input is smaller than the first,
so that partials the first call left in the shared scratch cannot leak into
the second. Each output is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

from gpu_cases import TOL, Step, max_abs_err, say
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def same_bits(a, b):
    ia = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
    ib = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
    return torch.equal(ia, ib)


def check_call(pa, name, partition):
    st = Step(SMALL[name])
    st.run_cache_ops(pa)
    need = pa.decode_workspace_bytes(st.spec.B, st.spec.Hq, st.spec.D, st.max_ctx, partition)
    say(f"[noalloc] {name} partition={partition}: {need} bytes of partials")
    out = torch.full_like(st.q, float("nan"))
    got = pa.decode_noalloc(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                            st.spec.scale, st.max_ctx, partition=partition, out=out)
    ref = st.decode(pa, partition=partition)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert same_bits(got, ref), f"{name}: differs from pa_decode with a workspace"
    err = max_abs_err(got, st.expect)
    say(f"    bit-identical to pa_decode; max abs err vs oracle {err:.3e}")
    assert err <= TOL[st.spec.dtype]
    return need


def test_noalloc_matches_decode_on_calls_in_a_row(pa):
    # the second call's input, and its partials, are smaller than the first's
    big = check_call(pa, "gqa8", 64)          # matrix-core kernel, fp16 partials
    small = check_call(pa, "mha_bf16", 64)    # vector kernel, fp16 partials
    assert 0 < small < big
    f32 = check_call(pa, "tiny", 16)          # fp32 partials
    assert 0 < f32 < big
    f32g = check_call(pa, "gqa8_f32", 64)     # fp32 matrix-core kernel, fp32 partials
    assert f32g > 0


def test_noalloc_without_split_and_oversized_split(pa):
    check_call(pa, "gqa2", 0)                 # no split: the scratch is not touched
    st = Step(SMALL["mha_bf16"], oracle_full=False)
    # a split whose partials exceed the scratch area is refused before any launch
    B, Hq, D, part = st.spec.B, st.spec.Hq, st.spec.D, 16
    max_ctx = 1 << 20
    need = pa.decode_workspace_bytes(B, Hq, D, max_ctx, part)
    assert need > pa.PA_NOALLOC_SCRATCH_BYTES
    out = torch.zeros_like(st.q)
    with pytest.raises(pa.PAError) as e:
        pa.decode_noalloc(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                          st.spec.scale, max_ctx, partition=part, out=out)
    assert e.value.status == pa.PA_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
