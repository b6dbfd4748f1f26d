"""Attention calls captured as HIP graphs (torch.cuda.CUDAGraph).

Given its output and workspace, a call allocates nothing and records no
memset, so its captured form must replay the eager result bit for bit:
multi-query attention on the matrix-core decode kernel and on the chunk
kernel with split partials and the merge, and shared-prefix decode in one
pass and in two, in bf16 and fp32. Before each replay the output is poisoned
with NaN and the workspace with other data; after it, the same call runs
eagerly on the same buffers (eager work between replays).
"""

import numpy as np
import pytest
import torch

from gpu_cases import Step, say
from test_gpu_multi_query import CHUNKS
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_410_amd as m
    return m


def replay_matches_eager(call, out, ws, what):
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    assert not torch.isnan(eager.float()).any(), what
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"{what}: replay {i}"
        call()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"{what}: eager {i}"


@pytest.mark.parametrize("name,partition", [
    ("mq_gqa8", 64),          # matrix-core decode kernel and chunk kernel, split
    ("mq_gqa8_d64", 128),     # chunk kernel at head_dim 64, split
    ("mq_gqa8_short", 32),    # one or two tiles per kv head
    ("mq_f32_gqa", 64),       # fp32 matrix-core kernel, split
])
def test_multi_query_graph_replays(pa, name, partition):
    say(f"[graph] multi_query {name} partition={partition}")
    st = Step(CHUNKS[name], oracle_full=False)
    st.run_cache_ops(pa)
    rows = st.q.shape[0]
    ws = torch.empty(max(16, pa.decode_workspace_bytes(rows, st.spec.Hq, st.spec.D, st.max_ctx,
                                                       partition)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q)

    def call():
        pa.multi_query(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                       st.query_start, st.spec.scale, st.max_ctx, st.max_q, partition=partition,
                       out=out, workspace=ws)

    replay_matches_eager(call, out, ws, name)


@pytest.mark.parametrize("name,partition,max_group", [
    ("cow_small", 0, None),       # one pass
    ("cow_small", 32, None),      # two passes: split shared part
    ("cow_gqa", 0, 4),            # 16 columns per kv head in one tile: one pass
    ("cow_gqa", 16, 8),           # two tiles per kv head: the chunk kernel's group pass
    ("cow_gqa_f32", 32, None),    # fp32: two passes on the fp32 matrix-core kernel
    ("cow_small_f32", 0, None),   # fp32, one head per kv head: the vector kernel's tail
])
def test_decode_shared_graph_replays(pa, name, partition, max_group):
    say(f"[graph] decode_shared {name} partition={partition} max_group={max_group}")
    st = Step(SMALL[name], oracle_full=False)
    st.run_cache_ops(pa)
    G = st.spec.Hq // st.spec.Hkv
    mg = max_group or 16 // G
    gs, sh = pa.shared_groups(st.tb.block_tables, st.tb.context_lens, mg)
    assert sh.max() > 0
    gs_d, sh_d = torch.from_numpy(gs).cuda(), torch.from_numpy(sh).cuda()
    B = st.q.shape[0]
    ws = torch.empty(max(16, pa.decode_shared_workspace_bytes(B, st.spec.Hq, st.spec.D,
                                                              int(sh.max()), partition)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q)

    def call():
        pa.decode_shared(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens, gs_d,
                         sh_d, st.spec.scale, st.max_ctx, mg, int(sh.max()), partition=partition,
                         out=out, workspace=ws)

    replay_matches_eager(call, out, ws, name)
