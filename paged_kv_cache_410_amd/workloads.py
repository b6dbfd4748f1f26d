"""Seeded synthetic workloads for paged decode attention.

This module draws the random inputs only: context-length mixes, the order of
the physical-block free list, and the q / K / V values. It holds none of the
attention arithmetic and none of the block bookkeeping: block tables, slots
and copy-on-write pairs come from whatever block manager the caller passes
in (the library's native manager in the benchmark, the oracle's in tests), so
both sides of every parity check read inputs from one generator.

Workloads (lengths, seeds and draw order are fixed here):

  tiny  fp32, 4 seqs, 8 heads (MHA), head_dim 64, contexts {1, 17, 100, 250},
        a 64-block pool handed out in a seeded random order.        seed 0
  7b    bf16, 64 seqs, 32/32 heads, head_dim 128, contexts U[128, 2048],
        pool = used blocks + 10% free.                              seed 1
  13b   bf16, 128 seqs, 40/40 heads, head_dim 128, contexts lognormal
        (median 500, sigma 0.7 in log space) clipped to [16, 2048].  seed 2
  gqa   bf16, 16 seqs, 64 q heads / 8 kv heads, head_dim 128, contexts
        U[8192, 32768], 512-token partitions.                      seed 3
  cow   bf16, 16 prompts x 8 samples, 32 heads, head_dim 128. Prompt length
        1024 - r, r ~ U{1..15} (so the last prompt block is partly filled and
        shared by 8 samples); each sample then gets a private tail of
        U{1..256} tokens.                                           seed 4
  prefix  bf16, 128 requests, 32/32 heads, head_dim 128, all starting with one
        1024-token system prompt (seeded token ids) followed by a private tail
        of U{16..512} tokens; the block manager must share prompt blocks
        across requests (prefix cache), so the 64 prompt blocks are held by
        all 128 sequences.                                          seed 7
  13b_verify4   the 13b shapes and length mix with 4 new tokens per
        sequence (several drafted tokens checked in one pass).      seed 5
  gqa_chunk512  bf16, 16 seqs, 64/8 heads, head_dim 128, contexts
        U[1024, 8192] whose last 512 tokens are the step's chunk (a prompt
        processed in 512-token chunks).                             seed 6
  gqa_chunk512_d64  the same recipe at head_dim 64.                 seed 11
  gqa_short  bf16, 128 seqs, 32 q heads / 8 kv heads, head_dim 128, the 13b
        length mix (a grouped-head layer at short contexts; no split at
        the library's default partition).                           seed 12

Draw order for a seed: lengths -> free-list permutation -> q -> K pool ->
V pool -> new K -> new V. Values are N(0, 1) in fp32, rounded to the
workload's element type by torch (round to nearest even for bf16).

Every workload has one decode step: each sequence's last token is appended
(through the block manager) and written with the step's new K/V, then all
sequences attend over their full context. For `cow`, the step's appended
tokens are the samples' whole tails, so the step carries the copy-on-write
copies of the shared, partly filled prompt blocks. A chunk workload
(spec.chunk) appends several new tokens per sequence (the last n_s tokens of
its context, n_s drawn after the lengths) and has one query row per new
token; its draw order is lengths -> new-token counts -> free-list
permutation -> q -> K pool -> V pool -> new K -> new V.
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class Spec:
    name: str
    dtype: str                 # "f32" | "bf16"
    B: int                     # sequences (cow: prompts * samples)
    Hq: int
    Hkv: int
    D: int
    seed: int
    lengths: tuple             # ("fixed", [..]) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    pool_blocks: int = 0       # fixed pool size; 0 = used blocks + pool_slack
    pool_slack: float = 0.10
    partition: int = 0         # tokens per split-context partition the benchmark uses (0 = none)
    bs: int = 16
    cow: dict = field(default_factory=dict)  # prompts, samples, prompt_len, r_max, tail_lo, tail_hi
    chunk: tuple = ()          # several new tokens per sequence: ("uniform", lo, hi) | ("all",)
    prefix: dict = field(default_factory=dict)  # shared, tail_lo, tail_hi, vocab

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)


CONFIGS = {
    "tiny": Spec("tiny", "f32", 4, 8, 8, 64, seed=0, lengths=("fixed", [1, 17, 100, 250]),
                 pool_blocks=64),
    "7b": Spec("7b", "bf16", 64, 32, 32, 128, seed=1, lengths=("uniform", 128, 2048)),
    "13b": Spec("13b", "bf16", 128, 40, 40, 128, seed=2, lengths=("lognormal", 500.0, 0.7, 16, 2048)),
    "gqa": Spec("gqa", "bf16", 16, 64, 8, 128, seed=3, lengths=("uniform", 8192, 32768), partition=512),
    "cow": Spec("cow", "bf16", 128, 32, 32, 128, seed=4, lengths=("cow",),
                cow=dict(prompts=16, samples=8, prompt_len=1024, r_max=15, tail_lo=1, tail_hi=256)),
    # several new tokens per sequence (multi-query attention, causal within the chunk)
    # requests sharing one system prompt through the prefix cache
    # the COW batch on a 64/8-head GQA layer: 8 samples x 8 query heads share
    # each prompt block (a study workload for the shared-prefix decode)
    "cow_gqa8": Spec("cow_gqa8", "bf16", 128, 64, 8, 128, seed=9, lengths=("cow",),
                     cow=dict(prompts=16, samples=8, prompt_len=1024, r_max=15, tail_lo=1,
                              tail_hi=256)),
    # the GQA batch at head_dim 64 (a study workload for the matrix-core
    # decode kernel's 64-dim tiles)
    "gqa_d64": Spec("gqa_d64", "bf16", 16, 64, 8, 64, seed=8, lengths=("uniform", 8192, 32768),
                    partition=512),
    # the GQA recipe in fp32 with shorter contexts (a study workload for fp32
    # grouped heads on the fp32 matrix-core kernel)
    "gqa_f32": Spec("gqa_f32", "f32", 16, 64, 8, 128, seed=10, lengths=("uniform", 2048, 8192),
                    partition=512),
    "prefix": Spec("prefix", "bf16", 128, 32, 32, 128, seed=7, lengths=("prefix",),
                   prefix=dict(shared=1024, tail_lo=16, tail_hi=512, vocab=32000)),
    "13b_verify4": Spec("13b_verify4", "bf16", 128, 40, 40, 128, seed=5,
                        lengths=("lognormal", 500.0, 0.7, 16, 2048), chunk=("uniform", 4, 4)),
    "gqa_chunk512": Spec("gqa_chunk512", "bf16", 16, 64, 8, 128, seed=6,
                         lengths=("uniform", 1024, 8192), chunk=("uniform", 512, 512)),
    # the same chunks at head_dim 64 (a study workload for the chunk kernel's
    # 128-byte rows)
    "gqa_chunk512_d64": Spec("gqa_chunk512_d64", "bf16", 16, 64, 8, 64, seed=11,
                             lengths=("uniform", 1024, 8192), chunk=("uniform", 512, 512)),
    # a grouped-head layer (4 query heads per kv head) over the 13b length mix:
    # a study workload for short contexts on the matrix-core decode kernel
    "gqa_short": Spec("gqa_short", "bf16", 128, 32, 8, 128, seed=12,
                      lengths=("lognormal", 500.0, 0.7, 16, 2048)),
}


def torch_dtype(spec):
    return torch.float32 if spec.dtype == "f32" else torch.bfloat16


def draw_lengths(spec, rng):
    """Final context lengths (history + the step's tokens), int64 [B].

    For cow also returns (prompt_lens [prompts], tail_lens [B]); for prefix
    ("prefix", shared prompt token ids, per-request tail token ids)."""
    kind = spec.lengths[0]
    if kind == "fixed":
        ctx = np.asarray(spec.lengths[1], dtype=np.int64)
        assert ctx.shape == (spec.B,)
        return ctx, None
    if kind == "uniform":
        lo, hi = spec.lengths[1], spec.lengths[2]
        return rng.integers(lo, hi, size=spec.B, endpoint=True).astype(np.int64), None
    if kind == "lognormal":
        med, sigma, lo, hi = spec.lengths[1:]
        raw = np.exp(rng.normal(math.log(med), sigma, size=spec.B))
        return np.clip(np.rint(raw), lo, hi).astype(np.int64), None
    if kind == "prefix":
        c = spec.prefix
        tails = rng.integers(c["tail_lo"], c["tail_hi"], size=spec.B, endpoint=True)
        shared = rng.integers(0, c["vocab"], size=c["shared"])
        tail_ids = [rng.integers(0, c["vocab"], size=int(t)) for t in tails]
        ctx = (c["shared"] + tails).astype(np.int64)
        return ctx, ("prefix", shared, tail_ids)
    if kind == "cow":
        c = spec.cow
        r = rng.integers(1, c["r_max"], size=c["prompts"], endpoint=True)
        prompt = c["prompt_len"] - r
        tails = rng.integers(c["tail_lo"], c["tail_hi"], size=c["prompts"] * c["samples"], endpoint=True)
        ctx = np.repeat(prompt, c["samples"]) + tails
        return ctx.astype(np.int64), (prompt.astype(np.int64), tails.astype(np.int64))
    raise ValueError(kind)


def _populate(spec, bm, ctx, cow_parts, n_new):
    """Drive a block manager through the workload's history and its step.

    Returns seq ids, the step's slots, the step's (src, dst) copy pairs, and
    for every step token its batch index and logical position.
    """
    seqs = []
    step_slots = []
    step_pairs = []
    step_seq = []
    step_pos = []

    def step(i, sid, n):
        start = bm.seq_len(sid)
        slots, pairs = bm.append(sid, n)
        step_slots.extend(slots)
        step_pairs.extend(pairs)
        step_seq.extend([i] * n)
        step_pos.extend(range(start, start + n))

    if cow_parts is not None and isinstance(cow_parts[0], str):
        # requests share the system prompt's full blocks through the prefix
        # cache: the first request registers them, the others reuse them
        _, shared, tail_ids = cow_parts
        for s in range(spec.B):
            tokens = np.concatenate([shared, tail_ids[s]]).astype(np.int32)
            sid, n_cached = bm.add_seq_cached(tokens[:-1])
            seqs.append(sid)
            bm.append_tokens(sid, tokens[n_cached:-1])       # history (untimed)
        for i, sid in enumerate(seqs):
            start = bm.seq_len(sid)
            tokens = np.concatenate([shared, tail_ids[i]]).astype(np.int32)
            slots, pairs = bm.append_tokens(sid, tokens[-1:])  # the step's token
            step_slots.extend(slots)
            step_pairs.extend(pairs)
            step_seq.append(i)
            step_pos.append(start)
    elif cow_parts is None:
        for s in range(spec.B):
            sid = bm.add_seq()
            seqs.append(sid)
            bm.append(sid, int(ctx[s]) - int(n_new[s]))   # history (untimed)
        for i, sid in enumerate(seqs):
            step(i, sid, int(n_new[i]))                    # the step's tokens
    else:
        prompt, tails = cow_parts
        c = spec.cow
        for p in range(c["prompts"]):
            parent = bm.add_seq()
            bm.append(parent, int(prompt[p]))          # prompt prefill (untimed)
            group = [parent] + [bm.fork(parent) for _ in range(c["samples"] - 1)]
            seqs.extend(group)
        for i, sid in enumerate(seqs):
            step(i, sid, int(tails[i]))                # divergent tails
    return seqs, step_slots, step_pairs, step_seq, step_pos


@dataclass
class Tables:
    spec: Spec
    NB: int
    MB: int
    free_order: np.ndarray      # int32 [NB]
    context_lens: np.ndarray    # int32 [B]
    block_tables: np.ndarray    # int32 [B, MB], unused = -1 (after the step)
    positions: np.ndarray       # int32 [B], the last position of each sequence
    slots: np.ndarray           # int32 [T], the step's slots (from the block manager)
    step_seq: np.ndarray        # int32 [T], batch index of each step token
    step_pos: np.ndarray        # int32 [T], logical position of each step token
    pairs: np.ndarray           # int32 [n, 2], the step's copy-on-write pairs
    query_start: np.ndarray     # int32 [B + 1], the step's new tokens per sequence (prefix sums)
    seqs: list
    bm: object


def draw_new_tokens(spec, ctx, rng):
    """New tokens per sequence in the step: 1 for a decode step; for a chunk
    workload U{lo..hi} clipped to the context, or the whole context ("all")."""
    if not spec.chunk:
        return np.ones(len(ctx), dtype=np.int64)
    if spec.chunk[0] == "all":
        return ctx.copy()
    lo, hi = spec.chunk[1], spec.chunk[2]
    return np.minimum(rng.integers(lo, hi, size=len(ctx), endpoint=True), ctx).astype(np.int64)


def make_tables(spec, bm_factory):
    """Block tables for `spec` built by `bm_factory(num_blocks, block_size, free_order)`."""
    rng = np.random.default_rng(spec.seed)
    ctx, cow_parts = draw_lengths(spec, rng)
    n_new = draw_new_tokens(spec, ctx, rng)
    if spec.pool_blocks:
        NB = spec.pool_blocks
    else:
        # dry run in an ample pool to count the blocks the workload holds
        big = int(sum(int(c) for c in ctx)) + spec.B + 16
        probe = bm_factory(big, spec.bs, np.arange(big, dtype=np.int32))
        _populate(spec, probe, ctx, cow_parts, n_new)
        used = big - probe.num_free()
        NB = int(math.ceil(used * (1.0 + spec.pool_slack)))
    free_order = rng.permutation(NB).astype(np.int32)
    bm = bm_factory(NB, spec.bs, free_order)
    seqs, slots, pairs, step_seq, step_pos = _populate(spec, bm, ctx, cow_parts, n_new)
    MB = max(len(bm.block_table(s)) for s in seqs)
    bt = np.asarray(bm.tables_array(seqs, MB), dtype=np.int32).reshape(spec.B, MB)
    lens = np.asarray([bm.seq_len(s) for s in seqs], dtype=np.int32)
    return Tables(spec=spec, NB=NB, MB=MB, free_order=free_order, context_lens=lens,
                  block_tables=bt, positions=(lens - 1).astype(np.int32),
                  slots=np.asarray(slots, dtype=np.int32),
                  step_seq=np.asarray(step_seq, dtype=np.int32),
                  step_pos=np.asarray(step_pos, dtype=np.int32),
                  pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
                  query_start=np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32),
                  seqs=seqs, bm=bm)


@dataclass
class Values:
    q: torch.Tensor         # [B, Hq, D]; chunk workloads: [T, Hq, D], one row per new token
    k_cache: torch.Tensor   # [NB, Hkv, bs, D]
    v_cache: torch.Tensor
    k_new: torch.Tensor     # [T, Hkv, D]
    v_new: torch.Tensor


def make_values(spec, NB, T, device="cpu"):
    """N(0,1) values in the workload's element type, drawn on `device`.

    The same seed gives the same values on the CPU every time; a GPU
    generator gives a different (still seeded) stream."""
    g = torch.Generator(device=device)
    g.manual_seed(spec.seed)
    dt = torch_dtype(spec)

    def draw(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(dt)

    q = draw(T if spec.chunk else spec.B, spec.Hq, spec.D)
    k = draw(NB, spec.Hkv, spec.bs, spec.D)
    v = draw(NB, spec.Hkv, spec.bs, spec.D)
    kn = draw(T, spec.Hkv, spec.D)
    vn = draw(T, spec.Hkv, spec.D)
    return Values(q, k, v, kn, vn)


def to_bits(t):
    """A torch tensor's raw element bits as numpy (uint16 for bf16, float32 for fp32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)
