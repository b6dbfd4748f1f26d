"""Benchmark of the paged decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 13b]

A step is one pass of the whole path over one batch of seeded synthetic
input, all of it already resident in HBM:
  copy-on-write block copies (workloads that have any) -> slot mapping and
  cache write of the step's new K/V (one fused launch) -> decode attention
  over every sequence (or causal attention of each sequence's new tokens).
W untimed steps, then exactly K timed steps between two device
synchronisations. HIP events on the launch stream bracket the decode call of
every n-th timed step (20 calls by default), inside the timed region, so the
decode kernel's average duration (and from it its achieved HBM bandwidth
against the 8 TB/s peak) is measured live.

Printed: one JSON line. `value` is the step's algorithmic HBM bytes over the
step time (GB/s); `decode_tokens_per_s` is the step's new tokens / step time
(one per sequence for a decode step). The `roofline` object covers the
attention kernel (bound: HBM, or the matrix peak for a chunk workload whose
arithmetic intensity passes the ridge); its `traffic` comes from the
committed rocprofv3 counter summary for that kernel and workload, or is null
when the kernel sources have changed since those counters were taken. The
`cpu_baseline` object is the fp64 CPU oracle on the same inputs, on this
host's cores (test infrastructure, timed for reference only).
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense matrix peak (fp32: vector peak)
PROFILES = os.path.join(ROOT, "profiles")
# Sources the decode kernels are built from: counters taken on another
# version of these no longer describe the kernel that runs.
DECODE_SOURCES = ["paged_kv_cache_410_amd/csrc/decode_valu.hip",
                  "paged_kv_cache_410_amd/csrc/decode_mfma.hip",
                  "paged_kv_cache_410_amd/csrc/decode_mfma_f32.hip",
                  "paged_kv_cache_410_amd/csrc/chunk_mfma.hip",
                  "paged_kv_cache_410_amd/csrc/chunk_ring.h",
                  "paged_kv_cache_410_amd/csrc/decode_reduce.hip",
                  "paged_kv_cache_410_amd/csrc/pa_device.h",
                  "paged_kv_cache_410_amd/csrc/pa_launch.h",
                  "paged_kv_cache_410_amd/csrc/pa_api.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_sources_sha():
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per decode launch from the committed counter summary, or None."""
    path = os.path.join(PROFILES, f"pa_decode_{workload}_pmc.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m_sha = re.search(r"^decode_sources_sha:\s*(\w+)", text, re.M)
    m_tr = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_tr:
        return None, "counter summary unreadable"
    if m_sha.group(1) != decode_sources_sha():
        return None, "decode sources changed since the counters were taken"
    return float(m_tr.group(1)), "ok"


def algorithmic_bytes(spec, tb):
    """Bytes the method must move, each element once (not what a kernel moves),
    and its flops (QK and PV, two per multiply-add)."""
    e = 4 if spec.dtype == "f32" else 2
    ctx = tb.context_lens.astype("int64")
    n = (tb.query_start[1:] - tb.query_start[:-1]).astype("int64")
    rows = int(n.sum()) if spec.chunk else spec.B
    kv = int(ctx.sum()) * spec.Hkv * spec.D * 2 * e                # every K and V row once
    qo = 2 * rows * spec.Hq * spec.D * e                           # q in, out
    meta = 4 * (int(((ctx + 15) // 16).sum()) + spec.B)            # table entries + lengths
    if spec.chunk:
        meta += 4 * (spec.B + 1)                                   # query_start
        # row i of a chunk of n attends over ctx - n + i + 1 tokens
        attended = int((n * (ctx - n) + n * (n + 1) // 2).sum())
    else:
        attended = int(ctx.sum())
    decode = kv + qo + meta
    T = len(tb.slots)
    write = 2 * 2 * T * spec.Hkv * spec.D * e                      # K, V rows: read + write
    slots = 4 * 4 * T                                              # seq, pos, table entry, slot
    copy = 2 * 2 * len(tb.pairs) * spec.Hkv * 16 * spec.D * e      # K, V blocks: read + write
    return dict(decode=decode, write=write, slots=slots, copy=copy,
                step=decode + write + slots + copy, flops=4 * attended * spec.Hq * spec.D)


def unique_decode_bytes(spec, tb):
    """For shared blocks: K/V bytes of each distinct (physical block, token) read."""
    e = 4 if spec.dtype == "f32" else 2
    # a shared block is read by each of its sharers; count its used rows once
    last_rows = {}
    for s in range(spec.B):
        L = int(tb.context_lens[s])
        for j in range((L + 15) // 16):
            b = int(tb.block_tables[s, j])
            last_rows[b] = max(last_rows.get(b, 0), min(16, L - 16 * j))
    rows = sum(last_rows.values())
    return rows * spec.Hkv * spec.D * 2 * e + 2 * spec.B * spec.Hq * spec.D * e


# Oracle work is bounded to about this many (row, token, dim) products per run
# (roughly 10-20 s on 16 host threads).
ORACLE_WORK_CAP = 1.5e11


def cpu_baseline(st_inputs, spec, tb, budget_s):
    """The fp64 oracle on the host, on the same inputs. The sample is the whole
    step when its work fits ORACLE_WORK_CAP, else the first k sequences that do;
    it is repeated until about `budget_s` seconds have been spent (at least
    once). Returns (sample rows' oracle output, row slice, the baseline object)."""
    import numpy as np

    import oracle
    q, k, v = st_inputs
    oracle.build()
    threads = oracle.max_threads()
    ctx = tb.context_lens.astype(np.int64)
    n = (tb.query_start[1:] - tb.query_start[:-1]).astype(np.int64)
    if spec.chunk:
        work = (n * (ctx - n) + n * (n + 1) // 2) * spec.Hq * spec.D * 2
    else:
        work = ctx * spec.Hq * spec.D * 2
    k_seq = max(1, int(np.searchsorted(np.cumsum(work), ORACLE_WORK_CAP, side="right")))
    k_seq = min(k_seq, spec.B)
    sub = type(tb)(**{**tb.__dict__, "context_lens": tb.context_lens[:k_seq],
                      "block_tables": tb.block_tables[:k_seq],
                      "query_start": tb.query_start[:k_seq + 1]})
    rows = slice(0, int(tb.query_start[k_seq])) if spec.chunk else slice(0, k_seq)
    sample_bytes = algorithmic_bytes(type(spec)(**{**spec.__dict__, "B": k_seq}), sub)["decode"]
    times = []
    out = None
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if spec.chunk:
            out = oracle.multi_query(q[rows], k, v, sub.block_tables, sub.context_lens,
                                     sub.query_start, spec.scale)
        else:
            out = oracle.decode(q[rows], k, v, sub.block_tables, sub.context_lens, spec.scale)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s or len(times) >= 20:
            break
    t = sorted(times)[len(times) // 2]
    what = "the whole" if k_seq == spec.B else f"the first {k_seq} of {spec.B} sequences of the"
    return out, rows, dict(
        value=round(sample_bytes / t / 1e9, 3), unit="GB/s", cores=threads, kind="oracle",
        host_cpus=os.cpu_count(), omp_num_threads=os.environ.get("OMP_NUM_THREADS"),
        sample=f"{what} {spec.name} step's attention ({spec.Hq} heads; fp64 oracle, OpenMP over "
               f"(query row, head)), median of {len(times)} runs; GB/s on that sample's "
               f"algorithmic bytes",
        seconds_per_run=round(t, 4), tokens_per_s=round((rows.stop - rows.start) / t, 2))


def host_bits(t):
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="13b",
                    choices=["tiny", "7b", "13b", "gqa", "gqa_d64", "gqa_f32", "cow", "cow_gqa8",
                             "prefix", "13b_verify4", "gqa_chunk512", "gqa_chunk512_d64",
                             "gqa_short"])
    ap.add_argument("--partition", type=int, default=None,
                    help="split-context partition in tokens (default: the library's choice, "
                         "or the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (e.g. under a counter profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--controls", choices=["all", "copy", "none"], default="all",
                    help="copy: only the device-to-device copy (profiled runs, where the "
                         "sequential-table launches would mix into the attention kernel's "
                         "statistics)")
    ap.add_argument("--no-controls", action="store_true", help="same as --controls none")
    ap.add_argument("--no-group", action="store_true",
                    help="attend over blocks shared by several sequences once per sequence "
                         "(pa_decode) instead of once per group of sharers (pa_decode_shared)")
    ap.add_argument("--max-group", type=int, default=16,
                    help="most sequences per group of sharers (pa_decode_shared)")
    ap.add_argument("--shared-partition", type=int, default=None,
                    help="partition length of the shared part in pa_decode_shared (0 = none; "
                         "default: the library's choice)")
    ap.add_argument("--event-every", type=int, default=None,
                    help="time the attention call with HIP events on every n-th timed step "
                         "(a pair of events between two kernels lengthens that step by about "
                         "6 microseconds; default: steps // 20, so that 20 calls are timed)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once as a HIP graph and replayed; the "
                         "replayed step then sets value and ms_per_step")
    args = ap.parse_args()
    if args.no_controls:
        args.controls = "none"

    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sequences or kv heads would shard with no exchange, but no multi-GPU run is "
              "built here)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_410_amd as pa
    from paged_kv_cache_410_amd import _lib, workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(_lib.LIB_PATH):
        print("bench.py: libpa.so is not built (python -m paged_kv_cache_410_amd.build)",
              file=sys.stderr)
        sys.exit(1)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = workloads.CONFIGS[args.workload]
    log(f"[bench] workload {spec.name}: building tables with the native block manager")
    tb = workloads.make_tables(spec, pa.BlockManager)
    T = len(tb.slots)
    vals = workloads.make_values(spec, tb.NB, T, device="cuda")
    k_cache, v_cache = vals.k_cache, vals.v_cache
    q, k_new, v_new = vals.q, vals.k_new, vals.v_new
    bt = torch.from_numpy(tb.block_tables).to(dev)
    cl = torch.from_numpy(tb.context_lens).to(dev)
    step_seq = torch.from_numpy(tb.step_seq).to(dev)
    step_pos = torch.from_numpy(tb.step_pos).to(dev)
    pairs = torch.from_numpy(np.ascontiguousarray(tb.pairs)).to(dev)
    max_ctx = int(tb.context_lens.max())
    rows = q.shape[0]                       # query rows: B, or every new token of a chunk
    qs = torch.from_numpy(tb.query_start).to(dev)
    max_q = int(np.diff(tb.query_start).max())
    partition = args.partition
    if partition is None:
        partition = spec.partition or pa.default_partition(rows, spec.Hq, spec.Hkv, spec.D,
                                                           max_ctx)
    ws_bytes = pa.decode_workspace_bytes(rows, spec.Hq, spec.D, max_ctx, partition)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    shared_kv = pa.shares_blocks(tb.block_tables)  # the caller's manager knows; so do the tables
    nbytes = algorithmic_bytes(spec, tb)
    log(f"[bench] NB={tb.NB} MB={tb.MB} T={T} pairs={len(tb.pairs)} max_ctx={max_ctx} "
        f"partition={partition} decode bytes={nbytes['decode'] / 1e9:.4f} GB")

    # The copy-on-write copies read blocks the step's writes then change, so a
    # repeated step starts from pools saved before the first one.
    if len(tb.pairs):
        dst = torch.from_numpy(tb.pairs[:, 1].astype(np.int64)).to(dev)
        k_saved, v_saved = k_cache[dst].clone(), v_cache[dst].clone()

    # Blocks shared by several sequences: read once per group of sharers.
    groups = None
    if shared_kv and not spec.chunk and not args.no_group and spec.dtype == "bf16" \
            and spec.D == 128:
        # groups of up to 16 sequences (past 16 columns per kv head the group
        # pass runs on the chunk kernel); once grouped, a pass reads through
        # the caches only where blocks still repeat within it
        plan = pa.shared_plan(tb.block_tables, tb.context_lens, spec.Hq, spec.Hkv,
                              args.max_group)
        if plan is not None:
            sp = plan["partition"] if args.shared_partition is None else args.shared_partition
            groups = dict(group_start=torch.from_numpy(plan["group_start"]).to(dev),
                          seq_shared=torch.from_numpy(plan["seq_shared"]).to(dev),
                          max_group=plan["max_group"], max_shared=plan["max_shared"],
                          partition=sp, own_repeats=plan["shared_kv"],
                          groups_overlap=plan["groups_overlap"],
                          workspace=torch.empty(max(1, pa.decode_shared_workspace_bytes(
                              spec.B, spec.Hq, spec.D, plan["max_shared"], sp)),
                              dtype=torch.uint8, device=dev))
            log(f"[bench] {len(plan['group_start']) - 1} groups of sharers, shared tokens "
                f"{sorted(set(plan['seq_shared'].tolist()))}, shared-part partition {sp}")

    def attend(tables, dest, shared):
        if groups is not None and tables is bt:
            pa.decode_shared(q, k_cache, v_cache, tables, cl, groups["group_start"],
                             groups["seq_shared"], spec.scale, max_ctx, groups["max_group"],
                             groups["max_shared"], partition=groups["partition"], out=dest,
                             workspace=groups["workspace"],
                             shared_kv=shared and groups["own_repeats"],
                             groups_overlap=shared and groups["groups_overlap"])
        elif spec.chunk:
            pa.multi_query(q, k_cache, v_cache, tables, cl, qs, spec.scale, max_ctx, max_q,
                           partition=partition, out=dest, workspace=workspace, shared_kv=shared)
        else:
            pa.decode(q, k_cache, v_cache, tables, cl, spec.scale, max_ctx, partition=partition,
                      out=dest, workspace=workspace, shared_kv=shared)

    def step(ev=None, parts=False):
        # ev: events before and after the attention call; with `parts`, also
        # before the copies and before the cache write (ev[2], ev[3])
        if parts:
            ev[2].record()
        if len(tb.pairs):
            pa.copy_blocks(k_cache, v_cache, pairs)
        if parts:
            ev[3].record()
        # slot mapping and the cache write, one launch
        pa.append_kv(k_new, v_new, k_cache, v_cache, bt, step_pos, seq_ids=step_seq,
                     slots_out=slots)
        if ev is not None:
            ev[0].record()
        attend(bt, out, shared_kv)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4))
           for _ in range(args.steps)]   # [2], [3]: the untimed per-kernel pass below
    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    every = max(1, args.steps // 20 if args.event_every is None else args.event_every)
    for i in range(args.steps):
        step(evs[i] if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [e[0].elapsed_time(e[1]) for e in evs[::every]]
    # The copies and the cache write, timed on their own in an untimed pass
    # (events between them would lengthen the timed step).
    for e in evs:
        step(e, parts=True)
    torch.cuda.synchronize()
    copy_ms = [e[2].elapsed_time(e[3]) for e in evs]
    write_ms = [e[3].elapsed_time(e[0]) for e in evs]
    pass_dec_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)   # cross-check of dec_ms
    ms_step = wall * 1e3 / args.steps
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    dec_sorted = sorted(dec_ms)
    dec_med_ms = dec_sorted[len(dec_ms) // 2]
    dec_p10_ms = dec_sorted[len(dec_ms) // 10]
    dec_p90_ms = dec_sorted[min(len(dec_ms) - 1, (9 * len(dec_ms)) // 10)]
    log(f"[bench] step {ms_step * 1e3:.1f} us, decode avg {dec_avg_ms * 1e3:.1f} us "
        f"(median {dec_med_ms * 1e3:.1f})")

    graph = None
    if args.graph:
        # The same launches captured once and replayed: no host launch latency
        # between the step's kernels. Every replay must reproduce the eager
        # step's output bits: the kernels are deterministic, and a repeated
        # step leaves every slot the attention reads as the first step left
        # it (a repeated copy-on-write step may change slots past contexts).
        eager_out = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        match = True
        for _ in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            match = match and torch.equal(out, eager_out)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} graph replays")
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        match = match and torch.equal(out, eager_out)
        graph = dict(ms_per_step=round(gms, 5), eager_ms_per_step=round(ms_step, 5),
                     replays_match_eager=bool(match))
        log(f"[bench] graph step {gms * 1e3:.1f} us (eager {ms_step * 1e3:.1f} us), "
            f"replays match eager: {match}")
        if not match:
            print("bench.py: graph replays differ from the eager step", file=sys.stderr)
            sys.exit(1)
        ms_step = gms
        del g

    controls = {}
    if args.controls != "none":
        # A plain device-to-device copy of the decode's K/V byte count: the
        # bandwidth a streaming kernel reaches here (and the reference the HBM
        # counters are scaled by).
        n = nbytes["decode"] // 2 // 16 * 16
        a = torch.empty(n // 2, dtype=torch.int16, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / reps
        controls["d2d_copy"] = dict(bytes_read=n, bytes_written=n, us=round(cms * 1e3, 2),
                                    GBps=round(2 * n / (cms * 1e-3) / 1e9, 1))
        del a, b
        # The same attention over sequentially placed blocks (sequence s holds
        # blocks base_s, base_s + 1, ...): what the block-table indirection and
        # scattered placement cost against a contiguous cache. The pool's
        # contents are whatever it holds; only the time is used.
        nblk = -(-tb.context_lens.astype(np.int64) // 16)
        if args.controls == "all" and int(nblk.sum()) <= tb.NB:
            seq_bt = np.full_like(tb.block_tables, -1)
            base = np.concatenate([[0], np.cumsum(nblk)[:-1]])
            for s_i, (b0, nb_i) in enumerate(zip(base, nblk)):
                seq_bt[s_i, :nb_i] = np.arange(b0, b0 + nb_i, dtype=np.int32)
            seq_bt_d = torch.from_numpy(seq_bt).to(dev)
            scratch_out = torch.empty_like(out)
            for _ in range(3):
                attend(seq_bt_d, scratch_out, False)
            e0.record()
            for _ in range(reps):
                attend(seq_bt_d, scratch_out, False)
            e1.record()
            torch.cuda.synchronize()
            ims = e0.elapsed_time(e1) / reps
            controls["sequential_tables"] = dict(
                us=round(ims * 1e3, 2), GBps=round(nbytes["decode"] / (ims * 1e-3) / 1e9, 1),
                paged_over_sequential=round(dec_avg_ms / ims, 4))
            del scratch_out, seq_bt_d

    if len(tb.pairs):
        k_cache[dst], v_cache[dst] = k_saved, v_saved
        step()
        torch.cuda.synchronize()

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        log("[bench] oracle on the host (cpu_baseline)")
        inputs = (host_bits(q), host_bits(k_cache), host_bits(v_cache))
        if spec.dtype == "f32":
            inputs = tuple(x.view(np.float32) for x in inputs)
        expect, sample_rows, cpu = cpu_baseline(inputs, spec, tb, args.cpu_seconds)
        got = out[sample_rows].float().cpu().numpy().astype(np.float64)
        parity = float(np.max(np.abs(got - expect)))
        log(f"[bench] oracle {cpu['seconds_per_run']} s/run on {cpu['cores']} threads; "
            f"max abs err vs oracle {parity:.3e}")

    traffic, why = read_traffic(spec.name)
    value = nbytes["step"] / (ms_step * 1e-3) / 1e9
    # The attention kernel's bound: HBM unless its arithmetic intensity passes
    # the ridge of the matrix peak over the HBM peak.
    mpeak = MFMA_PEAK_TFLOPS[spec.dtype]
    intensity = nbytes["flops"] / nbytes["decode"]
    if intensity > mpeak * 1e12 / (HBM_PEAK_GBPS * 1e9):
        bound, unit, peak = ("mfma" if spec.dtype == "bf16" else "alu"), "TFLOP/s", mpeak
        achieved = nbytes["flops"] / (dec_avg_ms * 1e-3) / 1e12
    else:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBPS
        # Blocks shared by several sequences are read from HBM once; their
        # repeats come from the caches. The HBM roofline therefore counts each
        # block's used rows once; the logical rate is reported beside it.
        hbm_bytes = unique_decode_bytes(spec, tb) if shared_kv else nbytes["decode"]
        achieved = hbm_bytes / (dec_avg_ms * 1e-3) / 1e9
    achieved_median = achieved * dec_avg_ms / dec_med_ms
    line = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + decode tokens/sec",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {"workload": f"{spec.name}: B={spec.B} Hq={spec.Hq} Hkv={spec.Hkv} "
                               f"D={spec.D} block_size=16 {spec.dtype}",
                   "batch": spec.B, "num_q_heads": spec.Hq, "num_kv_heads": spec.Hkv,
                   "head_dim": spec.D, "block_size": 16, "partition": partition,
                   "max_ctx": max_ctx, "mean_ctx": round(float(tb.context_lens.mean()), 1),
                   "pool_blocks": tb.NB, "new_tokens": T, "query_rows": rows,
                   "cow_pairs": len(tb.pairs), "shared_kv": shared_kv,
                   "shared_groups": (None if groups is None else
                                     dict(groups=int(groups["group_start"].shape[0] - 1),
                                          max_shared=groups["max_shared"],
                                          shared_partition=groups["partition"],
                                          shared_parts_overlap=groups["groups_overlap"],
                                          own_blocks_repeat=groups["own_repeats"])),
                   "parallelism": "none (one GPU)"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "attention_TFLOPs": round(nbytes["flops"] / (dec_avg_ms * 1e-3) / 1e12, 2),
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_us_median": round(dec_med_ms * 1e3, 2),
        "decode_us_p10_p90": [round(dec_p10_ms * 1e3, 2), round(dec_p90_ms * 1e3, 2)],
        "decode_timed_calls": len(dec_ms),
        "decode_timed_calls_note": f"{len(dec_ms)} of {args.steps} timed steps (every {every})",
        "decode_us_median_separate_pass": round(pass_dec_ms[len(pass_dec_ms) // 2] * 1e3, 2),
        "write_us": round(sum(write_ms) / len(write_ms) * 1e3, 2),
        "copy_us": round(sum(copy_ms) / len(copy_ms) * 1e3, 2) if len(tb.pairs) else None,
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "achieved_median": round(achieved_median, 1),
                     "frac_median": round(achieved_median / peak, 4),
                     "traffic": traffic,
                     "kernel": ("pa_decode_shared (group pass, tail pass, merge)"
                                if groups is not None else "attention (one launch per step"
                                + (", plus the partition merge)" if ws_bytes else ")")),
                     "traffic_note": why, "intensity_flop_per_byte": round(intensity, 2)},
        "cpu_baseline": cpu,
        "parity_max_abs_err_vs_oracle": parity,
        "controls": controls,
        "graph": graph,
    }
    if shared_kv:
        # blocks shared by several sequences: K/V bytes of each block counted once
        ub = unique_decode_bytes(spec, tb)
        line["unique_decode_bytes"] = ub
        line["roofline_unique_GBps"] = round(ub / (dec_avg_ms * 1e-3) / 1e9, 1)
        line["roofline"]["achieved_logical_GBps"] = round(
            nbytes["decode"] / (dec_avg_ms * 1e-3) / 1e9, 1)
        line["roofline"]["bytes"] = "unique (each shared block's used rows once)"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
