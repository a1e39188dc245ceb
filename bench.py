#!/usr/bin/env python3
"""PagedAttention decode benchmark on one MI355X.

One step = the decode step of the hot path over one batch: store each
sequence's new key/value token, split-K decode over the whole context, and
the split-K reduce.  --mode fused (default) makes it one call of
paged_attention_decode_step (the store inside the decode launch where the
shape allows, then the reduce);
--mode separate makes it paged_kv_write, paged_attention_decode_partials and
paged_attention_splitk_reduce.  Per-kernel times always come from the
separate launches.  The KV cache is prefilled once through the same library;
R copies of the pools ("layers", at least two and at least 2 GB of cache)
are cycled so that each step reads its KV from HBM, not from the 256 MB
Infinity Cache.

--prefill times chunked prefill instead: one step stores every sequence's
chunk of new key/value rows (paged_kv_write) and runs the causal attention
of the chunk's query rows over the paged cache (paged_attention_prefill), on
the chunked-prefill workload (16 sequences, 512-row chunks over 1k-8k
contexts); its roofline is the bf16 matrix-core peak.

Prints ONE JSON line on stdout; details go to stderr.

    python bench.py [--steps K] [--warmup W] [--config 3] [--gpus 1] [--mode fused]
    python bench.py --prefill
    python bench.py --swap

--swap times moving whole sequences of the GQA workload to a pinned host
pool and back: staged through a device pool and moved as whole-run
asynchronous copies (the headline), and by the block-move kernel straight
to the host; then
each form on a second stream beside a split-K decode of the other
sequences.  Its roofline is the host link (PCIe 5.0 x16, 64 GB/s each way).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode µs/step + effective KV GB/s as % of MI355X HBM peak"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, vendor figure
HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction
SWAP_METRIC = "KV swap to host and back: µs per round trip + host-link GB/s"
PREFILL_METRIC = "chunked prefill µs/step (store chunk + causal attention) + matrix-core TFLOP/s"
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}
# sources of the decode kernels: a counter file taken on other sources is stale
SRC_FILES = ("decode.hip", "decode_valu.h", "decode_f32.hip", "decode_bf16.hip", "decode_fp8.hip",
             "decode_mfma.hip", "decode_prefix.hip", "decode_common.h", "pkv_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = bf16 GQA)")
    p.add_argument("--partition", type=int, default=None, help="split-K tokens (default: workload's)")
    p.add_argument("--layers", type=int, default=0, help="pool copies cycled per step (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=400_000,
                   help="token budget of the oracle's timed sample")
    p.add_argument("--traffic-file", default=None)
    p.add_argument("--mode", choices=("fused", "separate"), default="fused")
    p.add_argument("--schedule", choices=("splitk", "streamk", "prefix", "queue"), default="splitk",
                   help="split-K partitions of --partition tokens, stream-K persistent waves, "
                        "the shared-prefix decode (shared blocks read once per 32 query rows), or "
                        "split-K with items taken from a work counter (fp8 matrix-core shape; "
                        "no step form: the store, then the decode and its reduce)")
    p.add_argument("--workers", type=int, default=0, help="stream-K waves (0 = resident count)")
    p.add_argument("--prefill", action="store_true",
                   help="time chunked prefill (store + causal attention) instead of decode")
    p.add_argument("--swap", action="store_true",
                   help="time swapping sequences to a pinned host pool and back")
    p.add_argument("--swap-seqs", type=int, default=16, help="sequences moved per swap")
    return p.parse_args()


def algorithmic_bytes(wl):
    c = wl.cfg
    L = wl.context_lens
    e, eq = ELEM[c.kv_dtype], ELEM[c.q_dtype]
    kv = int(L.sum()) * c.H_kv * c.d * 2 * e
    q = c.S * c.H_q * c.d * eq
    o = q
    tbl = int(((L + c.bs - 1) // c.bs).sum()) * 4 + c.S * 4
    write = c.S * c.H_kv * c.d * 2 * (ELEM[c.src_dtype] + e)
    # unique KV bytes: a shared prefix's full blocks counted once
    shared = (c.prefix // c.bs) * c.bs if c.prefix else 0
    kv_unique = (shared + int((L - shared).sum())) * c.H_kv * c.d * 2 * e if shared else kv
    return {"kv": kv, "kv_unique": kv_unique, "q": q, "o": o, "tables": tbl, "write": write,
            "decode": kv + q + o + tbl, "decode_unique": kv_unique + q + o + tbl,
            "step": kv + q + o + tbl + write}


def src_sha():
    h = hashlib.sha256()
    for f in SRC_FILES:
        with open(os.path.join(ROOT, "paged_kv_cache_211_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(path, workload_key, kernel):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counter runs,
    or None when absent, for another kernel or taken on other sources.
    workload_key names the workload, with "-p<P>" when the launch uses
    another split-K length than the workload's own."""
    path = path or os.path.join(ROOT, "profiles", f"traffic_{workload_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != src_sha() or t.get("kernel") != kernel:
        log(f"traffic file {path} is for another kernel or source; traffic = null")
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, token_budget):
    """Time the oracle (fp64 numpy) on a bounded sample of the same step."""
    import numpy as np

    from oracle import attention as OA
    from oracle.layout import write_kv
    from oracle.replay import OracleState

    c = wl.cfg
    order = np.random.default_rng([c.seed, 9]).permutation(c.S)
    sample, tok = [], 0
    for s in order:
        if sample and tok + int(wl.context_lens[s]) > token_budget:
            continue
        sample.append(int(s))
        tok += int(wl.context_lens[s])
    sample.sort()
    st = OracleState(wl, only_seqs=sample)
    st.run(wl, wl.prefill)
    dec = st.run(wl, wl.decode)
    slots = np.concatenate(dec)
    ks, vs = zip(*(wl.values(op[3], op[4], 1) for op in wl.decode))
    K, V = np.concatenate(ks)[sample], np.concatenate(vs)[sample]
    tables = st.tables(c.S)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    t0 = time.perf_counter()
    write_kv(st.kc, st.vc, K, V, slots[sample], bs=c.bs, src_dtype=c.src_dtype,
             cache_dtype=c.kv_dtype, k_scale=c.k_scale, v_scale=c.v_scale)
    OA.paged_decode(wl.q, c.q_dtype, st.kc, st.vc, tables, wl.context_lens, bs=c.bs,
                    cache_dtype=c.kv_dtype, scale=c.scale, k_scale=c.k_scale, v_scale=c.v_scale,
                    seqs=sample)
    dt = time.perf_counter() - t0
    frac = tok / wl.total_tokens
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(dt / frac * 1e6, 1), "unit": "us/step", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(sample)} of {c.S} sequences, {tok} of {wl.total_tokens} context tokens "
                      f"({100 * frac:.1f}%), timed {dt:.2f} s, scaled by tokens",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model}


def prefill_flops(c, lens, chunks):
    """Algorithmic flops of the causal attention: chunk row i of sequence s
    sees L_s - C_s + i + 1 tokens, 2 d flops each for QK^T and for PV, per
    query head."""
    vis = sum(int(C) * (int(L) - int(C)) + int(C) * (int(C) + 1) // 2 for L, C in zip(lens, chunks))
    return 4 * c.d * c.H_q * vis


def cpu_baseline_prefill(wl, chunks, q_bits, nseq):
    """Time the oracle's prefill on `nseq` sequences, scaled by flops."""
    import numpy as np

    from oracle import attention as OA
    from oracle.replay import OracleState

    c = wl.cfg
    sample = sorted(int(s) for s in np.random.default_rng([c.seed, 9]).permutation(c.S)[:nseq])
    st = OracleState(wl, only_seqs=sample)
    st.run(wl, wl.prefill)
    st.run(wl, wl.decode)
    qs = np.concatenate([[0], np.cumsum(chunks)])
    t0 = time.perf_counter()
    OA.paged_prefill(q_bits, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens, qs,
                     bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale, seqs=sample)
    dt = time.perf_counter() - t0
    frac = (prefill_flops(c, wl.context_lens[sample], chunks[sample])
            / prefill_flops(c, wl.context_lens, chunks))
    return {"value": round(dt / frac * 1e6, 1), "unit": "us/step", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"attention of {len(sample)} of {c.S} sequences ({100 * frac:.1f}% of the "
                      f"flops), timed {dt:.2f} s, scaled by flops; the chunk store not timed",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max((i.get("num_threads") or 1) for i in info) if info else 1
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def main_prefill(args):
    import numpy as np
    import torch

    import synth
    import paged_kv_cache_211_amd as pkv
    from synth import device as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.make(synth.PREFILL["full"])
    wl.cache_limit = 0
    c = wl.cfg
    chunks = synth.prefill_chunks(wl)
    q_bits = synth.prefill_queries(wl, chunks)
    flops = prefill_flops(c, wl.context_lens, chunks)
    T, maxC = int(chunks.sum()), int(chunks.max())
    log(f"[bench] prefill workload {c.key}: S={c.S} H_q={c.H_q} H_kv={c.H_kv} d={c.d} "
        f"bs={c.bs} context {wl.total_tokens} tokens, {T} chunk rows, {flops / 1e9:.1f} GFLOP")
    cache, _ = W.build(wl, poison=False, device=dev)
    inp = cache.decode_inputs(range(c.S), 0)
    tab, lens = inp["block_tables"], inp["context_lens"]
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)).to(dev)
    q = W.to_dev(q_bits, c.q_dtype, dev)
    out = torch.empty_like(q)
    # the chunk's key/value rows and their slots (positions L - C .. L - 1)
    tab_h = tab.cpu().numpy()
    ks, vs, slots = [], [], []
    for s in range(c.S):
        L, C = int(wl.context_lens[s]), int(chunks[s])
        k, v = wl.values(("seq", s), L - C, C)
        ks.append(k)
        vs.append(v)
        pos = np.arange(L - C, L)
        slots.append(tab_h[s, pos // c.bs].astype(np.int64) * c.bs + pos % c.bs)
    K = W.to_dev(np.concatenate(ks), c.src_dtype, dev)
    V = W.to_dev(np.concatenate(vs), c.src_dtype, dev)
    slot_dev = torch.from_numpy(np.concatenate(slots).astype(np.int32)).to(dev)
    kv_bytes = wl.total_tokens * c.H_kv * c.d * 2 * ELEM[c.kv_dtype]
    R = args.layers or max(2, math.ceil(2e9 / kv_bytes))
    layers = [(cache.key_cache, cache.value_cache)]
    for _ in range(R - 1):
        layers.append((cache.key_cache.clone(), cache.value_cache.clone()))

    def attend(i):
        kc, vc = layers[i % R]
        pkv.paged_attention_prefill(out, q, kc, vc, tab, lens, qs, maxC, c.scale)

    def step(i):
        kc, vc = layers[i % R]
        pkv.paged_kv_write(K, V, kc, vc, slot_dev)
        attend(i)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) / args.steps * 1e3
    # the roofline kernel alone, back to back on its stream
    for i in range(args.warmup):
        attend(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        attend(i)
    e1.record()
    torch.cuda.synchronize()
    kern_us = e0.elapsed_time(e1) / args.steps * 1e3
    tflops = flops / (kern_us * 1e-6) / 1e12
    log(f"[bench] prefill step {us_step:.1f} us; attention back to back {kern_us:.1f} us = "
        f"{tflops:.0f} TFLOP/s ({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of "
        f"{MFMA_BF16_PEAK_TFLOPS:.0f}); {R} pool layers")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample ...")
        cpu = cpu_baseline_prefill(wl, chunks, q_bits, 2)
        log(f"[bench] oracle: {cpu['value']} us/step est. ({cpu['sample']})")
    line = {
        "metric": PREFILL_METRIC, "value": round(us_step, 2), "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us_step / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{c.key}: {c.S} seqs, {c.H_q}/{c.H_kv} heads, head_dim {c.d}, "
                               f"block_size {c.bs}, bf16 KV, chunks of {maxC} rows over contexts "
                               f"of {int(wl.context_lens.min())}-{int(wl.context_lens.max())} "
                               f"tokens (seed {c.seed}), {R} pool layers",
                   "global_batch": c.S, "seq_len": int(wl.context_lens.max()),
                   "chunk_rows": T, "parallelism": "single GPU"},
        "kernel_us": {"prefill_attention_back_to_back": round(kern_us, 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel", "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main_swap(args):
    import numpy as np
    import torch

    import synth
    import paged_kv_cache_211_amd as pkv
    from synth import device as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.make(3)
    c = wl.cfg
    cache, step = W.build(wl, poison=False, device=dev)
    n = min(args.swap_seqs, c.S)
    seqs = list(range(n))
    nblocks = sum(len(cache.alloc.block_table(s)) for s in seqs)
    cache.host_pool(nblocks)
    block_bytes = c.H_kv * c.bs * c.d * ELEM[c.kv_dtype]
    moved = nblocks * block_bytes * 2            # key and value pools
    log(f"[bench] swap: {n} sequences, {nblocks} blocks, {moved / 1e6:.1f} MB each way")
    # the kernel alone, on fixed pairs (every device block of the sequences
    # to host slots 0.. and back), K launches each way between events
    dblk = np.concatenate([cache.alloc.block_table(s) for s in seqs]).astype(np.int32)
    hslot = np.arange(nblocks, dtype=np.int32)
    out_pairs = torch.from_numpy(np.stack([dblk, hslot], 1).copy()).to(dev)
    in_pairs = torch.from_numpy(np.stack([hslot, dblk], 1).copy()).to(dev)
    # the staged form: device blocks <-> a contiguous device staging pool (one
    # launch, HBM to HBM), staging pool <-> host slots as whole-run copies
    stage_k, stage_v = pkv.empty_pools(nblocks, c.H_kv, c.d, c.bs, cache.dtype, dev)
    gather_pairs = torch.from_numpy(np.stack([dblk, hslot], 1).copy()).to(dev)   # dev -> stage
    scatter_pairs = torch.from_numpy(np.stack([hslot, dblk], 1).copy()).to(dev)  # stage -> dev
    ident = np.stack([hslot, hslot], 1).copy()                                  # stage <-> host

    def d2h(stream=None, staged=False):
        if staged:
            pkv.paged_kv_swap_blocks(stage_k, stage_v, cache.key_cache, cache.value_cache,
                                     gather_pairs, stream=stream)
            pkv.paged_kv_swap_blocks_memcpy(cache.host_key, cache.host_value, stage_k, stage_v,
                                         ident, stream=stream)
        else:
            pkv.paged_kv_swap_blocks(cache.host_key, cache.host_value, cache.key_cache,
                                     cache.value_cache, out_pairs, stream=stream)

    def h2d(stream=None, staged=False):
        if staged:
            pkv.paged_kv_swap_blocks_memcpy(stage_k, stage_v, cache.host_key, cache.host_value,
                                         ident, stream=stream)
            pkv.paged_kv_swap_blocks(cache.key_cache, cache.value_cache, stage_k, stage_v,
                                     scatter_pairs, stream=stream)
        else:
            pkv.paged_kv_swap_blocks(cache.key_cache, cache.value_cache, cache.host_key,
                                     cache.host_value, in_pairs, stream=stream)

    def time_alone(staged):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(args.warmup):
            d2h(staged=staged)
            h2d(staged=staged)
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(args.steps):
            d2h(staged=staged)
        e[1].record()
        for _ in range(args.steps):
            h2d(staged=staged)
        e[2].record()
        torch.cuda.synchronize()
        return (e[0].elapsed_time(e[1]) / args.steps * 1e3,
                e[1].elapsed_time(e[2]) / args.steps * 1e3)

    out_us, in_us = time_alone(False)
    staged_out_us, staged_in_us = time_alone(True)
    # the whole call path: allocator swap pairs, the staging launch, the copies
    t0 = time.perf_counter()
    steps = max(1, args.steps // 5)
    for _ in range(steps):
        for s in seqs:
            cache.swap_out(s)
        for s in seqs:
            cache.swap_in(s)
    torch.cuda.synchronize()
    rt_us = (time.perf_counter() - t0) / steps * 1e6
    gbps_out, gbps_in = moved / (out_us * 1e-6) / 1e9, moved / (in_us * 1e-6) / 1e9
    log(f"[bench] swap kernel: device->host {out_us:.1f} us = {gbps_out:.1f} GB/s, host->device "
        f"{in_us:.1f} us = {gbps_in:.1f} GB/s; per-sequence engine calls round trip {rt_us:.0f} us")
    log(f"[bench] swap staged through a device pool, whole-run copies on the host link: "
        f"device->host {staged_out_us:.1f} us = "
        f"{moved / (staged_out_us * 1e-6) / 1e9:.1f} GB/s, host->device {staged_in_us:.1f} us = "
        f"{moved / (staged_in_us * 1e-6) / 1e9:.1f} GB/s")

    # overlap: the other sequences decode (split-K) on the main stream while
    # the victims' blocks go to the host pool and back on a second stream of
    # the same (default) priority
    main_st, side = torch.cuda.current_stream(), torch.cuda.Stream()
    residents = list(range(n, c.S))
    rin = cache.decode_inputs(residents, c.partition)
    rq = step["query"][residents].contiguous()
    rout = torch.empty_like(rq)

    def decode_residents():
        cache.decode(rq, rin, c.scale, out=rout)

    for _ in range(args.warmup):
        decode_residents()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record(main_st)
    for _ in range(5):
        decode_residents()
    ev[1].record(main_st)
    torch.cuda.synchronize()
    # enough decode steps to span one swap round trip
    n_dec = max(1, math.ceil((out_us + in_us) / (ev[0].elapsed_time(ev[1]) * 1e3 / 5)))
    ev[0].record(main_st)
    for _ in range(n_dec):
        decode_residents()
    ev[1].record(main_st)
    torch.cuda.synchronize()
    dec_alone = ev[0].elapsed_time(ev[1]) * 1e3 / n_dec

    def overlap_of(staged, rt_alone):
        # both at once: the side stream starts when the main stream does
        ev[2].record(main_st)
        side.wait_event(ev[2])
        d2h(side, staged)
        h2d(side, staged)
        ev[3].record(side)
        for _ in range(n_dec):
            decode_residents()
        ev[4].record(main_st)
        main_st.wait_event(ev[3])
        ev[5].record(main_st)
        torch.cuda.synchronize()
        dec_during = ev[2].elapsed_time(ev[4]) * 1e3 / n_dec
        swap_during = ev[2].elapsed_time(ev[3]) * 1e3
        both = ev[2].elapsed_time(ev[5]) * 1e3
        serial = dec_alone * n_dec + rt_alone
        log(f"[bench] overlap ({'staged, whole-run copies' if staged else 'swap kernel'}): {n_dec} decode steps "
            f"of {len(residents)} sequences {dec_alone:.1f} us each alone, {dec_during:.1f} us while "
            f"swapping; swap round trip {rt_alone:.0f} us alone, {swap_during:.0f} us beside the "
            f"decode; both {both:.0f} us vs {serial:.0f} us one after the other")
        return {"decode_us_alone": round(dec_alone, 2), "decode_us_during_swap": round(dec_during, 2),
                "swap_round_trip_us_alone": round(rt_alone, 1),
                "swap_round_trip_us_during_decode": round(swap_during, 1),
                "both_us": round(both, 1), "serial_us": round(serial, 1),
                "hidden_fraction": round((serial - both) / min(dec_alone * n_dec, rt_alone), 3)}

    overlap = {"decode_steps": n_dec, "decode_sequences": len(residents),
               "swap_kernel": overlap_of(False, out_us + in_us),
               "staged": overlap_of(True, staged_out_us + staged_in_us)}
    # the headline is the staged form (the engine's swap path)
    rt = staged_out_us + staged_in_us
    staged_gbps_out, staged_gbps_in = moved / (staged_out_us * 1e-6) / 1e9, moved / (staged_in_us * 1e-6) / 1e9
    slow = min(staged_gbps_out, staged_gbps_in)
    line = {
        "metric": SWAP_METRIC, "value": round(rt, 2), "unit": "us/round-trip",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(rt / 1e3, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{c.key}: sequences 0..{n - 1} ({nblocks} blocks of "
                               f"{block_bytes * 2} bytes) to a pinned host pool and back, "
                               f"staged through a device pool, whole-run copies on the host link",
                   "parallelism": "single GPU"},
        "kernel_us": {"swap_device_to_host": round(out_us, 2), "swap_host_to_device": round(in_us, 2),
                      "swap_calls_round_trip": round(rt_us, 1),
                      "staged_device_to_host": round(staged_out_us, 2),
                      "staged_host_to_device": round(staged_in_us, 2)},
        "overlap_with_decode": overlap,
        "roofline": {"bound": "host-link", "achieved": round(slow, 2), "peak": HOST_LINK_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(slow / HOST_LINK_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "staging launch + whole-run copies (slower direction)",
                     "algorithmic_bytes_per_launch": moved,
                     "device_to_host_GBps": round(staged_gbps_out, 2),
                     "host_to_device_GBps": round(staged_gbps_in, 2),
                     "swap_kernel_device_to_host_GBps": round(gbps_out, 2),
                     "swap_kernel_host_to_device_GBps": round(gbps_in, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); paged decode shards by sequence or kv head with no "
              "exchange, so per-GPU throughput is the one-GPU figure.", file=sys.stderr)
        sys.exit(2)
    if args.prefill:
        return main_prefill(args)
    if args.swap:
        return main_swap(args)

    import numpy as np
    import torch

    import synth
    import paged_kv_cache_211_amd as pkv
    from synth import device as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.make(args.config)
    wl.cache_limit = 0 if not args.no_cpu_baseline else 4
    c = wl.cfg
    P = c.partition if args.partition is None else args.partition
    ab = algorithmic_bytes(wl)
    log(f"[bench] workload {c.key}: S={c.S} H_q={c.H_q} H_kv={c.H_kv} d={c.d} bs={c.bs} "
        f"kv={c.kv_dtype} tokens={wl.total_tokens} blocks={wl.num_blocks} partition={P}")

    t0 = time.perf_counter()
    cache, step = W.build(wl, poison=False, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] prefill through the library: {time.perf_counter() - t0:.1f} s")

    pool_bytes = (cache.key_cache.numel() * cache.key_cache.element_size()) * 2
    R = args.layers or max(2, math.ceil(2e9 / max(ab["kv"], 1)))
    layers = [(cache.key_cache, cache.value_cache)]
    for _ in range(R - 1):
        layers.append((cache.key_cache.clone(), cache.value_cache.clone()))
    log(f"[bench] {R} pool layers of {pool_bytes / 1e9:.2f} GB")

    SK = args.schedule == "streamk"
    PF = args.schedule == "prefix"
    QU = args.schedule == "queue"
    if QU and not P:
        raise SystemExit("--schedule queue needs split-K partitions (--partition > 0)")
    if PF:
        inp = cache.decode_inputs(range(c.S), P, prefix=True, num_q_heads=c.H_q)
        ws = cache.workspace(inp["prefix_totals"][0], c.H_q, c.d)
        log(f"[bench] shared prefix: groups {inp['prefix']['group_offsets'].cpu().tolist()} "
            f"prefix blocks {inp['prefix']['group_prefix_blocks'].cpu().tolist()} "
            f"plan totals {inp['prefix_totals']}")
    elif SK:
        P = 0
        inp = cache.decode_inputs(range(c.S), streamk=True, num_q_heads=c.H_q,
                                  q_dtype=W.TORCH_CACHE[c.q_dtype], workers=args.workers or None)
        ws = cache.streamk_workspace(inp, c.H_q)
        log(f"[bench] stream-K: {inp['workers']} waves over {inp['total_tiles']} tiles per head group")
    else:
        inp = cache.decode_inputs(range(c.S), P)
        ws = cache.workspace(inp["total_partitions"], c.H_q, c.d) if P else None
    q, key, value, slots = step["query"], step["key"], step["value"], step["slots_dev"]
    out = torch.empty_like(q)
    tab, lens = inp["block_tables"], inp["context_lens"]
    # longest sequence's partition count: sizes the standalone reduce's launch
    max_parts = int(-(-int(inp["lens_host"].max()) // P)) if P else 0
    if PF:
        # the decode (prefix + suffix pass, storing the new tokens where each
        # (sequence, kv head) has one suffix wave -- the criterion of the
        # split-K step on these dtypes) and the reduce, or a store launch first
        n_launch = pkv.paged_attention_decode_step_launches(c.H_q, c.H_kv, c.d, c.bs, q.dtype,
                                                            cache.dtype, P)
    elif QU:
        n_launch = 3   # the store, the work-counter decode, the reduce
    elif SK:
        n_launch = 2 if pkv.paged_attention_decode_step_launches(c.H_q, c.H_kv, c.d, c.bs, q.dtype,
                                                                 cache.dtype, 0) == 1 else 3
    else:
        n_launch = pkv.paged_attention_decode_step_launches(c.H_q, c.H_kv, c.d, c.bs, q.dtype,
                                                            cache.dtype, P)

    def run_prefix(kc, vc):
        pkv.paged_attention_decode_prefix(out, q, kc, vc, tab, lens, c.scale, P, inp["prefix"],
                                          inp["prefix_totals"], ws, c.k_scale, c.v_scale)

    def run_queue(kc, vc):
        pkv.paged_attention_decode_queue(out, q, kc, vc, tab, lens, c.scale, c.k_scale, c.v_scale,
                                         P, inp["partition_offsets"], inp["total_partitions"], ws)

    def run_fused(i, ev=None):
        kc, vc = layers[i % R]
        if ev:
            ev[0].record()
        if PF:
            pkv.paged_attention_decode_prefix_step(out, q, key, value, kc, vc, tab, lens, c.scale,
                                                   P, inp["prefix"], inp["prefix_totals"], ws,
                                                   c.k_scale, c.v_scale)
        elif QU:
            pkv.paged_kv_write(key, value, kc, vc, slots, k_scale=c.k_scale, v_scale=c.v_scale)
            run_queue(kc, vc)
        elif SK:
            pkv.paged_attention_decode_step_streamk(out, q, key, value, kc, vc, tab, lens, c.scale,
                                                    inp["tile_offsets"], inp["total_tiles"],
                                                    inp["workers"], ws, c.k_scale, c.v_scale)
        else:
            pkv.paged_attention_decode_step(out, q, key, value, kc, vc, tab, lens, c.scale,
                                            c.k_scale, c.v_scale, P, inp["partition_offsets"],
                                            inp["total_partitions"], ws)
        if ev:
            ev[1].record()

    def run_separate(i, ev=None):
        kc, vc = layers[i % R]
        if ev:
            ev[0].record()
        pkv.paged_kv_write(key, value, kc, vc, slots, k_scale=c.k_scale, v_scale=c.v_scale)
        if ev:
            ev[1].record()
        if PF or QU:
            run_prefix(kc, vc) if PF else run_queue(kc, vc)
            if ev:
                ev[2].record()
        elif SK:
            pkv.paged_attention_decode_streamk_partials(out, q, kc, vc, tab, lens, c.scale,
                                                        inp["tile_offsets"], inp["total_tiles"],
                                                        inp["workers"], ws, c.k_scale, c.v_scale)
            if ev:
                ev[2].record()
            pkv.paged_attention_streamk_reduce(out, ws, inp["tile_offsets"], inp["total_tiles"],
                                               inp["workers"], c.H_kv, c.bs, cache.dtype)
        elif P:
            pkv.paged_attention_decode_partials(out, q, kc, vc, tab, lens, c.scale, c.k_scale,
                                                c.v_scale, P, inp["partition_offsets"],
                                                inp["total_partitions"], ws)
            if ev:
                ev[2].record()
            pkv.paged_attention_splitk_reduce(out, ws, inp["partition_offsets"],
                                              inp["total_partitions"], max_parts)
        else:
            pkv.paged_attention_decode(out, q, kc, vc, tab, lens, c.scale, c.k_scale, c.v_scale)
            if ev:
                ev[2].record()
        if ev:
            ev[3].record()

    run = run_fused if args.mode == "fused" else run_separate

    # streaming-copy reference (also the known-size kernel for counter scaling)
    copy_n = 1 << 30
    src_b = torch.empty(copy_n, dtype=torch.uint8, device=dev)
    dst_b = torch.empty_like(src_b)
    dst_b.copy_(src_b)
    torch.cuda.synchronize()
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    for _ in range(5):
        dst_b.copy_(src_b)
    ce1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * copy_n * 5 / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del dst_b
    # attainable streaming-read rate of this GPU: the library's read probe
    # (contiguous 32 KiB runs per workgroup, 16-byte non-temporal loads, 32768 workgroups) over 1 GiB
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        pkv.pkv_hbm_read_probe(src_b, sink, 32768)
    torch.cuda.synchronize()
    ce0.record()
    for _ in range(5):
        pkv.pkv_hbm_read_probe(src_b, sink, 32768)
    ce1.record()
    torch.cuda.synchronize()
    probe_gbps = copy_n * 5 / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del src_b, sink

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # region 1: the headline, K whole steps bracketed by events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps

    # region 2: the separate launches, an event around each kernel
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.warmup):
        run_separate(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        run_separate(i, evs[i])
    torch.cuda.synchronize()
    t_write = np.array([a.elapsed_time(b) for a, b, _, _ in evs]) * 1e3
    t_dec = np.array([b.elapsed_time(c2) for _, b, c2, _ in evs]) * 1e3
    t_red = np.array([c2.elapsed_time(d) for _, _, c2, d in evs]) * 1e3
    dec_us = float(np.mean(t_dec))

    # region 3: the step entry alone, events around each call
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup):
        run_fused(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        run_fused(i, fev[i])
    torch.cuda.synchronize()
    t_fused = np.array([a.elapsed_time(b) for a, b in fev]) * 1e3
    fused_us = float(np.mean(t_fused))

    # region 4: the roofline kernel alone, K back-to-back launches between two
    # events on its stream (cycling the pool layers): its average launch time
    def run_decode_only(i):
        kc, vc = layers[i % R]
        if PF:
            run_prefix(kc, vc)
        elif QU:
            run_queue(kc, vc)
        elif SK:
            pkv.paged_attention_decode_streamk_partials(out, q, kc, vc, tab, lens, c.scale,
                                                        inp["tile_offsets"], inp["total_tiles"],
                                                        inp["workers"], ws, c.k_scale, c.v_scale)
        elif P:
            pkv.paged_attention_decode_partials(out, q, kc, vc, tab, lens, c.scale, c.k_scale,
                                                c.v_scale, P, inp["partition_offsets"],
                                                inp["total_partitions"], ws)
        else:
            pkv.paged_attention_decode(out, q, kc, vc, tab, lens, c.scale, c.k_scale, c.v_scale)

    for i in range(args.warmup):
        run_decode_only(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        run_decode_only(i)
    e1.record()
    torch.cuda.synchronize()
    dec_only_us = e0.elapsed_time(e1) / args.steps * 1e3

    # the same reads without the arithmetic (split-K schedules): the rate the
    # decode's access pattern itself reaches on this device
    paged_probe_us = None
    if P and not (PF or SK):
        psink = torch.zeros(4, dtype=torch.int32, device=dev)

        def run_paged_probe(i):
            kc, vc = layers[i % R]
            pkv.pkv_paged_read_probe(kc, vc, tab, lens, c.H_q, q.dtype, P, inp["partition_offsets"],
                                     inp["total_partitions"], psink)

        for i in range(args.warmup):
            run_paged_probe(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            run_paged_probe(i)
        e1.record()
        torch.cuda.synchronize()
        paged_probe_us = e0.elapsed_time(e1) / args.steps * 1e3
        log(f"[bench] paged read probe (the decode's reads, no arithmetic): {paged_probe_us:.1f} us "
            f"= {ab['kv'] / (paged_probe_us * 1e-6) / 1e9:.0f} GB/s of KV; decode kernel / probe time "
            f"{dec_only_us / paged_probe_us:.3f}")

    us_step = ms_step * 1e3
    kv_gbps = ab["kv"] / (us_step * 1e-6) / 1e9
    if n_launch == 1:
        # the step is one kernel (store inside the decode, no partitions)
        kernel, kern_us, kern_bytes = "decode step (store + decode)", fused_us, ab["step"]
    elif PF:
        # the three launches of the shared-prefix decode, over the unique bytes
        kernel, kern_us, kern_bytes = "decode (shared prefix + suffix + reduce)", dec_only_us, ab["decode_unique"]
    elif QU:
        # the work-counter decode and its reduce (no partials-only form)
        kernel, kern_us, kern_bytes = "decode (work-counter split-K + reduce)", dec_only_us, ab["decode"]
    else:
        kernel = ("decode (stream-K)" if SK else "decode (split-K partials)" if P else "decode")
        kern_us, kern_bytes = dec_only_us, ab["decode"]
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    traffic = load_traffic(args.traffic_file,
                           c.key if P == c.partition or SK or PF else f"{c.key}-p{P}", kernel)
    log(f"[bench] mode {args.mode}: step {us_step:.1f} us (wall {wall / args.steps * 1e6:.1f} us); "
        f"step entry {fused_us:.1f} us in {n_launch} launch(es); separate launches: "
        f"write {np.mean(t_write):.1f} us, decode {dec_us:.1f} us "
        f"[p10 {np.percentile(t_dec, 10):.1f}, p90 {np.percentile(t_dec, 90):.1f}], "
        f"reduce {np.mean(t_red):.1f} us; decode back to back {dec_only_us:.1f} us")
    log(f"[bench] KV {ab['kv'] / 1e9:.3f} GB/step -> {kv_gbps:.0f} GB/s = "
        f"{100 * kv_gbps / HBM_PEAK_GBPS:.1f}% of {HBM_PEAK_GBPS:.0f}; {kernel} "
        f"{achieved:.0f} GB/s; device copy {copy_gbps:.0f} GB/s; read probe {probe_gbps:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample ...")
        cpu = cpu_baseline(wl, args.cpu_tokens)
        log(f"[bench] oracle: {cpu['value']} us/step est. ({cpu['sample']})")

    dtype = {"f32": "f32", "bf16": "bf16", "fp8": "fp8-kv/bf16-q"}[c.kv_dtype]
    line = {
        "metric": METRIC,
        "value": round(us_step, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{c.key}: {c.S} seqs, {c.H_q}/{c.H_kv} heads, head_dim {c.d}, "
                        f"block_size {c.bs}, {c.kv_dtype} KV, context {wl.total_tokens} tokens "
                        f"(seed {c.seed}), "
                        + (f"stream-K {inp['workers']} waves" if SK else
                           f"split-K {P} from a work counter" if QU else f"split-K {P}")
                        + f", {R} pool layers, {args.mode} step",
            "global_batch": c.S,
            "seq_len": int(wl.context_lens.max()),
            "mean_context": round(float(wl.context_lens.mean()), 1),
            "parallelism": "single GPU",
            "mode": args.mode,
            "schedule": args.schedule,
            "step_launches": n_launch if args.mode == "fused" else (3 if (P or SK) else 2),
        },
        "kv_GBps": round(kv_gbps, 1),
        "pct_hbm_peak": round(100 * kv_gbps / HBM_PEAK_GBPS, 2),
        "step_algorithmic_bytes": ab["step"],
        "kernel_us": {"paged_kv_write": round(float(np.mean(t_write)), 2),
                      "decode": round(dec_us, 2), "splitk_reduce": round(float(np.mean(t_red)), 2),
                      "decode_step_entry": round(fused_us, 2),
                      "decode_back_to_back": round(dec_only_us, 2)},
        "device_copy_GBps": round(copy_gbps, 1),
        "hbm_read_probe_GBps": round(probe_gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "algorithmic_bytes_per_launch": kern_bytes,
                     "frac_of_read_probe": round(achieved / probe_gbps, 4),
                     "paged_read_probe_us": round(paged_probe_us, 2) if paged_probe_us else None,
                     "paged_probe_over_kernel_time": round(paged_probe_us / kern_us, 4)
                     if paged_probe_us else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
