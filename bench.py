"""Benchmark: one decode step of a block-quantized paged KV cache on one
MI355X -- store each sequence's current token (re-quantizing its block) and
run the fused dequantizing split-K attention plus its log-sum-exp reduce, as
one paged_attn_decode_append call (paged_attn_decode_shared_prefix when the
sequences share a prefix); the same step as two calls (kv_quantize_store,
paged_attn_decode) is timed beside it.

Prints ONE JSON line.  ``value`` is the step's algorithmic HBM bytes per
second (GB/s = 1e9 B/s) with all inputs resident in HBM; the line also gives
tokens/s per layer, the fraction of the 8 TB/s HBM peak, the roofline of the
decode kernels measured with HIP events on their stream, and the CPU oracle
timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import dataclasses
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "quantized-KV decode attention GB/s (% of HBM peak) + tokens/s per layer"


def measured_traffic(workload):
    """HBM bytes per decode call from the committed rocprofv3 counter runs,
    or None when they are missing or were taken on a different kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from paged_block_quantized_amd.traffic import kernel_source_hash
    if rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_decode")


def _r5(x):
    x = float(x)
    return round(x, 5) if x == x else None


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and logical CPU count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def oracle_workers():
    """Worker processes for the oracle baseline: every host CPU, at most 16
    (the share of a one-GPU host this benchmark may occupy)."""
    return max(1, min(16, os.cpu_count() or 1))


def _oracle_decode_worker(units, bs, k_codec, v_codec, sm_scale, start_evt, seconds, out_q):
    """One worker process of the oracle baseline (spawned: imports numpy and
    the oracle only, never touches the GPU).  Each unit is one (sequence,
    KV head): fp16 history [ctx, D] of K and V and its query heads [G, D].
    The history up to the current token is quantized before the timed
    region; then, until `seconds` have passed, each unit in turn re-stores
    its current token (re-quantizing the block) and runs float64 attention
    over its dequantized context."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention, paged
    prepared = []
    for uid, hk, hv, q in units:
        ctx = hk.shape[0]
        nb = (ctx + bs - 1) // bs
        pool = paged.PoolArrays(nb, 1, bs, hk.shape[-1], k_codec=k_codec, v_codec=v_codec)
        paged.store_range(pool, list(range(nb)), hk[:, None], hv[:, None], 0, ctx - 1)
        prepared.append((uid, ctx, nb, pool, hk[:, None], hv[:, None], q))
    done = {uid: 0 for uid, *_ in units}
    start_evt.wait()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for uid, ctx, nb, pool, hk, hv, q in prepared:
                paged.store_range(pool, list(range(nb)), hk, hv, ctx - 1, ctx)
                khat, vhat = paged.gather_dequant(pool, list(range(nb)), ctx)
                attention.decode_attention(q, khat, vhat, sm_scale)
                done[uid] += 1
        dt = time.perf_counter() - t0
    out_q.put((done, dt))


def cpu_baseline(setup, seconds):
    """The oracle's decode step on the host's cores: (sequence, KV head)
    units of the workload's first sequences, spread over a pool of worker
    processes, each repeating the oracle's step (store the current token,
    float64 attention over the dequantized context) for `seconds`.
    Throughput is the algorithmic bytes of the unit-steps done (a unit's
    share of its sequence's step bytes) over the slowest worker's time."""
    import multiprocessing as mp

    import numpy as np

    from paged_block_quantized_amd import runner, workloads as W

    w = setup.w
    H, G = w.num_kv_heads, w.num_q_heads // w.num_kv_heads
    n_workers = oracle_workers()
    # units of whole sequences first, at most about 256 MiB of fp16 history
    unit_bytes = int(np.max(setup.ctx)) * w.head_dim * 4
    max_units = max(n_workers, min(w.num_seqs * H, (256 << 20) // unit_bytes))
    units, seq_of = [], {}
    for s in range(w.num_seqs):
        if len(units) >= max_units:
            break
        hk, hv = runner.sequence_history(setup, s)
        q = setup.q[s].cpu().numpy()
        for g in range(H):
            if len(units) >= max_units:
                break
            uid = len(units)
            seq_of[uid] = s
            units.append((uid, np.ascontiguousarray(hk[:, g]), np.ascontiguousarray(hv[:, g]),
                          np.ascontiguousarray(q[g * G:(g + 1) * G])))
    n_workers = min(n_workers, len(units))
    ctx_mp = mp.get_context("spawn")
    start_evt, out_q = ctx_mp.Event(), ctx_mp.Queue()
    procs = [ctx_mp.Process(target=_oracle_decode_worker,
                            args=(units[i::n_workers], w.block_size, W.k_codec_of(w), w.v_codec, setup.sm_scale,
                                  start_evt, seconds, out_q), daemon=True)
             for i in range(n_workers)]
    for p_ in procs:
        p_.start()
    time.sleep(0.5)
    start_evt.set()
    results = [out_q.get(timeout=seconds + 600) for _ in procs]
    for p_ in procs:
        p_.join(timeout=60)
    dt = max(r[1] for r in results)
    nbytes = 0
    steps = 0
    for done, _ in results:
        for uid, n in done.items():
            ctx1 = np.array([int(setup.ctx[seq_of[uid]])])
            sub = dataclasses.replace(w, num_seqs=1, prefix=0)
            per_seq = runner.decode_bytes(sub, ctx1) + runner.store_step_bytes(sub, ctx1, rewrite_tiles=False)
            nbytes += n * per_seq / H
            steps += n
    model, cpus = host_cpu()
    n_seqs = len(set(seq_of.values()))
    return {
        "value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": n_workers, "kind": "oracle",
        "host_cpus": cpus, "cpu_model": model,
        "tokens_per_s_per_layer": round(steps / H / dt, 2),
        "sample": (f"{steps} (sequence, KV head) unit-steps over {len(units)} units of the first {n_seqs} "
                   f"sequences of the same workload (oracle store of the current token + float64 attention), "
                   f"{n_workers} worker processes, {dt:.1f} s; shared prefixes counted per sequence"),
    }


def swap_plan_bytes(pool, plan):
    """Bytes a swap plan moves: whole blocks (codes, scales, zero points) and
    the held rows of each head of the tail slots (K and V, fp16)."""
    H, bs, D = pool.num_kv_heads, pool.block_size, pool.head_dim
    kb = H * bs * D
    block = ((kb // 2 if pool.k_int4 else kb) + (kb // 2 if pool.v_int4 else kb) + 4 * H
             + (H if pool.v_zp_used else 0) + (H if pool.k_zp_used else 0))
    total = 0
    for kind, _, _, rows in plan:
        total += block if kind < 2 else 4 * H * rows * D
    return total


def measure_swap(setup, reps):
    """A quarter of the batch swapped out to pinned host memory and back in,
    reps times: the swap kernel's rate per direction (HIP events around
    kv_swap_blocks on its stream), the host allocator's time per call, and
    the DMA engines' rate for one contiguous copy of the same size (torch
    copy_ between device and pinned host memory) as the link's practical
    peak.  Leaves the pool's tables changed: run it last."""
    import numpy as np
    import torch

    from paged_block_quantized_amd import _lib as L
    pool, w = setup.pool, setup.w
    group = list(range(0, w.num_seqs, 4))
    n_blocks = sum(len(pool.table(s)[0]) for s in group)
    pool.set_swap_space(n_blocks, len(group))
    stream = torch.cuda.current_stream()
    plan = torch.zeros((L.swap_plan_cap(pool.handle, group), 4), dtype=torch.int32, pin_memory=True)
    ms = {"out": [], "in": []}
    host_us = {"out": [], "in": []}
    nbytes = {}
    for i in range(reps + 1):
        for d, fn in (("out", L.kv_seq_swap_out), ("in", L.kv_seq_swap_in)):
            t0 = time.perf_counter()
            n = fn(pool.handle, group, plan)
            t1 = time.perf_counter()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            L.kv_swap_blocks(pool.desc, pool.mem, pool.host_desc, pool.host_mem, plan, n, stream)
            b.record(stream)
            torch.cuda.synchronize()          # the plan buffer is reused
            nbytes[d] = swap_plan_bytes(pool, plan[:n].tolist())
            if i:
                ms[d].append(a.elapsed_time(b))
                host_us[d].append((t1 - t0) * 1e6)
    size = nbytes["out"]
    dev = torch.empty(size, dtype=torch.uint8, device="cuda")
    host = torch.empty(size, dtype=torch.uint8, pin_memory=True)
    dma = {"d2h": [], "h2d": []}
    for i in range(reps + 1):
        for d, (dst, src) in (("d2h", (host, dev)), ("h2d", (dev, host))):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src, non_blocking=True)
            b.record(stream)
            torch.cuda.synchronize()
            if i:
                dma[d].append(a.elapsed_time(b))
    gbs = {d: nbytes[d] / (float(np.median(ms[d])) * 1e-3) / 1e9 for d in ms}
    dgbs = {d: size / (float(np.median(dma[d])) * 1e-3) / 1e9 for d in dma}
    return {
        "kernel": "kv_swap_blocks (one launch per plan; the device reads or writes pinned host memory)",
        "sequences": len(group), "blocks": n_blocks, "bytes_per_direction": size,
        "out_ms": round(float(np.median(ms["out"])), 4), "in_ms": round(float(np.median(ms["in"])), 4),
        "out_gbs": round(gbs["out"], 2), "in_gbs": round(gbs["in"], 2),
        "dma_d2h_gbs": round(dgbs["d2h"], 2), "dma_h2d_gbs": round(dgbs["h2d"], 2),
        "out_frac_of_dma": round(gbs["out"] / dgbs["d2h"], 4),
        "in_frac_of_dma": round(gbs["in"] / dgbs["h2d"], 4),
        "host_us_kv_seq_swap_out": round(float(np.median(host_us["out"])), 1),
        "host_us_kv_seq_swap_in": round(float(np.median(host_us["in"])), 1),
    }


MFMA_F16_PEAK_TFLOPS = 2500.0


def cpu_baseline_multi(setup, seconds):
    """The oracle's multi-query attention on a bounded sample: sequence 0's
    stored tokens quantized by the oracle, then its queries from the last one
    backwards, single-threaded, until `seconds` have passed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention, paged
    from paged_block_quantized_amd import runner, workloads as W

    w = setup.w
    bs, n = w.block_size, w.q_len
    ctx = int(setup.ctx[0])
    k, v = W.kv_tokens(w, 0, ctx, "cpu")
    nb = (ctx + bs - 1) // bs
    pool = paged.PoolArrays(nb, w.num_kv_heads, bs, w.head_dim, k_codec=W.k_codec_of(w), v_codec=w.v_codec)
    paged.store_range(pool, list(range(nb)), k.numpy(), v.numpy(), 0, ctx)
    q = setup.q[:n].cpu().numpy()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        khat, vhat = paged.gather_dequant(pool, list(range(nb)), ctx)
        flops, done = 0, 0
        while time.perf_counter() - t0 < seconds and done < n:
            i = n - 1 - done
            pos = ctx - n + i
            attention.decode_attention(q[i], khat[:, :pos + 1], vhat[:, :pos + 1], setup.sm_scale)
            flops += 4 * w.head_dim * w.num_q_heads * (pos + 1)
            done += 1
        dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"sequence 0 ({ctx} tokens stored): its last {done} of {n} queries, float64 "
                      f"numpy, dequantization included, {dt:.1f} s"}


def dense_attention_context(w, ctx, reps=10):
    """Context for the multi-query kernel: the library's dense fp16 attention
    (torch scaled_dot_product_attention, flash backend, else the
    memory-efficient one) on the workload's shape -- every sequence's
    q_len queries over its whole context, all query heads (K and V expanded
    to them beforehand), no quantization, no block tables and no mask, so
    every query sees every key -- over two sets of K and V used in turn.
    TFLOP/s counts 4 D per (query, key, head) as the kernel's figure does."""
    import numpy as np
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    S, Hq, D, n = w.num_seqs, w.num_q_heads, w.head_dim, w.q_len
    L_ = int(max(ctx))
    g = torch.Generator(device="cuda").manual_seed(17)
    q = torch.randn(S, Hq, n, D, dtype=torch.float16, device="cuda", generator=g)
    kv = [[torch.randn(S, Hq, L_, D, dtype=torch.float16, device="cuda", generator=g) for _ in range(2)]
          for _ in range(2)]
    stream = torch.cuda.current_stream()
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("memory-efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel(be):
                ms = []
                for i in range(reps + 4):
                    k, v = kv[i % 2]
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    F.scaled_dot_product_attention(q, k, v)
                    b.record(stream)
                    torch.cuda.synchronize()
                    if i >= 4:
                        ms.append(a.elapsed_time(b))
        except RuntimeError:
            continue
        t = float(np.median(ms))
        flops = 4 * D * Hq * n * L_ * S
        del q, kv
        return {"kernel": f"torch scaled_dot_product_attention ({name} backend), fp16, dense", "ms": round(t, 4),
                "flops": flops, "tflops": round(flops / (t * 1e-3) / 1e12, 1),
                "frac": round(flops / (t * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                "note": "context for roofline.frac: the same shape as dense fp16 tensors with every key "
                        "visible (no codes to convert, no tables, no mask), not a denominator"}
    return None


def bench_multi(w, args):
    """Multi-query (chunked prefill) attention: K timed calls of
    paged_attn_multi_query over the workload's pool."""
    import numpy as np
    import torch

    from paged_block_quantized_amd import runner, workloads as W
    print(f"setup {w.name}", file=sys.stderr, flush=True)
    setup = runner.setup_multi(w, partition=args.partition or 0)
    flops = runner.multi_flops(w, setup.ctx)
    nbytes = runner.multi_bytes(w, setup.ctx)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        setup.run()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        setup.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    call_ms = e0.elapsed_time(e1) / K
    tflops = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (call_ms * 1e-3) / 1e12
    T = w.num_seqs * w.q_len
    line = {
        "metric": "multi-query attention over the quantized paged cache, TFLOP/s (+ query tokens/s)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8" if w.v_codec != "fp8" else "fp8", "data": "synthetic",
        "config": {"workload": w.name, "layers": 1, "num_seqs": w.num_seqs, "context": int(setup.ctx.max()),
                   "query_tokens_per_seq": w.q_len, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "k_codec": W.k_codec_of(w), "v_codec": w.v_codec,
                   "partition": setup.partition or "library default"},
        "query_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "unique_bytes_gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
        "roofline": {"kernel": "paged_attn_multi_query (grouped-query MFMA kernel, multi-query mode; "
                               "plus the per-query reduce when partitions are split)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(w.name),
                     "flops_per_launch": flops, "bytes_per_launch": nbytes},
    }
    if not args.only_timed:
        print("dense attention context", file=sys.stderr, flush=True)
        line["roofline"]["library_dense_attention"] = dense_attention_context(w, setup.ctx)
    if not args.no_cpu_baseline:
        print("cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_multi(setup, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def cpu_baseline_store(setup, seconds):
    """The oracle's quantize-and-store of whole prompts (the same rows the
    GPU stores), single-threaded, for up to ``seconds``."""
    from threadpoolctl import threadpool_limits

    from oracle import paged
    from paged_block_quantized_amd import runner, workloads as W

    w, T = setup.w, setup.tokens
    H, D, bs = w.num_kv_heads, w.head_dim, w.block_size
    nb = (T + bs - 1) // bs
    per_prompt = runner.prefill_store_bytes(w) // w.num_seqs
    done, spent = 0, 0.0
    with threadpool_limits(1):
        for s in range(w.num_seqs):
            hk = setup.k[s * T:(s + 1) * T].cpu().numpy()
            hv = setup.v[s * T:(s + 1) * T].cpu().numpy()
            ref = paged.PoolArrays(nb, H, bs, D, w.v_codec == "i4", k_codec=W.k_codec_of(w), v_codec=w.v_codec)
            t0 = time.perf_counter()
            paged.store_range(ref, list(range(nb)), hk, hv, 0, T)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= seconds:
                break
    return {"value": round(done * per_prompt / spent / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_stored_per_s": round(done * T / spent, 1),
            "sample": f"{done} of the {w.num_seqs} prompts ({T} tokens each, all KV heads) stored by the oracle, "
                      f"{spent:.1f} s, one thread"}


def bench_store(w, args):
    """Quantize-and-store: K timed calls of kv_quantize_store that store every
    prompt of the workload (re-quantizing the same blocks each call), then
    the one-token append steps of the same workload, each timed alone."""
    import numpy as np
    import torch

    from paged_block_quantized_amd import runner, workloads as W
    print(f"setup {w.name}", file=sys.stderr, flush=True)
    setup = runner.setup_prefill_store(w)
    nbytes = runner.prefill_store_bytes(w)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        setup.run()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        setup.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    call_ms = e0.elapsed_time(e1) / K
    T = w.num_seqs * setup.tokens

    # one-token appends to 64 partially filled blocks, 16 steps (every block
    # crosses its fill point once); the host reserves the positions between
    # the timed calls
    print("appends", file=sys.stderr, flush=True)
    app = runner.setup_append(w)
    app_ms, app_bytes = [], []
    for step in range(16):
        args_ = app.inputs(step)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        app.pool.quantize_store(*args_, 1)
        b.record(stream)
        torch.cuda.synchronize()
        app_ms.append(a.elapsed_time(b))
        app_bytes.append(runner.store_step_bytes(w, app.fill + step + 1))
    line = {
        "metric": "quantize-and-store GB/s (% of HBM peak) + tokens stored/s",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "tokens_per_prompt": setup.tokens,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "k_codec": W.k_codec_of(w), "v_codec": w.v_codec, "pool_blocks": setup.pool.num_blocks},
        "pct_of_hbm_peak": round(100 * nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "tokens_stored_per_s": round(T / (ms_step * 1e-3), 1),
        "step_bytes": nbytes,
        "append": {"calls": 16, "sequences": w.num_seqs, "mean_us": round(1e3 * float(np.mean(app_ms)), 2),
                   "p10_us": round(1e3 * float(np.percentile(app_ms, 10)), 2),
                   "p90_us": round(1e3 * float(np.percentile(app_ms, 90)), 2),
                   "mean_bytes": int(np.mean(app_bytes)),
                   "note": "one kv_quantize_store call per step, each timed alone with HIP events "
                           "(launch-latency bound)"},
        "roofline": {"kernel": "kv_quantize_store (quantize_store_kernel), one call storing every prompt",
                     "bound": "hbm", "achieved": round(nbytes / (call_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name), "bytes_per_launch": nbytes},
    }
    if not args.only_timed:
        print("elementwise ceiling", file=sys.stderr, flush=True)
        line["roofline"]["plain_elementwise_ceiling"] = elementwise_ceiling(nbytes)
    if not args.no_cpu_baseline:
        print("cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_store(setup, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def elementwise_ceiling(nbytes, reps=10):
    """Context for the store: a plain contiguous elementwise kernel with the
    store's traffic mix (two bytes read per byte written), torch.add of two
    fp16 arrays into a third, moving the store call's bytes per call, over
    two sets of buffers used in turn (each larger than the last-level
    cache).  It does no scattering and no arithmetic beyond the add."""
    import numpy as np
    import torch

    n = nbytes // 6   # fp16 elements: 2 n B read twice, 2 n B written
    bufs = [[torch.randn(n, dtype=torch.float16, device="cuda") for _ in range(3)] for _ in range(2)]
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(reps + 2):
        x, y, z = bufs[i % 2]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        torch.add(x, y, out=z)
        b.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(a.elapsed_time(b))
    del bufs
    t = float(np.median(ms))
    moved = 6 * n
    return {"kernel": "torch.add (fp16, a + b -> c), contiguous", "bytes": moved,
            "gbs": round(moved / (t * 1e-3) / 1e9, 1), "frac": round(moved / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "context for roofline.frac: the store's 2:1 read:write mix in a plain elementwise kernel, "
                    "not a denominator"}


def read_ceiling(setup, reps=10):
    """The plain-read ceiling of the decode's access pattern, measured with
    kv_stream_read_tiles: exactly the tiles the decode reads (per sequence
    and KV head, its K tiles, then its V tiles, in table order; a shared
    prefix once), rotating over the pool copies as the timed steps do, and a
    sequential read of the same number of bytes.  GB/s over the tile bytes
    (the tile list itself, 4 bytes per tile, is read too and not counted)."""
    import numpy as np
    import torch

    from paged_block_quantized_amd import _lib as L
    w = setup.w
    H, bs, D = w.num_kv_heads, w.block_size, w.head_dim
    from paged_block_quantized_amd import workloads as W
    k_tile = bs * D // 2 if W.k_codec_of(w) == "i4" else bs * D
    v_tile = bs * D // 2 if w.v_codec == "i4" else bs * D
    if k_tile not in (1024, 2048, 4096) or v_tile not in (1024, 2048, 4096):
        return None
    tables = setup.tables.cpu().numpy()
    shared_blocks = setup.shared // bs
    ids = []
    for s_ in range(w.num_seqs):
        nb = (int(setup.ctx[s_]) + bs - 1) // bs
        first = shared_blocks if (setup.shared and s_ > 0) else 0
        blocks = tables[s_, first:nb].astype(np.int64)
        for h in range(H):
            ids.append(blocks * H + h)
    order = torch.from_numpy(np.concatenate(ids).astype(np.int32)).cuda()
    n = int(order.numel())
    sink = torch.empty(max(1, L.kv_stream_read_sink_words(n)), dtype=torch.int32, device="cuda")
    copies = [setup.pool.arrays] + [arr for _, arr in (setup.replicas or [])]
    stream = torch.cuda.current_stream()

    def run(ordered):
        ms = []
        for i in range(reps + 1):
            arr = copies[i % len(copies)]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for name, tb in (("k_codes", k_tile), ("v_codes", v_tile)):
                src = arr[name]
                L.kv_stream_read_tiles(src, src.numel() * src.element_size() // tb, tb,
                                       order if ordered else None, n, sink, stream)
            b.record(stream)
            torch.cuda.synchronize()
            if i:
                ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    nbytes = n * (k_tile + v_tile)
    t_tiles, t_seq = run(True), run(False)
    return {"kernel": "kv_stream_read_tiles (one launch per code array)", "bytes": nbytes,
            "decode_tiles_gbs": round(nbytes / (t_tiles * 1e-3) / 1e9, 1),
            "sequential_gbs": round(nbytes / (t_seq * 1e-3) / 1e9, 1),
            "decode_tiles_frac": round(nbytes / (t_tiles * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "sequential_frac": round(nbytes / (t_seq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "the decode's tile list over pool copies the timed steps rotate through; context "
                    "for roofline.frac (the decode's arithmetic made free), not a denominator"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the GPU's clocks take a few milliseconds of load to settle")
    ap.add_argument("--workload", default="llama7b")
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--rotate", type=int, default=4,
                    help="copies of the pool the timed steps cycle through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-timed", action="store_true",
                    help="skip the same-pool and cache-flush context measurements "
                         "(for profiling the timed loop alone)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, ROOT)
    from paged_block_quantized_amd import runner, workloads as W

    w = W.WORKLOADS[args.workload]
    if w.q_len:
        bench_multi(w, args)
        return
    if w.store_only:
        bench_store(w, args)
        return
    print(f"setup {w.name}", file=sys.stderr, flush=True)
    setup = runner.setup_decode(w, partition=args.partition)
    S = w.num_seqs
    dbytes = runner.decode_bytes(w, setup.ctx)
    # the timed steps store the same current token again and again: the
    # block's scale does not change after the first, so the store's
    # algorithmic writes are the token's own codes (not the whole tile)
    sbytes = runner.store_step_bytes(w, setup.ctx, rewrite_tiles=False)

    # The timed steps cycle through R copies of the pool at different
    # addresses, as the layers of a model would, so no step finds its codes in
    # a cache left by the step before (the 256 MB last-level cache is far
    # smaller than R copies).
    R = max(1, args.rotate)
    if R > 1:
        setup.add_replicas(R - 1)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        setup.step(r=i % R)
    torch.cuda.synchronize()

    def timed(steps, rot, fused=True):
        """Per step: events around the fused call (store + decode in one
        call), or around each of the two calls of the separate path."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(steps)] for _ in range(3)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            r = i % rot
            ev[0][i].record(stream)
            if fused:
                setup.step(r=r)
            else:
                setup.store_current(r=r)
            ev[1][i].record(stream)
            if not fused:
                setup.attend(r=r)
            ev[2][i].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        a_ = np.array([ev[0][i].elapsed_time(ev[1][i]) for i in range(steps)])
        b_ = np.array([ev[1][i].elapsed_time(ev[2][i]) for i in range(steps)])
        return (t1 - t0) * 1e3 / steps, a_, b_

    K = args.steps
    # the timed region: K steps (one call each) with events only at its two
    # ends, so that no event marker sits between the calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        setup.step(r=i % R)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    step_call_ms = e0.elapsed_time(e1) / K
    print(f"timed {K} steps over {R} pool copies: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    # the decode alone (no store), K calls with events only at the two ends
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(K):
        setup.attend(r=i % R)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_loop_ms = d0.elapsed_time(d1) / K
    # context: per-call events (spread of the call time)
    _, fused_ms, _ = timed(min(K, 20), R)
    # context: the same step as two calls (kv_quantize_store, paged_attn_decode)
    ms_sep, st_ms, dec = timed(min(K, 20), R, fused=False)
    store_ms, dec_ms = float(np.mean(st_ms)), float(np.mean(dec))
    dec_same, fl_w, fl_r, ceiling = np.array([np.nan]), [np.nan], [np.nan], None
    if not args.only_timed:
        # context: the same pool every step (its codes partly in the last-level cache)
        _, dec_same, _ = timed(min(K, 20), 1)
        # context: decode after a 1 GiB cache-clearing pass (outside the
        # events), once a write (torch zero_: it leaves dirty lines whose
        # write-back competes with the next reads) and once a plain read
        # (kv_stream_read_tiles: clean lines, so only the cache is cold)
        from paged_block_quantized_amd import _lib as L
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        n_fl = (1 << 30) // 4096
        sink = torch.empty(L.kv_stream_read_sink_words(n_fl), dtype=torch.int32, device="cuda")
        fl_w, fl_r = [], []
        for i in range(20):
            if i % 2 == 0:
                flush.zero_()
            else:
                L.kv_stream_read_tiles(flush, n_fl, 4096, None, n_fl, sink, stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            setup.attend()
            b.record(stream)
            torch.cuda.synchronize()
            (fl_w if i % 2 == 0 else fl_r).append(a.elapsed_time(b))
        del flush, sink
        print("read ceiling", file=sys.stderr, flush=True)
        ceiling = read_ceiling(setup)

    # context: with a shared prefix, the per-sequence step (the prefix read
    # by every sequence) for comparison with the shared-prefix call
    unshared = float("nan")
    if setup.shared:
        ua, ub = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_u = min(K, 20)
        torch.cuda.synchronize()
        ua.record(stream)
        for i in range(n_u):
            setup.step_unshared(r=i % R)
        ub.record(stream)
        torch.cuda.synchronize()
        unshared = ua.elapsed_time(ub) / n_u

    # context: host cost of a prefix-cached allocation (kv_seq_alloc_prefix) of
    # one of this workload's requests while the shared prefix is held
    host_prefix_us = None
    if w.prefix:
        from paged_block_quantized_amd import KVPool
        n_tok = int(setup.ctx.max())
        hp = KVPool(setup.pool.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.v_codec,
                    k_codec=W.k_codec_of(w),
                    max_seqs=4, device=None)
        ids = np.random.default_rng(0).integers(0, 32000, n_tok).astype(np.int32)
        hp.alloc_prefix(0, ids[:w.prefix])
        reps = 20
        t0 = time.perf_counter()
        from paged_block_quantized_amd import _lib as L
        for i in range(reps):
            cached = L.kv_seq_alloc_prefix(hp.handle, 1, ids)
            L.kv_seq_free(hp.handle, 1)
        host_prefix_us = round((time.perf_counter() - t0) * 1e6 / reps, 1)
        assert cached == w.prefix
        hp.close()

    step_bytes = dbytes + sbytes
    # paged_attn_decode reads a shared prefix once per sequence
    obytes = runner.decode_bytes(dataclasses.replace(w, prefix=0), setup.ctx) if w.prefix else dbytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = step_bytes / (step_call_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": w.name, "layers": 1, "num_seqs": S,
            "context": int(setup.ctx.max()) if w.ctx_kind == "fixed" else [int(setup.ctx.min()), int(setup.ctx.max())],
            "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size,
            "k_codec": {"i8": "int8_sym", "fp8": "fp8_e4m3", "i4": "int4_asym"}[W.k_codec_of(w)],
            "v_codec": {"i8": "int8_sym", "i4": "int4_asym", "i8a": "int8_asym", "fp8": "fp8_e4m3"}[w.v_codec],
            "partition": setup.partition, "shared_prefix": w.prefix,
            "pool_copies_rotated": R,
            "batch_order": "the workload's own order (single-pass grouped-query launches rank the "
                           "sequences by length inside the kernel)",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s_per_layer": round(S / (ms_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "kernels_ms": {"paged_attn_decode_append": round(step_call_ms, 5),
                       "paged_attn_decode_append_per_call_events": round(float(np.mean(fused_ms)), 5),
                       "paged_attn_decode_append_p10": round(float(np.percentile(fused_ms, 10)), 5),
                       "paged_attn_decode_append_p90": round(float(np.percentile(fused_ms, 90)), 5),
                       "paged_attn_decode": round(dec_loop_ms, 5),
                       "separate_step_ms_per_step": round(ms_sep, 5),
                       "separate_quantize_store_1tok": round(store_ms, 5),
                       "separate_paged_attn_decode_per_call_events": round(dec_ms, 5),
                       "paged_attn_decode_append_same_pool_back_to_back": _r5(np.mean(dec_same)),
                       "paged_attn_decode_after_1GiB_write_flush": _r5(np.median(fl_w)),
                       "paged_attn_decode_after_1GiB_read_flush": _r5(np.median(fl_r)),
                       "per_sequence_step_without_shared_prefix": _r5(unshared)},
        "host_us": {"kv_seq_alloc_prefix_plus_free": host_prefix_us},
        "roofline": {
            "kernel": (("paged_attn_decode_shared_prefix: the prefix's partitions once for all sequences "
                        "(grouped kernel), the store kernel, the per-sequence partitions, the reduce; one call")
                       if setup.shared else
                       ("paged_attn_decode_append: the current token's store fused into the split-K "
                        "decode (plus the reduce kernel when partitions are split), one call")),
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": step_bytes,
            "decode_only": {"kernel": ("paged_attn_decode (no store; a shared prefix read by every "
                                       "sequence), K calls between two events"),
                            "bytes_per_launch": obytes,
                            "achieved": round(obytes / (dec_loop_ms * 1e-3) / 1e9, 2),
                            "frac": round(obytes / (dec_loop_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "plain_read_ceiling": ceiling,
        },
    }
    if not args.no_cpu_baseline:
        print("cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(setup, args.cpu_seconds)
    if not args.only_timed:
        # context, not the step: swapping a quarter of the batch to host memory
        print("swap", file=sys.stderr, flush=True)
        line["swap"] = measure_swap(setup, 5)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
