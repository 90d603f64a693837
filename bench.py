"""Benchmark of the paged KV cache hot path on one MI355X.

One step = one decode pass over all 80 layers of the Llama-3-70B-shaped
workload (batch 32 x 8,192 tokens, 64 query / 8 KV heads of 128, bf16, 16-token
blocks under a shuffled table): the per-step split plan is uploaded, then
each layer runs as one launch that appends the step's token at position
len - 1 (RoPE there) and attends over the layer's cache.  The reported value
is the whole step's algorithmic HBM bytes (every cached K/V byte, q, out, lse,
the block-table entries and the appended token) divided by its time, in GB/s.

The injection workload runs after it: top-8 memory chunks of 64..256 tokens
from a 10,000-chunk store of unrotated bf16 K/V (32 layers x 8 KV heads x 128)
injected for 64 requests at non-consecutive positions, in one call per
repetition; reported as injected tokens/s and GB/s.

Each dominant kernel is also timed per launch with HIP events on the stream
it runs on.  The CPU oracle is timed on a bounded sample of the decode
workload.  One JSON line is printed on stdout; progress goes to stderr.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def recorded_traffic(kernel="decode_mfma_kernel", workload="70b", root=ROOT):
    """HBM bytes per launch of `kernel` on decode workload `workload` from the
    rocprofv3 counter summaries in profiles/, if one was taken on that
    workload with the current kernel sources (else None)."""
    import glob
    import hashlib
    src = os.path.join(root, "paged_kv_cache_inject_amd", "csrc", "pkv_kernels.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic-record:"):
                continue
            fields = dict(kv.split("=", 1) for kv in line.split()[1:])
            if (fields.get("kernel") == kernel and fields.get("workload") == workload
                    and fields.get("sources_sha256") == sha):
                return int(fields["bytes_per_launch"])
    return None


POOL_LAYOUT = os.environ.get("PKV_BENCH_LAYOUT", "block")


def layout_strides(layout, num_blocks, n_kv_heads, plane):
    """(layer, block, head strides, V offset) in elements of a pool layout:
    "block": [layer][block][K planes of all heads | V planes of all heads];
    "head": [layer][block][head][K plane | V plane];
    "plane": [layer][K | V][head][block], so that one head's planes of
    consecutive blocks are adjacent (a 32-token allocation block's two
    16-token planes form one contiguous run per head)."""
    if layout == "plane":
        head_stride = num_blocks * plane
        return 2 * n_kv_heads * head_stride, plane, head_stride, n_kv_heads * head_stride
    block_stride = 2 * n_kv_heads * plane
    if layout == "head":
        return num_blocks * block_stride, block_stride, 2 * plane, plane
    return num_blocks * block_stride, block_stride, plane, n_kv_heads * plane


def device_pool_fp8(n_layers, num_blocks, n_kv_heads, head_dim, seed, scale=0.01, layout=None,
                    per_block=False):
    """fp8 (E4M3) pool of random finite codes with one K and one V scale per
    (layer, KV head), or per (layer, block, KV head) (values in [scale,
    2 scale)); layouts as in device_pool."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    layout = layout or POOL_LAYOUT
    layer_stride, block_stride, head_stride, v_off = layout_strides(
        layout, num_blocks, n_kv_heads, 16 * head_dim)
    buf = torch.empty(n_layers * layer_stride, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    for layer in range(n_layers):
        g.manual_seed(seed * 1000 + layer)
        part = buf[layer * layer_stride:(layer + 1) * layer_stride]
        part.copy_(torch.randint(0, 0x7F, (layer_stride,), dtype=torch.uint8, device="cuda",
                                 generator=g))
        part |= torch.randint(0, 2, (layer_stride,), dtype=torch.uint8, device="cuda",
                              generator=g) << 7
    if per_block:
        g.manual_seed(seed * 1000 + 999)
        shape = (n_layers, num_blocks, n_kv_heads)
        ks = scale * (1 + torch.rand(shape, dtype=torch.float32, device="cuda", generator=g))
        vs = scale * (1 + torch.rand(shape, dtype=torch.float32, device="cuda", generator=g))
    else:
        ks = torch.full((n_layers, n_kv_heads), scale, dtype=torch.float32, device="cuda")
        vs = torch.full((n_layers, n_kv_heads), scale, dtype=torch.float32, device="cuda")
    desc = pkv.pkv_pool(n_layers, num_blocks, n_kv_heads, head_dim, pkv.PKV_FP8E4M3,
                        1 if per_block else 0, buf.data_ptr(), buf.data_ptr() + v_off,
                        layer_stride, block_stride, head_stride, ks.data_ptr(), vs.data_ptr())
    return (buf, ks, vs), desc


def device_pool(n_layers, num_blocks, n_kv_heads, head_dim, dtype, seed, layout=None):
    """Pool buffer filled with N(0,1) per layer, in one of the layouts of
    layout_strides."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from workloads.configs import device_normal
    layout = layout or POOL_LAYOUT
    layer_stride, block_stride, head_stride, v_off = layout_strides(
        layout, num_blocks, n_kv_heads, 16 * head_dim)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    buf = torch.empty(n_layers * layer_stride, dtype=tdt, device="cuda")
    if seed is not None:
        for layer in range(n_layers):
            buf[layer * layer_stride:(layer + 1) * layer_stride] = device_normal(
                layer_stride, dtype, seed * 1000 + layer)
    e = buf.element_size()
    desc = pkv.pkv_pool(n_layers, num_blocks, n_kv_heads, head_dim, pkv.DTYPE_CODES[dtype], 0,
                        buf.data_ptr(), buf.data_ptr() + v_off * e, layer_stride, block_stride,
                        head_stride)
    return buf, desc


def decode_bytes(lens, n_kv_heads, head_dim, n_q_heads, elem, kv_elem=None):
    """Algorithmic bytes of one decode launch (one layer): every cached K/V
    byte (kv_elem bytes per element, default elem), q, out, lse, the table
    entries (and the two scales per KV head of a quantised pool)."""
    kv_elem = elem if kv_elem is None else kv_elem
    kv = int(np.sum(lens)) * n_kv_heads * head_dim * kv_elem * 2
    if kv_elem == 1:
        kv += 2 * n_kv_heads * 4
    q = len(lens) * n_q_heads * head_dim * elem
    out = len(lens) * n_q_heads * head_dim * 4 + len(lens) * n_q_heads * 4
    tables = int(sum(-(-int(x) // 16) for x in lens)) * 4
    return kv + q + out + tables


def append_bytes(n_seqs, n_kv_heads, head_dim, elem, kv_elem=None):
    """Algorithmic bytes of one single-token append (one layer): the new K
    and V rows read and stored, the cos/sin row of each position, the
    position and the table entry of each sequence."""
    kv_elem = elem if kv_elem is None else kv_elem
    rows = n_seqs * n_kv_heads * head_dim
    return rows * 2 * (elem + kv_elem) + n_seqs * head_dim * 4 + n_seqs * 8


def item_balance(lens, part_tokens, n_kv_heads, n_cus=256):
    """Work items of a decode plan and how evenly they load the CUs.

    Items are the plan's token ranges (a sequence longer than part_tokens is
    split into ranges of that many tokens, the last shorter), launched
    longest first, every KV head of an item in turn.  The load model: one
    workgroup per CU at a time, time proportional to tokens, each workgroup
    starting on the CU that frees first.  `lpt_makespan_over_mean` is the
    model's finishing time over the perfectly even share (1.0 = balanced)."""
    import heapq
    items = []
    for n in lens:
        n = int(n)
        t = 0
        while t < n:
            items.append(min(part_tokens, n - t))
            t += part_tokens
    items.sort(reverse=True)
    free = [(0, c) for c in range(n_cus)]
    heapq.heapify(free)
    for x in items:
        for _ in range(n_kv_heads):
            t, c = heapq.heappop(free)
            heapq.heappush(free, (t + x, c))
    makespan = max(t for t, _ in free)
    mean = sum(items) * n_kv_heads / n_cus
    a = np.asarray(items)
    edges = [0] + [1 << k for k in range(4, 16)] + [1 << 30]
    hist = {}
    for lo, hi in zip(edges[:-1], edges[1:]):
        c = int(((a > lo) & (a <= hi)).sum())
        if c:
            hist["%d-%d" % (lo + 1, min(hi, int(a.max())))] = c
    return {"items": len(items), "workgroups": len(items) * n_kv_heads,
            "tokens_per_item_p0_p50_p90_p100": [int(a.min()), int(np.median(a)),
                                                int(np.percentile(a, 90)), int(a.max())],
            "tokens_per_item_histogram": hist,
            "lpt_makespan_over_mean": round(makespan / mean, 4),
            "model": "one workgroup per CU at a time, time proportional to tokens, "
                     "longest first, %d CUs" % n_cus}


def bw_probe(n_bytes=8 << 30, reps=5):
    import torch
    import paged_kv_cache_inject_amd as pkv
    src = torch.ones(n_bytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pkv.pkv_bw_probe(src, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        pkv.pkv_bw_probe(src, sink)
    e.record()
    torch.cuda.synchronize()
    gbps = n_bytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del src
    return gbps


def decode_workload(name):
    from workloads.configs import (LLAMA8B_1LAYER, LLAMA70B_80LAYER, MISTRAL_WINDOW, MQA_64,
                                   RAGGED_MHA, llama70b_structure, llama8b_structure,
                                   ragged_mha_structure, window_structure)
    if name == "mqa":
        return MQA_64, llama70b_structure(MQA_64)
    if name == "mistral-window":
        return MISTRAL_WINDOW, window_structure()
    if name in ("70b", "70b-fp8", "70b-fp8b"):
        return LLAMA70B_80LAYER, llama70b_structure(LLAMA70B_80LAYER)
    if name in ("70b-block32", "70b-block32-fp8"):
        return LLAMA70B_80LAYER, llama70b_structure(LLAMA70B_80LAYER, block_tokens=32)
    if name == "8b":
        return LLAMA8B_1LAYER, llama8b_structure(LLAMA8B_1LAYER)
    if name == "ragged":
        return RAGGED_MHA, ragged_mha_structure(RAGGED_MHA)
    raise ValueError(name)


def run_decode(steps, warmup, workload="70b", launch_steps=None, two_calls=True,
               attention_only=False):
    """One decode step per layer of `workload`: the one-launch append and
    attention (pkv_append_decode_attention), or with attention_only the
    attention call alone over the same cache (pkv_decode_attention), for
    comparing kernels."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from workloads.configs import host_normal, device_normal
    cfg, st = decode_workload(workload)
    lens = st["lens"]
    launch_steps = steps if launch_steps is None else launch_steps
    per_block = workload.endswith("-fp8b")     # fp8 with scales per (layer, block, head)
    fp8 = workload.endswith("-fp8") or per_block
    log("decode: allocating and filling %d layers x %d blocks%s"
        % (cfg.n_layers, st["num_blocks"], " (fp8)" if fp8 else ""))
    if fp8:
        buf, pool = device_pool_fp8(cfg.n_layers, st["num_blocks"], cfg.n_kv_heads,
                                    cfg.head_dim, cfg.seed, per_block=per_block)
    else:
        buf, pool = device_pool(cfg.n_layers, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim,
                                cfg.dtype, cfg.seed)
    q_host = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[cfg.dtype]
    q = torch.from_numpy(q_host.view(np.int16)).cuda().view(tdt)
    tables = torch.from_numpy(st["tables"]).cuda()
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, device="cuda")
    lse = torch.empty(cfg.batch, cfg.n_q_heads, device="cuda")
    part = int(os.environ.get("PKV_BENCH_PART", "0"))
    window = int(st.get("window", 0))
    plan = pkv.pkv_decode_plan_create(lens, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, part,
                                      window=window)
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    n_items = pkv.pkv_decode_plan_items(plan)
    part_tokens = pkv.pkv_decode_plan_part_tokens(plan)
    waves = pkv.pkv_decode_plan_waves(plan)
    # The step's own token: its K and V (per layer, unrotated) are appended
    # at position len - 1 with RoPE before the layer's decode reads the
    # cache, so the query attends to itself.  Every step rewrites that slot,
    # which keeps the context at the workload's length from step to step.
    first = torch.from_numpy((np.asarray(lens) - 1).astype(np.int32)).cuda()
    new_dt = "bf16" if fp8 else cfg.dtype
    n_new = cfg.batch * cfg.n_kv_heads * cfg.head_dim
    k_new = [device_normal(n_new, new_dt, cfg.seed * 7919 + 2 * layer)
             for layer in range(cfg.n_layers)]
    v_new = [device_normal(n_new, new_dt, cfg.seed * 7919 + 2 * layer + 1)
             for layer in range(cfg.n_layers)]
    max_pos = int(np.max(lens))
    cos_h, sin_h = pkv.pkv_rope_table(cfg.head_dim, cfg.rope_base, max_pos)
    dcos, dsin = torch.from_numpy(cos_h).cuda(), torch.from_numpy(sin_h).cuda()

    def step():
        pkv.pkv_decode_plan_upload(plan, ws)
        for layer in range(cfg.n_layers):
            if attention_only:
                pkv.pkv_decode_attention(plan, pool, layer, q, tables, out, lse, ws,
                                         q_dtype=new_dt)
            else:
                pkv.pkv_append_decode_attention(plan, pool, layer, q, tables, k_new[layer],
                                                v_new[layer], "pairs", dcos, dsin, max_pos, out,
                                                lse, ws, q_dtype=new_dt)

    def step_two_calls():
        pkv.pkv_decode_plan_upload(plan, ws)
        for layer in range(cfg.n_layers):
            pkv.pkv_append_kv(pool, layer, tables, first, 1, k_new[layer], v_new[layer], "pairs",
                              dcos, dsin, max_pos)
            pkv.pkv_decode_attention(plan, pool, layer, q, tables, out, lse, ws)

    log("decode: %d warmup steps" % warmup)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_s, t_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Timed region: exactly `steps` steps, no markers between the launches.
    log("decode: %d timed steps" % steps)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_s.record()
    for _ in range(steps):
        step()
    t_e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_s.elapsed_time(t_e)
    # The same step as two launches per layer (pkv_append_kv, then
    # pkv_decode_attention), for comparison.
    two_calls_ms = None
    if two_calls:
        u_s, u_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        step_two_calls()
        u_s.record()
        for _ in range(steps):
            step_two_calls()
        u_e.record()
        torch.cuda.synchronize()
        two_calls_ms = u_s.elapsed_time(u_e) / steps
    # Instrumented pass: the same number of steps again, each launch carrying
    # a start/stop event pair attached to its own dispatch (the kernel's
    # execution, as a profiler's kernel trace measures it).
    i_s, i_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pkv.pkv_kernel_timing(True)
    try:
        i_s.record()
        for _ in range(launch_steps):
            step()
        i_e.record()
        torch.cuda.synchronize()
    finally:
        pkv.pkv_kernel_timing(False)
    launch_ms = [float(x) for x in pkv.pkv_kernel_times()]
    assert len(launch_ms) == launch_steps * cfg.n_layers, len(launch_ms)
    # attended tokens: the last `window` positions under a sliding window
    attended = np.minimum(lens, window) if window > 0 else lens
    per_decode = decode_bytes(attended, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads, 2,
                              kv_elem=1 if fp8 else 2)
    per_append = 0 if attention_only else append_bytes(cfg.batch, cfg.n_kv_heads, cfg.head_dim,
                                                       2, kv_elem=1 if fp8 else 2)
    per_launch = per_decode + per_append
    ms_step = total_ms / steps
    res = dict(ms_per_step=ms_step, wall_ms_per_step=wall * 1e3 / steps,
               instrumented_ms_per_step=i_s.elapsed_time(i_e) / max(1, launch_steps),
               bytes_per_step=per_launch * cfg.n_layers,
               bytes_per_launch=per_launch, append_bytes_per_launch=per_append,
               two_calls_ms_per_step=two_calls_ms,
               # the timed region's duration per launch (the launches run back to back)
               launch_ms_avg=ms_step / cfg.n_layers,
               # per-dispatch events (the kernel and its dispatch) of the instrumented pass
               event_ms_avg=float(np.mean(launch_ms)), event_ms_p50=float(np.median(launch_ms)),
               event_ms_p10=float(np.percentile(launch_ms, 10)),
               event_ms_p90=float(np.percentile(launch_ms, 90)),
               seed=cfg.seed,
               tables_sha256=hashlib.sha256(np.ascontiguousarray(st["tables"]).tobytes()).hexdigest(),
               launches_timed=len(launch_ms),
               n_items=n_items, part_tokens=part_tokens, waves=waves,
               workload=cfg.workload + ((" (fp8 E4M3 cache, scales per block)" if per_block
                                         else " (fp8 E4M3 cache)") if fp8 else ""),
               dtype="fp8e4m3" if fp8 else cfg.dtype,
               batch=cfg.batch, context=int(lens.max()), layers=cfg.n_layers)
    res["value"] = res["bytes_per_step"] / (ms_step * 1e-3) / 1e9
    res["launch_gbps"] = per_launch / (res["launch_ms_avg"] * 1e-3) / 1e9
    if cfg.n_layers == 1:
        # A single layer re-reads the same bytes every step, part of which the
        # 256 MB last-level cache can hold: also time each step after reading
        # through a 1 GiB buffer (outside the events), which leaves none of the
        # layer in that cache and no dirty lines in it, median of the steps.
        # The same after writing the buffer instead: that step also carries
        # some of the write's aftermath.
        flush = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        pkv.pkv_bw_probe(flush, sink)
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

        def after(prep):
            times = []
            for k in range(steps):
                prep(k)
                c_s, c_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c_s.record()
                step()
                c_e.record()
                torch.cuda.synchronize()
                times.append(c_s.elapsed_time(c_e))
            return float(np.median(times))

        res["cold_ms_per_step"] = after(lambda k: pkv.pkv_bw_probe(flush, sink))
        res["cold_after_write_ms_per_step"] = after(lambda k: scratch.fill_(k & 0xFF))
        del flush, scratch, sink
        res["cold_gbps"] = res["bytes_per_step"] / (res["cold_ms_per_step"] * 1e-3) / 1e9
        res["cold_after_write_gbps"] = (res["bytes_per_step"] /
                                        (res["cold_after_write_ms_per_step"] * 1e-3) / 1e9)
        log("decode: cold caches %.4f ms/step, %.1f GB/s (after a 1 GiB write %.4f ms/step)"
            % (res["cold_ms_per_step"], res["cold_gbps"], res["cold_after_write_ms_per_step"]))
    log("decode: %.3f ms/step, %.1f GB/s; per launch %.1f us -> %.1f GB/s; as two calls "
        "per layer %s ms/step" % (ms_step, res["value"], res["launch_ms_avg"] * 1e3,
                                  res["launch_gbps"],
                                  "-" if two_calls_ms is None else "%.3f" % two_calls_ms))
    pkv.pkv_decode_plan_destroy(plan)
    del buf, ws, q, tables, out, lse, k_new, v_new, first, dcos, dsin
    torch.cuda.empty_cache()
    return res, st


def run_inject(reps):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from workloads.configs import INJECT_TOP8, inject_structure, device_normal
    cfg = INJECT_TOP8
    st = inject_structure(cfg)
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    n_src = st["n_src"]
    row = H * d
    log("inject: store of %d tokens x %d layers (%.1f GB)" %
        (n_src, L, 2 * n_src * L * row * 2 / 1e9))
    store_k = torch.empty(L * n_src * row, dtype=torch.bfloat16, device="cuda")
    store_v = torch.empty(L * n_src * row, dtype=torch.bfloat16, device="cuda")
    for layer in range(L):
        a, b = layer * n_src * row, (layer + 1) * n_src * row
        store_k[a:b] = device_normal(b - a, "bf16", cfg.seed * 1000 + 2 * layer)
        store_v[a:b] = device_normal(b - a, "bf16", cfg.seed * 1000 + 2 * layer + 1)
    buf, pool = device_pool(L, st["num_blocks"], H, d, "bf16", None)
    cache = pkv.pkv_cache_create(st["num_blocks"], cfg.batch, st["max_blocks"],
                                 st["free_list_seed"])
    for b, m in enumerate(st["mem_lens"]):
        pkv.pkv_alloc_blocks(cache, b, int(m))
    max_pos = 4096
    cos, sin = pkv.pkv_rope_table(d, cfg.rope_base, max_pos)
    dcos, dsin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    src = pkv.make_src(store_k, store_v, n_src * row, row, n_src)
    runs = pkv.make_runs(st["runs"])
    ws = torch.empty(pkv.pkv_inject_workspace_bytes(runs), dtype=torch.uint8, device="cuda")
    n_tok = int(sum(r[1] for r in st["runs"]))

    def once():
        pkv.pkv_inject(cache, pool, src, runs, 0, L, "pairs", dcos, dsin, max_pos, ws)

    once()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        once()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    bytes_call = n_tok * L * row * 2 * 2 * 2     # K and V, read and written
    res = dict(ms_per_call=ms, tokens=n_tok, tokens_per_s=n_tok / (ms * 1e-3),
               token_layers_per_s=n_tok * L / (ms * 1e-3), gbps=bytes_call / (ms * 1e-3) / 1e9,
               bytes_per_call=bytes_call, requests=cfg.batch, layers=L)
    log("inject: %.3f ms/call, %.3g tok/s, %.1f GB/s" % (ms, res["tokens_per_s"], res["gbps"]))
    pkv.pkv_cache_destroy(cache)
    res["request_path"] = run_request_path(cfg, st, pool, src, runs, dcos, dsin, max_pos, ws,
                                           reps=max(2, reps // 3))
    del store_k, store_v, buf, ws
    torch.cuda.empty_cache()
    return res


def run_request_path(cfg, st, pool, src, runs, dcos, dsin, max_pos, inject_ws, reps):
    """Every step of the path for one batch of requests, from an empty cache:
    reserve each request's blocks, inject the composed memory (all layers),
    extend by the 32-token suffix, export and upload the tables, append the
    suffix in every layer, extend by the decode token, export the tables
    again, plan, and run the decode step (the token appended at len - 1 and
    attended over) in every layer.  Timed from the host's first call to the
    end of the last kernel; the GPU time of each phase comes from events."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from workloads.configs import device_normal
    L, H, d, B = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.batch
    HQ, suffix = cfg.n_q_heads, cfg.extra["suffix"]
    row = H * d
    seqs = list(range(B))
    suf_k = [device_normal(B * suffix * row, "bf16", cfg.seed * 31 + 4 * l) for l in range(L)]
    suf_v = [device_normal(B * suffix * row, "bf16", cfg.seed * 31 + 4 * l + 1) for l in range(L)]
    tok_k = [device_normal(B * row, "bf16", cfg.seed * 31 + 4 * l + 2) for l in range(L)]
    tok_v = [device_normal(B * row, "bf16", cfg.seed * 31 + 4 * l + 3) for l in range(L)]
    q = device_normal(B * HQ * d, "bf16", cfg.seed * 37).view(B, HQ, d)
    out = torch.empty(B, HQ, d, device="cuda")
    lse = torch.empty(B, HQ, device="cuda")
    tdev = torch.empty(B, st["max_blocks"], dtype=torch.int32, device="cuda")
    fdev = torch.empty(B, dtype=torch.int32, device="cuda")
    lens_end = np.asarray(st["mem_lens"]) + suffix + 1
    probe = pkv.pkv_decode_plan_create(lens_end, HQ, H, d, 0)
    dws = torch.empty(pkv.pkv_decode_workspace_bytes(probe), dtype=torch.uint8, device="cuda")
    pkv.pkv_decode_plan_destroy(probe)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    host = {}

    def timed(key, fn, *a):
        t0 = time.perf_counter()
        r = fn(*a)
        host[key] = host.get(key, 0.0) + (time.perf_counter() - t0) * 1e3
        return r

    def reserve():
        c = pkv.pkv_cache_create(st["num_blocks"], B, st["max_blocks"], st["free_list_seed"])
        for b, m in enumerate(st["mem_lens"]):
            pkv.pkv_alloc_blocks(c, b, int(m))
        return c

    def tables_for(c, n_new):
        first = pkv.pkv_extend(c, seqs, n_new)
        table, lens = pkv.pkv_block_table(c, seqs, st["max_blocks"])
        return first, table, lens

    def batch():
        host.clear()
        c = timed("reserve", reserve)
        ev[0].record()
        timed("inject_call", pkv.pkv_inject, c, pool, src, runs, 0, L, "pairs", dcos, dsin,
              max_pos, inject_ws)
        ev[1].record()
        first, table, _ = timed("extend_and_tables", tables_for, c, suffix)
        tdev.copy_(torch.from_numpy(table))
        fdev.copy_(torch.from_numpy(first.astype(np.int32)))
        for layer in range(L):
            pkv.pkv_append_kv(pool, layer, tdev, fdev, suffix, suf_k[layer], suf_v[layer],
                              "pairs", dcos, dsin, max_pos)
        ev[2].record()
        _, table, lens = timed("extend_and_tables", tables_for, c, 1)
        tdev.copy_(torch.from_numpy(table))
        plan = timed("decode_plan", pkv.pkv_decode_plan_create, lens, HQ, H, d, 0)
        pkv.pkv_decode_plan_upload(plan, dws)
        for layer in range(L):
            pkv.pkv_append_decode_attention(plan, pool, layer, q, tdev, tok_k[layer], tok_v[layer],
                                            "pairs", dcos, dsin, max_pos, out, lse, dws)
        ev[3].record()
        return c, plan

    c, plan = batch()                      # warm-up
    torch.cuda.synchronize()
    pkv.pkv_decode_plan_destroy(plan)
    pkv.pkv_cache_destroy(c)
    wall, phases, hosts = [], [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        c, plan = batch()
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - t0) * 1e3)
        phases.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
        hosts.append(dict(host))
        pkv.pkv_decode_plan_destroy(plan)
        pkv.pkv_cache_destroy(c)
    ms = float(np.median(wall))
    ph = np.median(np.array(phases), axis=0)
    n_tok = int(sum(r[1] for r in st["runs"]))
    res = dict(ms_per_batch=ms, requests=B, layers=L, injected_tokens=n_tok,
               requests_per_s=B / (ms * 1e-3), injected_tokens_per_s=n_tok / (ms * 1e-3),
               gpu_ms_inject=float(ph[0]), gpu_ms_suffix_append=float(ph[1]),
               gpu_ms_decode_step=float(ph[2]),
               host_ms={k: float(np.median([h[k] for h in hosts])) for k in hosts[0]})
    log("request path: %.3f ms per batch of %d requests (inject %.3f, suffix append %.3f, "
        "decode step %.3f ms on the GPU; host %s)" % (ms, B, ph[0], ph[1], ph[2],
                                                      res["host_ms"]))
    del suf_k, suf_v, tok_k, tok_v, q, out, lse, tdev, fdev, dws
    return res


def run_inject_host(reps, n_chunks=250, batch=16, dma_compare=False):
    """The injection workload with the chunk store in pinned host memory
    ([InferScale] §6): 16 requests compose the prefix and top-8 of 250 chunks;
    the inject kernel reads only the runs' rows, over PCIe, while it writes the
    pool.  Reported against the same run's host-to-device DMA ceiling.

    The K and V stores are torch tensors allocated with pin_memory=True, so
    every torch copy into or out of them goes through torch's own
    pinned-memory path; the inject call reads them through their pinned
    addresses."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from workloads.configs import INJECT_TOP8, inject_structure, device_normal
    cfg = INJECT_TOP8
    st = inject_structure(cfg, n_chunks=n_chunks, batch=batch)
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    n_src, row = st["n_src"], H * d
    nbytes = L * n_src * row * 2                       # one of K, V
    log("inject (host store): %d tokens x %d layers in pinned host memory (%.1f GB)"
        % (n_src, L, 2 * nbytes / 1e9))
    stores = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    assert all(t.is_pinned() and t.numel() == nbytes for t in stores)
    try:
        for salt, store in enumerate(stores):
            for layer in range(L):
                a = layer * n_src * row * 2
                b = a + n_src * row * 2
                assert 0 <= a < b <= store.numel()
                t = device_normal(n_src * row, "bf16", cfg.seed * 1000 + 2 * layer + salt)
                store[a:b].copy_(t.view(torch.uint8))
                del t
        log("inject (host store): store filled")
        # DMA ceiling: 1 GiB pinned -> device
        pin = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dma = []
        for _ in range(4):
            s.record()
            dst.copy_(pin, non_blocking=True)
            e.record()
            torch.cuda.synchronize()
            dma.append((1 << 30) / (s.elapsed_time(e) * 1e-3) / 1e9)
        dma_gbps = float(np.median(dma[1:]))
        del pin, dst
        buf, pool = device_pool(L, st["num_blocks"], H, d, "bf16", None)
        cache = pkv.pkv_cache_create(st["num_blocks"], batch, st["max_blocks"], st["free_list_seed"])
        for b_, m in enumerate(st["mem_lens"]):
            pkv.pkv_alloc_blocks(cache, b_, int(m))
        max_pos = 4096
        cos, sin = pkv.pkv_rope_table(d, cfg.rope_base, max_pos)
        dcos, dsin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
        src = pkv.make_src(stores[0].data_ptr(), stores[1].data_ptr(), n_src * row, row, n_src,
                           dtype="bf16")
        runs = pkv.make_runs(st["runs"])
        ws = torch.empty(pkv.pkv_inject_workspace_bytes(runs), dtype=torch.uint8, device="cuda")
        n_tok = int(sum(r[1] for r in st["runs"]))
        for (_seq, n, _dst, src_tok) in st["runs"]:
            assert 0 <= src_tok and src_tok + n <= n_src

        def once():
            pkv.pkv_inject(cache, pool, src, runs, 0, L, "pairs", dcos, dsin, max_pos, ws)

        once()
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            once()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        src_bytes = n_tok * L * row * 2 * 2            # K and V rows read over PCIe
        # The alternative: a copy engine moves each run's rows (one
        # host-to-device copy per run, layer and K/V) from the same pinned
        # store into a device staging buffer for the kernel to scatter from.
        # Only the copies are timed.
        dma_runs_ms = None
        if dma_compare:
            staging = torch.empty(n_tok * row * 2, dtype=torch.uint8, device="cuda")

            def copies():
                for layer in range(L):
                    at = 0
                    for (_seq, n, _dst, src_tok) in st["runs"]:
                        nb_ = n * row * 2
                        assert (at + n) * row * 2 <= staging.numel()
                        for store in stores:
                            a = (layer * n_src + src_tok) * row * 2
                            assert a + nb_ <= nbytes
                            staging[at * row * 2:at * row * 2 + nb_].copy_(store[a:a + nb_],
                                                                           non_blocking=True)
                        at += n

            copies()
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            copies()
            torch.cuda.synchronize()
            dma_runs_ms = (time.perf_counter() - w0) * 1e3
            del staging
        res = dict(ms_per_call=ms, tokens=n_tok, requests=batch, layers=L,
                   tokens_per_s=n_tok / (ms * 1e-3), pcie_gbps=src_bytes / (ms * 1e-3) / 1e9,
                   dma_gbps=dma_gbps, src_bytes=src_bytes, store_gb=2 * nbytes / 1e9,
                   dma_per_run_ms=dma_runs_ms, dma_per_run_copies=len(st["runs"]) * L * 2)
        log("inject (host store): %.3f ms/call, %.3g tok/s, %.1f GB/s over PCIe (DMA ceiling %.1f)"
            % (ms, res["tokens_per_s"], res["pcie_gbps"], dma_gbps))
        pkv.pkv_cache_destroy(cache)
        del buf, ws
    finally:
        torch.cuda.synchronize()
        del stores
    torch.cuda.empty_cache()
    return res


def run_cow(reps):
    """Copy-on-write for beam search on the 70B-shaped cache (80 layers, 8 KV
    heads, d=128, bf16): 32 prompts of 200 tokens (12 full blocks and 8
    tokens), each forked into 4 beams; the first new token of beams 1-3
    copies the shared, partly filled last block (every layer, K and V), 96
    block copies per round.  Only pkv_copy_blocks is timed; fork, extend and
    free between rounds are host work."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    L, H, d = 80, 8, 128
    prompts, beams, plen = 32, 4, 200
    per_prompt = -(-plen // 16)
    nb = prompts * (per_prompt + beams) + 64
    buf, pool = device_pool(L, nb, H, d, "bf16", None)
    cache = pkv.pkv_cache_create(nb, prompts * beams, 16)
    for p_ in range(prompts):
        pkv.pkv_extend(cache, [p_], plen)
    beam_seqs = [prompts + p_ * (beams - 1) + b for p_ in range(prompts) for b in range(beams - 1)]
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times, pairs = [], 0
    for r in range(reps + 1):
        for p_ in range(prompts):
            for b in range(beams - 1):
                pkv.pkv_fork(cache, p_, prompts + p_ * (beams - 1) + b)
        pkv.pkv_extend(cache, beam_seqs, 1)
        pairs = len(pkv.pkv_pending_copies(cache))
        s.record()
        pkv.pkv_copy_blocks(cache, pool)
        e.record()
        torch.cuda.synchronize()
        if r > 0:
            times.append(s.elapsed_time(e))
        for x in beam_seqs:
            pkv.pkv_free_seq(cache, x)
    ms = float(np.median(times))
    moved = pairs * L * 2 * H * 16 * d * 2 * 2        # K and V planes, read and written
    res = dict(pairs=pairs, layers=L, bytes_moved=moved, us_per_round=ms * 1e3,
               gbps=moved / (ms * 1e-3) / 1e9,
               workload="beam search, 70B-shaped cache: 32 prompts x 200 tokens, 4 beams each; "
                        "the first new token of beams 1-3 copies the shared partial block")
    log("cow: %d block copies in %.1f us, %.1f GB/s (read + write)" % (pairs, ms * 1e3, res["gbps"]))
    pkv.pkv_cache_destroy(cache)
    del buf
    torch.cuda.empty_cache()
    return res


def run_tiny(reps=200):
    """The tiny fp32 workload (1 layer, 2 sequences of 37 and 100 tokens, 4
    query / 2 KV heads, d 64, 16-block pool under a permuted table): latency
    of injecting its 24-token unrotated chunk at positions 40..63 of
    sequence 1 (pkv_inject, one layer) and of one decode over both sequences
    (pkv_decode_attention).  Each call is timed from the host call to its
    completion (median) and by events around it on the stream."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from workloads.configs import TINY, tiny_inputs
    cfg = TINY
    w = tiny_inputs(cfg)
    L, H, d, hq = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    buf, pool = device_pool(L, w["num_blocks"], H, d, "f32", None)
    buf.zero_()
    cache = pkv.pkv_cache_create(w["num_blocks"], 2, w["max_blocks"])
    for sq in range(2):
        pkv.pkv_set_blocks(cache, sq, [b for b in w["tables"][sq] if b >= 0], 0)
    n_src = w["src_k"].shape[1]
    sk = torch.from_numpy(np.ascontiguousarray(w["src_k"]).reshape(-1)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w["src_v"]).reshape(-1)).cuda()
    src = pkv.make_src(sk, sv, n_src * H * d, H * d, n_src)
    max_pos = 128
    cos, sin = pkv.pkv_rope_table(d, cfg.rope_base, max_pos)
    dcos, dsin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    pkv.pkv_inject(cache, pool, src, w["prefill_runs"], 0, L, "pairs", dcos, dsin, max_pos, ws)
    table, lens = pkv.pkv_block_table(cache, [0, 1], w["max_blocks"])
    tdev = torch.from_numpy(table).cuda()
    q = torch.from_numpy(np.ascontiguousarray(w["q"]).reshape(-1)).cuda().view(2, hq, d)
    out = torch.empty(2, hq, d, device="cuda")
    lse = torch.empty(2, hq, device="cuda")
    plan = pkv.pkv_decode_plan_create(lens, hq, H, d, 0)
    dws = torch.empty(pkv.pkv_decode_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    pkv.pkv_decode_plan_upload(plan, dws)
    runs = pkv.make_runs(w["chunk_runs"])

    def inject():
        pkv.pkv_inject(cache, pool, src, runs, 0, L, "pairs", dcos, dsin, max_pos, ws)

    def decode():
        pkv.pkv_decode_attention(plan, pool, 0, q, tdev, out, lse, dws)

    res = {}
    for name, fn in (("inject_chunk", inject), ("decode", decode)):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        host, ev = [], []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            host.append((time.perf_counter() - t0) * 1e6)
            ev.append(a.elapsed_time(b) * 1e3)
        res[name] = {"host_call_to_done_us_p50": round(float(np.median(host)), 2),
                     "events_us_p50": round(float(np.median(ev)), 2)}
    pkv.pkv_decode_plan_destroy(plan)
    pkv.pkv_cache_destroy(cache)
    del buf, sk, sv, ws, dws
    log("tiny: inject %s, decode %s" % (res["inject_chunk"], res["decode"]))
    return res


def _oracle_tiny(reps):
    """The oracle on the tiny workload: prefill and chunk inject, then decode
    of both sequences; returns (ms for the chunk inject, ms for the decode,
    pid)."""
    from oracle import attention as o_att, inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.layout import PoolSpec
    from oracle.rope import rope_table
    from workloads.configs import TINY, tiny_inputs
    cfg = TINY
    w = tiny_inputs(cfg)
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    nb = w["num_blocks"]
    plane = 16 * d
    spec = PoolSpec(L, nb, H, d, "f32", nb * 2 * H * plane, 2 * H * plane, plane)
    pool = np.zeros(L * nb * 2 * H * plane, dtype=np.float32)
    model = AllocatorModel(nb, 2, w["max_blocks"])
    for sq in range(2):
        model.set_blocks(sq, [b for b in w["tables"][sq] if b >= 0], 0)
    cos, sin = rope_table(d, cfg.rope_base, 128)
    n_src = w["src_k"].shape[1]
    args = (w["src_k"].reshape(-1), w["src_v"].reshape(-1), n_src * H * d, H * d, 0, L, "pairs",
            cos, sin)
    lens = o_inject.inject(pool, pool[H * plane:], spec, model.tables, [0, 0], w["prefill_runs"],
                           *args)
    t_inj = t_dec = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        o_inject.inject(pool, pool[H * plane:], spec, model.tables, lens, w["chunk_runs"], *args)
        t1 = time.perf_counter()
        o_att.decode_paged(w["q"], pool, pool[H * plane:], spec, 0, model.tables, lens,
                           cfg.n_q_heads)
        t_dec += time.perf_counter() - t1
        t_inj += t1 - t0
    return t_inj / reps * 1e3, t_dec / reps * 1e3, os.getpid()


# ---------------------------------------------------------------------------
# CPU baseline: the oracle timed on the host's cores (a reported baseline, not
# a target).  Worker processes are spawned at the start of main(), before this
# process touches the GPU, and never import torch; each runs numpy with one
# BLAS thread.  Every unit builds fresh synthetic inputs of the workload's
# shape (not timed) and times only the oracle call.
# ---------------------------------------------------------------------------
CPU_SHARE = 16            # host cores one GPU's job may use on the GPU machine


def _worker_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:
        pass


def _worker_ready(pause):
    time.sleep(pause)          # keeps every worker busy so that each submit spawns one
    return os.getpid()


def start_cpu_pool():
    """Spawn one worker per host core (at most CPU_SHARE); returns (pool, n)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    n = max(1, min(CPU_SHARE, len(os.sched_getaffinity(0))))
    ex = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                             initializer=_worker_init)
    pids = list(ex.map(_worker_ready, [1.0] * n))
    return ex, len(set(pids))


def host_info():
    model, ram = "?", None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    return {"cpu_model": model, "host_ram_gib": ram}


def _oracle_decode_units(hq, hkv, d, dtype, lens, seed):
    """Oracle decode of one synthetic sequence per length (one layer each):
    a pool holding only that sequence's blocks under a shuffled table, N(0,1)
    values, and a query; times decode_paged alone.  Returns (kv bytes, s)."""
    from oracle import attention as o_att
    from oracle.layout import PoolSpec
    from workloads.configs import host_normal
    rng = np.random.default_rng(seed)
    plane = 16 * d
    bs = 2 * hkv * plane
    elem = 1 if dtype == "fp8" else (4 if dtype == "f32" else 2)
    by = secs = 0.0
    for ln in lens:
        nb = -(-int(ln) // 16)
        pool = host_normal(rng, (nb * bs,), dtype)
        table = [rng.permutation(nb).tolist()]
        q = host_normal(rng, (1, hq, d), dtype)
        spec = PoolSpec(1, nb, hkv, d, dtype, nb * bs, bs, plane)
        t0 = time.perf_counter()
        o_att.decode_paged(q, pool, pool[hkv * plane:], spec, 0, table, [int(ln)], hq, seqs=[0],
                           by_plane=True)
        secs += time.perf_counter() - t0
        by += int(ln) * hkv * d * elem * 2
    return by, secs, os.getpid()


def _oracle_inject_request(L, hkv, d, runs, seed):
    """Oracle inject of one request's runs (prefix, chunks, separators) over
    L layers from a store holding only the rows the runs name.  Returns
    (injected tokens x layers, s)."""
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.layout import PoolSpec
    from oracle.rope import rope_table
    from workloads.configs import host_normal
    rng = np.random.default_rng(seed)
    n_tok = sum(n for (_s, n, _p, _src) in runs)
    m = max(p + n for (_s, n, p, _src) in runs)
    local, at = [], 0
    for (_s, n, p, _src) in runs:                 # store rows renumbered 0..n_tok-1
        local.append((0, n, p, at))
        at += n
    row = hkv * d
    src_k = host_normal(rng, (L * n_tok * row,), "bf16")
    src_v = host_normal(rng, (L * n_tok * row,), "bf16")
    nb = -(-m // 16)
    model = AllocatorModel(nb, 1, nb)
    model.alloc_blocks(0, m)
    plane = 16 * d
    bs = 2 * hkv * plane
    spec = PoolSpec(L, nb, hkv, d, "bf16", nb * bs, bs, plane)
    pool = np.zeros(L * nb * bs, dtype=np.uint16)
    cos, sin = rope_table(d, 10000.0, m)
    t0 = time.perf_counter()
    o_inject.inject(pool, pool[hkv * plane:], spec, model.tables, [0], local, src_k, src_v,
                    n_tok * row, row, 0, L, "pairs", cos, sin)
    return n_tok * L, time.perf_counter() - t0, os.getpid()


def _parallel(ex, fn, jobs):
    """Run jobs on the pool; returns (total work, the busiest worker's summed
    oracle time, all workers' summed oracle time)."""
    futs = [ex.submit(fn, *j) for j in jobs]
    res = [f.result() for f in futs]
    per_pid = {}
    for work, secs, pid in res:
        per_pid[pid] = per_pid.get(pid, 0.0) + secs
    return sum(r[0] for r in res), max(per_pid.values()), sum(per_pid.values())


def cpu_baselines(ex, n_workers, units_70b=8):
    """The oracle on the host's cores, per workload: the 70B decode (a
    sample of (sequence, layer) units), the 8B-shaped layer (in full), the
    ragged MHA batch (a sample of its sequences) and the top-8 injection (a
    sample of requests over 8 of 32 layers).  Each reports the all-core
    rate (total work over the busiest worker's oracle time) and the rate of
    one worker running alone."""
    from workloads.configs import (INJECT_TOP8, LLAMA70B_80LAYER, LLAMA8B_1LAYER, RAGGED_MHA,
                                   inject_structure, llama8b_structure, ragged_mha_structure)
    info = host_info()
    out = {}
    # 70B-shaped decode: units of one (sequence, layer), 8,192 tokens, 64/8 heads
    c = LLAMA70B_80LAYER
    alone = ex.submit(_oracle_decode_units, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype,
                      [8192] * 2, 7).result()
    per_job = units_70b
    by, span, busy = _parallel(ex, _oracle_decode_units,
                               [(c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype, [8192] * per_job,
                                 100 + i) for i in range(n_workers)])
    out["decode_70b"] = dict(
        value=by / span / 1e9, unit="GB/s", cores=n_workers, kind="oracle",
        single_core_value=alone[0] / alone[1] / 1e9,
        sample="%d (sequence, layer) units of the 70B-shaped decode (8,192 tokens, 64 query / "
               "8 KV heads, d 128, bf16) out of %d, %d per worker; float64 numpy, one BLAS "
               "thread per worker; value = KV bytes / the busiest worker's oracle time; "
               "single_core_value = one worker alone on 2 units" % (per_job * n_workers,
                                                                     c.batch * c.n_layers, per_job),
        **info)
    # 8B-shaped layer, all 64 sequences
    c = LLAMA8B_1LAYER
    lens = [int(x) for x in llama8b_structure(c)["lens"]]
    by, span, busy = _parallel(ex, _oracle_decode_units,
                               [(c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype,
                                 lens[i::n_workers], 200 + i) for i in range(n_workers)])
    out["decode_8b"] = dict(value=by / span / 1e9, unit="GB/s", cores=n_workers, kind="oracle",
                            single_core_value=by / busy / 1e9,
                            sample="all 64 sequences of the 8B-shaped layer (lengths 512..4096), "
                                   "dealt over the workers; single_core_value = KV bytes over "
                                   "the summed per-worker times", **info)
    # ragged MHA: a seeded sample of 4 sequences per worker (lognormal lengths)
    c = RAGGED_MHA
    lens = [int(x) for x in ragged_mha_structure(c)["lens"]]
    pick = np.random.default_rng(5).choice(len(lens), min(len(lens), 4 * n_workers),
                                           replace=False)
    sample = [lens[i] for i in pick]
    by, span, busy = _parallel(ex, _oracle_decode_units,
                               [(c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype,
                                 sample[i::n_workers], 300 + i) for i in range(n_workers)])
    out["decode_ragged"] = dict(
        value=by / span / 1e9, unit="GB/s", cores=n_workers, kind="oracle",
        single_core_value=by / busy / 1e9,
        sample="%d of the 256 ragged MHA sequences (seeded draw, %d tokens), 64 heads, d 128, "
               "f16; single_core_value = KV bytes over the summed per-worker times"
               % (len(sample), sum(sample)), **info)
    # injection: one request per worker, 8 of its 32 layers
    c = INJECT_TOP8
    st = inject_structure(c)
    by_req = {}
    for r in st["runs"]:
        by_req.setdefault(r[0], []).append(r)
    reqs = sorted(by_req)[:n_workers]
    tl, span, busy = _parallel(ex, _oracle_inject_request,
                               [(8, c.n_kv_heads, c.head_dim,
                                 sorted(by_req[b], key=lambda r: r[2]), 400 + b) for b in reqs])
    out["inject"] = dict(
        value=tl / c.n_layers / span, unit="tokens/s", cores=n_workers, kind="oracle",
        single_core_value=tl / c.n_layers / busy,
        sample="%d requests of the top-8 injection (prefix, 8 chunks and their separators), 8 "
               "of 32 layers each, rows of the retrieved chunks only; tokens/s counts a token "
               "once for all 32 layers (token-layers / 32)" % len(reqs), **info)
    return out


def _r4(x):
    return None if x is None else round(x, 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--inject-reps", type=int, default=10)
    ap.add_argument("--no-inject", action="store_true")
    ap.add_argument("--inject-only", action="store_true",
                    help="time only the injection workload (no JSON line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache decode figure")
    ap.add_argument("--no-cow", action="store_true", help="skip the copy-on-write figure")
    ap.add_argument("--no-window", action="store_true",
                    help="skip the sliding-window decode figure")
    ap.add_argument("--no-host-store", action="store_true",
                    help="skip the pinned-host-store inject figure")
    ap.add_argument("--host-store-only", action="store_true",
                    help="time only the pinned-host-store inject (no JSON line)")
    ap.add_argument("--cow-reps", type=int, default=10)
    ap.add_argument("--dma-compare", action="store_true",
                    help="also time moving the host store's run rows by one copy per run "
                         "(17,408 copies; off by default to keep the run short)")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the 8B-shaped and ragged-MHA decode figures")
    ap.add_argument("--no-two-calls", action="store_true",
                    help="skip the comparison timing of the step as two launches per layer")
    ap.add_argument("--attention-only", action="store_true",
                    help="time the attention call alone (no fused append) in the decode step")
    ap.add_argument("--decode-kernel", default="auto", choices=["auto", "dot2"],
                    help="dot2: packed dot products on the VALU where they apply (query groups "
                         "of at most 4, 8-wave workgroups, attention alone)")
    ap.add_argument("--decode-workload", default="70b",
                    choices=["70b", "8b", "ragged", "70b-fp8", "70b-fp8b", "mistral-window",
                             "70b-block32", "70b-block32-fp8", "mqa"],
                    help="decode workload timed (the reported line uses 70b)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the hot path here runs on a single MI355X; "
              "multi-GPU sharding is design-only. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    cpu_pool = n_cpu = None
    if not args.no_cpu_baseline and not (args.inject_only or args.host_store_only):
        # the oracle's worker processes start before this process touches the GPU
        cpu_pool, n_cpu = start_cpu_pool()
        log("cpu baseline: %d worker processes" % n_cpu)
    import torch
    import paged_kv_cache_inject_amd as pkv
    pkv.load_library()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log("device:", props.name, getattr(props, "gcnArchName", "?"), "%d CUs" % props.multi_processor_count)
    if args.inject_only:
        run_inject(args.inject_reps)
        return
    if args.host_store_only:
        run_inject_host(max(2, args.inject_reps // 3))
        return
    probe = bw_probe()
    log("bw probe: %.1f GB/s" % probe)
    two = not args.no_two_calls
    if args.decode_kernel == "dot2":
        os.environ["PKV_DECODE_KERNEL"] = "2"
    dec, _ = run_decode(args.steps, args.warmup, args.decode_workload,
                        two_calls=two and not args.attention_only,
                        attention_only=args.attention_only)
    fp8 = fp8b = None
    if not args.no_fp8 and args.decode_workload == "70b":
        fp8, _ = run_decode(args.steps, args.warmup, "70b-fp8", two_calls=two)
        fp8b, _ = run_decode(args.steps, args.warmup, "70b-fp8b", two_calls=False)
    win = None
    if not args.no_window and args.decode_workload == "70b":
        win, _ = run_decode(args.steps, args.warmup, "mistral-window", two_calls=two)
    inj = None if args.no_inject else run_inject(args.inject_reps)
    cow = None if args.no_cow else run_cow(args.cow_reps)
    inj_host = None if args.no_host_store else run_inject_host(
        max(2, args.inject_reps // 3), dma_compare=args.dma_compare)
    shapes = {}
    if not args.no_shapes and args.decode_workload == "70b":
        # the other decode shapes (one layer each; also timed with the last-level
        # cache flushed between steps)
        for name in ("8b", "ragged"):
            shapes[name] = run_decode(args.steps, args.warmup, name, two_calls=False)
    tiny = run_tiny() if args.decode_workload == "70b" else None
    cpu = {}
    if cpu_pool is not None:
        log("cpu baseline: the oracle on %d cores" % n_cpu)
        cpu = cpu_baselines(cpu_pool, n_cpu)
        if tiny is not None:
            ti, td, _ = cpu_pool.submit(_oracle_tiny, 20).result()
            tiny["oracle_ms"] = {"inject_chunk": round(ti, 3), "decode": round(td, 3),
                                 "cores": 1}
        cpu_pool.shutdown()
        log("cpu baseline: %s" % {k: round(v["value"], 3) for k, v in cpu.items()})
    line = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) + injected tokens/s",
        "value": round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dec["dtype"],
        "data": "synthetic",
        "pct_of_peak": round(100 * dec["value"] / PEAK_HBM_GBPS, 2),
        "config": {"workload": dec["workload"], "batch": dec["batch"], "context": dec["context"],
                   "layers": dec["layers"], "part_tokens": dec["part_tokens"],
                   "work_items": dec["n_items"], "waves_per_workgroup": dec["waves"],
                   "pool_layout": POOL_LAYOUT,
                   "step": ("per layer: pkv_decode_attention alone (%s kernel)"
                            % args.decode_kernel) if args.attention_only else
                           "per layer: pkv_append_decode_attention (the step's token "
                           "appended at position len-1 with RoPE, then attention over len "
                           "tokens, one launch)"},
        "roofline": {"bound": "hbm", "achieved": round(dec["launch_gbps"], 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(dec["launch_gbps"] / PEAK_HBM_GBPS, 4),
                     "traffic": recorded_traffic(workload=args.decode_workload),
                     "kernel": "decode_mfma_kernel (pkv_append_decode_attention, one layer)",
                     "bytes_per_launch": dec["bytes_per_launch"],
                     "launch_us_avg": round(dec["launch_ms_avg"] * 1e3, 2),
                     "dispatch_event_us_p10_p50_p90": [round(dec["event_ms_p10"] * 1e3, 2),
                                                       round(dec["event_ms_p50"] * 1e3, 2),
                                                       round(dec["event_ms_p90"] * 1e3, 2)],
                     "frac_of_bw_probe": round(dec["launch_gbps"] / probe, 4),
                     "append_bytes_per_launch": dec["append_bytes_per_launch"],
                     "launch_timing": "launch_us_avg: HIP events around the timed region "
                                      "(%d steps of %d back-to-back launches) divided by the "
                                      "launches; dispatch_event_us: start/stop events attached "
                                      "to each of %d dispatches (hipExtLaunchKernel, via "
                                      "pkv_kernel_timing) in a pass after the timed steps, "
                                      "which include the dispatch itself"
                                      % (args.steps, dec["layers"], dec["launches_timed"])},
        "two_calls_ms_per_step": _r4(dec["two_calls_ms_per_step"]),
        "bw_probe_gbps": round(probe, 1),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", "?"),
                   "compute_units": props.multi_processor_count},
        "inputs": {"seed": dec["seed"], "tables_sha256": dec["tables_sha256"]},
        "cpu_baseline": cpu.get("decode_70b"),
    }
    if tiny is not None:
        line["tiny"] = dict(workload="tiny fp32 reference: 1 layer, 2 sequences (37 and 100 "
                                     "tokens), 4 query / 2 KV heads, d 64, 16-block pool; a "
                                     "24-token chunk injected at 40..63 of sequence 1",
                            latency_only=True, **tiny)
    if fp8 is not None:
        line["decode_fp8"] = {
            "workload": "the same decode workload with an fp8 (E4M3) cache, per-(layer, KV head) "
                        "scales, bf16 queries",
            "ms_per_step": round(fp8["ms_per_step"], 4), "gbps": round(fp8["value"], 1),
            "pct_of_peak": round(100 * fp8["value"] / PEAK_HBM_GBPS, 2),
            "launch_us_avg": round(fp8["launch_ms_avg"] * 1e3, 2),
            "two_calls_ms_per_step": _r4(fp8["two_calls_ms_per_step"]),
            "step_speedup_vs_bf16": round(dec["ms_per_step"] / fp8["ms_per_step"], 3)}
    if fp8b is not None:
        line["decode_fp8_block_scales"] = {
            "workload": "the same decode workload with an fp8 (E4M3) cache whose scales are "
                        "per (layer, block, KV head), bf16 queries",
            "ms_per_step": round(fp8b["ms_per_step"], 4), "gbps": round(fp8b["value"], 1),
            "pct_of_peak": round(100 * fp8b["value"] / PEAK_HBM_GBPS, 2),
            "launch_us_avg": round(fp8b["launch_ms_avg"] * 1e3, 2),
            "vs_per_head_scales": round(fp8b["ms_per_step"] / fp8["ms_per_step"], 3)}
    if win is not None:
        line["decode_window"] = {
            "workload": win["workload"], "ms_per_step": round(win["ms_per_step"], 4),
            "gbps": round(win["value"], 1), "pct_of_peak": round(100 * win["value"] / PEAK_HBM_GBPS, 2),
            "launch_us_avg": round(win["launch_ms_avg"] * 1e3, 2),
            "launch_gbps": round(win["launch_gbps"], 1), "layers": win["layers"],
            "two_calls_ms_per_step": _r4(win["two_calls_ms_per_step"]),
            "bytes_per_launch": win["bytes_per_launch"]}
    if inj is not None:
        line["inject"] = {"tokens_per_s": round(inj["tokens_per_s"], 1), "unit": "tokens/s",
                          "token_layers_per_s": round(inj["token_layers_per_s"], 1),
                          "gbps": round(inj["gbps"], 1), "ms_per_call": round(inj["ms_per_call"], 4),
                          "tokens_per_call": inj["tokens"], "requests": inj["requests"],
                          "layers": inj["layers"],
                          "workload": "top-8 of 10k chunks (64..256 tokens), 32 layers x 8 x 128 "
                                      "bf16, 64 requests, gaps of 1..15 positions",
                          "cpu_baseline": cpu.get("inject")}
        rp = inj["request_path"]
        line["request_path"] = {
            "workload": "the same 64 requests from an empty cache: reserve blocks, inject, "
                        "32-token suffix append, decode step (token appended at len-1 and "
                        "attended) over 32 layers; host planning and table uploads included",
            "ms_per_batch": round(rp["ms_per_batch"], 3),
            "requests_per_s": round(rp["requests_per_s"], 1),
            "injected_tokens_per_s": round(rp["injected_tokens_per_s"], 1),
            "gpu_ms": {"inject": round(rp["gpu_ms_inject"], 3),
                       "suffix_append": round(rp["gpu_ms_suffix_append"], 3),
                       "decode_step": round(rp["gpu_ms_decode_step"], 3)},
            "host_ms": {k: round(v, 3) for k, v in rp["host_ms"].items()},
            "host_ms_meaning": "reserve: cache create + 64 block reservations; inject_call: "
                               "the inject call (host planning, descriptor upload, launch); "
                               "extend_and_tables: two extends with table exports; "
                               "decode_plan: planning the decode step"}
    if inj_host is not None:
        line["inject_host_store"] = {
            "workload": "top-8 of 250 chunks (64..256 tokens) + prefix, 16 requests, 32 layers x "
                        "8 x 128 bf16; store in pinned host memory, rows read over PCIe by the "
                        "inject kernel",
            "tokens_per_s": round(inj_host["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_call": round(inj_host["ms_per_call"], 3),
            "tokens_per_call": inj_host["tokens"], "requests": inj_host["requests"],
            "pcie_gbps": round(inj_host["pcie_gbps"], 2),
            "dma_h2d_ceiling_gbps": round(inj_host["dma_gbps"], 2),
            "frac_of_dma_ceiling": round(inj_host["pcie_gbps"] / inj_host["dma_gbps"], 3),
            "store_gb": round(inj_host["store_gb"], 2),
            "dma_per_run_ms": _r4(inj_host["dma_per_run_ms"]),
            "dma_per_run_copies": inj_host["dma_per_run_copies"],
            "dma_per_run_meaning": "the same rows moved by the copy engine instead, one "
                                   "host-to-device copy per run, layer and K/V into a device "
                                   "staging buffer (copies alone, no scatter)"}
    if cow is not None:
        line["cow"] = {"workload": cow["workload"], "block_copies": cow["pairs"],
                       "layers": cow["layers"], "bytes_moved": cow["bytes_moved"],
                       "us": round(cow["us_per_round"], 1), "gbps": round(cow["gbps"], 1),
                       "pct_of_peak": round(100 * cow["gbps"] / PEAK_HBM_GBPS, 2),
                       "kernel": "copy_blocks_kernel (pkv_copy_blocks)"}
    for name, key in (("8b", "decode_8b"), ("ragged", "decode_ragged")):
        if name not in shapes:
            continue
        r, st = shapes[name]
        line[key] = {
            "workload": r["workload"], "dtype": r["dtype"],
            "ms_per_step": round(r["ms_per_step"], 4), "gbps": round(r["value"], 1),
            "pct_of_peak": round(100 * r["value"] / PEAK_HBM_GBPS, 2),
            "cold_ms_per_step": round(r["cold_ms_per_step"], 4),
            "cold_gbps": round(r["cold_gbps"], 1),
            "cold_after_write_ms_per_step": round(r["cold_after_write_ms_per_step"], 4),
            "cold_after_write_gbps": round(r["cold_after_write_gbps"], 1),
            "launch_us_p10_p50_p90": [round(r["event_ms_p10"] * 1e3, 2),
                                      round(r["event_ms_p50"] * 1e3, 2),
                                      round(r["event_ms_p90"] * 1e3, 2)],
            "bytes_per_step": r["bytes_per_step"], "work_items": r["n_items"],
            "part_tokens": r["part_tokens"], "waves_per_workgroup": r["waves"],
            "seed": r["seed"], "tables_sha256": r["tables_sha256"],
            "cold_meaning": "each step timed after reading through a 1 GiB buffer, so the "
                            "256 MB last-level cache holds none of the layer (and no dirty "
                            "lines); cold_after_write: after writing that buffer instead, "
                            "which leaves some of the write's aftermath in the timed step",
            "cpu_baseline": cpu.get(key)}
        line[key]["balance"] = item_balance(st["lens"], r["part_tokens"],
                                            decode_workload(name)[0].n_kv_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
