"""Benchmark: paged-KV decode steps on one MI355X.

One timed step is one decode step of the whole batch through ``--layers``
attention layers (distinct K/V pools per layer, one block table shared by all
layers, as a model's layers share page ids):

  host   : the page allocator grows every sequence by one token
           (pkv_alloc_reserve_batch); when a sequence starts a new page, the
           block table is copied to the device (async, pinned);
  device : per layer, append the new token's K/V and run paged decode
           attention (fused append + partition kernel + log-sum-exp reduce,
           or separate append with ``--separate-append``).

Positions advance every step, so the context grows and sequences cross page
boundaries as they do in serving. Inputs are seeded synthetic data
(``workloads``): layer 0 is the workload as drawn, the other layers get their
own random pools drawn on the device. The first step of layer 0 is checked
against the fp64 oracle on sampled sequences.

Timing: HIP events on the launch stream bracket the whole timed region
(``ms_per_step``, ``value``) and one decode call per step, the layer rotating
with the step (``roofline.avg_launch_us``); an event record costs a few
microseconds of GPU time, so not every call is bracketed.

Output: one JSON line on stdout (rank 0, N = 1).
"""

import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3,
                    help="workload number (3 = Llama-3-8B GQA, shared prefix; 6 = 4096-token sliding window)")
    ap.add_argument("--page-size", type=int, default=None, help="page size (workload 5 only)")
    ap.add_argument("--layers", type=int, default=8, help="distinct layer pools per step (working set >> 256 MB MALL)")
    ap.add_argument("--partition", type=int, default=None, help="partition tokens (0 = unsplit)")
    ap.add_argument("--separate-append", action="store_true", help="kv_append launch + decode instead of fused")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="treat a shared prefix like private tokens (read once per sequence)")
    ap.add_argument("--graph", action="store_true",
                    help="replay a captured HIP graph of each step's layer calls instead of launching them from "
                         "Python (slower on this stack: graph launch costs more than it saves)")
    ap.add_argument("--patch-max", type=int, default=1024,
                    help="table changes per step applied in place by pkv_block_table_patch; more -> full upload")
    ap.add_argument("--n-query", type=int, default=1,
                    help="chunk of K new tokens per sequence and step (one chunk append, then one causal "
                         "multi-query attention call, pkv_paged_decode_attention_multi); tokens/s counts B * K per "
                         "layer-step")
    ap.add_argument("--int8-keys", action="store_true",
                    help="keys as int8 codes with a per-token fp32 scale, values fp16 (pkv_kv_append_k8 + "
                         "pkv_paged_decode_attention_k8)")
    ap.add_argument("--no-stream-peak", action="store_true",
                    help="skip the streaming-read ceiling measurement (pkv_probe_stream_read)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time for the CPU baseline")
    ap.add_argument("--check-sequences", type=int, default=8)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (3 times) so HBM counters can be "
                         "scaled against a kernel of known traffic")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True).stdout.strip() or None
    except Exception:
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or None


def algorithmic_bytes(lens, B, Hq, Hkv, D, P, shared_tokens, k_bytes=None, n_query=1):
    """Unique bytes one layer-step must move: every attended K/V byte once
    (shared-prefix tokens once for the whole batch), q in, out, new K/V in and
    written, the block-table entries and lengths. ``k_bytes``: stored bytes of
    one token's key per KV head (2 D for fp16, D + 4 for int8 codes + scale)."""
    kb = 2 * D if k_bytes is None else k_bytes
    lens = np.asarray(lens, dtype=np.int64)
    kv_tokens = int(lens.sum()) - shared_tokens * (len(lens) - 1)
    kv = kv_tokens * Hkv * (kb + 2 * D)
    q_out = 2 * n_query * B * Hq * D * 2
    new_kv = n_query * B * Hkv * (2 * 2 * D + kb + 2 * D)   # read k_new/v_new (fp16), write them to the pools
    table = int(sum(-(-int(n) // P) for n in lens)) * 4 + B * 4
    return kv + q_out + new_kv + table, kv


def algorithmic_bytes_window(lens, B, Hq, Hkv, D, P, window, k_bytes=None):
    """Unique bytes of one sliding-window layer-step: the K/V of the last
    ``window`` tokens of each sequence, q in, out, the new K/V read and
    written, the ring entries the window touches and the lengths. ``k_bytes``:
    stored bytes of one token's key per KV head (2 D for fp16, D + 4 for int8)."""
    kb = 2 * D if k_bytes is None else k_bytes
    lens = np.asarray(lens, dtype=np.int64)
    lo = np.maximum(lens - window, 0)
    kv_tokens = int((lens - lo).sum())
    kv = kv_tokens * Hkv * (kb + 2 * D)
    q_out = 2 * B * Hq * D * 2
    new_kv = B * Hkv * (2 * 2 * D + kb + 2 * D)
    table = int(((lens - 1) // P - lo // P + 1).clip(min=0).sum()) * 4 + B * 4
    return kv + q_out + new_kv + table, kv


def kernel_source_digest():
    """sha256 of the device source with comments and whitespace removed, so a
    comment edit does not orphan the committed counter summary."""
    import hashlib
    import re
    path = os.path.join(ROOT, "paged_kv_cache_279_amd", "csrc", "pkv_device.hip")
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic(workload_name, config_key):
    """HBM bytes per partition-kernel launch from the committed rocprofv3
    counter summary, if it was taken on this exact kernel source and
    configuration; else None.

    FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the
    same counter reads for a plain device copy of known size (the summary
    records both factors)."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_code_sha256") != kernel_source_digest():
        return None
    entry = rec.get("configs", {}).get(config_key)
    if not entry or entry.get("workload") != workload_name:
        return None
    k = entry["partition_kernel"]
    return (k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"]) * 1024


def streaming_peak(torch, pkv, nbytes, stream, n_buf=8, reps=4):
    """Streaming-read rate over the decode call's byte count: pkv_probe_stream_read
    over random 4 KiB tiles of n_buf rotating buffers (so the 256 MB
    Infinity Cache holds none of them), timed back to back with HIP events."""
    n_tiles = max(1, int(nbytes) // 4096)
    bufs = [torch.ones(n_tiles * 4096, dtype=torch.uint8, device="cuda") for _ in range(n_buf)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    order = torch.randperm(n_tiles, device="cuda", generator=gen).to(torch.int32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b in bufs:
        pkv.probe_stream_read(b, order, sink, stream=stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for r in range(n_buf * reps):
        pkv.probe_stream_read(bufs[r % n_buf], order, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (n_buf * reps)
    del bufs
    torch.cuda.empty_cache()
    return n_tiles * 4096 / us / 1e3, us, n_tiles * 4096


def logical_table(ring, n_tokens, P):
    """Block table of logical pages 0 .. ceil(n / P) - 1 of ring-paged
    sequences (logical page j in ring entry j % R), for the oracle's append."""
    R = ring.shape[1]
    width = max(1, -(-int(n_tokens) // P))
    return np.ascontiguousarray(ring[:, np.arange(width) % R])


def cpu_baseline(w, seconds):
    """Time the oracle (as it stands) on layer 0 of the workload: append then
    decode for every sequence, repeated until ``seconds`` have passed."""
    import oracle
    from threadpoolctl import threadpool_limits
    step = 0
    lens = w.lens(step)
    passes = 0
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    logical = logical_table(w.block_table, int(lens.max()), w.P) if w.window else w.block_table
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        while True:
            kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new[step], w.v_new[step], logical,
                                      w.pos(step), w.P)
            if w.window:
                oracle.decode_attention_window(w.q, kp, vp, w.block_table, lens, w.window, w.scale, w.P)
            else:
                oracle.decode_attention(w.q, kp, vp, w.block_table, lens, w.scale, w.P)
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {
        "value": passes * w.B / dt,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d pass(es) of append + decode over layer 0 of workload '%s' (%d sequences, %d cached tokens), "
                  "numpy fp64 with %d BLAS threads (the oracle's Python loops run on one); %.1f s"
                  % (passes, w.name, w.B, int(lens.sum()), cores, dt),
        "cpu_model": cpu_model(),
        "host_cores_available": len(os.sched_getaffinity(0)),
        "numpy": np.__version__,
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import oracle
    import paged_kv_cache_279_amd as pkv
    from workloads import workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pkv.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    w = workload(args.workload, page_size=args.page_size)
    B, Hq, Hkv, D, P = w.B, w.Hq, w.Hkv, w.D, w.P
    part = w.partition_tokens if args.partition is None else args.partition
    R = args.layers
    total_steps = args.warmup + args.steps
    k8 = args.int8_keys
    KQ = args.n_query
    fused = not args.separate_append and KQ == 1
    prefix_tokens = 0 if args.no_shared_prefix else w.shared_prefix_pages * w.P
    W = w.window
    if W and (KQ > 1 or not fused or args.graph):
        raise SystemExit("the sliding-window workload runs one query, the fused append, eagerly")
    if w.steps == 0:
        raise SystemExit("workload %d has no append; pick 2-5" % args.workload)
    if KQ > 1 and args.graph:
        raise SystemExit("--n-query runs without graphs")
    log("workload %s: B=%d Hq=%d Hkv=%d D=%d P=%d part=%d layers=%d fused=%s" % (w.name, B, Hq, Hkv, D, P, part, R,
                                                                                  fused))

    # ---- a1: page allocator (host). Pages for every step are drawn on demand;
    # a sliding window holds a fixed ring of pages per sequence, reserved once.
    prefix_pages = w.shared_prefix_pages
    final_ctx = w.context.astype(np.int64) + KQ * max(total_steps, w.steps)   # tokens after the last step
    if W:
        need = w.N
        max_pages = w.max_pages
    else:
        need = prefix_pages + sum(-(-int(n) // P) - prefix_pages for n in final_ctx)
        max_pages = max(-(-int(n) // P) for n in final_ctx)
    N = max(need, w.N)
    free_order = np.concatenate([w.perm, np.arange(w.N, N, dtype=np.int32)]).astype(np.int32)
    alloc = pkv.PageAllocator(N, P, free_order=free_order)
    seqs = np.arange(B, dtype=np.int32)
    if prefix_pages:
        owner = B
        alloc.reserve(owner, prefix_pages * P)
        for b in range(B):
            alloc.share_prefix(b, alloc.table(owner))
    bt_np = np.full((B, max_pages), -1, dtype=np.int32)          # the allocator's table (host)
    # the workload reserves pages for all of its own steps up front (page-sweep: 64 steps)
    alloc.reserve_batch(seqs, np.full(B, max_pages * P) if W else w.context + w.steps, bt_np)
    assert np.array_equal(bt_np[:, :w.max_pages], w.block_table), "allocator layout differs from the workload"

    # ---- device buffers
    def put(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + args.workload)
    k_pools, v_pools = [], []

    def random_k8_pool():
        # codes uniform in [-127, 127], positive fp32 scales: timing does not depend on the values
        codes = torch.randint(-127, 128, (N, Hkv, P // 16, 16 * D), dtype=torch.int8, device=dev, generator=gen)
        scales = torch.randn((N, Hkv, P // 16, 16), device=dev, generator=gen).abs_().mul_(0.05).add_(0.005)
        return torch.cat([codes.view(torch.uint8), scales.view(torch.uint8)], dim=-1).contiguous()

    for layer in range(R):
        vp = pkv.empty_pool(N, Hkv, P, D, device=dev)
        if k8:
            kp = random_k8_pool()
        else:
            kp = pkv.empty_pool(N, Hkv, P, D, device=dev)
        if layer == 0:
            if not k8:
                kp[:w.N].copy_(put(w.k_pool))
            vp[:w.N].copy_(put(w.v_pool))
            if N > w.N:
                if not k8:
                    kp[w.N:].normal_(generator=gen)
                vp[w.N:].normal_(generator=gen)
        else:
            if not k8:
                kp.normal_(generator=gen)
            vp.normal_(generator=gen)
        k_pools.append(kp)
        v_pools.append(vp)
    k8_layer0 = k_pools[0].cpu().numpy() if k8 else None
    q = put(w.q)
    knew = torch.empty((total_steps, B, Hkv, D), dtype=torch.float16, device=dev)
    vnew = torch.empty_like(knew)
    knew.normal_(generator=gen)
    vnew.normal_(generator=gen)
    knew[0].copy_(put(w.k_new[0]))
    vnew[0].copy_(put(w.v_new[0]))
    bt_dev = torch.from_numpy(bt_np).to(dev)
    lens_all = torch.from_numpy((w.context[None, :] + KQ * (1 + np.arange(total_steps)[:, None])).astype(np.int32)).to(dev)
    pos_all = lens_all - 1
    if KQ > 1:
        # the chunk's K positions per step, and K tokens (step 0: the workload's token first) per step
        pos_chunk = (lens_all - KQ).contiguous()                    # [steps][B]: first position of each chunk
        knew_mq = torch.empty((total_steps, B, KQ, Hkv, D), dtype=torch.float16, device=dev)
        vnew_mq = torch.empty_like(knew_mq)
        knew_mq.normal_(generator=gen)
        vnew_mq.normal_(generator=gen)
        knew_mq[0, :, 0].copy_(put(w.k_new[0]))
        vnew_mq[0, :, 0].copy_(put(w.v_new[0]))
        q_mq = torch.empty((B, KQ, Hq, D), dtype=torch.float16, device=dev)
        q_mq.normal_(generator=gen)
        out_mq = torch.empty((B, KQ, Hq, D), dtype=torch.float16, device=dev)
    max_context = int(final_ctx.max())
    ws_bytes = pkv.decode_workspace_bytes_multi(B, KQ, Hq, D, W or max_context, part, prefix_tokens)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    k_pool_bytes = pkv.k8_pool_bytes(N, Hkv, P, D) if k8 else N * Hkv * P * D * 2
    mem_gb = R * (k_pool_bytes + N * Hkv * P * D * 2) / 1e9
    log("pools: N=%d pages/layer, %.2f GB over %d layers" % (N, mem_gb, R))

    scale = w.scale

    def layer_call(layer, lens, pos, kn, vn, s):
        if W:
            window_call = pkv.paged_decode_attention_window_k8 if k8 else pkv.paged_decode_attention_window
            window_call(q, k_pools[layer], v_pools[layer], bt_dev, lens, W, scale, part, k_new=kn, v_new=vn,
                        out=out, workspace=workspace, stream=s)
        elif KQ > 1:
            # pos [B], kn / vn [B][K][Hkv][D]: the chunk's K tokens in one append launch, then its attention
            if k8:
                pkv.kv_append_k8_chunk(kn, vn, k_pools[layer], v_pools[layer], bt_dev, pos, stream=s)
                pkv.paged_decode_attention_multi_k8(q_mq, k_pools[layer], v_pools[layer], bt_dev, lens, max_context,
                                                    scale, part, prefix_tokens=prefix_tokens, out=out_mq,
                                                    workspace=workspace, stream=s)
            else:
                pkv.kv_append_chunk(kn, vn, k_pools[layer], v_pools[layer], bt_dev, pos, stream=s)
                pkv.paged_decode_attention_multi(q_mq, k_pools[layer], v_pools[layer], bt_dev, lens, max_context,
                                                 scale, part, out=out_mq, workspace=workspace, stream=s,
                                                 prefix_tokens=prefix_tokens)
        elif k8:
            if not fused:
                pkv.kv_append_k8(kn, vn, k_pools[layer], v_pools[layer], bt_dev, pos, stream=s)
            pkv.paged_decode_attention_k8(q, k_pools[layer], v_pools[layer], bt_dev, lens, max_context, scale, part,
                                          prefix_tokens, k_new=kn if fused else None, v_new=vn if fused else None,
                                          out=out, workspace=workspace, stream=s)
        elif prefix_tokens:
            if not fused:
                raise SystemExit("the shared-prefix bench path runs with the fused append")
            pkv.paged_decode_attention_shared_prefix(
                q, k_pools[layer], v_pools[layer], bt_dev, lens, max_context, scale, part, prefix_tokens,
                k_new=kn, v_new=vn, out=out, workspace=workspace, stream=s)
        elif fused:
            pkv.append_paged_decode_attention(q, kn, vn, k_pools[layer], v_pools[layer], bt_dev, lens, max_context,
                                              scale, part, out=out, workspace=workspace, stream=s)
        else:
            pkv.kv_append(kn, vn, k_pools[layer], v_pools[layer], bt_dev, pos, stream=s)
            pkv.paged_decode_attention(q, k_pools[layer], v_pools[layer], bt_dev, lens, max_context, scale, part,
                                       out=out, workspace=workspace, stream=s)

    def layer_step(step, layer):
        if KQ > 1:
            layer_call(layer, lens_all[step], pos_chunk[step], knew_mq[step], vnew_mq[step], stream)
        else:
            layer_call(layer, lens_all[step], pos_all[step], knew[step], vnew[step], stream)

    last_bt = bt_np.copy()
    host_t = {"alloc": 0.0, "upload": 0.0}
    # table uploads go through a ring of pinned staging buffers; a buffer is
    # refilled only once the stream has finished the copy that last used it
    n_stage = 4
    stage = [torch.empty((B, max_pages), dtype=torch.int32).pin_memory() for _ in range(n_stage)]
    stage_ev = [torch.cuda.Event() for _ in range(n_stage)]
    stage_used = [False] * n_stage
    n_upload = 0

    def host_step(step):
        # a1: grow every sequence to hold this step's token; upload the table if it changed
        nonlocal last_bt, n_upload
        if W:
            return                       # the ring is fixed: nothing to allocate or upload
        t0 = time.perf_counter()
        alloc.reserve_batch(seqs, w.context + KQ * (step + 1), bt_np)
        changed = not np.array_equal(bt_np, last_bt)
        t1 = time.perf_counter()
        if changed:
            rows, cols = np.nonzero(bt_np != last_bt)
            if len(rows) <= args.patch_max:
                # a few new pages: patch the device table in place (entries in the kernel arguments)
                pkv.block_table_patch(bt_dev, rows, cols, bt_np[rows, cols], stream=stream)
            else:
                i = n_upload % n_stage
                if stage_used[i]:
                    stage_ev[i].synchronize()
                stage[i].numpy()[...] = bt_np
                bt_dev.copy_(stage[i], non_blocking=True)
                stage_ev[i].record(stream)
                stage_used[i] = True
                n_upload += 1
            last_bt = bt_np.copy()
        host_t["alloc"] += t1 - t0
        host_t["upload"] += time.perf_counter() - t1

    # ---- parity check: step 0, layer 0, sampled sequences, against the oracle
    if KQ > 1:
        # the pools before the call (pages past the workload's pool are drawn on the device): the oracle
        # appends the chunk itself
        k_init, v_init = k_pools[0].cpu().numpy(), v_pools[0].cpu().numpy()
    host_step(0)
    layer_step(0, 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # the split schedule's header (private blocks per KV head, then the private
    # and prefix blocks per workgroup piece) as the partition kernel left it
    sched = workspace[:12].view(torch.int32).cpu().numpy().tolist() if part > 0 else None
    sample = np.linspace(0, B - 1, min(B, args.check_sequences)).astype(int)
    if KQ > 1:
        got = out_mq.cpu().numpy().astype(np.float64)
        kp0, vp0 = w.k_pool, w.v_pool
        bt0 = bt_np[:, :]
        kn0, vn0 = knew_mq[0].cpu().numpy(), vnew_mq[0].cpu().numpy()
        # token i of sequence b goes to position context[b] + i (the oracle's token writes, in place on
        # one copy of the pools; int8 keys quantised by the oracle's quantiser)
        kpool_full, vpool_full = k_init.copy(), v_init.copy()
        for b in range(B):
            for i in range(KQ):
                page, off = oracle.token_slot(bt0[b], int(w.context[b]) + i, P)
                for h in range(Hkv):
                    if k8:
                        codes, sc = oracle.quantize_k(kn0[b, i, h])
                        oracle.k8_write_token(kpool_full, page, h, off, codes, sc, D)
                    else:
                        oracle.write_token(kpool_full, page, h, off, kn0[b, i, h], "k")
                    oracle.write_token(vpool_full, page, h, off, vn0[b, i, h], "v")
        # query i of a chunk is the single-token decode of its own prefix (the oracle's chunk
        # definition); long chunks are checked on the first, second, middle and last queries
        qi = np.arange(KQ) if KQ <= 8 else np.unique(np.array([0, 1, KQ // 2, KQ - 1]))
        one = oracle.decode_attention_k8 if k8 else oracle.decode_attention
        qh = q_mq.cpu().numpy()[sample]
        lens0 = (w.context + KQ).astype(np.int32)[sample]
        ref = np.stack([one(qh[:, i], kpool_full, vpool_full, bt0[sample], lens0 - KQ + i + 1, scale, P) for i in qi],
                       axis=1)
        got = got[:, qi]
    elif W:
        logical = logical_table(w.block_table, int(w.lens(0).max()), P)
        if k8:
            kp0, vp0 = oracle.kv_append_k8(k8_layer0[:w.N], w.v_pool, w.k_new[0], w.v_new[0], logical, w.pos(0), P)
            ref = oracle.decode_attention_window_k8(w.q[sample], kp0, vp0, w.block_table[sample], w.lens(0)[sample],
                                                    W, scale, P)
        else:
            kp0, vp0 = oracle.kv_append(w.k_pool, w.v_pool, w.k_new[0], w.v_new[0], logical, w.pos(0), P)
            ref = oracle.decode_attention_window(w.q[sample], kp0, vp0, w.block_table[sample], w.lens(0)[sample], W,
                                                 scale, P)
    elif k8:
        kp0, vp0 = oracle.kv_append_k8(k8_layer0[:w.N], w.v_pool, w.k_new[0], w.v_new[0], w.block_table, w.pos(0), P)
        ref = oracle.decode_attention_k8(w.q[sample], kp0, vp0, w.block_table[sample], w.lens(0)[sample], scale, P)
    else:
        kp0, vp0 = oracle.kv_append(w.k_pool, w.v_pool, w.k_new[0], w.v_new[0], w.block_table, w.pos(0), P)
        ref = oracle.decode_attention(w.q[sample], kp0, vp0, w.block_table[sample], w.lens(0)[sample], scale, P)
    err = np.abs(got[sample].astype(np.float64) - ref)
    max_err = float(err.max())
    # the worst element beside half a step of the fp16 output grid at its
    # value: what rounding the exact result to fp16 alone leaves there
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    worst_ref = float(ref[worst])
    worst_half_step = float(np.spacing(np.float16(abs(worst_ref)))) / 2
    log("parity (layer 0, step 0, %d sequences): max_abs_err=%.3e at an output of %.3f (half an fp16 step there: %.3e)"
        % (len(sample), max_err, worst_ref, worst_half_step))
    if not max_err <= 4e-3:
        raise SystemExit("parity check failed: %.3e" % max_err)
    # the check ran step 0 on layer 0 already; restore its pools so every layer starts alike
    if k8:
        k_pools[0].copy_(put(k8_layer0))
    else:
        k_pools[0][:w.N].copy_(put(w.k_pool))
    v_pools[0][:w.N].copy_(put(w.v_pool))

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of %d MiB (read %d B + write %d B each)" % (args.copy_calibration_mib, n, n))
        del src, dst

    # ---- launch mode. Graph: the R layer calls of a step are captured once as
    # a HIP graph over fixed step buffers; each step copies its lengths and new
    # tokens into them, then replays the graph (no Python per layer).
    graph = None
    if args.graph:
        lens_cur = lens_all[0].clone()
        pos_cur = pos_all[0].clone()
        kn_cur = knew[0].clone()
        vn_cur = vnew[0].clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for layer in range(R):
                layer_call(layer, lens_cur, pos_cur, kn_cur, vn_cur, cap)
        torch.cuda.synchronize()

    def run_step(step, per_call_events=None, kernel_events=None):
        if graph is not None:
            lens_cur.copy_(lens_all[step], non_blocking=True)
            pos_cur.copy_(pos_all[step], non_blocking=True)
            kn_cur.copy_(knew[step], non_blocking=True)
            vn_cur.copy_(vnew[step], non_blocking=True)
            if per_call_events is not None:
                per_call_events[0].record(stream)
            graph.replay()
            if per_call_events is not None:
                per_call_events[1].record(stream)
        else:
            # one call per step is bracketed by events (the layer rotates with the
            # step): an event record costs a few microseconds of GPU time itself
            timed = step % R
            for layer in range(R):
                if per_call_events is not None and layer == timed:
                    per_call_events[0].record(stream)
                if kernel_events is not None and layer == timed:
                    # the partition kernel of this call records its own start and stop
                    pkv.profile_next_partition_kernel(*kernel_events)
                layer_step(step, layer)
                if per_call_events is not None and layer == timed:
                    per_call_events[1].record(stream)

    # ---- warmup
    for step in range(args.warmup):
        host_step(step)
        run_step(step)
    torch.cuda.synchronize()

    # ---- timed: HIP events on the launch stream around the decode calls (the
    # graph replay of a step's R calls, or one eager call per step)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    kev = None
    if graph is None:
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for pair in kev:                       # torch creates an event on its first record
            for e in pair:
                e.record(stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    host_s = launch_s = 0.0
    host_t["alloc"] = host_t["upload"] = 0.0
    for i in range(args.steps):
        step = args.warmup + i
        h0 = time.perf_counter()
        host_step(step)
        h1 = time.perf_counter()
        # eager: even timed steps time the partition kernel (its own launch events),
        # odd ones the whole call, so that no step carries both
        if kev is not None and i % 2 == 0:
            run_step(step, None, kev[i])
        elif kev is not None:
            run_step(step, ev[i], None)
        else:
            run_step(step, ev[i])
        host_s += h1 - h0
        launch_s += time.perf_counter() - h1
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    log("host per step: allocator %.1f us, table upload %.1f us, launching the layer calls %.1f us; GPU %.1f us "
        "per step" % (host_t["alloc"] / args.steps * 1e6, host_t["upload"] / args.steps * 1e6,
                      launch_s / args.steps * 1e6, total_ms / args.steps * 1e3))
    if graph is not None:
        call_ms = np.array([e[0].elapsed_time(e[1]) / R for e in ev])
        kernel_ms = None
    else:
        call_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(1, args.steps, 2)])
        kernel_ms = np.array([kev[i][0].elapsed_time(kev[i][1]) for i in range(0, args.steps, 2)])
    ms_per_step = total_ms / args.steps
    ms_per_layer = ms_per_step / R

    config_key = "%s:P%d:part%d:%s:%s%s" % (w.name, P, part, "fused" if fused else "separate",
                                           "prefix" if prefix_tokens else "noprefix", ":k8" if k8 else "")
    # algorithmic bytes of the timed steps (lengths grow by one per step)
    bytes_steps = []
    kv_steps = []
    for i in range(args.steps):
        step = args.warmup + i
        if W:
            tot, kv = algorithmic_bytes_window(w.context + step + 1, B, Hq, Hkv, D, P, W,
                                               k_bytes=(D + 4) if k8 else None)
        else:
            tot, kv = algorithmic_bytes(w.context + KQ * (step + 1), B, Hq, Hkv, D, P, prefix_pages * P,
                                        k_bytes=(D + 4) if k8 else None, n_query=KQ)
        bytes_steps.append(tot)
        kv_steps.append(kv)
    bytes_per_call = float(np.mean(bytes_steps))
    kv_per_call = float(np.mean(kv_steps))
    call_avg_s = float(call_ms.mean()) / 1e3 if len(call_ms) else float("nan")
    call_gbps = bytes_per_call / call_avg_s / 1e9
    # the dominant kernel: the partition kernel, timed by its own start/stop events;
    # in split mode the merge kernel writes the output rows, so they are not its bytes
    split = part > 0
    kernel_bytes = bytes_per_call - (2 * B * KQ * Hq * D if split else 0)
    kernel_avg_s = float(kernel_ms.mean()) / 1e3 if kernel_ms is not None else call_avg_s
    achieved = kernel_bytes / kernel_avg_s / 1e9
    tokens_per_s = B * KQ / (ms_per_layer / 1e3)

    result = {
        "metric": "decode tokens/s and effective KV-read HBM GB/s (% of peak), GQA 32/8, d=128",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_size": P,
            "kv_dtype": "k int8 + fp32 scale per token and head, v f16" if k8 else "f16", "accumulate": "f32",
            "arithmetic": "matrix-core products on f16 operands (q, K, V and the softmax weights P rounded to f16; int8 "
                          "key codes widened to f16 exactly) with f32 accumulation; softmax statistics and the "
                          "log-sum-exp merge in f32; f16 output",
            "mean_context": float(np.mean(w.context + KQ * (args.warmup + 1 + (args.steps - 1) / 2))),
            "queries_per_sequence": KQ,
            "window_tokens": W or None,
            "ring_pages": max_pages if W else None,
            "shared_prefix_tokens": prefix_pages * P,
            "partition_tokens": part,
            "split_schedule": None if sched is None else {
                "private_blocks_per_kv_head": sched[0],
                "private_piece_blocks": sched[1], "private_piece_tokens": sched[1] * 16,
                "prefix_piece_blocks": sched[2] if prefix_tokens else None,
                "note": "partition_tokens is the minimum piece; each workgroup takes one piece of this many "
                        "16-token blocks from each work list (pieces may cross sequence boundaries)"},
            "layers_per_step": R,
            "append": "fused" if fused else "separate",
            "launch": "eager" if graph is None else "hip graph per step (%d layer calls)" % R,
            "shared_prefix_path": bool(prefix_tokens),
            "tokens_per_s_definition": ("batch * queries per sequence / (time of one attention layer-step: "
                                        "chunk append + chunk attention), i.e. tokens verified per second through one "
                                        "layer") if KQ > 1 else
                                       "batch / (time of one attention layer-step: append + decode), "
                                       "i.e. sequences advanced per second through one layer",
            "tokens_per_s_32_layers": round(tokens_per_s / 32, 1),
            "ms_per_layer_step": round(ms_per_layer, 5),
            "kv_gbps": round(kv_per_call / (ms_per_layer / 1e3) / 1e9, 1),
            "kv_frac_of_peak": round(kv_per_call / (ms_per_layer / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
            "parity_max_abs_err": max_err,
            "parity_worst_output": round(worst_ref, 5),
            "parity_worst_fp16_half_step": worst_half_step,
            "working_set_gb": round(mem_gb, 2),
            "wall_s": round(wall, 3),
            "git": git_sha(),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_partition_kernel (%s%s%s%s%s)" % (
                "split" if split else "unsplit",
                ", shared prefix" if prefix_tokens else "", ", int8 keys" if k8 else "",
                ", %d-query chunks" % KQ if KQ > 1 else ", sliding window" if W else "",
                ", fused append" if fused else ""),
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": measured_traffic(w.name, config_key),
            "traffic_unit": "HBM bytes per partition-kernel launch (FETCH_SIZE x fetch scale + WRITE_SIZE x write "
                            "scale)",
            "bytes_per_launch": round(kernel_bytes),
            "avg_launch_us": round(kernel_avg_s * 1e6, 3),
            "timing": ("hipExtLaunchKernel start/stop events of the partition kernel: one layer call on every even "
                       "timed step (odd steps time the whole call)"
                       if kernel_ms is not None else "graph replay events / layers (whole call)"),
            "call": {
                "what": "whole decode call: partition kernel%s, launch gap and two event records" % (
                    " + log-sum-exp merge kernel" if split else ""),
                "avg_us": round(call_avg_s * 1e6, 3) if len(call_ms) else None,
                "bytes": round(bytes_per_call),
                "achieved_gbps": round(call_gbps, 1) if len(call_ms) else None,
                "frac": round(call_gbps / PEAK_HBM_GBPS, 4) if len(call_ms) else None,
            },
        },
    }
    if not args.no_stream_peak:
        peak_gbps, peak_us, peak_bytes = streaming_peak(torch, pkv, kernel_bytes, stream)
        log("streaming-read ceiling: %.1f MB in %.2f us = %.0f GB/s" % (peak_bytes / 1e6, peak_us, peak_gbps))
        result["roofline"]["streaming_read_peak"] = {
            "value": round(peak_gbps, 1), "unit": "GB/s", "bytes": peak_bytes, "us": round(peak_us, 3),
            "how": "pkv_probe_stream_read: the call's byte count as random 4 KiB tiles, non-temporal 16-byte "
                   "loads, 8 rotating buffers, back-to-back launches"}
        result["roofline"]["frac_of_streaming_peak"] = round(achieved / peak_gbps, 4)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (>= %.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
