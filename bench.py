"""Benchmark: one paged decode step of a 70B-shaped model on one MI355X.

A step is the whole hot path over one batch: the host block manager appends
one token to each of the 100 sequences (slots, any copy-on-write pairs,
tables), the tables / lengths are uploaded, then for each of the 80 layers
one launch writes the new token's K/V into its slot and runs paged decode
attention over every sequence's ~4K-token history (split-context form,
paged_attn_decode_append).  --separate-cache-write times the two-call form
instead (reshape_and_cache, then paged_attn_decode, per layer).

Workload (synthetic, seeded): 80 layers, 64 query / 8 KV heads, head_dim 128,
bf16, 16-token blocks, 100 sequences with contexts ~N(4096, 256) clipped to
[3072, 5120], blocks placed by a seeded permutation of a pool 1.02x the
blocks needed (+ room for the appended tokens).  Cached K/V are N(0, 1)
draws made on the device.

Prints one JSON line: KV-read GB/s (whole step), seq-steps/s, % of the MI355X
HBM peak, a roofline entry for the decode kernel (HIP events around each timed
step's decode launches), and the fp64 CPU oracle timed on a bounded sample of
the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--partition P]
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0    # MI355X HBM3E, AMD's published peak
KV_DTYPES = {"bf16": 0, "fp8": 1, "int8": 2, "int8_tensor": 3, "int8_channel": 4, "int4": 5,
             "int8_kchannel_vtensor": 6}
TENSOR_SCALE = 0.035     # per-tensor K and V scale of the 8-bit runs (fp8 and int8_tensor)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def scale_regions(pool, kvt):
    """(byte offset, float count) of each scale region the pool holds: per
    (token, head) for int8, per (layer, KV head, dim) for the calibrated
    channel scales (K and V, or K only when V has one scale per tensor)."""
    import paged_kv_cache_436_amd as pkv
    c = pool.cfg
    _, _, ks_off, vs_off = pool.region_offsets()
    if kvt == pkv.PKV_KV_INT8:
        n = c.num_layers * c.num_blocks * c.num_kv_heads * c.block_size
    else:
        n = c.num_layers * c.num_kv_heads * c.head_dim
    return [(off, n) for off in (ks_off, vs_off) if off is not None]


def tensor_scales(kvt):
    """(K, V) per-tensor scales the 8-bit runs pass with each call."""
    import paged_kv_cache_436_amd as pkv
    k = TENSOR_SCALE if kvt in (pkv.PKV_KV_FP8_E5M2, pkv.PKV_KV_INT8_TENSOR) else 1.0
    v = TENSOR_SCALE if kvt in (pkv.PKV_KV_FP8_E5M2, pkv.PKV_KV_INT8_TENSOR,
                                pkv.PKV_KV_INT8_KCHANNEL_VTENSOR) else 1.0
    return k, v


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="tokens per KV block of the 70B step (default 16)")
    ap.add_argument("--partition", type=int, default=-1,
                    help="split-context partition size in tokens (-1: the whole table span, one partition)")
    ap.add_argument("--layers", type=int, default=80,
                    help="layers per step (the workload has 80; fewer only for quick experiments)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-cache-write", action="store_true",
                    help="per layer, reshape_and_cache then paged_attn_decode (two launches)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: each layer's call attends to the last N positions only "
                         "(paged_attn_decode_ex; bytes counted over those positions)")
    ap.add_argument("--kv-dtype", default="bf16", choices=sorted(KV_DTYPES),
                    help="KV storage of the pool (8-bit pools hold random codes; the oracle sample runs for bf16 only)")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="with --config cow_prefix: decode through paged_attn_decode_shared_prefix, which reads the "
                         "93 shared prefix blocks once per KV head instead of once per sequence")
    ap.add_argument("--config", default="", choices=["", "llama8b", "long32k_fp8", "long32k_int8", "cow_prefix"],
                    help="instead of the 70B step: one decode layer of another workload (8B-shaped: 64 seqs, "
                         "ctx 512..4096; 32K quantised: 8 seqs x 32768, block 32, partition 512), rotating over "
                         "three pool copies so the 256 MB MALL does not hold the working set; cow_prefix: the "
                         "shared-prefix copy-on-write run, 200 sequences forked from a 1500-token prefix, each "
                         "generating 64..512 tokens)")
    ap.add_argument("--prefix-cache", type=int, default=0,
                    help="host only: N requests sharing a 1500-token system prompt through the block manager's "
                         "prefix cache; report microseconds per request and the prefill tokens it saves")
    ap.add_argument("--prefix-kind", default="hash", choices=["hash", "radix"],
                    help="with --prefix-cache: the SHA-256 block chain or the radix tree over token ids")
    ap.add_argument("--swap", type=int, default=0,
                    help="instead of the decode step: swap N blocks of the 70B-shaped pool out to pinned host "
                         "memory and back (swap_blocks), and report GB/s each way")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the decode step: paged prefill after a prefix-cache hit (200 prompts = a "
                         "1500-token system prompt, cached and shared, + 64..512 own tokens; 70B-shaped heads), "
                         "one layer per call; TFLOP/s against the bf16 matrix-core peak")
    ap.add_argument("--prefill-workload", default="prefix_cache", choices=["prefix_cache", "full_prompt"],
                    help="with --prefill: prefix_cache (above) or full_prompt (16 whole 4096-token prompts)")
    ap.add_argument("--p-one-part", action="store_true",
                    help="with --prefill: PKV_PREFILL_P_ONE_PART (softmax weights meet V rounded once, one "
                         "matrix-core product per P.V tile instead of two)")
    ap.add_argument("--compute-probe", action="store_true",
                    help="instead of the decode step: time the compute of one 16-token bf16 block of one KV head "
                         "per wave (matrix cores vs vector ALU, no HBM traffic; libpkv_probe.so) against the "
                         "time the block takes to stream from HBM")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB three times (torch copy kernel): the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


PROFILE = os.path.join(ROOT, "profiles", "pa_split_kernel_llama70b_bf16.md")
PREFILL_PROFILE = os.path.join(ROOT, "profiles", "pa_prefill_kernel_prefix_prefill.md")
_CSRC = os.path.join(ROOT, "paged_kv_cache_436_amd", "csrc")
# the sources each kernel is compiled from, hashed in this order
KERNEL_SRCS = [os.path.join(_CSRC, f) for f in ("decode_kernels.hip", "decode_common.h", "pkv_codecs.h")]
PREFILL_SRCS = [os.path.join(_CSRC, f) for f in ("prefill_kernels.hip", "decode_common.h", "pkv_codecs.h")]


CONFIGS_PROFILE = os.path.join(ROOT, "profiles", "pa_split_kernel_configs.md")


def measured_traffic(profile=PROFILE, srcs=KERNEL_SRCS, key=None):
    """HBM bytes per launch from a committed rocprofv3 counter summary (the
    line for workload `key` when given), or None when the kernel's sources
    have changed since the counters were taken (the summary records the
    sha256 of the sources concatenated)."""
    import hashlib
    import re
    try:
        text = open(profile, encoding="utf-8").read()
        src = b"".join(open(f, "rb").read() for f in srcs)
    except OSError:
        return None
    tag = re.escape(f"[{key}]") if key else ""
    m = re.search(r"traffic_bytes_per_launch" + tag + r" = (\d+); kernel_source_sha256 = ([0-9a-f]{64})", text)
    if not m or m.group(2) != hashlib.sha256(src).hexdigest():
        return None
    return int(m.group(1))


HOST_LINK_GBS = 64.0     # PCIe Gen5 x16, one direction


def config_bench(args):
    """One appending decode call per launch on another workload's layer,
    rotating over three pool copies; HIP events around K back-to-back calls."""
    import torch

    import paged_kv_cache_436_amd as pkv
    import workloads

    if args.config == "llama8b":
        w = workloads.llama8b()
    else:
        w = workloads.long_quant(pkv.PKV_KV_FP8_E5M2 if args.config == "long32k_fp8" else pkv.PKV_KV_INT8)
    S, Hq, Hkv, D, B, W = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.table_width
    kvt = w.kv_dtype
    e = 2 if kvt == pkv.PKV_KV_BF16 else 1
    P = args.partition if args.partition > 0 else (w.partition_size or (W * B + 31) // 32 * 32)
    cfg = pkv.make_config(1, w.num_blocks, B, Hkv, D, kvt)
    dev = torch.device("cuda:0")
    pools = []
    for i in range(3):
        pool = pkv.Pool(cfg, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(436006 + i)
        k_off, v_off, ks_off, vs_off = pool.region_offsets()
        lb = pool.desc.layer_bytes
        for off in (k_off, v_off):
            region = pool.memory[off: off + lb]
            if e == 2:
                region.view(torch.bfloat16).normal_(generator=g)
            else:
                region.random_(0, 120 if kvt == pkv.PKV_KV_FP8_E5M2 else 256, generator=g)
        for off, n in scale_regions(pool, kvt):
            pool.memory[off: off + 4 * n].view(torch.float32).uniform_(0.02, 0.05)
        pools.append(pool)
    tables = torch.from_numpy(workloads.static_tables(w)).to(dev)
    ctx = torch.from_numpy(np.asarray(w.context_lens, np.int32) ).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(436007)
    q = torch.randn((S, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    newk = torch.randn((S, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    newv = torch.randn((S, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(pkv.paged_attn_workspace_bytes(S, Hq, D, W, B, P), dtype=torch.uint8, device=dev)
    sc = TENSOR_SCALE if kvt == pkv.PKV_KV_FP8_E5M2 else 1.0
    st = torch.cuda.current_stream()

    def call(i):
        pkv.paged_attn_decode_append(out, q, pools[i % 3], 0, newk, newv, tables, ctx, w.scale, k_scale=sc,
                                     v_scale=sc, partition_size=P, workspace=ws, stream=st)

    for i in range(3 * args.warmup):
        call(i)
    torch.cuda.synchronize()
    K = 3 * args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()                      # no garbage-collector pass between the timed launches
    e0.record(st)
    for i in range(K):
        call(i)
    e1.record(st)
    torch.cuda.synchronize()
    gc.enable()
    per = e0.elapsed_time(e1) * 1e-3 / K
    tok = int(np.asarray(w.context_lens, np.int64).sum())
    nbytes = tok * Hkv * (2 * D * e + (8 if kvt == pkv.PKV_KV_INT8 else 0))
    gbs = nbytes / per / 1e9
    name = {"llama8b": "8B-shaped decode layer: 64 seqs x ctx 512..4096, 32q/8kv heads, head_dim 128, bf16 KV, "
                       "block 16",
            "long32k_fp8": "32K quantised decode layer: 8 seqs x 32768, 64q/8kv heads, head_dim 128, fp8 e5m2 KV, "
                           "block 32, partition 512",
            "long32k_int8": "32K quantised decode layer: 8 seqs x 32768, 64q/8kv heads, head_dim 128, int8 "
                            "per-token KV, block 32, partition 512"}[args.config]
    res = {"metric": "paged decode KV-read GB/s (% of MI355X HBM peak) + decode seq-steps/s", "value": round(gbs, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": 3 * args.warmup, "us_per_call": round(per * 1e6, 2),
           "higher_is_better": True, "dtype": {1: "fp8", 2: "int8"}.get(kvt, "bf16"), "data": "synthetic",
           "config": {"workload": name, "partition_size": P, "kv_bytes_per_call": nbytes, "pool_copies": 3},
           "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(CONFIGS_PROFILE, KERNEL_SRCS, args.config),
                        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"}}
    print(json.dumps(res), flush=True)


def cow_bench(args):
    """The shared-prefix copy-on-write run: 200 sequences (40 KV heads, MHA,
    head_dim 128, block 16) forked from one 1500-token prefix whose last block
    is partly filled, each generating 64..512 tokens.  Every step: host
    block-manager append (step 0 copies the shared partial block for 199 of
    the 200 sharers), upload of tables and lengths, copy_blocks when there
    are pairs, and one appending decode launch for the active sequences.  The
    whole run is timed between synchronisations, after warm-up decodes of the
    shared state.  Logical bytes count every sequence's whole context; unique
    bytes count the shared prefix blocks once."""
    import torch

    import paged_kv_cache_436_amd as pkv
    import workloads

    w = workloads.cow_prefix()
    S, H, D, B, W = w.num_seqs, w.num_kv_heads, w.head_dim, w.block_size, w.table_width
    gen = np.asarray(w.extra["gen_steps"], np.int64)
    prefix = int(w.extra["prefix"])
    dev = torch.device("cuda:0")
    cfg = pkv.make_config(1, w.num_blocks, B, H, D)
    pool = pkv.Pool(cfg, device=dev)
    pool.memory.zero_()
    bm = pkv.BlockManager(w.num_blocks, B, w.block_order)
    bm.add_seq(0, prefix)
    for i in range(1, S):
        bm.fork(0, i)
    tab0, _ = bm.block_tables([0], W)
    g = torch.Generator(device=dev)
    g.manual_seed(436009)
    k_pre = torch.randn((prefix, H, D), generator=g, device=dev).to(torch.bfloat16)
    v_pre = torch.randn((prefix, H, D), generator=g, device=dev).to(torch.bfloat16)
    pre_slots = np.array([tab0[0][t // B] * B + t % B for t in range(prefix)], np.int64)
    pkv.reshape_and_cache(pool, 0, k_pre, v_pre, torch.from_numpy(pre_slots).to(dev))
    steps = int(gen.max())
    q_all = torch.randn((S, H, D), generator=g, device=dev).to(torch.bfloat16)
    kn = torch.randn((S, H, D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((S, H, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((S, H, D), dtype=torch.float32, device=dev)
    P = (W * B + 31) // 32 * 32
    prefix_blocks = prefix // B                  # full prefix blocks stay shared for the whole run
    shared = bool(args.shared_prefix)
    if shared:
        # the shared blocks named once: the decode reads them once per KV head
        d_prefix = torch.from_numpy(np.ascontiguousarray(tab0[0][:prefix_blocks], np.int32)).to(dev)
        ws = torch.empty(pkv.paged_attn_shared_prefix_workspace_bytes(S, H, H, D, W, B, pkv.PKV_KV_BF16,
                                                                      prefix_blocks * B),
                         dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(pkv.paged_attn_workspace_bytes(S, H, D, W, B, P), dtype=torch.uint8, device=dev)

    def decode(o, q, tab, ctx, key=None, value=None, st=None, shared_form=shared):
        if shared_form:
            pkv.paged_attn_decode_shared_prefix(o, q, pool, 0, tab, ctx, w.scale, d_prefix, prefix_blocks * B,
                                                partition_size=P, workspace=ws, key=key, value=value, stream=st)
        else:
            # the tables share the prefix's blocks: K/V loaded with the default
            # cache policy, so that a block's other readers find it in L2
            pkv.paged_attn_decode_ex(o, q, pool, 0, tab, ctx, w.scale, partition_size=P, workspace=ws, key=key,
                                     value=value, keep_kv_cached=True, stream=st)
    st = torch.cuda.current_stream()
    # two sets of pinned staging and device tables: the host prepares step
    # i + 1 while the GPU runs step i
    # (tables and lengths share one staging buffer: one host-to-device copy per step)
    stage_h = [torch.empty(S * W + S, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    stage_d = [torch.empty(S * W + S, dtype=torch.int32, device=dev) for _ in range(2)]
    tab_h = [b[:S * W].view(S, W) for b in stage_h]
    ctx_h = [b[S * W:] for b in stage_h]
    tab_d = [b[:S * W].view(S, W) for b in stage_d]
    ctx_d = [b[S * W:] for b in stage_d]
    done = [None, None]
    # warm-up: decodes of the shared state (no append, nothing changes)
    t0s, c0s = bm.block_tables(np.arange(S, dtype=np.int32), W)
    td, cd = torch.from_numpy(t0s).to(dev), torch.from_numpy(c0s).to(dev)
    for _ in range(args.warmup):
        decode(out, q_all, td, cd, st=st)
    # the block copy the first step makes runs once untimed too (between two
    # blocks that hold nothing yet), so that no first-launch cost of its
    # kernel lands inside the timed run
    spare = np.setdiff1d(np.arange(w.num_blocks), t0s[:, :prefix_blocks + 1])[:2]
    pkv.copy_blocks(pool, torch.from_numpy(spare.reshape(1, 2).astype(np.int64)).to(dev), stream=st)
    for k in range(2):                # and so do the staging uploads and the timing events
        stage_d[k].copy_(stage_h[k], non_blocking=True)
    ew = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ew[0].record(st)
    ew[1].record(st)
    torch.cuda.synchronize()
    logical = unique = seq_steps = pairs_total = 0
    ev = []
    waited = 0.0                      # host time spent waiting for the GPU (staging reuse)
    marks = []                        # host clock at each step's start
    # no garbage-collector pass inside the timed run (a full pass over the
    # process's objects stalled one step for ~37 ms)
    gc.collect()
    gc.disable()
    t_start = time.perf_counter()
    for step in range(steps):
        marks.append(time.perf_counter())
        k = step & 1
        active = np.nonzero(gen > step)[0].astype(np.int32)
        n = active.size
        slots, pairs = bm.append(active)
        if done[k] is not None:
            tw = time.perf_counter()
            done[k].synchronize()     # the copy out of this staging set (two steps ago) is done
            waited += time.perf_counter() - tw
        tab_np, ctx_np = bm.block_tables(active, W, out=tab_h[k].numpy()[:n], ctx_out=ctx_h[k].numpy()[:n])
        stage_d[k].copy_(stage_h[k], non_blocking=True)
        if pairs.shape[0]:
            pkv.copy_blocks(pool, torch.from_numpy(pairs).to(dev, non_blocking=False), stream=st)
            pairs_total += pairs.shape[0]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        decode(out[:n], q_all[:n], tab_d[k][:n], ctx_d[k][:n], kn[:n], vn[:n], st=st)
        e1.record(st)
        ev.append((e0, e1))
        done[k] = e1
        ctx64 = ctx_np.astype(np.int64)
        logical += int(ctx64.sum()) * H * 2 * D * 2
        unique += (int((ctx64 - prefix_blocks * B).sum()) + prefix_blocks * B) * H * 2 * D * 2
        seq_steps += n
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gc.enable()
    gpu = sum(a.elapsed_time(b) for a, b in ev) * 1e-3
    blk_bytes = H * 2 * D * 2 * B
    # the final shared state through both forms: the shared-prefix decode
    # against the plain one (the GPU parity tests compare both with the oracle)
    tf, cf = bm.block_tables(np.arange(S, dtype=np.int32), W)
    tfd, cfd = torch.from_numpy(tf).to(dev), torch.from_numpy(cf).to(dev)
    o_a = torch.empty_like(out)
    o_b = torch.empty_like(out)
    decode(o_a, q_all, tfd, cfd, st=st)
    ws_plain = torch.empty(pkv.paged_attn_workspace_bytes(S, H, D, W, B, P), dtype=torch.uint8, device=dev)
    pkv.paged_attn_decode(o_b, q_all, pool, 0, tfd, cfd, w.scale, partition_size=P, workspace=ws_plain, stream=st)
    torch.cuda.synchronize()
    form_diff = float((o_a - o_b).abs().max())
    res = {"metric": "paged decode KV-read GB/s (% of MI355X HBM peak) + decode seq-steps/s",
           "value": round(seq_steps / wall, 1), "unit": "seq-steps/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "shared-prefix copy-on-write run: 200 seqs forked from a 1500-token prefix, "
                                  "40q/40kv heads, head_dim 128, bf16 KV, block 16, 64..512 generated tokens each, "
                                  "appending decode per step",
                      "decode_call": ("paged_attn_decode_shared_prefix (the 93 shared blocks read once per KV head)"
                                      if shared else "paged_attn_decode_ex, appending, PKV_DECODE_KEEP_KV_CACHED"),
                      "seq_steps": seq_steps, "cow_pairs": pairs_total},
           "final_state_max_abs_diff_vs_plain_decode": form_diff,
           "wall_s": round(wall, 4), "decode_gpu_s": round(gpu, 4),
           "host_wait_s": round(waited, 4),
           "longest_steps_ms": [[int(i), round(float(d) * 1e3, 3)] for d, i in
                                sorted(zip(np.diff(marks + [t_start + wall]), range(steps)), reverse=True)[:4]],
           "logical_kv_gbs_decode": round(logical / gpu / 1e9, 1),
           "unique_kv_gbs_decode": round(unique / gpu / 1e9, 1),
           "unique_pct_of_hbm_peak": round(100 * unique / gpu / 1e9 / HBM_PEAK_GBS, 2),
           "bytes_saved_by_sharing_at_end": (S - 1) * prefix_blocks * blk_bytes,
           "roofline": {"bound": "hbm", "achieved": round(unique / gpu / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(unique / gpu / 1e9 / HBM_PEAK_GBS, 4),
                        "bytes": "unique KV bytes (shared prefix counted once) / summed decode launch time"}}
    log(f"cow run: {steps} steps, {seq_steps} seq-steps in {wall:.3f} s wall, decode launches {gpu:.3f} s; "
        f"logical {logical / gpu / 1e9:.0f} GB/s, unique {unique / gpu / 1e9:.0f} GB/s")
    print(json.dumps(res), flush=True)


def prefix_cache_bench(args):
    """The shared-system-prompt scenario of the bjdmk.com.cn article (§3.2:
    a 1500-token system prompt, 200 concurrent requests): every request is
    that prompt plus 64..512 private tokens; time kv_bm_add_seq_tokens per
    request (SHA-256 keys over every full block, lookups, allocation), or
    kv_bm_add_seq_radix (the walk down the radix tree, which also reuses the
    system prompt's last 12 tokens through a block copy) with
    --prefix-kind radix."""
    import paged_kv_cache_436_amd as pkv

    n = args.prefix_cache
    B = 16
    rng = np.random.default_rng(436004)
    system = rng.integers(0, 32000, size=1500).tolist()
    prompts = [np.asarray(system + rng.integers(0, 32000, size=int(rng.integers(64, 513))).tolist(), np.int32)
               for _ in range(n)]
    nb = sum(-(-len(p) // B) for p in prompts) + 8
    radix = args.prefix_kind == "radix"
    times, saved, copies = [], 0, 0
    for rep in range(args.warmup + args.steps):
        bm = pkv.BlockManager(nb, B)
        t0 = time.perf_counter()
        if radix:
            res = [bm.add_seq_radix(i, p) for i, p in enumerate(prompts)]
            cached = [c for c, _ in res]
        else:
            cached = [bm.add_seq_tokens(i, p) for i, p in enumerate(prompts)]
        t1 = time.perf_counter()
        if rep >= args.warmup:
            times.append(t1 - t0)
            saved = sum(cached)
            copies = sum(1 for _, pr in res if pr is not None) if radix else 0
        if radix:
            lookups, hits, keys, _ = bm.radix_stats()
        else:
            lookups, hits, keys = bm.prefix_stats()
        used = bm.stats()[0]
        bm.close()
    per = float(np.median(times)) / n
    total_tokens = sum(len(p) for p in prompts)
    res = {"metric": f"prefix-cache admission ({args.prefix_kind}): microseconds per request (host)",
           "value": round(per * 1e6, 2),
           "unit": "us/request", "n_gpus": 0, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": False, "dtype": "int32", "data": "synthetic",
           "config": {"workload": f"{n} requests = one 1500-token system prompt + 64..512 private tokens, "
                                  "block 16", "prompt_tokens": total_tokens},
           "prefill_tokens_reused": saved, "prefill_fraction_reused": round(saved / total_tokens, 4),
           ("token_lookups" if radix else "block_lookups"): lookups, ("token_hits" if radix else "block_hits"): hits,
           "blocks_used": used, "blocks_without_sharing": nb - 8}
    if radix:
        res["partial_block_copies"] = copies
    print(json.dumps(res), flush=True)


def swap_bench(args):
    """swap_blocks of N blocks (80 layers, K and V: 2.6 MB each in the 70B
    shape) device -> pinned host -> device, timed with HIP events; the bytes
    are checked to come back unchanged."""
    import torch

    import paged_kv_cache_436_amd as pkv
    import workloads

    w = workloads.llama70b(num_layers=80, extra_steps=1)
    n = args.swap
    cfg = pkv.make_config(80, n, w.block_size, w.num_kv_heads, w.head_dim, pkv.PKV_KV_BF16)
    nbytes = pkv.kv_pool_bytes(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(436005)
    dev_mem = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    host_mem = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    back_mem = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src, host, back = pkv.Pool(cfg, memory=dev_mem), pkv.Pool(cfg, memory=host_mem), pkv.Pool(cfg, memory=back_mem)
    rng = np.random.default_rng(436005)
    out_pairs = torch.from_numpy(np.stack([np.arange(n), rng.permutation(n)], 1).astype(np.int64)).cuda()
    in_pairs = torch.from_numpy(np.stack([out_pairs[:, 1].cpu().numpy(), np.arange(n)], 1)).cuda()
    moved = n * 80 * 2 * w.num_kv_heads * w.block_size * w.head_dim * 2
    st = torch.cuda.current_stream()
    times = {"out": [], "in": []}
    for rep in range(args.warmup + args.steps):
        for name, a, b, pr in (("out", src, host, out_pairs), ("in", host, back, in_pairs)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            pkv.swap_blocks(a, b, pr, stream=st)
            e1.record(st)
            torch.cuda.synchronize()
            if rep >= args.warmup:
                times[name].append(e0.elapsed_time(e1) * 1e-3)
    assert torch.equal(back_mem[:nbytes], dev_mem), "swap round trip changed bytes"
    gbs = {k: moved / float(np.median(v)) / 1e9 for k, v in times.items()}
    res = {"metric": "swap_blocks GB/s (device -> pinned host, host -> device)",
           "value": round(min(gbs.values()), 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "dtype": "u8", "data": "synthetic",
           "config": {"workload": f"swap {n} blocks of the 70B-shaped pool (80 layers, 8 KV heads, head_dim 128, "
                                  "bf16, block 16) out and back", "bytes_each_way": moved},
           "swap_out_gbs": round(gbs["out"], 2), "swap_in_gbs": round(gbs["in"], 2),
           "roofline": {"bound": "host link", "peak": HOST_LINK_GBS, "unit": "GB/s",
                        "achieved": round(min(gbs.values()), 2),
                        "frac": round(min(gbs.values()) / HOST_LINK_GBS, 4)}}
    print(json.dumps(res), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


def prefill_bench(args):
    """paged_attn_prefill over the prefix-cache workload: each of the 200
    prompts attends causally to the shared cached system prompt and to its own
    tokens.  HIP events around K back-to-back calls; algorithmic flops =
    sum over new tokens of (positions attended) * Hq * 4 * D.  A few
    sequences are checked against the oracle, which is timed on them."""
    import torch
    from threadpoolctl import threadpool_info

    import paged_kv_cache_436_amd as pkv
    import workloads

    w = workloads.prefix_prefill() if args.prefill_workload == "prefix_cache" else workloads.full_prefill()
    S, Hq, Hkv, D, B, W = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.table_width
    ctx_np = np.asarray(w.context_lens, np.int64)
    chunk = np.asarray(w.extra["chunk"], np.int64)
    qs_np = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    T = int(qs_np[-1])
    dev = torch.device("cuda:0")
    kvt = KV_DTYPES[args.kv_dtype]
    cfg = pkv.make_config(1, w.num_blocks, B, Hkv, D, kvt)
    pool = pkv.Pool(cfg, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(436008)
    k_off, v_off, ks_off, vs_off = pool.region_offsets()
    lb = pool.desc.layer_bytes
    for off in (k_off, v_off):
        if kvt == pkv.PKV_KV_BF16:
            pool.memory[off: off + lb].view(torch.bfloat16).normal_(generator=g)
        else:   # random codes (e5m2: finite patterns below the exponent-31 codes)
            pool.memory[off: off + lb].random_(0, 120 if kvt == pkv.PKV_KV_FP8_E5M2 else 256, generator=g)
    # int8 per-token scales, or the calibrated per-channel ones (int8, int4)
    lo, hi = (0.3, 0.6) if kvt == pkv.PKV_KV_INT4 else (0.02, 0.05)
    for off, n in scale_regions(pool, kvt):
        pool.memory[off: off + 4 * n].view(torch.float32).uniform_(lo, hi, generator=g)
    sck, scv = tensor_scales(kvt)
    tables = torch.from_numpy(w.extra["tables"]).to(dev)
    ctx = torch.from_numpy(ctx_np.astype(np.int32)).to(dev)
    qs = torch.from_numpy(qs_np).to(dev)
    q = torch.randn((T, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream()
    maxq = int(chunk.max())

    def call():
        pkv.paged_attn_prefill(out, q, pool, 0, tables, ctx, qs, w.scale, maxq, k_scale=sck, v_scale=scv,
                               p_one_part=args.p_one_part, stream=st)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(K):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) * 1e-3 / K
    # keys attended: token k of a chunk of n over a prompt of c sees c - n + k + 1 positions
    keys = int(sum(n * (c - n) + n * (n + 1) // 2 for c, n in zip(ctx_np, chunk)))
    flops = keys * Hq * 4 * D
    tfs = flops / per / 1e12
    log(f"prefill: {T} new tokens, {keys} (token, position) pairs per head; {per * 1e3:.3f} ms per call, "
        f"{tfs:.1f} TFLOP/s")

    cpu = parity = None
    if kvt == pkv.PKV_KV_BF16:   # the oracle sample copies the K/V regions only (no scale regions)
        # oracle on a bounded sample of sequences (gather + causal attention, fp64)
        from oracle import attention, layout
        tile = pool.desc.tile_bytes
        gpu_out = out.cpu().numpy()
        qbits = q.view(torch.int16).cpu().numpy().view(np.uint16)
        tabs = w.extra["tables"]
        rng = np.random.default_rng(437)
        spent, keys_done, worst, seqs = 0.0, 0, 0.0, 0
        for s in rng.permutation(S):
            c, n = int(ctx_np[s]), int(chunk[s])
            nblk = math.ceil(c / B)
            sub = layout.PoolShape(1, nblk, B, Hkv, D)
            img = layout.empty_image(sub)
            idx = torch.from_numpy(tabs[s, :nblk].astype(np.int64)).to(dev)
            for region, dst in ((k_off, img.k), (v_off, img.v)):
                lay = pool.memory[region: region + lb].view(w.num_blocks, Hkv * tile)
                dst[:] = lay.index_select(0, idx).cpu().numpy().view(np.uint16).reshape(-1)
            t0 = time.perf_counter()
            ref = attention.paged_prefill(qbits[qs_np[s]:qs_np[s + 1]], img, 0, np.arange(nblk, dtype=np.int32)[None, :],
                                          np.array([c]), np.array([0, n]), w.scale)
            spent += time.perf_counter() - t0
            worst = max(worst, float(np.max(np.abs(gpu_out[qs_np[s]:qs_np[s + 1]] - ref))))
            keys_done += n * (c - n) + n * (n + 1) // 2
            seqs += 1
            if spent >= args.cpu_seconds:
                break
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
        cpu_tfs = keys_done * Hq * 4 * D / spent / 1e12
        log(f"cpu oracle: {cpu_tfs:.6f} TFLOP/s over {seqs} sequences; parity max abs err {worst:.2e}")
        cpu = {"value": round(cpu_tfs, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
               "sample": f"{seqs} sequences' prefill ({keys_done} (token, position) pairs per head), "
                         f"{spent:.1f} s of fp64 numpy causal attention"}
        parity = {"sequences_checked": seqs, "max_abs_err": worst, "bar": 1e-2}
    kv_name = {v: k for k, v in KV_DTYPES.items()}[kvt]
    res = {"metric": "paged prefill TFLOP/s (algorithmic, % of MI355X bf16 matrix-core peak)",
           "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_call": round(per * 1e3, 4), "higher_is_better": True,
           "dtype": {"bf16": "bf16", "fp8": "fp8"}.get(kv_name, "int8" if kv_name.startswith("int8") else "int4"),
           "data": "synthetic",
           "config": {"kv_storage": kv_name, "workload": ("paged prefill after a prefix-cache hit: 200 prompts = 1500-token shared system "
                                   "prompt (93 cached blocks) + 64..512 own tokens, 64q/8kv heads, head_dim 128, "
                                   "bf16 KV, block 16, one layer") if args.prefill_workload == "prefix_cache" else
                                  ("paged prefill of 16 whole 4096-token prompts, 64q/8kv heads, head_dim 128, bf16 "
                                   "KV, block 16, one layer"),
                      "new_tokens": T, "max_query_len": maxq, "flops_per_call": flops,
                      "p_operand": "one rounded part" if args.p_one_part else "hi + lo parts"},
           "roofline": {"bound": "mfma", "kernel": "pa_prefill_kernel", "achieved": round(tfs, 2),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": (measured_traffic(PREFILL_PROFILE, PREFILL_SRCS)
                                    if args.prefill_workload == "prefix_cache" and kvt == pkv.PKV_KV_BF16
                                    and not args.p_one_part else None),
                        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"},
           "cpu_baseline": cpu, "parity_sample": parity}
    print(json.dumps(res), flush=True)


def copy_calibration():
    """A plain device copy of known size, for calibrating HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def compute_probe_bench(args):
    """Per-block compute time of the decode step's arithmetic, with no HBM
    traffic: q.K^T, softmax update and P.V of one 16-token bf16 block of one
    KV head (head dim 128) per wave, on the matrix cores (the decode kernel's
    way) and on the vector ALU, one workgroup of four waves per CU.  The
    slope between two loop lengths removes launch and prologue time."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_436_amd", "libpkv_probe.so"))
    lib.pkv_probe_compute.restype = ctypes.c_int
    lib.pkv_probe_compute.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    seed = torch.randn(8192, generator=g, device=dev).to(torch.bfloat16).view(torch.int32)
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    names = {0: "loop and operand changes only", 1: "matrix cores (decode kernel's arithmetic)",
             2: "vector ALU, 8 query heads per KV head", 3: "vector ALU, 4 query heads per KV head"}
    n_short, n_long = 2000, 6000

    def run(variant, chunks, reps):
        rc = lib.pkv_probe_compute(variant, seed.data_ptr(), out.data_ptr(), chunks, wgs, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"pkv_probe_compute({variant}) returned hipError {rc}")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            lib.pkv_probe_compute(variant, seed.data_ptr(), out.data_ptr(), chunks, wgs, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps           # us per launch

    res = {}
    for v in (0, 1, 2, 3):
        log(f"probe variant {v}: {names[v]}")
        for _ in range(max(args.warmup, 1)):
            run(v, n_short, 1)
        t_s = run(v, n_short, args.steps)
        t_l = run(v, n_long, args.steps)
        res[v] = (t_l - t_s) * 1e3 / (n_long - n_short)   # ns per block per wave
        log(f"  {t_s:.1f} us / {n_short} blocks, {t_l:.1f} us / {n_long} blocks: {res[v]:.1f} ns per block")
    # one 16-token bf16 block of one KV head: K and V, 16 x 128 x 2 bytes each,
    # streamed by each of the chip's 4 x CUs waves at once
    waves = 4 * wgs
    blk = 2 * 16 * 128 * 2
    mem_peak_ns = blk * waves / 8000e9 * 1e9
    line = {"metric": "per-block compute ns per wave (16-token bf16 block, head dim 128, no HBM traffic)",
            "unit": "ns", "waves": waves, "block_bytes": blk,
            "hbm_ns_per_block_at_peak": round(mem_peak_ns, 1),
            "variants": {names[v]: round(res[v], 1) for v in res},
            "compute_ns": {names[v]: round(res[v] - res[0], 1) for v in (1, 2, 3)},
            "steps": args.steps, "warmup": args.warmup}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.compute_probe:
        compute_probe_bench(args)
        return
    if args.swap:
        swap_bench(args)
        return
    if args.prefill:
        prefill_bench(args)
        return
    if args.prefix_cache:
        prefix_cache_bench(args)
        return
    if args.config == "cow_prefix":
        cow_bench(args)
        return
    if args.config:
        config_bench(args)
        return
    import torch

    import paged_kv_cache_436_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps_total = args.warmup + args.steps + 1
    w = workloads.llama70b(num_layers=80, extra_steps=steps_total, block_size=args.block_size)
    L = args.layers
    S, Hq, Hkv, D, B, W = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.table_width
    P = args.partition if args.partition > 0 else (W * B + 31) // 32 * 32

    # ---------------------------------------------------------------- state
    bm = pkv.BlockManager(w.num_blocks, B, w.block_order)
    for s in range(S):
        bm.add_seq(s, int(w.context_lens[s]) - 1)      # history; each step appends one token
    kvt = KV_DTYPES[args.kv_dtype]
    e = 2 if kvt == pkv.PKV_KV_BF16 else 1                          # bytes per stored element (INT4: two per byte)
    token_scales = 2 * 4 if kvt == pkv.PKV_KV_INT8 else 0          # int8: fp32 K and V scale per (token, head)
    tok_bytes = Hkv * (2 * D * e // (2 if kvt == pkv.PKV_KV_INT4 else 1) + token_scales)   # KV bytes per token per layer
    ks_t, vs_t = tensor_scales(kvt)
    if kvt != pkv.PKV_KV_BF16:
        args.no_cpu_baseline = True
    cfg = pkv.make_config(w.num_layers, w.num_blocks, B, Hkv, D, kvt)
    log(f"pool: {pkv.kv_pool_bytes(cfg) / 1e9:.1f} GB, {w.num_blocks} blocks/layer x {w.num_layers} layers")
    pool = pkv.Pool(cfg, device=dev)
    k_off, v_off, ks_off, vs_off = pool.region_offsets()
    lb = pool.desc.layer_bytes
    t0 = time.time()
    for layer in range(w.num_layers):
        g = torch.Generator(device=dev)
        g.manual_seed(436003 * 1000 + layer)
        for off in (k_off, v_off):
            region = pool.memory[off + layer * lb: off + (layer + 1) * lb]
            if e == 2:
                region.view(torch.bfloat16).normal_(generator=g)
            else:   # random codes (int8: +-127 range; e5m2: finite patterns below the exponent-31 codes)
                region.random_(0, 120 if kvt == pkv.PKV_KV_FP8_E5M2 else 256, generator=g)
    for off, n in scale_regions(pool, kvt):   # int8 scales: per-token ones, or the calibrated per-channel ones
        pool.memory[off: off + 4 * n].view(torch.float32).uniform_(0.02, 0.05)
    torch.cuda.synchronize()
    log(f"pool filled in {time.time() - t0:.1f} s")

    g = torch.Generator(device=dev)
    g.manual_seed(436003)
    q = torch.randn((L, S, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    newk = torch.randn((L, S, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    newv = torch.randn((L, S, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, pkv.paged_attn_workspace_bytes(S, Hq, D, W, B, P)), dtype=torch.uint8, device=dev)
    scale = w.scale

    # double-buffered pinned host staging for tables / lengths / slots
    seqs = np.arange(S, dtype=np.int32)
    h_tab = [torch.empty((S, W), dtype=torch.int32).pin_memory() for _ in range(2)]
    h_ctx = [torch.empty(S, dtype=torch.int32).pin_memory() for _ in range(2)]
    h_slot = [torch.empty(S, dtype=torch.int64).pin_memory() for _ in range(2)]
    h_done = [torch.cuda.Event() for _ in range(2)]
    d_tab = torch.empty((S, W), dtype=torch.int32, device=dev)
    d_ctx = torch.empty(S, dtype=torch.int32, device=dev)
    d_slot = torch.empty(S, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    kv_bytes = []
    dec_events = []

    separate = args.separate_cache_write
    window = args.window
    if window and separate:
        sys.exit("--window runs the appending form only")

    def decode(layer):
        if window:
            pkv.paged_attn_decode_ex(out, q[layer], pool, layer, d_tab, d_ctx, scale, k_scale=ks_t,
                                     v_scale=vs_t, partition_size=P, workspace=ws, key=newk[layer], value=newv[layer], sliding_window=window,
                                     stream=stream)
        elif separate:
            pkv.paged_attn_decode(out, q[layer], pool, layer, d_tab, d_ctx, scale, k_scale=ks_t, v_scale=vs_t,
                                  partition_size=P,
                                  workspace=ws, stream=stream)
        else:
            pkv.paged_attn_decode_append(out, q[layer], pool, layer, newk[layer], newv[layer], d_tab, d_ctx,
                                         scale, k_scale=ks_t, v_scale=vs_t, partition_size=P, workspace=ws, stream=stream)

    def step(i, timed):
        b = i % 2
        h_done[b].synchronize()                       # staging buffer b is free again
        slots, pairs = bm.append(seqs)
        assert pairs.shape[0] == 0                    # no sharing in this workload
        bm.block_tables(seqs, W, out=h_tab[b].numpy(), ctx_out=h_ctx[b].numpy())
        d_tab.copy_(h_tab[b], non_blocking=True)
        d_ctx.copy_(h_ctx[b], non_blocking=True)
        if separate:
            h_slot[b].numpy()[:] = slots
            d_slot.copy_(h_slot[b], non_blocking=True)
        h_done[b].record(stream)
        ctxs = h_ctx[b].numpy().astype(np.int64)
        ctx_sum = int((np.minimum(ctxs, window) if window else ctxs).sum())   # positions attended
        kv_bytes.append(ctx_sum * tok_bytes * L)
        # HIP events on the launch stream.  A timing event between two launches
        # costs ~10 us of idle GPU (the next launch no longer follows the
        # previous one directly), so the appending form, whose 80 decode
        # launches run back to back with nothing else between them, is
        # bracketed once per step; the two-call form per decode call.
        if timed and not separate:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        for layer in range(L):
            if separate:
                pkv.reshape_and_cache(pool, layer, newk[layer], newv[layer], d_slot, k_scale=ks_t, v_scale=vs_t,
                                      stream=stream)
                if timed:
                    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    c0.record(stream)
            decode(layer)
            if timed and separate:
                c1.record(stream)
                dec_events.append((c0, c1, ctx_sum, 1))
        if timed and not separate:
            e1.record(stream)
            dec_events.append((e0, e1, ctx_sum, L))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    log("warmup done")
    kv_bytes.clear()
    gc.collect()
    gc.disable()                      # no garbage-collector pass inside the timed steps
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    kv_per_step = sum(kv_bytes) / args.steps
    gbs = sum(kv_bytes) / elapsed / 1e9
    dec_ms = [e0.elapsed_time(e1) / n for e0, e1, _, n in dec_events]
    # per call: every context token's K and V once; the appending form also
    # writes the new token's K and V
    dec_bytes = [(c + (0 if separate else S)) * tok_bytes for _, _, c, _ in dec_events]
    avg_dec_ms = float(np.mean(dec_ms))
    avg_dec_bytes = float(np.mean(dec_bytes))
    achieved = avg_dec_bytes / (avg_dec_ms * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {gbs:.1f} GB/s; "
        f"decode call avg {avg_dec_ms * 1e3:.1f} us = {achieved:.1f} GB/s")

    # ---------------------------------------------------------------- sampled parity + CPU baseline
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(args, pkv, w, pool, decode, q, out, d_tab, d_ctx, scale)
    workload = ("70B-shaped paged decode step: 80 layers x 100 seqs x ~4K ctx, "
                f"64q/8kv heads, head_dim 128, {args.kv_dtype} KV, block {B}")
    if window:
        workload += f", sliding window of the last {window} positions"

    call = "paged_attn_decode" if separate else "paged_attn_decode_append"
    res = {
        "metric": "paged decode KV-read GB/s (% of MI355X HBM peak) + decode seq-steps/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.kv_dtype,
        "data": "synthetic",
        "config": {"workload": workload,
                   "sliding_window": window, "layers": L, "seqs": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block_size": B, "partition_size": P, "kv_bytes_per_step": int(kv_per_step),
                   "layer_calls": ("reshape_and_cache + paged_attn_decode" if separate
                                   else "paged_attn_decode_append")},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(S / (elapsed / args.steps), 1),
        "seq_tokens_per_s": round(kv_per_step / (tok_bytes * L) / (elapsed / args.steps), 1),
        "roofline": {"bound": "hbm", "kernel": f"pa_split_kernel (the one launch of a split-context {call} call)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if (window or kvt != pkv.PKV_KV_BF16) else measured_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                     "avg_call_us": round(avg_dec_ms * 1e3, 2), "bytes_per_call": int(avg_dec_bytes)},
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    print(json.dumps(res), flush=True)


def cpu_baseline(args, pkv, w, pool, decode, q, out, d_tab, d_ctx, scale):
    """Time the fp64 oracle on a bounded sample (layer after layer, sequence by
    sequence, until the time budget is spent) and check the GPU's output of
    each sampled layer on that sample.  The GPU call is the timed step's own
    (the appending form writes the last step's token again, the same bytes)."""
    import torch
    from threadpoolctl import threadpool_info

    from oracle import attention, layout

    S, Hq, Hkv, D, B, W = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.table_width
    tabs = d_tab.cpu().numpy()
    ctxs = d_ctx.cpu().numpy()
    k_off, v_off, _, _ = pool.region_offsets()
    tile = pool.desc.tile_bytes
    rng = np.random.default_rng(436)
    spent, done, worst, layers = 0.0, [], 0.0, 0
    for layer in range(args.layers):
        decode(layer)
        torch.cuda.synchronize()
        gpu_out = out.cpu().numpy()
        qbits = q[layer].view(torch.int16).cpu().numpy().view(np.uint16)
        layers += 1
        for s in rng.permutation(S):
            n = int(ctxs[s])
            nblk = math.ceil(n / B)
            # copy this sequence's tiles of the layer to the host as a small pool
            sub = layout.PoolShape(1, nblk, B, Hkv, D)
            img = layout.empty_image(sub)
            idx = torch.from_numpy(tabs[s, :nblk].astype(np.int64)).to(pool.memory.device)
            for region, dst in ((k_off, img.k), (v_off, img.v)):
                base = region + layer * pool.desc.layer_bytes
                lay = pool.memory[base: base + pool.desc.layer_bytes].view(w.num_blocks, Hkv * tile)
                dst[:] = lay.index_select(0, idx).cpu().numpy().view(np.uint16).reshape(-1)
            local = np.arange(nblk, dtype=np.int32)
            t0 = time.perf_counter()
            ref = attention.paged_decode(qbits[s:s + 1], img, 0, local[None, :], np.array([n]), scale,
                                         window=args.window)
            spent += time.perf_counter() - t0
            done.append(min(n, args.window) if args.window else n)   # positions attended
            worst = max(worst, float(np.max(np.abs(gpu_out[s] - ref[0]))))
            if spent >= args.cpu_seconds:
                break
        if spent >= args.cpu_seconds:
            break
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    bytes_done = sum(done) * Hkv * 2 * D * 2
    cpu = {"value": round(bytes_done / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{len(done)} (sequence, layer) decodes of the same step over {layers} layer(s), "
                     f"{sum(done)} tokens, {spent:.1f} s of fp64 numpy decode (gather + softmax attention)",
           "host_cpus": len(os.sched_getaffinity(0))}
    parity = {"decodes_checked": len(done), "max_abs_err": worst, "bar": 1e-2}
    log(f"cpu oracle: {cpu['value']} GB/s on {threads} threads; parity max abs err {worst:.2e}")
    return cpu, parity


if __name__ == "__main__":
    main()
