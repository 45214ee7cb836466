"""Benchmark: one routed MoE layer (exact routing -> union -> fused 4-bit
SwiGLU experts -> combine) on one MI355X.

A step is one call of the whole layer (router gate matvec, softmax/top-k,
union and pair lists, gate_up, down, combine) on one fresh batch.  Steps
rotate over a stack of distinct layers resident in HBM (16 by default) so
that the weights stream from HBM, not from the 256 MB Infinity Cache.  Each
call's arguments are marshalled once; before anything is timed, every
rotated layer runs at both batch sizes and then for 0.3 s more (clocks and
caches in their steady state whatever --steps and --warmup are).

Prints one JSON line:
  value       tokens/s of the decode layer (d=4096, 128 experts, top-8,
              ffn 1536, B=1), whole job, inputs resident in HBM;
  effective_gbps / hbm_frac   bytes of the distinct routed experts per step
              (packed words + bf16 scales + biases) / step time, vs 8 TB/s;
  roofline    the dominant kernel (gate_up) timed with HIP events on its
              launch stream over a fixed 1000 back-to-back launches:
              algorithmic bytes per launch / mean duration;
  kernels_back_to_back   the same for the down kernel;
  secondary   the same layer as a 64-token prefill chunk, and the 256-expert
              fused layer (d=2048, ffn 512) at B=1 and B=64, each with its
              FFN kernels' rates;
  calibration a plain streaming read of 4 GiB (smoe_stream_read);
  stack       the 94-layer stacked harness;
  cpu_baseline  the CPU oracle on bounded samples of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer tokens/s and effective expert-weight GB/s (% HBM peak), B=1 and B=64"


_T0 = time.time()


def progress(msg):
    """One line on stderr as each part of the run ends (the JSON line stays
    the only thing on stdout)."""
    print(f"bench: {msg} ({time.time() - _T0:.1f} s)", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000, help="timed decode steps")
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--prefill-steps", type=int, default=200)
    p.add_argument("--layers", type=int, default=16, help="distinct layers rotated through")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-fused", action="store_true",
                   help="leave out the 256-expert fused layer (B=1 and B=64)")
    p.add_argument("--workloads", default="decode,prefill,fused_b1,fused_b64",
                   help="comma list of decode, prefill, fused_b1, fused_b64 (the value line "
                        "needs decode; the others go to secondary)")
    p.add_argument("--stack", action="store_true",
                   help="run only the stacked harness (94 layers: prompt chunks, then decode)")
    p.add_argument("--no-stack", action="store_true", help="leave the stacked harness out")
    p.add_argument("--attention", action="store_true",
                   help="only the attention block around the layer (decode and 64-token chunks)")
    p.add_argument("--shared", action="store_true",
                   help="only the layer with a shared expert (decode and prefill), beside the "
                        "same layer without one")
    p.add_argument("--stack-layers", type=int, default=94)
    p.add_argument("--stack-prompt", type=int, default=512)
    p.add_argument("--stack-decode", type=int, default=128)
    p.add_argument("--no-calibration", action="store_true",
                   help="leave out the stream-read and launch/barrier calibration (profiling "
                        "passes)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a device-to-device copy of COPY_BYTES (for the counter scale)")
    p.add_argument("--summarize-counters", nargs="+",
                   metavar="OUT LABEL COPY_FETCH_CSV COPY_WRITE_CSV CSV",
                   help="write a per-kernel summary of rocprofv3 --pmc counter CSVs (any "
                        "counters; FETCH_SIZE/WRITE_SIZE scaled by the copy calibration) to OUT "
                        "and exit")
    p.add_argument("--summarize-trace", nargs=4, metavar=("OUT", "LABEL", "COMMAND", "STATS_CSV"),
                   help="write a rocprofv3 kernel_stats.csv as the per-kernel table in profiles/ "
                        "(label and the command that made it in the header) and exit")
    p.add_argument("--counter-command", default=None,
                   help="with --summarize-counters: the command the rocprofv3 passes ran, for the "
                        "summary's header")
    p.add_argument("--trace-csv", default=None,
                   help="with --summarize-counters: the kernel_stats.csv of the same command, "
                        "for kernel durations (MFMA rates)")
    return p.parse_args()


class Stack:
    """n distinct layers of one shape in device memory plus shared buffers.
    Calls are marshalled once per (layer, input) and then repeated."""

    def __init__(self, smoe, cfg, n_layers, max_batch):
        import torch

        import synth.gpu as sg
        self.cfg, self.smoe = cfg, smoe
        self.desc = smoe.make_desc(cfg.d_model, cfg.ffn_dim, cfg.num_experts, cfg.top_k,
                                   cfg.norm_topk_prob, cfg.router_bf16, cfg.shared_ffn_dim)
        self.layers = []
        for l in range(n_layers):
            W = sg.make_layer(cfg, layer=l)
            self.layers.append((W, smoe.experts_of(self.desc, W)))
        dev = torch.device("cuda:0")
        self.ws = torch.zeros(smoe.workspace_size(self.desc, max_batch), dtype=torch.uint8,
                              device=dev)
        smoe.workspace_init(self.ws)
        self.un = smoe.UnionBuffers.alloc(cfg.num_experts, max_batch * cfg.top_k, dev)
        self.idx = torch.zeros(max_batch, cfg.top_k, dtype=torch.int32, device=dev)
        self.w = torch.zeros(max_batch, cfg.top_k, dtype=torch.float32, device=dev)
        self.out = torch.zeros(max_batch, cfg.d_model, dtype=torch.float32, device=dev)
        self._calls = {}
        torch.cuda.synchronize()

    def prepared(self, l, x, stage=None, single=False):
        key = (l, x.data_ptr(), x.shape[0], stage, single)
        c = self._calls.get(key)
        if c is None:
            W, ex = self.layers[l]
            B = x.shape[0]
            c = self.smoe.prepare_moe_layer(self.desc, W["router"], ex, x, self.out[:B],
                                            self.idx[:B], self.w[:B], self.un, self.ws,
                                            stage=stage, single=single)
            self._calls[key] = c
        return c

    def call(self, l, x):
        self.prepared(l, x)()

    def stage(self, st, l, x):
        self.prepared(l, x, st)()


def x_pool(cfg, B, n):
    import synth.gpu as sg
    return [sg.hidden(cfg.seed, 0, 1000 + i, B, cfg.d_model) for i in range(n)]


def warm_pass(stack, pools, seconds=0.3):
    """Untimed: every rotated layer with every batch size, then more layer
    calls until `seconds` have passed, so that clocks and caches are in their
    steady state before anything is timed, whatever --steps and --warmup are."""
    import torch
    nl = len(stack.layers)
    for xs in pools:
        for l in range(nl):
            stack.call(l, xs[l % len(xs)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(32):
            xs = pools[i % len(pools)]
            stack.call(i % nl, xs[i % len(xs)])
            i += 1
        torch.cuda.synchronize()


HOLD_US = 200


def time_layer(stack, xs, steps, warmup, single=False):
    """Seconds for `steps` whole-layer calls, rotating layers and inputs, timed
    with events between two synchronisations after `warmup` untimed calls
    (single: the layer as one cooperative launch, smoe_moe_layer_single).
    A device-side wait of HOLD_US queued before the first event keeps the GPU
    busy while the host enqueues the first calls: without it the region
    opens with the host's latency to its first launch (about 20 us, a
    microsecond a step over 20 steps), which is not the layer's."""
    import torch
    nl = len(stack.layers)
    calls = [stack.prepared(s % nl, xs[s % len(xs)], single=single)
             for s in range(max(steps, warmup))]
    for s in range(warmup):
        calls[s]()
    torch.cuda.synchronize()
    stack.smoe.gpu_sleep(HOLD_US)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        calls[s]()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3


ROOFLINE_LAUNCHES = 1000


def time_stage(stack, xs, stage, launches=ROOFLINE_LAUNCHES):
    """Mean duration (s) of one stage's kernel: HIP events on its launch stream
    around `launches` back-to-back launches over the rotating layers, all with
    the routing of one input (the route stage runs once first, so every
    launch sees that input's union).  A fixed count, independent of --steps.
    Events around each single launch would add the runtime's marker overhead
    (a few microseconds) to every sample; back to back, consecutive kernels
    overlap one's tail with the next one's start instead."""
    import torch
    smoe = stack.smoe
    nl = len(stack.layers)
    stack.stage(smoe.SMOE_STAGE_ROUTE, 0, xs[0])
    calls = [stack.prepared(i % nl, xs[0], stage) for i in range(nl)]
    for i in range(50):
        calls[i % nl]()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(launches):
        calls[i % nl]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / launches / 1e3


def union_sizes(stack, xs, steps):
    """|U| of every timed step (the routing is deterministic; re-run untimed)."""
    import torch
    nl = len(stack.layers)
    sizes = []
    for s in range(steps):
        stack.call(s % nl, xs[s % len(xs)])
        sizes.append(stack.un.n_union.clone())
    torch.cuda.synchronize()
    return [int(t.item()) for t in sizes]


def gate_up_bytes(cfg):
    """Packed words + scales + biases of one expert's gate and up projections."""
    d, f = cfg.d_model, cfg.ffn_dim
    return 2 * (f * d // 2 + 2 * 2 * f * d // 64)


def down_bytes(cfg):
    d, f = cfg.d_model, cfg.ffn_dim
    return d * f // 2 + 2 * 2 * d * f // 64


def layer_entry(stack, cfg, xs, steps, warmup, kernels=True):
    """One workload's figures: step time, tokens/s, effective expert GB/s and
    its fraction of the HBM peak, and (kernels) each FFN kernel's mean
    duration back to back with its algorithmic bytes and rate."""
    B = cfg.batch
    t = time_layer(stack, xs, steps, warmup)
    sz = union_sizes(stack, xs, min(steps, 256))
    u = sum(sz) / len(sz)
    step = t / steps
    eb = cfg.expert_bytes()
    gbps = u * eb / step / 1e9
    e = {"workload": cfg.name, "batch": B, "steps": steps, "ms_per_step": round(step * 1e3, 5),
         "tokens_per_s": round(B / step, 1), "mean_union": u,
         "effective_bytes_per_step": int(u * eb), "effective_gbps": round(gbps, 1),
         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    if kernels:
        smoe = stack.smoe
        u0 = union_sizes(stack, xs[:1], 1)[0]
        ks = {}
        for name, st, nbytes in (("gate_up", smoe.SMOE_STAGE_GATE_UP, gate_up_bytes(cfg)),
                                 ("down", smoe.SMOE_STAGE_DOWN, down_bytes(cfg))):
            ts = time_stage(stack, xs, st)
            b = u0 * nbytes
            ks[name] = {"mean_launch_us": round(ts * 1e6, 3), "bytes_per_launch": int(b),
                        "gbps": round(b / ts / 1e9, 1), "frac": round(b / ts / 1e9 / HBM_PEAK_GBPS, 4)}
        e["kernels_back_to_back"] = ks
    return e


STREAM_BYTES = 4 << 30


def stream_read_calibration(smoe):
    """Read bandwidth of a plain stream of 16-byte nontemporal loads over a
    4 GiB buffer (smoe_stream_read, far larger than the 256 MB memory-side
    cache), for several workgroup counts: the rate this part reaches on a
    pure stream, context for the kernels' fractions of the 8 TB/s peak."""
    import torch
    dev = torch.device("cuda:0")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.ones(STREAM_BYTES // 4, dtype=torch.int32, device=dev)
    out = {}
    for per_cu in (2, 4, 8):
        sink = torch.zeros(ncu * per_cu, dtype=torch.int32, device=dev)
        for _ in range(3):
            smoe.stream_read(buf, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            smoe.stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / n
        out[f"{per_cu}_blocks_per_cu"] = round(STREAM_BYTES / t / 1e9, 1)
    # the direct global -> LDS copy path of the prefill FFN kernels, on rows of
    # the decode/prefill layer's gate_up (d = 4096: 2048 B) and down (f = 1536:
    # 768 B) matrices, in the kernels' pattern and in memory order
    dma = {}
    for row_bytes in (2048, 768):
        units = STREAM_BYTES // (64 * row_bytes)
        nbytes = units * 64 * row_bytes
        sink = torch.zeros((units + 3) // 4, dtype=torch.int32, device=dev)
        r = {}
        for mode, name in ((0, "ffn_pattern_gbps"), (1, "memory_order_gbps")):
            for _ in range(3):
                smoe.dma_read(buf, sink, row_bytes, mode, nbytes=nbytes)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 10
            e0.record()
            for _ in range(n):
                smoe.dma_read(buf, sink, row_bytes, mode, nbytes=nbytes)
            e1.record()
            torch.cuda.synchronize()
            r[name] = round(nbytes / (e0.elapsed_time(e1) / 1e3 / n) / 1e9, 1)
        dma[f"rows_{row_bytes}B"] = r
    del buf
    torch.cuda.empty_cache()
    best = max(out.values())
    return {"kernel": "k_stream_read (smoe_stream_read)", "bytes": STREAM_BYTES,
            "gbps_by_grid": out, "best_gbps": best, "best_frac": round(best / HBM_PEAK_GBPS, 4),
            "dma_read": {"kernel": "k_dma_read (smoe_dma_read): global -> LDS copies, three "
                                   "4 KB stages a wave, two workgroups of four waves per CU",
                         **dma}}


def sync_calibration(smoe):
    """What a kernel boundary costs against its in-kernel alternative:
      * launch_us: mean cost of one more launch in a stream of back-to-back
        launches of an empty kernel (one workgroup per CU), HIP events around
        1000 launches enqueued by one call;
      * grid_barrier_us: one device-wide barrier of a cooperative grid of one
        256-thread workgroup per CU (smoe_grid_barrier: one device-scope
        release per workgroup, then acquire polls), from the kernel's own
        s_memrealtime stamps: first start to last exit, and last arrival to
        last exit (the polls' share), medians of 20."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    smoe.empty_launch(ncu, 100)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1000
    e0.record()
    smoe.empty_launch(ncu, n)                        # enqueued from C, back to back
    e1.record()
    torch.cuda.synchronize()
    launch_us = e0.elapsed_time(e1) * 1e3 / n
    counter = torch.zeros(1, dtype=torch.int32, device=dev)
    timed_out = torch.zeros(1, dtype=torch.int32, device=dev)
    stamps = torch.zeros(3 * ncu, dtype=torch.int64, device=dev)
    whole, polls = [], []
    for rep in range(25):
        counter.zero_()
        smoe.grid_barrier(ncu, counter, stamps, timed_out)
        st = stamps.view(ncu, 3).cpu().numpy().astype(np.int64)
        if rep >= 5:
            whole.append((st[:, 2].max() - st[:, 0].min()) * 0.01)
            polls.append((st[:, 2].max() - st[:, 1].max()) * 0.01)
    return {"launch_us": round(launch_us, 2), "workgroups": ncu,
            "grid_barrier_us": round(float(np.median(whole)), 2),
            "grid_barrier_polls_us": round(float(np.median(polls)), 2),
            "grid_barrier_timed_out": bool(int(timed_out.cpu()[0]))}


def shared_bench(smoe, args):
    """The decode and prefill layer with a shared expert (fs = 3072 beside the
    routed experts), and the same layer without one in the same run: the
    shared expert's bytes are read once per call for every token."""
    import torch
    from synth import configs
    res = {}
    for name, cfg in (("shared", configs.DECODE_SHARED), ("plain", configs.DECODE)):
        st = Stack(smoe, cfg, args.layers, max_batch=64)
        xs1 = x_pool(cfg, 1, 257)
        t1 = time_layer(st, xs1, args.steps, args.warmup) / args.steps
        u1 = sum(union_sizes(st, xs1, 256)) / 256
        xs64 = x_pool(cfg, 64, 17)
        t64 = time_layer(st, xs64, args.prefill_steps, 5) / args.prefill_steps
        u64 = sum(union_sizes(st, xs64, args.prefill_steps)) / args.prefill_steps
        res[name] = (t1, u1, t64, u64)
        del st
        torch.cuda.empty_cache()
    cfg = configs.DECODE_SHARED
    eb = cfg.expert_bytes()
    sb = 3 * (cfg.shared_ffn_dim * cfg.d_model // 2 + 2 * 2 * cfg.shared_ffn_dim * cfg.d_model // 64)
    t1, u1, t64, u64 = res["shared"]
    p1, _, p64, _ = res["plain"]
    g1 = (u1 * eb + sb) / t1 / 1e9
    g64 = (u64 * eb + sb) / t64 / 1e9
    return {
        "metric": "layer with a shared expert: decode tokens/s (B=1)", "value": round(1 / t1, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t1 * 1e3, 5), "higher_is_better": True, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: the routed layer (d=4096, 128 experts, top-8, ffn "
                               "1536) plus a shared expert of width 3072 on every token, 4-bit g64",
                   "shared_expert_bytes": sb, "effective_bytes_per_step": int(u1 * eb + sb)},
        "effective_gbps": round(g1, 1), "hbm_frac": round(g1 / HBM_PEAK_GBPS, 4),
        "plain_layer_us": round(p1 * 1e6, 3), "shared_cost_us": round((t1 - p1) * 1e6, 3),
        "shared_bytes_time_at_peak_us": round(sb / HBM_PEAK_GBPS / 1e3, 3),
        "secondary": {"workload": f"{configs.PREFILL_SHARED.name}: the same, 64-token chunk",
                      "tokens_per_s": round(64 / t64, 1), "ms_per_step": round(t64 * 1e3, 5),
                      "mean_union": u64, "effective_gbps": round(g64, 1),
                      "hbm_frac": round(g64 / HBM_PEAK_GBPS, 4),
                      "plain_layer_us": round(p64 * 1e6, 3),
                      "shared_cost_us": round((t64 - p64) * 1e6, 3)},
    }


def _blas_threads():
    """Threads numpy's BLAS uses (the attention oracle's matrix products)."""
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        return os.cpu_count() or 1


ATTN_SHAPE = dict(d_model=4096, num_heads=64, num_kv_heads=4, ctx=4096, rope_theta=1.0e6)


def attention_bench(smoe, args):
    """The attention block around the layer (d 4096, 64 query and 4 key/value
    heads of 128, a 4096-slot bf16 KV ring, RoPE theta 1e6): decode steps at
    B = 1 with the ring full (each step appends and wraps), over 16 distinct
    layers resident in HBM; then 64-token chunks.  Weights bf16 N(0, 0.02),
    prior ring contents N(0, 1), hidden states RMS-normalised N(0, 1)."""
    import numpy as np
    import torch

    import synth
    import synth.gpu as sg
    from oracle import attention as A
    sh = ATTN_SHAPE
    d, H, G, ctx = sh["d_model"], sh["num_heads"], sh["num_kv_heads"], sh["ctx"]
    hd = 128
    rows = (H + 2 * G) * hd
    desc = smoe.make_attn_desc(d, H, G, ctx, rope_theta=sh["rope_theta"])
    nl = args.layers
    layers = []
    for l in range(nl):
        wqkv = sg.bf16_matrix(0, l, synth.T_ATTN_QKV, rows, d, 0.02)
        wo = sg.bf16_matrix(0, l, synth.T_ATTN_O, d, H * hd, 0.02)
        kc = sg.bf16_matrix(0, l, synth.T_K_CACHE, G * ctx, hd, 1.0)
        vc = sg.bf16_matrix(0, l, synth.T_V_CACHE, G * ctx, hd, 1.0)
        layers.append((wqkv, wo, kc, vc))
    dev = torch.device("cuda:0")
    ws = torch.zeros(smoe.attn_workspace_size(desc, 64), dtype=torch.uint8, device=dev)
    xs1 = [sg.hidden(0, 0, 3000 + i, 1, d) for i in range(64)]
    out = torch.empty(64, d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i, B, xs, pos):
        wqkv, wo, kc, vc = layers[i % nl]
        smoe.attn_forward(desc, wqkv, wo, xs[i % len(xs)], pos, kc, vc, out[:B], ws)

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    pos_base = ctx - 1                     # the ring is full from the first step on
    t1 = timed(lambda i: step(i, 1, xs1, pos_base + i // nl), args.steps, args.warmup)
    # the QKV projection alone, back to back (HIP events on its launch stream)
    def qkv_only(i):
        wqkv, wo, kc, vc = layers[i % nl]
        smoe.attn_forward_stage(0, desc, wqkv, wo, xs1[i % 64], pos_base, kc, vc, out[:1], ws)

    tq = timed(qkv_only, min(args.steps, 2000), 20)
    qkv_bytes = rows * d * 2
    kv_bytes = 2 * G * ctx * hd * 2
    step_bytes = qkv_bytes + d * H * hd * 2 + kv_bytes
    xs64 = [sg.hidden(0, 0, 4000 + i, 64, d) for i in range(4)]
    t64 = timed(lambda i: step(i, 64, xs64, pos_base + 64 * (i // nl + 1)),
                max(4, args.prefill_steps // 10), 2)
    # the oracle (as it stands) on one decode step of layer 0, from CPU-generated inputs
    cfg = A.AttnConfig(d_model=d, num_heads=H, num_kv_heads=G, ctx=ctx, rope_theta=sh["rope_theta"])
    Wq = synth.bf16_matrix(0, 0, synth.T_ATTN_QKV, rows, d, 0.02)
    Wo_ = synth.bf16_matrix(0, 0, synth.T_ATTN_O, d, H * hd, 0.02)
    kc64 = A.bf16_bits_to_f64(synth.bf16_matrix(0, 0, synth.T_K_CACHE, G * ctx, hd, 1.0)).reshape(G, ctx, hd)
    vc64 = A.bf16_bits_to_f64(synth.bf16_matrix(0, 0, synth.T_V_CACHE, G * ctx, hd, 1.0)).reshape(G, ctx, hd)
    x0 = synth.hidden(0, 0, 3000, 1, d)
    n_cpu, t0 = 0, time.perf_counter()
    while True:
        A.attention_block(cfg, Wq, Wo_, x0, pos_base + n_cpu, kc64, vc64)
        n_cpu += 1
        if time.perf_counter() - t0 > min(args.cpu_seconds, 10.0) or n_cpu >= 20:
            break
    cpu_s = (time.perf_counter() - t0) / n_cpu
    del layers
    torch.cuda.empty_cache()
    return {
        "metric": "attention block: decode tokens/s (B=1, full 4096-slot KV ring)",
        "value": round(1.0 / t1, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t1 * 1e3, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "attn_d4096_h64_kv4_hd128_ctx4096: RMS norm, bf16 QKV projection, "
                               "QK-norm, RoPE (theta 1e6), K/V append, causal GQA attention over the "
                               "full ring, bf16 O projection + residual; B=1 decode",
                   "layers_rotated": nl, "effective_bytes_per_step": step_bytes},
        "effective_gbps": round(step_bytes / t1 / 1e9, 1),
        "hbm_frac": round(step_bytes / t1 / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "k_gemv_bf16<1, 8> (QKV projection)",
                     "achieved": round(qkv_bytes / tq / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(qkv_bytes / tq / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": qkv_bytes,
                     "mean_launch_us": round(tq * 1e6, 3)},
        "secondary": {"workload": "the same block on 64-token chunks (each projection one "
                                  "pass of bf16 MFMA tiles over the weights)",
                      "tokens_per_s": round(64 / t64, 1), "ms_per_step": round(t64 * 1e3, 4)},
        "cpu_baseline": {"value": round(1.0 / cpu_s, 3), "unit": "tokens/s", "cores": _blas_threads(),
                         "kind": "oracle",
                         "sample": f"{n_cpu} decode steps of layer 0 at a full ring, numpy float64"},
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_layer(W):
    """Host copies of one device layer's input bytes (router, gate, up, down)
    for the oracle: the generator's bytes, the same as the CPU generator's."""
    import numpy as np
    import torch

    def h(t):
        return tuple(t_.cpu().numpy().view(np.uint32 if t_.dtype == torch.int32 else np.uint16)
                     for t_ in t)
    return {"router": W["router"].cpu().numpy().view(np.uint16), "gate": h(W["gate"]),
            "up": h(W["up"]), "down": h(W["down"])}


def cpu_baseline(cfg, L, seconds):
    """The oracle (as it stands) on bounded samples of the same workload, on
    the host cores: exact routing plus the layer-major FFN of layer 0
    (L: host copies of its weights), timed with perf_counter.
      * decode tokens (B = 1) on every core OpenMP gives it, for ~seconds/2;
      * the same on one core, for ~seconds/4;
      * one 64-token prefill chunk on every core (all of its ~126 union
        experts).  Weight copies to the host are not timed."""
    import numpy as np

    import oracle
    import synth
    from synth import configs
    tokens = [synth.hidden(cfg.seed, 0, 1000 + i, 1, cfg.d_model) for i in range(8)]

    def decode_rate(budget):
        done, t0 = 0, time.perf_counter()
        while True:
            x = tokens[done % len(tokens)]
            _, idx, w = oracle.route(L["router"], x, cfg.top_k, cfg.norm_topk_prob)
            oracle.moe(L["gate"], L["up"], L["down"], x, idx, w, layer_major=True)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done / el, done, el

    all_cores = oracle.num_threads()
    v_all, n_all, el_all = decode_rate(seconds / 2)
    oracle.set_num_threads(1)
    try:
        v_one, n_one, el_one = decode_rate(seconds / 4)
    finally:
        oracle.set_num_threads(all_cores)
    pre = configs.PREFILL
    x64 = synth.hidden(pre.seed, 0, 1000, pre.batch, pre.d_model)
    t0 = time.perf_counter()
    _, idx, w = oracle.route(L["router"], x64, pre.top_k, pre.norm_topk_prob)
    oracle.moe(L["gate"], L["up"], L["down"], x64, idx, w, layer_major=True)
    el64 = time.perf_counter() - t0
    return {"value": round(v_all, 3), "unit": "tokens/s", "cores": all_cores, "kind": "oracle",
            "sample": f"{n_all} single-token decode calls of layer 0 of the decode layer "
                      f"(routing + layer-major FFN), {el_all:.1f} s on {all_cores} threads",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_core": {"value": round(v_one, 3), "unit": "tokens/s", "cores": 1,
                            "sample": f"{n_one} decode calls, {el_one:.1f} s"},
            "prefill_chunk_b64": {"value": round(pre.batch / el64, 2), "unit": "tokens/s",
                                  "cores": all_cores,
                                  "sample": f"one 64-token chunk of layer 0 "
                                            f"({len(np.unique(idx))} union experts), "
                                            f"{el64:.1f} s"}}


# ------------------------------------------------------------------ stack
STACK_CHUNK = 64
STACK_IN_FLIGHT = 4        # prompt chunks in flight in the stacked harness


def stack_stats(idx_pre, nu_pre, idx_dec, E):
    """Routing statistics of a stacked run (host arrays).

    idx_pre [chunks, layers, tokens, K], nu_pre [chunks, layers]: prompt
    chunks; idx_dec [steps, layers, 1, K]: decode steps.  Union size of a
    (chunk, layer) = its distinct experts (checked against the device's
    count); adjacent-step reuse of layer l at step n >= 1 = the share of
    step n's K experts that step n-1 also used in layer l."""
    import numpy as np
    from synth import configs
    C, L, T, K = idx_pre.shape
    distinct = np.array([[len(np.unique(idx_pre[c, l])) for l in range(L)] for c in range(C)])
    if not np.array_equal(distinct, nu_pre):
        raise RuntimeError("device union sizes differ from the routing's distinct experts")
    S = idx_dec.shape[0]
    reuse = np.zeros((max(S - 1, 0), L))
    for n in range(1, S):
        for l in range(L):
            reuse[n - 1, l] = len(np.intersect1d(idx_dec[n, l, 0], idx_dec[n - 1, l, 0])) / K
    per_step = reuse.mean(axis=1) if S > 1 else np.zeros(0)
    return {
        "prefill_union_mean": float(distinct.mean()), "prefill_union_min": int(distinct.min()),
        "prefill_union_max": int(distinct.max()),
        "prefill_union_expected_uniform": round(configs.expected_union(E, K, T), 3),
        "prefill_union_per_chunk": [round(float(v), 2) for v in distinct.mean(axis=1)],
        "decode_reuse_mean": float(reuse.mean()) if S > 1 else None,
        "decode_reuse_expected_uniform": K / E,
        "decode_reuse_per_step": [round(float(v), 4) for v in per_step],
        "decode_union_per_layer": K,
    }


def stack_graph_decode(smoe, desc, args, cfg, n_layers, steps, h_out, idx_out, tmp, un, ws):
    """The decode steps again with each token's whole stack captured once in a
    HIP graph and replayed (the token's input copied into the graph's static
    buffer first).  Every replay's output and routing must equal the stream
    launches' bits for the same input (h_out, idx_out: the eager results)."""
    import torch

    import synth.gpu as sg
    d, K = cfg.d_model, cfg.top_k
    dev = torch.device("cuda:0")
    ins = [sg.hidden(cfg.seed, 0, 6000 + n, 1, d) for n in range(min(steps, 16))]
    hg = torch.zeros(1, d, dtype=torch.float32, device=dev)
    idx_g = torch.zeros(n_layers, 1, K, dtype=torch.int32, device=dev)
    w_g = torch.zeros(n_layers, 1, K, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hg.copy_(ins[0])
        smoe.stack_forward(desc, args, hg, tmp[:1], idx_g, w_g, un, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        smoe.stack_forward(desc, args, hg, tmp[:1], idx_g, w_g, un, ws)
    torch.cuda.synchronize()
    equal = True
    for n in range(len(ins)):
        hg.copy_(ins[n])
        g.replay()
        torch.cuda.synchronize()
        equal = equal and torch.equal(hg, h_out[n]) and torch.equal(idx_g, idx_out[n])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for n in range(steps):
        hg.copy_(ins[n % len(ins)])
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) / steps
    return {"decode_graph_ms_per_token": round(t, 4), "decode_graph_tokens_per_s": round(1e3 / t, 2),
            "decode_graph_replays_equal_stream_bits": bool(equal)}


def near_tie(row, K):
    """True when a token's K-th and (K+1)-th oracle logits are within fp32
    rounding noise, so that two correct implementations may pick either."""
    import numpy as np
    srt = np.sort(row.astype(np.float64))[::-1]
    return K < len(srt) and (srt[K - 1] - srt[K]) <= 1e-5 * max(1.0, float(np.abs(srt).max()))


def stack_oracle_points(smoe, desc, Ws, ex, cfg, n_layers, prompt, steps):
    """The stack's share of the CPU baseline: the oracle on sampled (decode
    step, layer) and (prompt chunk, layer) points, teacher-forced.  A point's
    input is the GPU's own input to layer l (its stream's hidden state through
    the stack's first l layers); layer l then runs alone on the GPU and in the
    oracle, on host copies of the experts the point routes to (copies not
    timed).  The oracle routes on its own logits; a token whose experts differ
    from the GPU's must be at a near-tie, and takes the GPU's set with the
    oracle's weights for it.  Per point: the oracle's seconds and the relative
    L2 of MoE_l(x) over the point and over its worst token."""
    import numpy as np
    import torch

    import oracle
    import synth.gpu as sg
    E, K, d = cfg.num_experts, cfg.top_k, cfg.d_model
    dev = torch.device("cuda:0")
    ws = torch.zeros(smoe.workspace_size(desc, STACK_CHUNK), dtype=torch.uint8, device=dev)
    smoe.workspace_init(ws)
    un = smoe.UnionBuffers.alloc(E, STACK_CHUNK * K, dev)
    layers = sorted({0, n_layers // 2, n_layers - 1})
    points = [("decode", n, l) for n in sorted({0, steps - 1}) for l in layers]
    points += [("prefill", 0, l) for l in sorted({0, n_layers - 1})]
    out_points = []
    for kind, n, l in points:
        x = (sg.hidden(cfg.seed, 0, 6000 + n, 1, d) if kind == "decode"
             else sg.hidden(cfg.seed, 0, 5000, prompt, d)[:STACK_CHUNK].clone())
        B = x.shape[0]
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        if l > 0:
            args = smoe.StackArgs([W["router"] for W in Ws[:l]], ex[:l])
            smoe.stack_forward(desc, args, x, torch.zeros(B, d, **f32), torch.zeros(l, B, K, **i32),
                               torch.zeros(l, B, K, **f32), un, ws)
        out = torch.empty(B, d, **f32)
        idx_g = torch.zeros(B, K, **i32)
        w_g = torch.zeros(B, K, **f32)
        smoe.moe_layer(desc, Ws[l]["router"], ex[l], x, out, idx_g, w_g, un, ws)
        torch.cuda.synchronize()
        xh, outg, idxg = x.cpu().numpy(), out.cpu().numpy(), idx_g.cpu().numpy()
        Wr = Ws[l]["router"].cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        lg_ref, idx_ref, w_ref = oracle.route(Wr, xh, K, cfg.norm_topk_prob)
        t_route = time.perf_counter() - t0
        flips = [t for t in range(B) if not np.array_equal(idxg[t], idx_ref[t])]
        if any(not near_tie(lg_ref[t], K) for t in flips):
            raise RuntimeError(f"stack point {kind} {n} layer {l}: routing differs off a near-tie")
        idx_use, w_use = idx_ref.copy(), w_ref.copy()
        for t in flips:
            idx_use[t] = idxg[t]
            w_use[t] = oracle.weights_of(lg_ref[t:t + 1], idxg[t:t + 1], cfg.norm_topk_prob)[0]
        used = np.unique(idx_use)
        sel = torch.from_numpy(used.astype(np.int64)).to(dev)

        def host(mat):
            return tuple(m.index_select(0, sel).cpu().numpy().view(
                np.uint32 if m.dtype == torch.int32 else np.uint16) for m in mat)
        gate, up, down = host(Ws[l]["gate"]), host(Ws[l]["up"]), host(Ws[l]["down"])
        cidx = np.searchsorted(used, idx_use).astype(np.int32)
        t1 = time.perf_counter()
        ref = oracle.moe(gate, up, down, xh, cidx, w_use, layer_major=True)
        t_ffn = time.perf_counter() - t1
        diff = (outg.astype(np.float64) - ref.astype(np.float64))
        ref64 = ref.astype(np.float64)
        tok = np.linalg.norm(diff, axis=1) / np.maximum(np.linalg.norm(ref64, axis=1), 1e-30)
        out_points.append({"point": f"{kind} {'step' if kind == 'decode' else 'chunk'} {n}, "
                                    f"layer {l}", "tokens": B, "union": int(len(used)),
                           "oracle_s": round(t_route + t_ffn, 3),
                           "rel_l2": float(f"{np.linalg.norm(diff) / np.linalg.norm(ref64):.3e}"),
                           "worst_token_rel_l2": float(f"{tok.max():.3e}"),
                           "near_tie_flips": len(flips)})
    del ws
    torch.cuda.empty_cache()
    return {"kind": "oracle", "cores": oracle.num_threads(),
            "sample": "teacher-forced (step or chunk, layer) points of the 94-layer stack; "
                      "MoE_l of the GPU's own input to layer l, oracle against GPU",
            "points": out_points}


def stack_harness(smoe, n_layers, prompt, steps, oracle_points=False):
    """The stacked routed-expert path: n_layers layers of the decode shape
    resident in HBM; a prompt of `prompt` tokens in chunks of 64, layer-major
    (each chunk through every layer, its union streamed once per layer), then
    `steps` single-token decode steps through every layer; h <- RMSNorm(h +
    MoE(h)) between layers, attention left out.  The prompt runs with
    STACK_IN_FLIGHT chunks at once (smoe_stack_forward_chunks: each chunk a
    layer behind the previous one, on its own stream), and once more one chunk
    at a time (smoe_stack_forward), which must give the same bits.  Inputs:
    RMS-normalised N(0, 1) rows, prompt from one seeded stream, decode step n
    from its own."""
    import numpy as np
    import torch

    import synth.gpu as sg
    from synth import configs
    cfg = configs.STACK
    E, K, d = cfg.num_experts, cfg.top_k, cfg.d_model
    if prompt % STACK_CHUNK:
        raise ValueError("the prompt is a whole number of 64-token chunks")
    chunks = prompt // STACK_CHUNK
    t0 = time.perf_counter()
    Ws = [sg.make_layer(cfg, layer=l) for l in range(n_layers)]
    ex = [smoe.Experts(smoe.qmat(*W["gate"]), smoe.qmat(*W["up"]), smoe.qmat(*W["down"]))
          for W in Ws]
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    args = smoe.StackArgs([W["router"] for W in Ws], ex)
    desc = smoe.make_desc(d, cfg.ffn_dim, E, K, cfg.norm_topk_prob, cfg.router_bf16)
    dev = torch.device("cuda:0")
    # one workspace, union and scratch per chunk in flight
    wss = [torch.zeros(smoe.workspace_size(desc, STACK_CHUNK), dtype=torch.uint8, device=dev)
           for _ in range(STACK_IN_FLIGHT)]
    for w_ in wss:
        smoe.workspace_init(w_)
    uns = [smoe.UnionBuffers.alloc(E, STACK_CHUNK * K, dev) for _ in range(STACK_IN_FLIGHT)]
    tmps = [torch.zeros(STACK_CHUNK, d, dtype=torch.float32, device=dev)
            for _ in range(STACK_IN_FLIGHT)]
    ws, un, tmp = wss[0], uns[0], tmps[0]
    streams = [None] + [torch.cuda.Stream() for _ in range(STACK_IN_FLIGHT - 1)]
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    idx_pre = torch.zeros(chunks, n_layers, STACK_CHUNK, K, **i32)
    w_pre = torch.zeros(chunks, n_layers, STACK_CHUNK, K, **f32)
    nu_pre = torch.zeros(chunks, n_layers, **i32)
    idx_dec = torch.zeros(steps, n_layers, 1, K, **i32)
    w_dec = torch.zeros(steps, n_layers, 1, K, **f32)
    nu_dec = torch.zeros(steps, n_layers, **i32)
    h_pre = sg.hidden(cfg.seed, 0, 5000, prompt, d)
    h_dec = [sg.hidden(cfg.seed, 0, 6000 + n, 1, d) for n in range(steps)]
    def rows(h, c):
        return h[c * STACK_CHUNK:(c + 1) * STACK_CHUNK]

    # warm-up: one chunk, the chunks in flight and one decode step through the
    # stack, on copies
    warm = h_pre[:STACK_CHUNK].clone()
    smoe.stack_forward(desc, args, warm, tmp, idx_pre[0], w_pre[0], un, ws, n_union=nu_pre[0])
    warm = h_pre[:STACK_CHUNK * STACK_IN_FLIGHT].clone()
    smoe.stack_forward_chunks(desc, args, [
        dict(h=rows(warm, j), tmp=tmps[j], topk_idx=idx_pre[j], topk_w=w_pre[j],
             n_union=nu_pre[j], un=uns[j], ws=wss[j], stream=streams[j])
        for j in range(min(STACK_IN_FLIGHT, chunks))])
    warm = h_dec[0].clone()
    smoe.stack_forward(desc, args, warm, tmp[:1], idx_dec[0], w_dec[0], un, ws,
                       n_union=nu_dec[0])
    torch.cuda.synchronize()
    h_one = h_pre.clone()                          # the prompt again, one chunk at a time
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    ev[0].record()
    for c0 in range(0, chunks, STACK_IN_FLIGHT):
        group = list(range(c0, min(c0 + STACK_IN_FLIGHT, chunks)))
        smoe.stack_forward_chunks(desc, args, [
            dict(h=rows(h_pre, c), tmp=tmps[j], topk_idx=idx_pre[c], topk_w=w_pre[c],
                 n_union=nu_pre[c], un=uns[j], ws=wss[j], stream=streams[j])
            for j, c in enumerate(group)])
    ev[1].record()
    for n in range(steps):
        smoe.stack_forward(desc, args, h_dec[n], tmp[:1], idx_dec[n], w_dec[n], un, ws,
                           n_union=nu_dec[n])
    ev[2].record()
    ev[3].record()
    for c in range(chunks):
        smoe.stack_forward(desc, args, rows(h_one, c), tmp, idx_pre[c], w_pre[c], un, ws,
                           n_union=nu_pre[c])
    ev[4].record()
    torch.cuda.synchronize()
    if any(smoe.read_status(w_) != 0 for w_ in wss):
        raise RuntimeError("the stack reported a bad expert id")
    pre_s = ev[0].elapsed_time(ev[1]) / 1e3
    dec_s = ev[1].elapsed_time(ev[2]) / 1e3
    one_s = ev[3].elapsed_time(ev[4]) / 1e3
    in_flight_equal = bool(torch.equal(h_pre.view(torch.int32), h_one.view(torch.int32)))
    if not in_flight_equal:
        raise RuntimeError("chunks in flight differ from one chunk at a time")
    graph = stack_graph_decode(smoe, desc, args, cfg, n_layers, steps, h_dec, idx_dec, tmp, un, ws)
    st = stack_stats(idx_pre.cpu().numpy(), nu_pre.cpu().numpy(), idx_dec.cpu().numpy(), E)
    if not np.all(nu_dec.cpu().numpy() == K):
        raise RuntimeError("a decode step's union is not its K experts")
    finite = bool(torch.isfinite(h_pre).all()) and all(bool(torch.isfinite(h).all()) for h in h_dec)
    eb = cfg.expert_bytes()
    pre_bytes = float(nu_pre.sum().item()) * eb
    dec_bytes = steps * n_layers * K * eb
    out = {
        "workload": f"{cfg.name}: {n_layers} stacked routed layers (d=4096, 128 experts, top-8, "
                    f"ffn 1536, 4-bit g64), h <- RMSNorm(h + MoE(h)); prompt {prompt} tokens "
                    f"in chunks of {STACK_CHUNK}, layer-major; then {steps} decode steps at B=1",
        "resident_expert_gb": round(n_layers * E * eb / 1e9, 2),
        "weight_generation_s": round(gen_s, 2),
        "prefill_s": round(pre_s, 5), "prefill_tokens_per_s": round(prompt / pre_s, 1),
        "prefill_effective_gbps": round(pre_bytes / pre_s / 1e9, 1),
        "prefill_chunks_in_flight": STACK_IN_FLIGHT,
        "prefill_us_per_chunk_layer": round(pre_s / (chunks * n_layers) * 1e6, 1),
        "prefill_one_chunk_at_a_time_us_per_chunk_layer": round(one_s / (chunks * n_layers) * 1e6, 1),
        "prefill_one_chunk_at_a_time_s": round(one_s, 5),
        "prefill_in_flight_equals_one_at_a_time": in_flight_equal,
        "decode_ms_per_token": round(dec_s / steps * 1e3, 4),
        "decode_tokens_per_s": round(steps / dec_s, 2),
        "decode_effective_gbps": round(dec_bytes / dec_s / 1e9, 1),
        "decode_hbm_frac": round(dec_bytes / dec_s / 1e9 / HBM_PEAK_GBPS, 4),
        "outputs_finite": finite,
    }
    out.update(graph)
    out.update(st)
    if oracle_points:
        out["oracle_points"] = stack_oracle_points(smoe, desc, Ws, ex, cfg, n_layers, prompt,
                                                   steps)
    del Ws, ex, args
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ traffic
# HBM traffic of the roofline kernel comes from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) over a short run of this script,
# each scaled by what the same counter reads for a plain device-to-device
# copy of COPY_BYTES.  The summary records a hash of the kernel's sources;
# once they change, the figure is stale and `traffic` is reported as null.
COPY_BYTES = 1 << 30
ROOFLINE_KERNEL = "k_gate_up_gemv<1, 64, 1, true, false>"
ROOFLINE_SOURCES = ["exact_routing_bit_amd/csrc/ffn_gemv.hip", "exact_routing_bit_amd/csrc/ffn_mfma.hip",
                    "exact_routing_bit_amd/csrc/router.hip", "exact_routing_bit_amd/csrc/device.hpp",
                    "exact_routing_bit_amd/csrc/smoe_internal.hpp",
                    "exact_routing_bit_amd/csrc/route_dev.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gate_up_gemv_decode_b1_traffic.txt")


def sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ROOFLINE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def copy_calibration():
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "repeats": 3}), flush=True)


def _counter_rows(path, counter=None):
    """(kernel, grid size, counter, value) of every dispatch row of a
    rocprofv3 --pmc CSV (one counter, or all)."""
    import csv
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if counter is None or r.get("Counter_Name") == counter:
                yield (r["Kernel_Name"], int(r.get("Grid_Size") or 0), r["Counter_Name"],
                       float(r["Counter_Value"]), r.get("Dispatch_Id"))


def short_kernel(name):
    import re
    n = name.replace("smoe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    n = re.sub(r"^void ", "", n)
    i = n.find("(")
    j = n.find(">")
    # keep template arguments, drop the parameter list
    if i >= 0 and (j < 0 or i < n.find("<") or j < i):
        n = n[:i]
    elif i >= 0:
        k = n.find("(", j)
        n = n[:k] if k >= 0 else n
    return n.strip()


def _copy_scale(path, counter):
    vals = [v for k, _, c, v, _ in _counter_rows(path, counter) if "copyBuffer" in k or
            "copy" in k.lower()]
    if not vals:
        raise SystemExit(f"no copy-kernel rows for {counter} in {path}")
    return COPY_BYTES / (max(vals) * 1024.0), max(vals)


def summarize_counters(out, label, copy_fetch_csv, copy_write_csv, *csvs, trace_csv=None,
                       command=None):
    """Per (kernel, grid size): the mean of every collected counter per
    dispatch.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are turned into
    HBM bytes with the scale that makes the same counter read a 1 GiB device
    copy as 1 GiB.  With the kernel_stats.csv of the same command, MFMA
    counters become rates: MOPS_F16 x 512 flops over the kernel's mean
    duration, and MFMA busy cycles over GUI-active cycles x 1024 SIMDs."""
    import csv
    from collections import defaultdict
    f_scale, cf = _copy_scale(copy_fetch_csv, "FETCH_SIZE")
    w_scale, cw = _copy_scale(copy_write_csv, "WRITE_SIZE")
    acc = defaultdict(lambda: defaultdict(list))
    for path in csvs:
        for k, g, c, v, _ in _counter_rows(path):
            acc[(short_kernel(k), g)][c].append(v)
    dur = {}
    if trace_csv:
        with open(trace_csv) as fh:
            for r in csv.DictReader(fh):
                dur[short_kernel(r["Name"])] = float(r["AverageNs"]) / 1e3
    rows = []
    for (k, g), cs in sorted(acc.items(), key=lambda kv: kv[0]):
        if "copyBuffer" in k or k.startswith("at::") or k.startswith("k_quant") or k in (
                "k_hidden", "k_router", "k_fill_u32"):
            continue
        r = {"kernel": k, "grid": g, "dispatches": max(len(v) for v in cs.values())}
        for c, vals in cs.items():
            r[c] = sum(vals) / len(vals)
        if "FETCH_SIZE" in r:
            r["hbm_read_bytes"] = r["FETCH_SIZE"] * 1024.0 * f_scale
        if "WRITE_SIZE" in r:
            r["hbm_write_bytes"] = r["WRITE_SIZE"] * 1024.0 * w_scale
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in r and k in dur:
            r["mfma_f16_tflops"] = r["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / (dur[k] * 1e-6) / 1e12
        if "SQ_VALU_MFMA_BUSY_CYCLES" in r and r.get("GRBM_GUI_ACTIVE"):
            r["mfma_busy_pct"] = 100.0 * r["SQ_VALU_MFMA_BUSY_CYCLES"] / (r["GRBM_GUI_ACTIVE"] * 1024)
        if "SQ_LDS_BANK_CONFLICT" in r and r.get("SQ_LDS_IDX_ACTIVE"):
            r["lds_conflict_per_active"] = r["SQ_LDS_BANK_CONFLICT"] / r["SQ_LDS_IDX_ACTIVE"]
        rows.append(r)
    cols = ["hbm_read_bytes", "hbm_write_bytes", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
            "SQ_INSTS_VALU_MFMA_MOPS_F16", "mfma_f16_tflops", "mfma_busy_pct", "SQ_INSTS_LDS",
            "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "lds_conflict_per_active",
            "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES",
            "GRBM_GUI_ACTIVE"]
    if command:
        passes = []
        for i, pth in enumerate(csvs):
            names = sorted({c for _, _, c, _, _ in _counter_rows(pth)})
            passes.append(f"#   rocprofv3 --pmc {' '.join(names)} --output-format csv -d <out>/p{i} "
                          f"-o p{i} -- {command}")
        passes += [f"#   durations: rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace "
                   f"-o t -- {command}",
                   "#   copy scale: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv "
                   "... -- python3 bench.py --copy-calibration",
                   "#   summary: python3 bench.py --summarize-counters <this file> <label> <copy fetch "
                   "csv> <copy write csv> <pass csvs> --trace-csv <kernel_stats.csv> "
                   "--counter-command '<command>'"]
    else:
        passes = [f"#   {p}" for p in csvs]
    lines = [f"# rocprofv3 --pmc counters per dispatch: {label}",
             "# passes (one rocprofv3 run each, from /tmp, TMPDIR=/tmp):",
             *passes,
             f"# FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}: the same counters "
             f"read {cf:.0f} / {cw:.0f} KiB for a {COPY_BYTES}-byte device copy "
             "(python3 bench.py --copy-calibration)",
             f"# kernel sources sha256: {sources_sha()}", ""]
    for r in rows:
        lines.append(f"kernel: {r['kernel']}  grid: {r['grid']}  dispatches: {r['dispatches']}")
        for c in cols:
            if c in r:
                v = r[c]
                lines.append(f"  {c}: {v:.4g}" if isinstance(v, float) else f"  {c}: {v}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    # the roofline kernel's traffic line (read by traffic_per_launch)
    for r in rows:
        if r["kernel"] == ROOFLINE_KERNEL and "hbm_read_bytes" in r and "hbm_write_bytes" in r:
            t = r["hbm_read_bytes"] + r["hbm_write_bytes"]
            tl = [f"# HBM traffic per launch of {ROOFLINE_KERNEL} on the decode layer (B=1)",
                  f"# from {out}",
                  f"kernel: {ROOFLINE_KERNEL}",
                  f"kernel_sources_sha256: {sources_sha()}",
                  f"fetch_kib_per_dispatch: {r['FETCH_SIZE']:.1f}",
                  f"write_kib_per_dispatch: {r['WRITE_SIZE']:.1f}",
                  f"copy_fetch_kib: {cf:.1f}  (scale {f_scale:.4f})",
                  f"copy_write_kib: {cw:.1f}  (scale {w_scale:.4f})",
                  f"traffic_bytes_per_launch: {t:.0f}"]
            with open(TRAFFIC_FILE, "w") as fh:
                fh.write("\n".join(tl) + "\n")


def traffic_per_launch():
    """Bytes per launch from the committed counter summary, or None when it is
    missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(l.split(":", 1) for l in fh if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("kernel_sources_sha256", "").strip() != sources_sha():
        return None
    return float(kv["traffic_bytes_per_launch"].split()[0])


def summarize_trace(out, label, command, stats_csv):
    """A kernel_stats.csv of rocprofv3 --kernel-trace --stats as a table of
    per-kernel calls and durations (microseconds), longest total first."""
    import csv
    rows = []
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            rows.append((short_kernel(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda t: -t[5])
    lines = [f"# kernel trace: {label}", f"# command: {command}",
             "# rocprofv3 --kernel-trace --stats (kernel_stats.csv), durations in microseconds", "",
             f"{'kernel':70s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for k, c, a, lo, hi, pct in rows:
        lines.append(f"{k[:70]:70s} {c:7d} {a:9.2f} {lo:9.2f} {hi:9.2f} {pct:6.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        if len(args.summarize_counters) < 5:
            raise SystemExit("--summarize-counters OUT LABEL COPY_FETCH_CSV COPY_WRITE_CSV CSV...")
        summarize_counters(*args.summarize_counters, trace_csv=args.trace_csv,
                           command=args.counter_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this build runs the layer on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return

    import exact_routing_bit_amd as smoe
    from synth import configs
    torch.cuda.set_device(0)
    if args.shared:
        print(json.dumps(shared_bench(smoe, args)), flush=True)
        return
    if args.attention:
        print(json.dumps(attention_bench(smoe, args)), flush=True)
        return
    if args.stack:
        r = stack_harness(smoe, args.stack_layers, args.stack_prompt, args.stack_decode)
        print(json.dumps({"metric": "stacked routed path: decode tokens/s (B=1 through every "
                                    "layer) and prompt tokens/s",
                          "value": r["decode_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "higher_is_better": True, "dtype": "f16", "data": "synthetic",
                          "config": {"workload": r.pop("workload")}, "stack": r}), flush=True)
        return

    wl = set(w.strip() for w in args.workloads.split(",") if w.strip())
    if args.no_prefill:
        wl -= {"prefill", "fused_b64"}
    if args.no_fused:
        wl -= {"fused_b1", "fused_b64"}
    # the decode layer (B = 1) and its 64-token prefill chunk over 16 rotated layers
    dec, pre = configs.DECODE, configs.PREFILL
    result, sec, L0 = {}, {}, None
    if "decode" in wl or "prefill" in wl:
        stack = Stack(smoe, dec, args.layers, max_batch=64)
        xs1 = x_pool(dec, 1, 257)
        xs64 = x_pool(pre, 64, 17)
        warm_pass(stack, [xs1, xs64])
    if "decode" in wl:
        main_e = layer_entry(stack, dec, xs1, args.steps, args.warmup)
        progress("decode layer timed")
        gu = main_e["kernels_back_to_back"]["gate_up"]
        result = {
            "metric": METRIC, "value": main_e["tokens_per_s"], "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": main_e["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": f"{dec.name}: one routed MoE layer, d=4096, 128 experts, top-8 "
                                   "norm_topk_prob, ffn 1536, 4-bit g64 experts, B=1 decode",
                       "layers_rotated": args.layers, "mean_union": main_e["mean_union"],
                       "effective_bytes_per_step": main_e["effective_bytes_per_step"],
                       "warm_pass": "every rotated layer at B=1 and B=64, then 0.3 s of layer calls"},
            "effective_gbps": main_e["effective_gbps"], "hbm_frac": main_e["hbm_frac"],
            "roofline": {"bound": "hbm", "kernel": ROOFLINE_KERNEL,
                         "achieved": gu["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gu["frac"], "traffic": traffic_per_launch(),
                         "bytes_per_launch": gu["bytes_per_launch"],
                         "mean_launch_us": gu["mean_launch_us"], "launches": ROOFLINE_LAUNCHES},
            "kernels_back_to_back": main_e["kernels_back_to_back"],
        }
        # the same layer as one cooperative launch (route, gate_up and down in
        # one grid behind two device-wide barriers), beside the three launches
        st = max(args.steps, 200)
        t_single = time_layer(stack, xs1, st, args.warmup, single=True)
        t_three = time_layer(stack, xs1, st, args.warmup)
        sec["decode_single_launch"] = {
            "workload": dec.name + ": the same layer, smoe_moe_layer_single", "steps": st,
            "ms_per_step": round(t_single / st * 1e3, 5),
            "tokens_per_s": round(st / t_single, 1),
            "hbm_frac": round(dec.expert_bytes() * 8 / (t_single / st) / 1e9 / HBM_PEAK_GBPS, 4),
            "three_launches_ms_per_step": round(t_three / st * 1e3, 5)}
        progress("single-launch decode layer timed")
    if "prefill" in wl:
        sec["prefill_b64"] = layer_entry(stack, pre, xs64, args.prefill_steps, 5)
        progress("prefill chunk timed")
    if "decode" in wl or "prefill" in wl:
        if not args.no_cpu and "decode" in wl:
            L0 = host_layer(stack.layers[0][0])
        del stack
        torch.cuda.empty_cache()
    if "fused_b1" in wl or "fused_b64" in wl:
        f1, f64 = configs.FUSED_B1, configs.FUSED_B64
        fst = Stack(smoe, f1, args.layers, max_batch=64)
        xf1, xf64 = x_pool(f1, 1, 257), x_pool(f64, 64, 17)
        warm_pass(fst, [xf1, xf64])
        if "fused_b1" in wl:
            sec["fused_b1"] = layer_entry(fst, f1, xf1, max(args.steps, 200), args.warmup)
        if "fused_b64" in wl:
            sec["fused_b64"] = layer_entry(fst, f64, xf64, args.prefill_steps, 5)
            progress("256-expert layer timed")
        del fst
        torch.cuda.empty_cache()
    if sec:
        result["secondary"] = sec
    if not args.no_calibration:
        result["calibration"] = stream_read_calibration(smoe)
        result["calibration"]["sync"] = sync_calibration(smoe)
        progress("calibrations done")
    stack_points = None
    if not args.no_stack and "decode" in wl:
        result["stack"] = stack_harness(smoe, args.stack_layers, args.stack_prompt,
                                        args.stack_decode, oracle_points=not args.no_cpu)
        stack_points = result["stack"].pop("oracle_points", None)
        progress("94-layer stack done")
    if L0 is not None:
        result["cpu_baseline"] = cpu_baseline(dec, L0, args.cpu_seconds)
        if stack_points is not None:
            result["cpu_baseline"]["stack_points"] = stack_points
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
