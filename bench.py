#!/usr/bin/env python3
"""Benchmark of the MLA latent-KV decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]

Timed step: one decode step of the batched ragged workload (B=8 rows, H=64,
qk_nope=128, qk_rope=64, v_head=128, kv_lora_rank=512, per-row cache lengths
drawn from U{1024..32768}, bf16 cache, fp32 accumulation) over L distinct layer
instances (default 8, about 1.25 GB of caches, beyond the 256 MB last-level
cache).  Per layer the step runs the whole chain through the C ABI:
  decode query (absorb_q and the RoPE of q_rope in one launch) -> latent
  attention (split-T partials) -> combine and absorb_v (one launch).  The split partials are
  one workspace shared by the layers, as an engine keeps them.
The step is captured once in a HIP graph and replayed; W warmup replays, then
K timed replays between synchronisations.

Printed: one JSON line.  value = rows*layers/s of the step.  roofline = the
latent attention kernel (the dominant kernel): algorithmic cache bytes per
launch (attended tokens x 1152 B) / its mean launch time: the attention
launches of all layers captured alone in a HIP graph (kernels run back to
back), HIP events around the replays.  traffic = HBM bytes per launch from the
FETCH_SIZE / WRITE_SIZE counter runs recorded in the committed profile, only
while the kernel sources still hash to the recorded digest.  stream_probe_* =
the same bytes streamed with the attention's launch geometry and copy
schedule and no arithmetic (the floor of that copy path at this shape);
attn_plus_merge_* = the attention and the merge (fused with absorb_v) per
layer.  cpu_baseline = the CPU oracle's reconstructed decode on a bounded
sample of the same rows (and its absorbed form on the same rows).  extra = the
dense (chained and layer-stacked), DSA (chain, layer-stacked and top-k
selection), full-layer and prefill workloads.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
TOKEN_BYTES = (512 + 64) * 2    # latent + rope per cached token, bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the 4096-token prefill leg (for MFMA counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (for FETCH_SIZE / WRITE_SIZE scaling)")
    return ap.parse_args()


class DecodeLayer:
    """Device tensors of one layer instance of a decode workload, packed cache [B, W, 576]."""

    def __init__(self, cfg, layer, torch, cf, dev, batch=None, spare_slots=0):
        inp = cf.decode_inputs(cfg, layer=layer, batch=batch)
        self.inp = inp
        import numpy as np
        cache = np.concatenate([inp.latent, inp.rope], axis=-1)
        if spare_slots:   # room to append the step's token at slot = width
            cache = np.concatenate([cache, np.zeros((cache.shape[0], spare_slots, cache.shape[2]), cache.dtype)], 1)
        self.cache = torch.from_numpy(cache.view(np.int16)).to(dev).view(torch.bfloat16)
        del cache
        self.latent = self.cache[..., : cfg.kv_lora_rank]
        self.rope = self.cache[..., cfg.kv_lora_rank:]
        b = inp.q_nope.shape[0]
        self.q_nope = torch.from_numpy(inp.q_nope.view(np.int16)).to(dev).view(torch.bfloat16)
        self.q_rope_raw = torch.from_numpy(inp.q_rope_raw.view(np.int16)).to(dev).view(torch.bfloat16)
        self.w = torch.from_numpy(inp.w_kvb.view(np.int16)).to(dev).view(torch.bfloat16)
        self.sel = torch.from_numpy(inp.sel_idx).to(dev) if inp.sel_idx is not None else None
        self.kv_len = [int(v) for v in inp.kv_len]
        self.sel_count = None if inp.sel_count is None else [int(v) for v in inp.sel_count]
        self.offsets = [int(v) for v in inp.offsets]
        self.n_att = [c if self.sel_count is not None and c > 0 else n
                      for n, c in zip(self.kv_len, self.sel_count or [-1] * b)]
        self.q_rope = torch.empty_like(self.q_rope_raw)
        self.q_lat = torch.empty((b, cfg.heads, cfg.kv_lora_rank), dtype=self.cache.dtype, device=dev)
        self.o_lat = torch.empty((b, cfg.heads, cfg.kv_lora_rank), dtype=torch.float32, device=dev)
        self.lse = torch.empty((b, cfg.heads), dtype=torch.float32, device=dev)
        self.ctx = torch.empty((b, cfg.heads * cfg.v_head), dtype=torch.float32, device=dev)
        self.cfg = cfg
        self.layer_id = layer
        # drop the host copies of the large arrays
        inp.latent = inp.rope = None

    def plan(self, mla, slots, torch, dev):
        self.chunk = mla.plan_chunk_len(self.n_att, slots)
        self.n_splits = [mla.split_count(n, self.chunk) for n in self.n_att]
        self.s_max = max(self.n_splits)
        b = len(self.kv_len)
        # bf16 split partials for the bf16 cache (one rounding of each
        # normalised split context; half the partial bytes of fp32)
        self.part_o = torch.empty((b, self.cfg.heads, self.s_max, self.cfg.kv_lora_rank), dtype=self.cache.dtype,
                                  device=dev)
        self.part_lse = torch.empty((b, self.cfg.heads, self.s_max), dtype=torch.float32, device=dev)

    def attn(self, mla):
        c = self.cfg
        mla.mla_decode_latent_attn(self.q_lat, self.q_rope, self.latent, self.rope, self.kv_len, c.softmax_scale,
                                   self.chunk, sel_idx=self.sel, sel_count=self.sel_count, part_o=self.part_o,
                                   part_lse=self.part_lse, s_max=self.s_max)

    def step(self, mla):
        c = self.cfg
        mla.mla_decode_query(self.q_nope, self.q_rope_raw, self.w, c.v_head, self.offsets, c.theta, q_lat=self.q_lat,
                             q_rope_out=self.q_rope)
        self.attn(mla)
        mla.mla_decode_combine_v(self.part_o, self.part_lse, self.n_splits, self.w, c.qk_nope, c.v_head, ctx=self.ctx)

    def full_layer_setup(self, torch, cf, dev, hidden):
        """Tensors of the whole layer around the hot path: the kv_a output of the
        step's token (appended at slot = width, each row at its own RoPE
        position) and the o_proj weight (synthetic hidden size)."""
        import numpy as np
        from synth import generators as gen
        c = self.cfg
        b = len(self.kv_len)
        r, dr = c.kv_lora_rank, c.qk_rope
        t = lambda x: torch.from_numpy(cf.store(x, cf.BF16).view(np.int16)).to(dev).view(torch.bfloat16)
        self.kv_a = t(gen.normal_f32(c.config_id, gen.T_MISC, (b, 1, r + dr), layer=500 + self.layer_id))
        self.norm_w = t(np.float32(1) + gen.normal_f32(c.config_id, gen.T_MISC, (r,), std=0.1, layer=600))
        self.w_o = t(gen.normal_f32(c.config_id, gen.T_MISC, (hidden, c.heads * c.v_head),
                                    std=(c.heads * c.v_head) ** -0.5, layer=700 + self.layer_id))
        self.out = torch.empty((b, hidden), dtype=torch.float32, device=dev)
        self.slot = self.cache.shape[1] - 1
        self.kv_len_new = [n + 1 for n in self.kv_len]

    def full_step(self, mla):
        """append -> query (absorb_q + RoPE) -> attention over kv_len + 1 -> combine + absorb_v -> o_proj."""
        c = self.cfg
        mla.mla_append_compressed(self.kv_a, self.norm_w, 1e-6, self.offsets, c.theta, self.latent, self.rope,
                                  self.slot)
        mla.mla_decode_query(self.q_nope, self.q_rope_raw, self.w, c.v_head, self.offsets, c.theta, q_lat=self.q_lat,
                             q_rope_out=self.q_rope)
        mla.mla_decode_latent_attn(self.q_lat, self.q_rope, self.latent, self.rope, self.kv_len_new,
                                   c.softmax_scale, self.chunk, part_o=self.part_o, part_lse=self.part_lse,
                                   s_max=self.s_max)
        mla.mla_decode_combine_v(self.part_o, self.part_lse, self.n_splits, self.w, c.qk_nope, c.v_head, ctx=self.ctx)
        mla.mla_o_proj(self.ctx, self.w_o, out=self.out)

    @property
    def cache_bytes(self):
        return sum(self.n_att) * TOKEN_BYTES


def share_partials(layers, torch, dev):
    """One split-partial workspace for every layer instance, as a decode engine
    keeps one: the partials are scratch that the combine consumes within the
    same layer, so the layers need not hold them apart."""
    s_max = max(ly.s_max for ly in layers)
    b = max(len(ly.kv_len) for ly in layers)
    c = layers[0].cfg
    po = torch.empty((b, c.heads, s_max, c.kv_lora_rank), dtype=layers[0].part_o.dtype, device=dev)
    pl = torch.empty((b, c.heads, s_max), dtype=torch.float32, device=dev)
    for ly in layers:
        ly.part_o, ly.part_lse, ly.s_max = po, pl, s_max


def time_graph(torch, fn, steps, warmup, blocks=1):
    """Capture fn() in a HIP graph; mean ms per replay over `steps` replays
    (with blocks > 1: the median over `blocks` consecutive timed blocks of
    `steps` replays each)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()   # eager run on the capture stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(blocks):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / steps)
    return sorted(times)[len(times) // 2], g


def kernel_sources_digest(names):
    """sha256 over what the kernel is compiled from, to tie recorded counters to
    a kernel version: whole csrc files, and for "file:first:last" entries the
    lines of that file from the one starting with `first` through the one
    starting with `last` (its parameter block inside a shared header)."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        name, *rng = n.split(":")
        with open(os.path.join(ROOT, "mla_latent_kv_partial_amd", "csrc", name), "rb") as f:
            data = f.read()
        if rng:
            lines = data.decode().splitlines(keepends=True)
            i = next(k for k, ln in enumerate(lines) if ln.startswith(rng[0]))
            j = next(k for k, ln in enumerate(lines) if k >= i and ln.startswith(rng[1]))
            data = "".join(lines[i:j + 1]).encode()
        h.update(data)
    return h.hexdigest()[:16]


# the attention kernel: its file, the device headers it includes and its
# parameter block (with the row limit) in launch.hpp
ATTN_SOURCES = ("decode_mfma.hip", "cdna4.hpp", "common.hpp", "launch.hpp:constexpr int kDecodeRowsPerLaunch:constexpr",
                "launch.hpp:struct DecodeRows:hipError_t launch_decode(")
ATTN_PROFILE = os.path.join(ROOT, "profiles", "decode_attn_ragged_bf16.md")


def recorded_traffic(digest):
    """HBM bytes per attention launch recorded by the FETCH_SIZE / WRITE_SIZE runs
    of the committed profile, if they were taken on kernel sources with this digest."""
    try:
        with open(ATTN_PROFILE) as f:
            text = f.read()
    except OSError:
        return None
    import re
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)\s+sources_sha256:\s*([0-9a-f]+)", text)
    if not m or m.group(2) != digest:
        return None
    return float(m.group(1))


def cpu_baseline(cf, oracle, layer0, budget_s=12.0):
    """The oracle's reconstructed decode (the plain definition) on rows of layer 0
    of the timed workload, until about `budget_s` seconds of CPU work."""
    import numpy as np
    import threadpoolctl
    inp = cf.decode_inputs(layer0.cfg, layer=0)
    c = inp.cfg
    q_rope = oracle.rope_partial_interleaved(cf.values(inp.q_rope_raw)[:, None], [int(o) for o in inp.offsets],
                                             c.qk_rope, c.theta)[:, 0]
    lat, rope, w = cf.values(inp.latent), cf.values(inp.rope), cf.values(inp.w_kvb)
    q_nope = cf.values(inp.q_nope)
    order = np.argsort(inp.kv_len)            # shortest rows first keeps the sample bounded
    rows, tokens, t0 = 0, 0, time.perf_counter()
    for b in order:
        oracle.decode_reconstructed(q_nope[b:b + 1], q_rope[b:b + 1], lat[b:b + 1], rope[b:b + 1], w,
                                    inp.kv_len[b:b + 1], None, c.softmax_scale, c.qk_nope, c.v_head)
        rows += 1
        tokens += int(inp.kv_len[b])
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    # the absorbed form (q_lat = W_UK^T q_nope, attention over latent||rope,
    # W_UV o_lat) on the same rows, fp64
    ta = time.perf_counter()
    for b in order[:rows]:
        oracle.decode_absorbed(q_nope[b:b + 1], q_rope[b:b + 1], lat[b:b + 1], rope[b:b + 1], w,
                               inp.kv_len[b:b + 1], None, c.softmax_scale, c.qk_nope, c.v_head)
    dta = time.perf_counter() - ta
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    return {
        "value": rows / dt, "unit": "rows*layers/s", "cores": int(threads), "kind": "oracle",
        "sample": f"reconstructed fp64 decode of {rows} row(s) of layer 0 ({tokens} cached tokens) in {dt:.1f}s",
        "cache_GBps": tokens * TOKEN_BYTES / dt / 1e9,
        "absorbed_value": rows / dta, "absorbed_cache_GBps": tokens * TOKEN_BYTES / dta / 1e9,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def prefill_leg(torch, mla, cf, dev, tokens=None, left_pad=0):
    """Reconstructed causal prefill over 4096 keys: ms per call and algorithmic TFLOP/s.
    tokens < 4096: the last `tokens` queries over a cached prefix of 4096 - tokens
    keys (chunked prefill); left_pad: keys before it are masked (padded row)."""
    pcfg = cf.PREFILL_BF16
    import numpy as np
    pin = cf.prefill_inputs(pcfg, tokens=tokens or pcfg.tokens, keys=pcfg.keys)
    t = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    c_q, w_qb, latent, w_kvb = t(pin.c_q), t(pin.w_qb), t(pin.latent), t(pin.w_kvb)
    rope = t(pin.k_rope_raw)
    mla.mla_rope_partial_interleaved(rope, 0, pcfg.qk_rope, pcfg.theta, out=rope)
    need = mla.prefill_workspace_bytes(torch.bfloat16, 1, pcfg.tokens, pcfg.keys, pcfg.heads, pcfg.q_lora_rank,
                                       pcfg.kv_lora_rank, pcfg.qk_nope, pcfg.qk_rope, pcfg.v_head)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    tt, kk, h = pin.c_q.shape[1], pin.latent.shape[1], pcfg.heads
    ctx = torch.empty((1, tt, pcfg.heads * pcfg.v_head), dtype=torch.float32, device=dev)
    offs = [int(o) for o in pin.q_offsets]
    run = lambda: mla.mla_prefill_reconstructed(c_q, w_qb, latent, rope, w_kvb, pcfg.heads, pcfg.qk_nope,
                                                pcfg.qk_rope, pcfg.v_head, offs, pcfg.theta, workspace=ws,
                                                ctx=ctx, left_pad=[left_pad] if left_pad else None)
    ms_p = time_graph(torch, run, 10, 5)[0]   # steady clocks: the first calls run slower
    prefix = kk - tt
    visible = sum(max(0, prefix + t + 1 - left_pad) for t in range(tt))   # causal pairs past the pad
    flops = (2 * tt * pcfg.q_lora_rank * h * (pcfg.qk_nope + pcfg.qk_rope)
             + 2 * kk * pcfg.kv_lora_rank * h * (pcfg.qk_nope + pcfg.v_head)
             + 2 * h * visible * (pcfg.qk_nope + pcfg.qk_rope + pcfg.v_head))
    out = {"tokens": tt, "keys": kk, "left_pad": left_pad, "ms": ms_p, "algorithmic_GFLOP": flops / 1e9,
           "TFLOPs": flops / (ms_p * 1e-3) / 1e12,
           "frac_bf16_mfma": flops / (ms_p * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    del c_q, w_qb, latent, w_kvb, rope, ws, ctx
    torch.cuda.empty_cache()
    return out


def o_proj_prefill_leg(torch, mla, cf, dev, rows=4096, hidden=6144):
    """o_proj after a 4096-token prefill (hidden size synthetic): TFLOP/s."""
    import numpy as np
    from synth import generators as gen
    width = 64 * 128
    ctx = torch.from_numpy(gen.normal_f32(5, gen.T_MISC, (rows, width))).to(dev)
    w = torch.from_numpy(cf.store(gen.normal_f32(5, gen.T_MISC, (hidden, width), std=width ** -0.5, layer=1),
                                  cf.BF16).view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((rows, hidden), dtype=torch.float32, device=dev)
    ws = torch.empty(rows * width * 2, dtype=torch.uint8, device=dev)
    ms = time_graph(torch, lambda: mla.mla_o_proj(ctx, w, out=out, workspace=ws), 10, 5)[0]
    flops = 2 * rows * width * hidden
    return {"rows": rows, "in": width, "hidden": hidden, "ms": ms, "TFLOPs": flops / (ms * 1e-3) / 1e12,
            "frac_bf16_mfma": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode and prefill "
              "paths here run on a single GPU (rows or sequence slices would shard across GPUs with one "
              "exchange of split partials per row)", file=sys.stderr)
        sys.exit(2)
    import torch
    import mla_latent_kv_partial_amd as mla
    from synth import configs as cf
    dev = torch.device("cuda:0")
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_leg(torch, mla, cf, dev)}), flush=True)
        return
    props = torch.cuda.get_device_properties(dev)
    slots = props.multi_processor_count
    log(f"device {props.name} CUs={slots}")

    # ------------------------------------------------------------- timed step
    cfg = cf.RAGGED_BF16
    layers = []
    for l in range(args.layers):
        layers.append(DecodeLayer(cfg, l, torch, cf, dev))
        layers[-1].plan(mla, slots, torch, dev)
        log(f"layer {l}: rows {layers[-1].kv_len} chunk {layers[-1].chunk} splits {sum(layers[-1].n_splits)}")
    share_partials(layers, torch, dev)
    rows = len(layers[0].kv_len)

    def step():
        for ly in layers:
            ly.step(mla)

    ms_step, _ = time_graph(torch, step, args.steps, args.warmup)
    cache_bytes = sum(ly.cache_bytes for ly in layers)
    log(f"step {ms_step:.3f} ms  ({cache_bytes / 1e6:.0f} MB of cache per step)")

    # dominant kernel: latent attention alone, one launch per layer captured in
    # a graph (back-to-back kernels, no host gaps), events around the replays
    ms_attn = time_graph(torch, lambda: [ly.attn(mla) for ly in layers], args.steps, args.warmup,
                         blocks=3)[0] / len(layers)
    per_launch_bytes = cache_bytes / len(layers)
    achieved = per_launch_bytes / (ms_attn * 1e-3) / 1e9
    log(f"attention {ms_attn * 1e3:.1f} us/launch  {achieved:.0f} GB/s")
    # the streaming probe: the same bytes, launch geometry and copy schedule,
    # no arithmetic and no partials
    ms_probe = time_graph(torch, lambda: [mla.mla_decode_stream_probe(ly.latent, ly.rope, ly.kv_len, ly.chunk)
                                          for ly in layers], args.steps, args.warmup, blocks=3)[0] / len(layers)
    probe_gbps = per_launch_bytes / (ms_probe * 1e-3) / 1e9
    log(f"stream probe {ms_probe * 1e3:.1f} us/launch  {probe_gbps:.0f} GB/s")
    # attention + merge (the merge fused with absorb_v, as in the step)
    def attn_merge():
        for ly in layers:
            ly.attn(mla)
            mla.mla_decode_combine_v(ly.part_o, ly.part_lse, ly.n_splits, ly.w, ly.cfg.qk_nope, ly.cfg.v_head,
                                     ctx=ly.ctx)
    ms_am = time_graph(torch, attn_merge, args.steps, args.warmup)[0] / len(layers)

    result = {
        "metric": "MLA decode rows*layers/s and achieved latent-cache HBM GB/s (% of peak)",
        "value": rows * len(layers) / (ms_step * 1e-3),
        "unit": "rows*layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, fan-in scaled weights)",
        "config": {
            "workload": "ragged_bf16 decode: B=8, H=64, qk_nope=128, qk_rope=64, v_head=128, kv_lora_rank=512, "
                        "lengths U{1024..32768}, 1 query token, bf16 cache, fp32 accumulate",
            "layers": len(layers), "rows": rows, "cache_MB_per_step": cache_bytes / 1e6,
            "step_GBps_cache": cache_bytes / (ms_step * 1e-3) / 1e9,
            "chain": "decode_query (absorb_q + q RoPE, one launch) -> latent_attn -> combine_v (combine + "
                     "absorb_v, one launch) per layer, HIP graph",
        },
        "roofline": {
            "kernel": "mla_decode_latent_attn (decode_mfma_kernel)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(kernel_sources_digest(ATTN_SOURCES)),
            "per_launch_bytes": per_launch_bytes, "launch_us": ms_attn * 1e3,
            "stream_probe_us": ms_probe * 1e3, "stream_probe_GBps": probe_gbps,
            "frac_of_stream_probe": achieved / probe_gbps,
            "attn_plus_merge_us": ms_am * 1e3, "attn_plus_merge_GBps": per_launch_bytes / (ms_am * 1e-3) / 1e9,
            "sources_sha256": kernel_sources_digest(ATTN_SOURCES),
        },
    }

    # ------------------------------------------------------------- extras
    if not args.no_extra:
        extra = {}
        # the ragged workload's 8 layer instances as the 64 rows of one launch:
        # the same kernel with its per-launch costs (dispatch, first tiles,
        # partial burst, kernel boundary) spread over 1351 MB; a model's
        # layers run one after the other, so this is not the step's figure
        wmax = max(ly.cache.shape[1] for ly in layers)
        rows_all = sum(ly.cache.shape[0] for ly in layers)
        rs = torch.empty((rows_all, wmax, cfg.kv_lora_rank + cfg.qk_rope), dtype=torch.bfloat16, device=dev)
        r0 = 0
        for ly in layers:   # rows stay right-aligned: valid tokens at [wmax - len, wmax)
            rs[r0:r0 + ly.cache.shape[0], wmax - ly.cache.shape[1]:].copy_(ly.cache)
            r0 += ly.cache.shape[0]
        r_lens = [n for ly in layers for n in ly.kv_len]
        r_q_lat = torch.cat([ly.q_lat for ly in layers], dim=0)
        r_q_rope = torch.cat([ly.q_rope for ly in layers], dim=0)
        r_chunk = mla.plan_chunk_len(r_lens, slots)
        r_ns = [mla.split_count(n, r_chunk) for n in r_lens]
        r_po = torch.empty((rows_all, cfg.heads, max(r_ns), cfg.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        r_pl = torch.empty((rows_all, cfg.heads, max(r_ns)), dtype=torch.float32, device=dev)
        ms_r = time_graph(torch, lambda: mla.mla_decode_latent_attn(
            r_q_lat, r_q_rope, rs[..., :cfg.kv_lora_rank], rs[..., cfg.kv_lora_rank:], r_lens, cfg.softmax_scale,
            r_chunk, part_o=r_po, part_lse=r_pl, s_max=max(r_ns)), args.steps, args.warmup, blocks=3)[0]
        extra["ragged_stacked_attn"] = {"rows": rows_all, "chunk": r_chunk, "splits": sum(r_ns),
                                        "launch_us": ms_r * 1e3, "cache_MB": cache_bytes / 1e6,
                                        "cache_GBps": cache_bytes / (ms_r * 1e-3) / 1e9,
                                        "frac_hbm": cache_bytes / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del rs, r_q_lat, r_q_rope, r_po, r_pl
        torch.cuda.empty_cache()
        # dense workload, 64 layer instances: chained (one graph) and stacked (one launch, 64 rows)
        dcfg = cf.DENSE_BF16
        n_dense = 64
        dl = [DecodeLayer(dcfg, l, torch, cf, dev) for l in range(n_dense)]
        for ly in dl:
            ly.plan(mla, slots, torch, dev)
        share_partials(dl, torch, dev)
        ms_d, _ = time_graph(torch, lambda: [ly.step(mla) for ly in dl], args.steps, args.warmup)
        extra["dense_chained"] = {"layers": n_dense, "ms_per_step": ms_d,
                                  "rows_layers_per_s": n_dense / (ms_d * 1e-3),
                                  "cache_GBps": sum(ly.cache_bytes for ly in dl) / (ms_d * 1e-3) / 1e9}
        stacked = torch.cat([ly.cache for ly in dl], dim=0)          # [64, 4096, 576]
        q_lat = torch.cat([ly.q_lat for ly in dl], dim=0)
        q_rope = torch.cat([ly.q_rope for ly in dl], dim=0)
        lens = [dcfg.tokens] * n_dense
        chunk = mla.plan_chunk_len(lens, slots)
        ns = [mla.split_count(n, chunk) for n in lens]
        po = torch.empty((n_dense, dcfg.heads, max(ns), dcfg.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        pl = torch.empty((n_dense, dcfg.heads, max(ns)), dtype=torch.float32, device=dev)
        ms_s = time_graph(torch, lambda: mla.mla_decode_latent_attn(
            q_lat, q_rope, stacked[..., :512], stacked[..., 512:], lens, dcfg.softmax_scale, chunk, part_o=po,
            part_lse=pl, s_max=max(ns)), args.steps, args.warmup)[0]
        sb = n_dense * dcfg.tokens * TOKEN_BYTES
        extra["dense_stacked_attn"] = {"rows": n_dense, "chunk": chunk, "launch_us": ms_s * 1e3,
                                       "cache_GBps": sb / (ms_s * 1e-3) / 1e9,
                                       "frac_hbm": sb / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del dl, stacked, q_lat, q_rope, po, pl
        torch.cuda.empty_cache()
        # DSA workload, 8 layer instances (each 131072-token cache, 2048 selected)
        scfg = cf.DSA_BF16
        sl = [DecodeLayer(scfg, l, torch, cf, dev) for l in range(args.layers)]
        for ly in sl:
            ly.plan(mla, slots, torch, dev)
        share_partials(sl, torch, dev)
        ms_dsa, _ = time_graph(torch, lambda: [ly.step(mla) for ly in sl], args.steps, args.warmup)
        ms_dsa_attn = time_graph(torch, lambda: [ly.attn(mla) for ly in sl], args.steps, args.warmup)[0] / len(sl)
        gb = scfg.selected * TOKEN_BYTES
        extra["dsa_chained"] = {"layers": len(sl), "ms_per_step": ms_dsa,
                                "rows_layers_per_s": len(sl) / (ms_dsa * 1e-3),
                                "attn_launch_us": ms_dsa_attn * 1e3,
                                "gathered_GBps": gb / (ms_dsa_attn * 1e-3) / 1e9}
        # layer-stacked: the layers' selections as rows of one launch
        st_cache = torch.cat([ly.cache for ly in sl], dim=0)
        st_q_lat = torch.cat([ly.q_lat for ly in sl], dim=0)
        st_q_rope = torch.cat([ly.q_rope for ly in sl], dim=0)
        st_sel = torch.cat([ly.sel for ly in sl], dim=0)
        st_len = [n for ly in sl for n in ly.kv_len]
        st_cnt = [c for ly in sl for c in ly.sel_count]
        st_chunk = mla.plan_chunk_len(st_cnt, slots)
        st_ns = [mla.split_count(c, st_chunk) for c in st_cnt]
        st_po = torch.empty((len(st_len), scfg.heads, max(st_ns), scfg.kv_lora_rank), dtype=torch.bfloat16,
                            device=dev)
        st_pl = torch.empty((len(st_len), scfg.heads, max(st_ns)), dtype=torch.float32, device=dev)
        ms_dst = time_graph(torch, lambda: mla.mla_decode_latent_attn(
            st_q_lat, st_q_rope, st_cache[..., :512], st_cache[..., 512:], st_len, scfg.softmax_scale, st_chunk,
            sel_idx=st_sel, sel_count=st_cnt, part_o=st_po, part_lse=st_pl, s_max=max(st_ns)),
            args.steps, args.warmup)[0]
        extra["dsa_stacked_attn"] = {"rows": len(st_len), "chunk": st_chunk, "launch_us": ms_dst * 1e3,
                                     "gathered_GBps": len(st_len) * gb / (ms_dst * 1e-3) / 1e9}
        del sl, st_cache, st_q_lat, st_q_rope, st_sel, st_po, st_pl
        torch.cuda.empty_cache()
        # DSA top-k selection over the 131072-token context (synthetic fp32 scores)
        import numpy as np
        from synth import generators as gen
        n_ctx, k_sel = scfg.tokens, scfg.selected
        scores = torch.from_numpy(gen.normal_f32(scfg.config_id, gen.T_DSA_SCORES, (args.layers, n_ctx))).to(dev)
        sel_buf = torch.empty(args.layers * k_sel, dtype=torch.int32, device=dev)
        lens = [n_ctx] * args.layers
        ws = torch.empty(max(mla.dsa_topk_workspace_bytes(lens, k_sel), 1), dtype=torch.uint8, device=dev)
        topk = {}
        for rows in (args.layers, 1):
            for two in (True, False):
                ms_sel = time_graph(torch, lambda: mla.mla_dsa_topk_select(
                    scores[:rows], lens[:rows], k_sel, sel_idx=sel_buf, workspace=ws, two_stage=two),
                    args.steps, args.warmup)[0]
                topk[f"{rows}_rows_{'two_stage' if two else 'one_workgroup'}_us"] = ms_sel * 1e3
        extra["dsa_topk"] = {"context": n_ctx, "top_k": k_sel, **topk,
                             "scores_GBps_8_rows": args.layers * n_ctx * 4 /
                             (topk[f"{args.layers}_rows_two_stage_us"] * 1e-6) / 1e9}
        del scores, sel_buf, ws
        extra["prefill"] = prefill_leg(torch, mla, cf, dev)
        # the whole layer around the hot path: append + chain + o_proj (hidden 6144, synthetic)
        fl = [DecodeLayer(cfg, l, torch, cf, dev, spare_slots=1) for l in range(args.layers)]
        for ly in fl:
            ly.n_att = [n + 1 for n in ly.n_att]   # attention covers kv_len + 1 tokens
            ly.plan(mla, slots, torch, dev)
            ly.full_layer_setup(torch, cf, dev, hidden=6144)
        share_partials(fl, torch, dev)
        ms_full, _ = time_graph(torch, lambda: [ly.full_step(mla) for ly in fl], args.steps, args.warmup)
        ms_oproj = time_graph(torch, lambda: [mla.mla_o_proj(ly.ctx, ly.w_o, out=ly.out) for ly in fl],
                              args.steps, args.warmup)[0] / len(fl)
        extra["decode_full_layer"] = {
            "layers": len(fl), "hidden": 6144, "ms_per_step": ms_full,
            "rows_layers_per_s": rows * len(fl) / (ms_full * 1e-3),
            "chain": "append -> decode_query -> latent_attn -> combine_v -> o_proj",
            "o_proj_us": ms_oproj * 1e3,
            "o_proj_weight_GBps": 6144 * cfg.heads * cfg.v_head * 2 / (ms_oproj * 1e-3) / 1e9}
        del fl
        torch.cuda.empty_cache()
        extra["prefill_chunked"] = prefill_leg(torch, mla, cf, dev, tokens=1024, left_pad=0)
        extra["prefill_left_padded"] = prefill_leg(torch, mla, cf, dev, tokens=4096, left_pad=1024)
        extra["o_proj_prefill"] = o_proj_prefill_leg(torch, mla, cf, dev)
        result["extra"] = extra

    if args.copy_calibration:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle")
        result["cpu_baseline"] = cpu_baseline(cf, oracle, layers[0])

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
