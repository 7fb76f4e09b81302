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
K timed replays between synchronisations.  The default W = 50: the chip's
clocks take ~10-15 ms of continuous work to settle, and with 5 warmup replays
the first timed steps ran up to 20 % slower (every timed measurement here
replays its graph W times first).

Printed: one JSON line.  value = rows*layers/s of the step (ms_per_step_spread:
p10/p50/p90 of the per-step event timings).  roofline = the latent attention
kernel (the dominant kernel): algorithmic cache bytes per launch (attended
tokens x 1152 B) / its mean launch time: the attention launches of all layers
captured alone in a HIP graph (kernels run back to back), HIP events around
the replays (on the stream they run on).  traffic = HBM bytes per launch from
the FETCH_SIZE / WRITE_SIZE counter runs recorded in the committed profile,
only while the kernel sources still hash to the recorded digest.
stream_probe_* = the same bytes streamed with the attention's launch geometry
and copy schedule and no arithmetic (the floor of that copy path at this
shape).  roofline.k3_k4 = the attention and the merge (fused with absorb_v)
over the same cache bytes: per layer, and for the ragged layers, 64 dense
layer instances and 64 DSA selections stacked as the rows of one launch each.
cpu_baseline = the CPU oracle (reconstructed and absorbed forms) on every
workload, each on the sample it names (median of 3; one run for the ragged
rows and the prefill), with the CPU model and thread count.  extra = the
step launched eagerly (no graph: the host's launch work in the timed
region), the stacked legs, the dense and DSA chains, the top-k selection,
the full layer and the prefill legs.
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
    ap.add_argument("--warmup", type=int, default=50)
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
    """Capture fn() in a HIP graph and replay it: `warmup` untimed replays, then
    `blocks` timed blocks of `steps` replays, with a HIP event on the current
    stream (where the replays run) before every replay and after the last.
    Returns (ms per replay: the median over the blocks of each block's mean,
    graph, per-replay samples in ms over all blocks)."""
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
    means, samples = [], []
    for _ in range(blocks):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for k in range(steps):
            g.replay()
            ev[k + 1].record()
        torch.cuda.synchronize()
        per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
        samples += per
        means.append(ev[0].elapsed_time(ev[steps]) / steps)
    return sorted(means)[len(means) // 2], g, samples


def spread(samples, scale=1.0):
    """p10 / p50 / p90 of per-replay samples (ms), times `scale`."""
    import numpy as np
    a = np.asarray(samples, dtype=np.float64) * scale
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90))}


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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def _oracle_decode_args(cf, oracle, inp, rows):
    """The oracle's arguments for `rows` of a decode workload (exact fp64 values
    of the stored inputs; the query's rope part rotated by the oracle)."""
    import numpy as np
    c = inp.cfg
    rows = list(rows)
    q_rope = oracle.rope_partial_interleaved(cf.values(inp.q_rope_raw[rows])[:, None],
                                             [int(inp.offsets[b]) for b in rows], c.qk_rope, c.theta)[:, 0]
    sel = None
    if inp.sel_count is not None:
        sel = [inp.attended(b) if inp.sel_count[b] > 0 else None for b in rows]
    return (cf.values(inp.q_nope[rows]), q_rope, cf.values(inp.latent[rows]), cf.values(inp.rope[rows]),
            cf.values(inp.w_kvb), np.asarray(inp.kv_len)[rows], sel, c.softmax_scale, c.qk_nope, c.v_head)


def cpu_baseline(cf, oracle):
    """The oracle (plain fp64 NumPy, BLAS threads as found) on every workload:
    decode in rows*layers/s and effective cache GB/s, prefill in GFLOP/s, each
    in its reconstructed (plain definition) and absorbed forms.  Median of 3
    runs, one run for the ragged rows and the prefill, each on the sample
    named in `sample`."""
    import numpy as np
    import threadpoolctl
    out = {}

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return _median(ts), len(ts)

    def decode_cfg(name, inp, rows, reps, sample):
        toks = sum(len(inp.attended(b)) for b in rows)
        res = {"sample": sample, "rows": len(rows), "attended_tokens": toks, "runs": reps}
        args = _oracle_decode_args(cf, oracle, inp, rows)
        for form in ("reconstructed", "absorbed"):
            fn = oracle.decode_reconstructed if form == "reconstructed" else oracle.decode_absorbed
            dt, n = timed(lambda: fn(*args), reps)
            res[form] = {"s": dt, "rows_layers_per_s": len(rows) / dt, "cache_GBps": toks * TOKEN_BYTES / dt / 1e9}
        out[name] = res
        log(f"cpu baseline {name}: {res['reconstructed']['s']:.2f} s reconstructed, {res['absorbed']['s']:.2f} s absorbed")

    inp = cf.decode_inputs(cf.TINY_F32)
    decode_cfg("tiny_f32", inp, [0], 3, "the whole workload (1 row, 128 tokens)")
    inp = cf.decode_inputs(cf.DENSE_BF16)
    decode_cfg("dense_bf16", inp, [0], 3, "the whole workload (1 row, 4096 tokens)")
    inp = cf.decode_inputs(cf.DSA_BF16)
    decode_cfg("dsa_bf16", inp, [0], 3, "the whole workload (1 row, 2048 selected of 131072)")
    inp.latent = inp.rope = None
    # ragged rows: rows of layer 0 in a seeded random order, each taken while
    # the sample stays within 10000 cached tokens (about 15 s of the plain
    # definition on 16 cores); the rate is also scaled to the whole layer by
    # its cached tokens (the oracle's cost is linear in the tokens of a row)
    inp = cf.decode_inputs(cf.RAGGED_BF16, layer=0)
    order = np.random.default_rng(2026).permutation(len(inp.kv_len))
    rows, toks = [], 0
    for b in order:
        if toks + int(inp.kv_len[b]) <= 10000:
            rows.append(int(b))
            toks += int(inp.kv_len[b])
    if not rows:
        rows, toks = [int(np.argmin(inp.kv_len))], int(np.min(inp.kv_len))
    layer_toks = int(np.sum(inp.kv_len))
    decode_cfg("ragged_bf16", inp, rows, 1,
               f"rows {rows} of layer 0 ({toks} of its {layer_toks} cached tokens; rows in a seeded random order, "
               f"each taken while the sample stays within 10000 tokens)")
    for form in ("reconstructed", "absorbed"):
        r = out["ragged_bf16"][form]
        r["layer_rows_layers_per_s"] = len(inp.kv_len) / (r["s"] * layer_toks / toks)
    inp = None
    # prefill: every key expanded, 64 query rows drawn at random (seeded)
    pc = cf.PREFILL_BF16
    pin = cf.prefill_inputs(pc)
    qrows = np.sort(np.random.default_rng(2027).choice(pc.tokens, size=64, replace=False))
    rr = oracle.rope_partial_interleaved(cf.values(pin.k_rope_raw), 0, pc.qk_rope, pc.theta)
    args = (cf.values(pin.c_q), cf.values(pin.w_qb), cf.values(pin.latent), rr, cf.values(pin.w_kvb), pin.q_offsets,
            pc.theta, None, pc.softmax_scale, pc.heads, pc.qk_nope, pc.qk_rope, pc.v_head)
    dt, _ = timed(lambda: oracle.prefill_reconstructed(*args, query_rows=qrows), 1)
    h, t, k = pc.heads, len(qrows), pc.keys
    flops = (2 * t * pc.q_lora_rank * h * (pc.qk_nope + pc.qk_rope) + 2 * k * pc.kv_lora_rank * h * (pc.qk_nope + pc.v_head)
             + 2 * h * int(np.sum(qrows + 1)) * (pc.qk_nope + pc.qk_rope + pc.v_head))
    out["prefill_bf16"] = {"sample": f"64 query rows of 4096 drawn at random, all {k} keys expanded", "runs": 1,
                           "reconstructed": {"s": dt, "GFLOPs": flops / dt / 1e9, "algorithmic_GFLOP": flops / 1e9}}
    log(f"cpu baseline prefill: {dt:.2f} s")
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    r = out["ragged_bf16"]
    return {
        "value": r["reconstructed"]["layer_rows_layers_per_s"], "unit": "rows*layers/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"ragged_bf16: {r['sample']}; reconstructed fp64 decode in {r['reconstructed']['s']:.1f} s, scaled "
                  f"to the whole 8-row layer by cached tokens",
        "cache_GBps": r["reconstructed"]["cache_GBps"],
        "absorbed_value": r["absorbed"]["layer_rows_layers_per_s"],
        "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
        "configs": out,
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
    ms_p = time_graph(torch, run, 10, 20)[0]   # 20 warmup calls (~14 ms): clocks settle first
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
    """o_proj after a 4096-token prefill (hidden size synthetic): TFLOP/s, after
    100 untimed replays (~40 ms) so that the clocks have settled."""
    import numpy as np
    from synth import generators as gen
    width = 64 * 128
    ctx = torch.from_numpy(gen.normal_f32(5, gen.T_MISC, (rows, width))).to(dev)
    w = torch.from_numpy(cf.store(gen.normal_f32(5, gen.T_MISC, (hidden, width), std=width ** -0.5, layer=1),
                                  cf.BF16).view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((rows, hidden), dtype=torch.float32, device=dev)
    ws = torch.empty(rows * width * 2, dtype=torch.uint8, device=dev)
    ms = time_graph(torch, lambda: mla.mla_o_proj(ctx, w, out=out, workspace=ws), 10, 100)[0]
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

    ms_step, _, step_samples = time_graph(torch, step, args.steps, args.warmup)
    cache_bytes = sum(ly.cache_bytes for ly in layers)
    log(f"step {ms_step:.3f} ms  ({cache_bytes / 1e6:.0f} MB of cache per step)")
    nl = len(layers)

    # dominant kernel: latent attention alone, one launch per layer captured in
    # a graph (back-to-back kernels, no host gaps), events around the replays
    ms_attn, _, attn_samples = time_graph(torch, lambda: [ly.attn(mla) for ly in layers], args.steps, args.warmup,
                                          blocks=3)
    ms_attn /= nl
    per_launch_bytes = cache_bytes / nl
    achieved = per_launch_bytes / (ms_attn * 1e-3) / 1e9
    log(f"attention {ms_attn * 1e3:.1f} us/launch  {achieved:.0f} GB/s")
    # the streaming probe: the same bytes, launch geometry and copy schedule,
    # no arithmetic and no partials
    ms_probe = time_graph(torch, lambda: [mla.mla_decode_stream_probe(ly.latent, ly.rope, ly.kv_len, ly.chunk)
                                          for ly in layers], args.steps, args.warmup, blocks=3)[0] / nl
    probe_gbps = per_launch_bytes / (ms_probe * 1e-3) / 1e9
    log(f"stream probe {ms_probe * 1e3:.1f} us/launch  {probe_gbps:.0f} GB/s")
    # attention + merge (the merge fused with absorb_v, as in the step): the
    # pair the latent-cache bandwidth target is judged on
    def attn_merge():
        for ly in layers:
            ly.attn(mla)
            mla.mla_decode_combine_v(ly.part_o, ly.part_lse, ly.n_splits, ly.w, ly.cfg.qk_nope, ly.cfg.v_head,
                                     ctx=ly.ctx)
    ms_am, _, am_samples = time_graph(torch, attn_merge, args.steps, args.warmup, blocks=3)
    ms_am /= nl
    am_gbps = per_launch_bytes / (ms_am * 1e-3) / 1e9
    log(f"attention + merge {ms_am * 1e3:.1f} us/layer  {am_gbps:.0f} GB/s")

    result = {
        "metric": "MLA decode rows*layers/s and achieved latent-cache HBM GB/s (% of peak)",
        "value": rows * nl / (ms_step * 1e-3),
        "unit": "rows*layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_spread": spread(step_samples),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, fan-in scaled weights)",
        "config": {
            "workload": "ragged_bf16 decode: B=8, H=64, qk_nope=128, qk_rope=64, v_head=128, kv_lora_rank=512, "
                        "lengths U{1024..32768}, 1 query token, bf16 cache, fp32 accumulate",
            "layers": nl, "rows": rows, "cache_MB_per_step": cache_bytes / 1e6,
            "step_GBps_cache": cache_bytes / (ms_step * 1e-3) / 1e9,
            "chain": "decode_query (absorb_q + q RoPE, one launch) -> latent_attn (bf16 split partials) -> "
                     "combine_v (combine + absorb_v, one launch) per layer, HIP graph",
        },
        "roofline": {
            "kernel": "mla_decode_latent_attn (decode_mfma_kernel)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(kernel_sources_digest(ATTN_SOURCES)),
            "per_launch_bytes": per_launch_bytes, "launch_us": ms_attn * 1e3,
            "launch_us_spread": spread(attn_samples, 1e3 / nl),
            "stream_probe_us": ms_probe * 1e3, "stream_probe_GBps": probe_gbps,
            "frac_of_stream_probe": achieved / probe_gbps,
            # the attention and the merge (K3 + K4) over the same cache bytes
            "k3_k4": {"per_layer": {"us": ms_am * 1e3, "us_spread": spread(am_samples, 1e3 / nl),
                                    "GBps": am_gbps, "frac": am_gbps / HBM_PEAK_GBS,
                                    "frac_of_stream_probe": am_gbps / probe_gbps}},
            "sources_sha256": kernel_sources_digest(ATTN_SOURCES),
        },
    }
    k3k4 = result["roofline"]["k3_k4"]

    # ------------------------------------------------------------- extras
    if not args.no_extra:
        extra = {}

        # the same step launched eagerly (no graph): the host's launch work
        # for the 24 kernels is then inside the timed region
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(args.steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        ms_eager = ev0.elapsed_time(ev1) / args.steps
        extra["step_eager"] = {"ms_per_step": ms_eager, "rows_layers_per_s": rows * nl / (ms_eager * 1e-3)}
        log(f"eager step {ms_eager:.3f} ms")

        def stacked_leg(q_lat, q_rope, latent, rope, lens, w, cfg_, sel_idx=None, sel_count=None):
            """One launch of the attention over all the rows, then (a second
            graph) the attention and the merge + projection of those rows."""
            n_att = [c if sel_count is not None and c > 0 else n
                     for n, c in zip(lens, sel_count or [-1] * len(lens))]
            chunk = mla.plan_chunk_len(n_att, slots)
            ns = [mla.split_count(n, chunk) for n in n_att]
            po = torch.empty((len(lens), cfg_.heads, max(ns), cfg_.kv_lora_rank), dtype=torch.bfloat16, device=dev)
            pl = torch.empty((len(lens), cfg_.heads, max(ns)), dtype=torch.float32, device=dev)
            ctx = torch.empty((len(lens), cfg_.heads * cfg_.v_head), dtype=torch.float32, device=dev)
            attn = lambda: mla.mla_decode_latent_attn(q_lat, q_rope, latent, rope, lens, cfg_.softmax_scale, chunk,
                                                      sel_idx=sel_idx, sel_count=sel_count, part_o=po, part_lse=pl,
                                                      s_max=max(ns))
            ms_a, _, sa = time_graph(torch, attn, args.steps, args.warmup, blocks=3)
            def both():
                attn()
                mla.mla_decode_combine_v(po, pl, ns, w, cfg_.qk_nope, cfg_.v_head, ctx=ctx)
            ms_b, _, sb = time_graph(torch, both, args.steps, args.warmup, blocks=3)
            byts = sum(n_att) * TOKEN_BYTES
            return {"rows": len(lens), "chunk": chunk, "splits": sum(ns), "cache_MB": byts / 1e6,
                    "attn_us": ms_a * 1e3, "attn_us_spread": spread(sa, 1e3),
                    "attn_GBps": byts / (ms_a * 1e-3) / 1e9, "attn_frac_hbm": byts / (ms_a * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "k3_k4_us": ms_b * 1e3, "k3_k4_us_spread": spread(sb, 1e3),
                    "k3_k4_GBps": byts / (ms_b * 1e-3) / 1e9,
                    "k3_k4_frac_hbm": byts / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS}

        # the ragged workload's 8 layer instances as the 64 rows of one launch:
        # the same kernels with their per-launch costs (dispatch, first tiles,
        # partial burst, kernel boundary) spread over 1351 MB; a model's layers
        # run one after the other, so this is kernel throughput, not the step
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
        extra["ragged_stacked"] = stacked_leg(r_q_lat, r_q_rope, rs[..., :cfg.kv_lora_rank], rs[..., cfg.kv_lora_rank:],
                                              r_lens, layers[0].w, cfg)
        k3k4["stacked_ragged"] = {k: extra["ragged_stacked"][k] for k in ("k3_k4_us", "k3_k4_GBps", "k3_k4_frac_hbm")}
        log(f"stacked ragged: attn {extra['ragged_stacked']['attn_us']:.1f} us, attn + merge "
            f"{extra['ragged_stacked']['k3_k4_us']:.1f} us")
        del rs, r_q_lat, r_q_rope
        torch.cuda.empty_cache()
        # dense workload, 64 layer instances: chained (one graph) and stacked (one launch, 64 rows)
        dcfg = cf.DENSE_BF16
        n_dense = 64
        dl = [DecodeLayer(dcfg, l, torch, cf, dev) for l in range(n_dense)]
        for ly in dl:
            ly.plan(mla, slots, torch, dev)
        share_partials(dl, torch, dev)
        ms_d, _, _ = time_graph(torch, lambda: [ly.step(mla) for ly in dl], args.steps, args.warmup)
        extra["dense_chained"] = {"layers": n_dense, "ms_per_step": ms_d,
                                  "rows_layers_per_s": n_dense / (ms_d * 1e-3),
                                  "cache_GBps": sum(ly.cache_bytes for ly in dl) / (ms_d * 1e-3) / 1e9}
        stacked = torch.cat([ly.cache for ly in dl], dim=0)          # [64, 4096, 576]
        q_lat = torch.cat([ly.q_lat for ly in dl], dim=0)
        q_rope = torch.cat([ly.q_rope for ly in dl], dim=0)
        extra["dense_stacked"] = stacked_leg(q_lat, q_rope, stacked[..., :512], stacked[..., 512:],
                                             [dcfg.tokens] * n_dense, dl[0].w, dcfg)
        k3k4["stacked_dense"] = {k: extra["dense_stacked"][k] for k in ("k3_k4_us", "k3_k4_GBps", "k3_k4_frac_hbm")}
        del dl, stacked, q_lat, q_rope
        torch.cuda.empty_cache()
        # DSA workload, 8 layer instances (each 131072-token cache, 2048 selected)
        import numpy as np
        scfg = cf.DSA_BF16
        sl = [DecodeLayer(scfg, l, torch, cf, dev) for l in range(args.layers)]
        for ly in sl:
            ly.plan(mla, slots, torch, dev)
        share_partials(sl, torch, dev)
        ms_dsa, _, _ = time_graph(torch, lambda: [ly.step(mla) for ly in sl], args.steps, args.warmup)
        ms_dsa_attn = time_graph(torch, lambda: [ly.attn(mla) for ly in sl], args.steps, args.warmup)[0] / len(sl)
        gb = scfg.selected * TOKEN_BYTES
        extra["dsa_chained"] = {"layers": len(sl), "ms_per_step": ms_dsa,
                                "rows_layers_per_s": len(sl) / (ms_dsa * 1e-3),
                                "attn_launch_us": ms_dsa_attn * 1e3,
                                "gathered_GBps": gb / (ms_dsa_attn * 1e-3) / 1e9}
        # layer-stacked: 64 selections of 2048 (fresh sorted indices) as the rows
        # of one launch, row r over the 131072-token window that starts r/16 of
        # a cache into the 8 caches laid end to end (rows overlap; the 64 x 2048
        # gathered tokens, 151 MB, come from 5 caches, beyond the last-level cache)
        from synth import generators as gen
        n_sel_rows = 64
        st_cache = torch.cat([ly.cache for ly in sl], dim=0)            # [8, W, 576]
        wd = scfg.tokens
        win = torch.as_strided(st_cache, (n_sel_rows, wd, 576), (wd * 576 // 16, 576, 1))
        st_q_lat = torch.cat([ly.q_lat for ly in sl] * (n_sel_rows // len(sl)), dim=0)
        st_q_rope = torch.cat([ly.q_rope for ly in sl] * (n_sel_rows // len(sl)), dim=0)
        st_sel = torch.from_numpy(np.concatenate([gen.dsa_positions(scfg.config_id, wd, scfg.selected, layer=100 + r)
                                                  for r in range(n_sel_rows)])).to(dev)
        extra["dsa_stacked"] = stacked_leg(st_q_lat, st_q_rope, win[..., :512], win[..., 512:], [wd] * n_sel_rows,
                                           sl[0].w, scfg, sel_idx=st_sel, sel_count=[scfg.selected] * n_sel_rows)
        k3k4["stacked_dsa"] = {k: extra["dsa_stacked"][k] for k in ("k3_k4_us", "k3_k4_GBps", "k3_k4_frac_hbm")}
        del sl, st_cache, win, st_q_lat, st_q_rope, st_sel
        torch.cuda.empty_cache()
        # DSA top-k selection over the 131072-token context (synthetic fp32 scores)
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
        ms_full, _, _ = time_graph(torch, lambda: [ly.full_step(mla) for ly in fl], args.steps, args.warmup)
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
        result["cpu_baseline"] = cpu_baseline(cf, oracle)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
