"""GPU parity of the decode chain (RoPE -> absorb_q -> latent attention -> combine
-> absorb_v) against the oracle on the four decode workloads, and the bitwise
invariants of the attention kernel."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf
from synth import generators as gen
from tests.gpu_util import TOL, assert_close, bitwise_equal, dev, host_values, say

pytestmark = pytest.mark.gpu

CHUNK = {"tiny_f32": 32, "dense_bf16": 256, "ragged_bf16": 512, "dsa_bf16": 256}


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


class Step:
    """Device tensors of one decode workload and the GPU chain over them."""

    def __init__(self, inp: cf.DecodeInputs, packed: bool = True):
        self.inp = inp
        c = inp.cfg
        self.cfg = c
        self.q_nope = dev(inp.q_nope)
        self.q_rope = dev(inp.q_rope_raw)
        self.w = dev(inp.w_kvb)
        if packed:
            cache = np.concatenate([inp.latent, inp.rope], axis=-1)
            self.cache = dev(cache)
            self.latent = self.cache[..., : c.kv_lora_rank]
            self.rope = self.cache[..., c.kv_lora_rank:]
        else:
            self.latent = dev(inp.latent)
            self.rope = dev(inp.rope)
        self.sel = dev(inp.sel_idx) if inp.sel_idx is not None else None
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(self, chunk, part_dtype=torch.float32):
        mla = _mla()
        c, inp = self.cfg, self.inp
        q_rope = self.q_rope.clone()
        view = q_rope.view(q_rope.shape[0], 1, c.heads, c.qk_rope)
        mla.mla_rope_partial_interleaved(view, [int(o) for o in inp.offsets], c.qk_rope, c.theta, out=view)
        q_lat = mla.mla_absorb_q(self.q_nope, self.w, c.v_head)
        po, pl, ns = mla.mla_decode_latent_attn(q_lat, q_rope, self.latent, self.rope, inp.kv_len, c.softmax_scale,
                                                chunk, sel_idx=self.sel, sel_count=inp.sel_count, dev_err=self.err,
                                                part_dtype=part_dtype)
        o_lat, lse = mla.mla_decode_combine(po, pl, ns)
        ctx = mla.mla_absorb_v(o_lat, self.w, c.qk_nope, c.v_head)
        # the same merge and projection in one launch
        o_lat_v, lse_v = torch.empty_like(o_lat), torch.empty_like(lse)
        ctx_v = mla.mla_decode_combine_v(po, pl, ns, self.w, c.qk_nope, c.v_head, o_lat=o_lat_v, lse=lse_v)
        torch.cuda.synchronize()
        return dict(q_rope=q_rope, q_lat=q_lat, part_o=po, part_lse=pl, n_splits=ns, o_lat=o_lat, lse=lse, ctx=ctx,
                    o_lat_v=o_lat_v, lse_v=lse_v, ctx_v=ctx_v)


def _selections(inp):
    if inp.sel_count is None:
        return None
    return [inp.attended(b) if inp.sel_count[b] > 0 else None for b in range(len(inp.kv_len))]


def _oracle(inp, reconstructed=False):
    c = inp.cfg
    q_rope = oracle.rope_partial_interleaved(cf.values(inp.q_rope_raw)[:, None], [int(o) for o in inp.offsets],
                                             c.qk_rope, c.theta)[:, 0]
    args = (cf.values(inp.q_nope), q_rope, cf.values(inp.latent), cf.values(inp.rope), cf.values(inp.w_kvb),
            inp.kv_len, _selections(inp), c.softmax_scale, c.qk_nope, c.v_head)
    out = oracle.decode_absorbed(*args)
    out["q_rope"] = q_rope
    if reconstructed:
        out["ctx_rec"] = oracle.decode_reconstructed(*args)
    return out


@pytest.mark.parametrize("plan", ["fixed", "bench"])
@pytest.mark.parametrize("cfg", cf.DECODE_CONFIGS, ids=lambda c: c.name)
def test_decode_chain_matches_oracle(cfg, plan):
    """Every decode workload at full size, with a fixed chunk and with the
    split plan bench.py times (256 concurrent workgroups)."""
    say(f"decode chain {cfg.name} ({plan} chunk): generating")
    inp = cf.decode_inputs(cfg)
    step = Step(inp)
    n_att = [int(c) if inp.sel_count is not None and c > 0 else int(n)
             for n, c in zip(inp.kv_len, inp.sel_count if inp.sel_count is not None else [-1] * len(inp.kv_len))]
    chunk = CHUNK[cfg.name] if plan == "fixed" else _mla().plan_chunk_len(n_att, 256)
    say(f"decode chain {cfg.name}: gpu, chunk {chunk}")
    got = step.run(chunk)
    assert int(step.err.item()) == 0
    say(f"decode chain {cfg.name}: oracle")
    ref = _oracle(inp, reconstructed=cfg.name in ("tiny_f32", "dense_bf16"))
    assert_close(host_values(got["q_lat"]), ref["q_lat"], cfg.dtype, "q_lat")
    assert_close(host_values(got["o_lat"]), ref["o_lat"], cfg.dtype, "o_lat")
    assert_close(host_values(got["lse"]), ref["lse"], cfg.dtype, "lse")
    assert_close(host_values(got["ctx"]), ref["ctx"], cfg.dtype, "ctx vs absorbed oracle")
    assert_close(host_values(got["ctx_v"]), ref["ctx"], cfg.dtype, "fused combine_v ctx vs absorbed oracle")
    # the fused entry's merge is the combine's own code: identical o_lat and lse
    assert bitwise_equal(got["o_lat_v"], got["o_lat"]) and bitwise_equal(got["lse_v"], got["lse"])
    if "ctx_rec" in ref:
        assert_close(host_values(got["ctx"]), ref["ctx_rec"], cfg.dtype, "ctx vs reconstructed oracle")
        assert_close(host_values(got["ctx_v"]), ref["ctx_rec"], cfg.dtype, "fused ctx vs reconstructed oracle")


@pytest.mark.parametrize("cfg", [cf.DENSE_BF16, cf.RAGGED_BF16, cf.DSA_BF16], ids=lambda c: c.name)
def test_decode_chain_bf16_partials(cfg):
    """The bf16 workloads at full size in the split plan bench.py times, with
    the split partials stored in bf16: the chain against the oracle at the bf16
    bar, and the partials bit-identical to the fp32 partials of the same call
    rounded to bf16 (one rounding of the same normalised values)."""
    mla = _mla()
    say(f"bf16 partials {cfg.name}: generating")
    inp = cf.decode_inputs(cfg)
    step = Step(inp)
    n_att = [int(c) if inp.sel_count is not None and c > 0 else int(n)
             for n, c in zip(inp.kv_len, inp.sel_count if inp.sel_count is not None else [-1] * len(inp.kv_len))]
    chunk = mla.plan_chunk_len(n_att, 256)
    got = step.run(chunk, part_dtype=torch.bfloat16)
    ref32 = step.run(chunk)
    assert int(step.err.item()) == 0
    assert got["part_o"].dtype == torch.bfloat16
    for b, n in enumerate(got["n_splits"]):
        assert bitwise_equal(got["part_o"][b, :, :n], ref32["part_o"][b, :, :n].to(torch.bfloat16))
        assert bitwise_equal(got["part_lse"][b, :, :n], ref32["part_lse"][b, :, :n])
    say(f"bf16 partials {cfg.name}: oracle")
    ref = _oracle(inp)
    assert_close(host_values(got["o_lat"]), ref["o_lat"], cfg.dtype, "o_lat (bf16 partials)")
    assert_close(host_values(got["lse"]), ref["lse"], cfg.dtype, "lse (bf16 partials)")
    assert_close(host_values(got["ctx"]), ref["ctx"], cfg.dtype, "ctx (bf16 partials)")
    assert_close(host_values(got["ctx_v"]), ref["ctx"], cfg.dtype, "fused combine_v ctx (bf16 partials)")


def _small_ragged(lengths=(700, 1, 333), seed_layer=5):
    """The ragged workload's head geometry at short, fixed per-row lengths."""
    return cf.decode_inputs(cf.RAGGED_BF16, layer=seed_layer, lengths=lengths)


@pytest.mark.parametrize("chunk", [1, 7, 64, 100, 256, 1024])
def test_partials_match_oracle(chunk):
    """The attention kernel alone: seeded latent-space and rotated queries go to
    both sides unchanged, so the partials of every split are compared directly."""
    inp = _small_ragged(lengths=(40, 1, 9) if chunk == 1 else (700, 1, 333), seed_layer=7)
    c = inp.cfg
    b = len(inp.kv_len)
    ql = cf.store(gen.normal_f32(c.config_id, gen.T_MISC, (b, c.heads, c.kv_lora_rank), layer=100 + chunk), c.dtype)
    qr = cf.store(gen.normal_f32(c.config_id, gen.T_MISC, (b, c.heads, c.qk_rope), layer=200 + chunk), c.dtype)
    got_o, got_l, got_ns = _mla().mla_decode_latent_attn(dev(ql), dev(qr), dev(inp.latent), dev(inp.rope), inp.kv_len,
                                                         c.softmax_scale, chunk)
    torch.cuda.synchronize()
    po, pl, ns = oracle.latent_attention_partials(cf.values(ql), cf.values(qr), cf.values(inp.latent),
                                                  cf.values(inp.rope), inp.kv_len, None, c.softmax_scale, chunk)
    assert list(ns) == got_ns
    gpo, gpl = host_values(got_o), host_values(got_l)
    for b in range(len(ns)):
        n = int(ns[b])
        assert_close(gpo[b, :, :n], po[b, :, :n], c.dtype, f"part_o row {b}")
        assert_close(gpl[b, :, :n], pl[b, :, :n], c.dtype, f"part_lse row {b}")


def test_batched_rows_equal_separate_calls_bitwise():
    inp = _small_ragged(lengths=(700, 5, 333), seed_layer=8)
    step = Step(inp, packed=True)
    mla = _mla()
    c = inp.cfg
    q_lat = mla.mla_absorb_q(step.q_nope, step.w, c.v_head)
    po, pl, ns = mla.mla_decode_latent_attn(q_lat, step.q_rope, step.latent, step.rope, inp.kv_len,
                                            c.softmax_scale, 128)
    w = step.latent.shape[1]
    for b in range(3):
        n = int(inp.kv_len[b])
        po_b, pl_b, ns_b = mla.mla_decode_latent_attn(
            q_lat[b:b + 1], step.q_rope[b:b + 1], step.latent[b:b + 1, w - n:], step.rope[b:b + 1, w - n:], [n],
            c.softmax_scale, 128, s_max=po.shape[2])
        assert ns_b[0] == ns[b]
        assert bitwise_equal(po_b[0, :, :ns[b]], po[b, :, :ns[b]])
        assert bitwise_equal(pl_b[0, :, :ns[b]], pl[b, :, :ns[b]])


def test_query_copy_and_register_loads_agree_bitwise():
    """Queries with 16-byte aligned rope rows are copied to LDS with the cache
    tiles; a rope view whose rows are not aligned takes the register loads.
    Both read the same values: identical partials."""
    inp = _small_ragged(lengths=(700, 5, 333), seed_layer=12)
    step = Step(inp, packed=True)
    mla = _mla()
    c = inp.cfg
    q_lat = mla.mla_absorb_q(step.q_nope, step.w, c.v_head)
    b = step.q_rope.shape[0]
    wide = torch.zeros((b, c.heads, c.qk_rope + 1), dtype=step.q_rope.dtype, device="cuda")
    odd = wide[:, :, 1:]                      # rows 130 B apart, starting 2 B in: not 16-byte aligned
    odd.copy_(step.q_rope)
    args = (step.latent, step.rope, inp.kv_len, c.softmax_scale, 128)
    po_a, pl_a, ns_a = mla.mla_decode_latent_attn(q_lat, step.q_rope, *args)
    po_b, pl_b, ns_b = mla.mla_decode_latent_attn(q_lat, odd, *args)
    torch.cuda.synchronize()
    assert list(ns_a) == list(ns_b)
    for r in range(b):                        # splits past a row's count are never written
        n = int(ns_a[r])
        assert bitwise_equal(po_a[r, :, :n], po_b[r, :, :n])
        assert bitwise_equal(pl_a[r, :, :n], pl_b[r, :, :n])


def test_selection_of_all_equals_dense_bitwise():
    inp = _small_ragged(lengths=(700, 5, 333), seed_layer=9)
    step = Step(inp)
    mla = _mla()
    c = inp.cfg
    q_lat = mla.mla_absorb_q(step.q_nope, step.w, c.v_head)
    dense = mla.mla_decode_latent_attn(q_lat, step.q_rope, step.latent, step.rope, inp.kv_len, c.softmax_scale, 64)
    sel = torch.cat([torch.arange(int(n), dtype=torch.int32) for n in inp.kv_len]).cuda()
    counts = [int(n) for n in inp.kv_len]
    picked = mla.mla_decode_latent_attn(q_lat, step.q_rope, step.latent, step.rope, inp.kv_len, c.softmax_scale, 64,
                                        sel_idx=sel, sel_count=counts)
    for b in range(3):
        n = dense[2][b]
        assert bitwise_equal(dense[0][b, :, :n], picked[0][b, :, :n])
        assert bitwise_equal(dense[1][b, :, :n], picked[1][b, :, :n])


def test_dsa_gather_equals_compacted_dense_bitwise():
    """Full-size DSA workload: gathering 2048 of 131072 tokens is bit-identical to
    attending a cache that holds exactly those tokens in the same order."""
    inp = cf.decode_inputs(cf.DSA_BF16)
    step = Step(inp)
    mla = _mla()
    c = inp.cfg
    q_lat = mla.mla_absorb_q(step.q_nope, step.w, c.v_head)
    sparse = mla.mla_decode_latent_attn(q_lat, step.q_rope, step.latent, step.rope, inp.kv_len, c.softmax_scale,
                                        256, sel_idx=step.sel, sel_count=inp.sel_count, dev_err=step.err)
    idx = torch.from_numpy(inp.sel_idx.astype(np.int64)).cuda() + (step.latent.shape[1] - int(inp.kv_len[0]))
    compact = step.cache[:, idx].contiguous()
    dense = mla.mla_decode_latent_attn(q_lat, step.q_rope, compact[..., :512], compact[..., 512:],
                                       [len(inp.sel_idx)], c.softmax_scale, 256)
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    assert sparse[2] == dense[2] == [8]
    assert bitwise_equal(sparse[0], dense[0]) and bitwise_equal(sparse[1], dense[1])


def test_selection_permutation_within_tolerance_and_bad_index_flagged():
    inp = _small_ragged(lengths=(700, 5, 333), seed_layer=10)
    step = Step(inp)
    mla = _mla()
    c = inp.cfg
    q_lat = mla.mla_absorb_q(step.q_nope, step.w, c.v_head)
    rng = np.random.default_rng(0)
    rows = [np.sort(rng.choice(700, 300, replace=False)), np.array([4, 0, 2]), np.sort(rng.choice(333, 50, False))]
    counts = [len(r) for r in rows]

    def run(rws, err=None):
        sel = torch.from_numpy(np.concatenate(rws).astype(np.int32)).cuda()
        po, pl, ns = mla.mla_decode_latent_attn(q_lat, step.q_rope, step.latent, step.rope, inp.kv_len,
                                                c.softmax_scale, 64, sel_idx=sel, sel_count=[len(r) for r in rws],
                                                dev_err=err)
        o, lse = mla.mla_decode_combine(po, pl, ns)
        return host_values(o), host_values(lse)

    a = run(rows)
    b = run([rng.permutation(r) for r in rows])
    assert_close(b[0], a[0], c.dtype, "permuted selection o_lat")
    # an index outside [0, kv_len) is skipped and flagged
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = [rows[0], np.array([4, 0, 2, 5, -1]), rows[2]]
    got = run(bad, err)
    torch.cuda.synchronize()
    assert int(err.item()) != 0
    assert_close(got[0], a[0], c.dtype, "masked bad indices")


def test_single_token_and_uniform_closed_forms():
    inp = _small_ragged(lengths=(1, 40, 9), seed_layer=11)
    step = Step(inp)
    mla = _mla()
    c = inp.cfg
    q_lat = mla.mla_absorb_q(step.q_nope, step.w, c.v_head)
    po, pl, ns = mla.mla_decode_latent_attn(q_lat, step.q_rope, step.latent, step.rope, inp.kv_len,
                                            c.softmax_scale, 16)
    o, lse = mla.mla_decode_combine(po, pl, ns)
    c0 = step.latent[0, -1].float()
    assert torch.equal(o[0], c0.expand_as(o[0])), "one attended token must be returned exactly"
    zq = torch.zeros_like(q_lat)
    zr = torch.zeros_like(step.q_rope)
    po, pl, ns = mla.mla_decode_latent_attn(zq, zr, step.latent, step.rope, inp.kv_len, c.softmax_scale, 16)
    o, lse = mla.mla_decode_combine(po, pl, ns)
    for b in range(3):
        n = int(inp.kv_len[b])
        mean = host_values(step.latent[b, -n:]).mean(axis=0)
        assert_close(host_values(o[b]), np.broadcast_to(mean, (c.heads, mean.size)), c.dtype, f"uniform row {b}",
                     tol=1e-5)
        assert np.allclose(host_values(lse[b]), math.log(n), rtol=1e-5)


@pytest.mark.parametrize("dtype,batch", [(cf.F32, 1), (cf.BF16, 1), (cf.BF16, 8), (cf.BF16, 33)])
def test_absorb_matches_oracle(dtype, batch):
    cfg = cf.TINY_F32 if dtype == cf.F32 else cf.DENSE_BF16
    from synth import generators as g
    h, dn, dv, r = cfg.heads, cfg.qk_nope, cfg.v_head, cfg.kv_lora_rank
    q = cf.store(g.normal_f32(95, 1, (batch, h, dn)), dtype)
    w = cf.store(g.normal_f32(95, 2, (h * (dn + dv), r), std=1 / math.sqrt(r)), dtype)
    o = g.normal_f32(95, 3, (batch, h, r))
    mla = _mla()
    q_lat = mla.mla_absorb_q(dev(q), dev(w), dv)
    ctx = mla.mla_absorb_v(dev(o), dev(w), dn, dv)
    torch.cuda.synchronize()
    assert_close(host_values(q_lat), oracle.absorb_q(cf.values(q), cf.values(w), dn, dv), dtype, "absorb_q")
    assert_close(host_values(ctx), oracle.absorb_v(o.astype(np.float64), cf.values(w), dn, dv), dtype, "absorb_v",
                 tol=TOL[dtype] if dtype == cf.F32 else 2e-2)


def test_absorb_unit_query_selects_weight_row_exactly():
    cfg = cf.DENSE_BF16
    from synth import generators as g
    h, dn, dv, r = cfg.heads, cfg.qk_nope, cfg.v_head, cfg.kv_lora_rank
    w = cf.store(g.normal_f32(96, 2, (h * (dn + dv), r), std=1 / math.sqrt(r)), cf.BF16)
    q = np.zeros((2, h, dn), dtype=np.float32)
    q[0, :, 5] = 1.0
    q[1, :, 127] = 1.0
    q_lat = _mla().mla_absorb_q(dev(cf.store(q, cf.BF16)), dev(w), dv)
    wt = dev(w).float().view(h, dn + dv, r)
    assert torch.equal(q_lat[0], wt[:, 5]) and torch.equal(q_lat[1], wt[:, 127])


@pytest.mark.parametrize("heads", [16, 32, 48, 128])
@pytest.mark.parametrize("packed", [True, False])
def test_head_counts_match_oracle(heads, packed):
    """The MFMA kernel's head-group variants (16, 32, 64 x 2 heads per launch)
    and a head count it has no grouping for (48: the generic kernel) on ragged
    rows, packed and separate latent / rope caches."""
    cfg = cf.with_shape(cf.RAGGED_BF16, heads=heads)
    inp = cf.decode_inputs(cfg, layer=heads, lengths=(300, 1, 77))
    say(f"heads={heads} packed={packed}")
    got = Step(inp, packed=packed).run(64)
    ref = _oracle(inp)
    assert_close(host_values(got["ctx"]), ref["ctx"], cfg.dtype, "ctx")
    assert_close(host_values(got["lse"]), ref["lse"], cfg.dtype, "lse")


@pytest.mark.parametrize("heads", [16, 32, 48, 128])
def test_head_counts_gathered_match_oracle(heads):
    cfg = cf.with_shape(cf.DSA_BF16, heads=heads, tokens=4096, selected=300)
    inp = cf.decode_inputs(cfg, layer=heads)
    say(f"gathered heads={heads}")
    step = Step(inp)
    got = step.run(64)
    assert int(step.err.item()) == 0
    ref = _oracle(inp)
    assert_close(host_values(got["ctx"]), ref["ctx"], cfg.dtype, "ctx")


@pytest.mark.parametrize("heads,r,n_splits,s_max,misalign", [
    (3, 512, (1, 7, 33, 600, 700), 700, False),   # several load batches, > 512 splits
    (2, 36, (40, 3), 40, False),                  # 16-byte path with a short feature axis
    (2, 30, (9, 1), 10, False),                   # scalar path: r not a multiple of 4
    (2, 512, (5, 70), 70, True),                  # scalar path: misaligned partials
    (1, 8, (5000,), 5000, False),                 # split lse beyond the LDS copy
])
def test_combine_direct_partials(heads, r, n_splits, s_max, misalign):
    """The merge on given partials against the oracle's merge, with empty
    splits (lse = -inf) whose partials hold NaN: such splits add nothing, and a
    (row, head) with no non-empty split gives o = 0 and lse = -inf."""
    mla = _mla()
    b = len(n_splits)
    say(f"combine heads={heads} r={r} n_splits={n_splits} s_max={s_max} misalign={misalign}")
    po = gen.normal_f32(96, 1, (b, heads, s_max, r))
    pl = 3.0 * gen.normal_f32(96, 2, (b, heads, s_max))
    rng = np.random.default_rng(7)
    empty = rng.random((b, heads, s_max)) < 0.2
    empty[0, 0, :] = True                           # a (row, head) with no split
    pl[empty] = -np.inf
    po_gpu = po.copy()
    po_gpu[empty] = np.nan
    flat = torch.empty(po.size + 1, dtype=torch.float32, device="cuda")
    view = (flat[1:] if misalign else flat[:-1]).view(b, heads, s_max, r)
    view.copy_(torch.from_numpy(po_gpu))
    o, lse = mla.mla_decode_combine(view, dev(pl), list(n_splits))
    po_ref = np.where(empty[..., None], 0.0, po)
    o_ref, lse_ref = oracle.combine_partials(po_ref, pl, n_splits)
    o_h, lse_h = host_values(o), host_values(lse)
    assert not np.isnan(o_h).any()
    assert np.array_equal(o_h[0, 0], np.zeros(r)) and lse_h[0, 0] == -np.inf
    assert_close(o_h, o_ref, cf.F32, "combined o_lat", tol=1e-5)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_h), fin)
    assert np.allclose(lse_h[fin], lse_ref[fin], rtol=0, atol=1e-5)


@pytest.mark.parametrize("fused", [False, True])
def test_merge_of_bf16_partials(fused):
    """The merge (and the fused merge + projection) reading bf16 partials, with
    empty splits, against the oracle's merge of the same (exactly widened) values."""
    mla = _mla()
    n_splits = (1, 9, 31, 40)
    b, heads, r, dn, dv = len(n_splits), 8, 512, 128, 128
    s_max = max(n_splits)
    po = cf.store(gen.normal_f32(98, 1, (b, heads, s_max, r)), cf.BF16)
    pl = 3.0 * gen.normal_f32(98, 2, (b, heads, s_max))
    empty = np.random.default_rng(12).random((b, heads, s_max)) < 0.2
    empty[0, 0, :] = True
    pl[empty] = -np.inf
    w = cf.store(gen.normal_f32(98, 3, (heads * (dn + dv), r), std=r ** -0.5), cf.BF16)
    po_ref = np.where(empty[..., None], 0.0, cf.values(po))
    o_ref, lse_ref = oracle.combine_partials(po_ref, pl, n_splits)
    o_lat = torch.empty((b, heads, r), dtype=torch.float32, device="cuda")
    lse = torch.empty((b, heads), dtype=torch.float32, device="cuda")
    if fused:
        ctx = mla.mla_decode_combine_v(dev(po), dev(pl), list(n_splits), dev(w), dn, dv, o_lat=o_lat, lse=lse)
    else:
        mla.mla_decode_combine(dev(po), dev(pl), list(n_splits), o_lat=o_lat, lse=lse)
    torch.cuda.synchronize()
    assert_close(host_values(o_lat), o_ref, cf.F32, "merged o_lat of bf16 partials", tol=1e-5)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(host_values(lse)), fin)
    if fused:
        assert_close(host_values(ctx), oracle.absorb_v(o_ref, cf.values(w), dn, dv), cf.F32, "fused ctx", tol=1e-5)


@pytest.mark.parametrize("wdt,heads,r,dn,dv,n_splits", [
    (cf.BF16, 8, 512, 128, 128, (1, 9, 31, 40)),   # bf16, r = 512: the row-pair kernel
    (cf.BF16, 3, 512, 64, 96, (5, 2, 7)),          # row-pair kernel with an odd row count, dv < 128
    (cf.BF16, 3, 448, 32, 64, (5, 2)),              # fast path, r / 64 = 7, one pass of columns
    (cf.BF16, 2, 1024, 16, 40, (3, 12)),            # r beyond the fast path: one thread per column
    (cf.BF16, 2, 512, 128, 192, (4, 6)),            # dv beyond the fast path
    (cf.F32, 4, 64, 32, 32, (4, 1)),                # fp32 weights
    (cf.F32, 2, 30, 8, 12, (9, 1)),                 # scalar merge (r not a multiple of 4)
])
def test_combine_v_direct_partials(wdt, heads, r, dn, dv, n_splits):
    """The fused merge + value projection on given partials (empty splits with
    NaN partials, one (row, head) with no split at all) against the oracle's
    merge followed by its absorb_v."""
    mla = _mla()
    b = len(n_splits)
    s_max = max(n_splits)
    say(f"combine_v {wdt} heads={heads} r={r} dn={dn} dv={dv} n_splits={n_splits}")
    po = gen.normal_f32(97, 1, (b, heads, s_max, r))
    pl = 3.0 * gen.normal_f32(97, 2, (b, heads, s_max))
    empty = np.random.default_rng(11).random((b, heads, s_max)) < 0.2
    empty[0, 0, :] = True
    pl[empty] = -np.inf
    po_gpu = po.copy()
    po_gpu[empty] = np.nan
    w = cf.store(gen.normal_f32(97, 3, (heads * (dn + dv), r), std=r ** -0.5), wdt)
    o_lat = torch.empty((b, heads, r), dtype=torch.float32, device="cuda")
    ctx = mla.mla_decode_combine_v(dev(po_gpu), dev(pl), list(n_splits), dev(w), dn, dv, o_lat=o_lat)
    torch.cuda.synchronize()
    o_ref, _ = oracle.combine_partials(np.where(empty[..., None], 0.0, po), pl, n_splits)
    ctx_ref = oracle.absorb_v(o_ref, cf.values(w), dn, dv)
    got = host_values(ctx)
    assert not np.isnan(got).any()
    assert np.array_equal(got[0, :dv], np.zeros(dv))   # row 0, head 0: no split, o = 0
    assert_close(host_values(o_lat), o_ref, cf.F32, "fused merge o_lat", tol=1e-5)
    assert_close(got, ctx_ref, cf.F32, "fused ctx", tol=1e-5)


@pytest.mark.parametrize("pdt,rows,heads,dv,max_splits", [
    (cf.F32, 37, 8, 128, 20),    # 16-row blocks with a ragged last block; batches of 8 splits and a tail
    (cf.BF16, 64, 16, 96, 6),    # bf16 partials, dv < 128 (columns past dv idle in the projection)
    (cf.BF16, 16, 4, 128, 1),    # one split per row, the fewest rows that take the many-row kernel
])
def test_combine_v_many_rows(pdt, rows, heads, dv, max_splits):
    """The fused merge + projection of a many-row launch (one workgroup per
    head and 16 rows) against the oracle: empty splits with NaN partials,
    a (row, head) with no split, split counts spanning several batches."""
    mla = _mla()
    r, dn = 512, 128
    n_splits = [int(v) for v in np.random.default_rng(rows).integers(1, max_splits, size=rows, endpoint=True)]
    s_max = max(n_splits)
    say(f"combine_v many rows: {pdt} rows={rows} heads={heads} dv={dv} s_max={s_max}")
    po = gen.normal_f32(96, 1, (rows, heads, s_max, r))
    pl = 3.0 * gen.normal_f32(96, 2, (rows, heads, s_max))
    empty = np.random.default_rng(13).random((rows, heads, s_max)) < 0.2
    empty[0, 0, :] = True
    pl[empty] = -np.inf
    po_store = cf.store(po, pdt)
    po_gpu = dev(po_store)
    po_gpu[torch.from_numpy(empty).to(po_gpu.device)] = float("nan")
    w = cf.store(gen.normal_f32(96, 3, (heads * (dn + dv), r), std=r ** -0.5), cf.BF16)
    o_lat = torch.empty((rows, heads, r), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    ctx = mla.mla_decode_combine_v(po_gpu, dev(pl), n_splits, dev(w), dn, dv, o_lat=o_lat, lse=lse)
    o_sep, lse_sep = mla.mla_decode_combine(po_gpu, dev(pl), n_splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.combine_partials(np.where(empty[..., None], 0.0, cf.values(po_store)), pl, n_splits)
    ctx_ref = oracle.absorb_v(o_ref, cf.values(w), dn, dv)
    got = host_values(ctx)
    assert not np.isnan(got).any()
    assert np.array_equal(got[0, :dv], np.zeros(dv))   # row 0, head 0: no split, o = 0
    assert_close(host_values(o_lat), o_ref, cf.F32, "many-row merge o_lat", tol=1e-5)
    assert_close(host_values(o_lat), host_values(o_sep), cf.F32, "many-row merge vs combine", tol=1e-6)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(host_values(lse)), fin)
    assert np.allclose(host_values(lse)[fin], lse_ref[fin], rtol=0, atol=1e-5)
    assert_close(got, ctx_ref, cf.F32, "many-row ctx", tol=1e-5)


def test_stream_probe_runs_and_writes_nothing():
    """The attention's streaming probe reads the ragged rows' cache and leaves it as it was."""
    mla = _mla()
    inp = cf.decode_inputs(cf.RAGGED_BF16, lengths=(700, 1, 333, 64))
    cache = dev(np.concatenate([inp.latent, inp.rope], axis=-1))
    before = cache.clone()
    c = cf.RAGGED_BF16
    mla.mla_decode_stream_probe(cache[..., :c.kv_lora_rank], cache[..., c.kv_lora_rank:], inp.kv_len, 64)
    torch.cuda.synchronize()
    assert torch.equal(cache.view(torch.int16), before.view(torch.int16))
