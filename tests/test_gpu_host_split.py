"""GPU parity of the batches the host splits into several launches: the
attention's row tables hold 128 rows per launch (the selection offsets carry
across launches), the merge's 256 rows per launch.  Page "mlx-bun 0.0.11 ->
0.0.13", glm52-mla.ts, Glm52Mla.forward loops over rows; every row of a split
batch must equal the oracle and the same row in a call of its own."""

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf
from synth import generators as gen
from tests.gpu_util import assert_close, bitwise_equal, dev, host_values, say

pytestmark = pytest.mark.gpu

CFG = cf.RAGGED_BF16
SEED = 41


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


def _rows_problem(rows=130, width=200):
    """Ragged rows, every third one (b % 3 == 1) attending a sorted selection of
    its valid slice; pad slots hold NaN."""
    c = CFG
    lens = gen.rng_for(SEED, gen.T_LENGTHS).integers(1, width, size=rows, endpoint=True).astype(np.int32)
    lat = gen.normal_f32(SEED, gen.T_LATENT, (rows, width, c.kv_lora_rank))
    rope = gen.normal_f32(SEED, gen.T_ROPE, (rows, width, c.qk_rope))
    for b in range(rows):
        lat[b, : width - lens[b]] = np.nan
        rope[b, : width - lens[b]] = np.nan
    ql = cf.store(gen.normal_f32(SEED, gen.T_MISC, (rows, c.heads, c.kv_lora_rank), layer=1), cf.BF16)
    qr = cf.store(gen.normal_f32(SEED, gen.T_MISC, (rows, c.heads, c.qk_rope), layer=2), cf.BF16)
    g = gen.rng_for(SEED, gen.T_SELECTION)
    counts, sels = [], []
    for b in range(rows):
        if b % 3 == 1:
            k = int(g.integers(1, lens[b], endpoint=True))
            sels.append(np.sort(g.choice(int(lens[b]), size=k, replace=False)).astype(np.int32))
            counts.append(k)
        else:
            sels.append(None)
            counts.append(-1)
    sel_idx = np.concatenate([s for s in sels if s is not None]).astype(np.int32)
    return dict(lens=lens, lat=cf.store(lat, cf.BF16), rope=cf.store(rope, cf.BF16), ql=ql, qr=qr, counts=counts,
                sels=sels, sel_idx=sel_idx)


def test_attention_130_rows_mixed_selection():
    """130 rows = launches of 128 and 2 rows; selected rows on both sides of the
    boundary, so the second launch starts inside the concatenated index list."""
    mla = _mla()
    p = _rows_problem()
    rows = len(p["lens"])
    chunk = 64
    say(f"attention {rows} rows, {sum(c > 0 for c in p['counts'])} selected, chunk {chunk}")
    cache = dev(np.concatenate([p["lat"], p["rope"]], axis=-1))
    lat, rope = cache[..., :CFG.kv_lora_rank], cache[..., CFG.kv_lora_rank:]
    ql, qr, sel = dev(p["ql"]), dev(p["qr"]), dev(p["sel_idx"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens = [int(v) for v in p["lens"]]
    po, pl, ns = mla.mla_decode_latent_attn(ql, qr, lat, rope, lens, CFG.softmax_scale, chunk, sel_idx=sel,
                                            sel_count=p["counts"], dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_o, ref_l, ref_ns = oracle.latent_attention_partials(cf.values(p["ql"]), cf.values(p["qr"]),
                                                            cf.values(p["lat"]), cf.values(p["rope"]), p["lens"],
                                                            p["sels"], CFG.softmax_scale, chunk)
    assert list(ref_ns) == ns
    gpo, gpl = host_values(po), host_values(pl)
    for b in (0, 1, 2, 100, 126, 127, 128, 129):
        n = ns[b]
        assert_close(gpo[b, :, :n], ref_o[b, :, :n], cf.BF16, f"part_o row {b}")
        assert_close(gpl[b, :, :n], ref_l[b, :, :n], cf.BF16, f"part_lse row {b}")
    o_all, _ = oracle.combine_partials(ref_o, ref_l, ref_ns)
    o_gpu, _ = mla.mla_decode_combine(po, pl, ns)
    assert_close(host_values(o_gpu), o_all, cf.BF16, "merged o_lat, all rows")
    # the rows of the second launch, in a call of their own: bitwise equal
    off = sum(c for c in p["counts"][:128] if c > 0)
    po2, pl2, _ = mla.mla_decode_latent_attn(ql[128:], qr[128:], lat[128:], rope[128:], lens[128:],
                                             CFG.softmax_scale, chunk, sel_idx=sel[off:], sel_count=p["counts"][128:],
                                             s_max=po.shape[2])
    torch.cuda.synchronize()
    for j, b in enumerate((128, 129)):
        n = ns[b]
        assert bitwise_equal(po2[j, :, :n], po[b, :, :n]) and bitwise_equal(pl2[j, :, :n], pl[b, :, :n])


def test_merge_260_rows():
    """mla_decode_combine and mla_decode_combine_v over 260 rows (launches of
    256 and 4 rows) against the oracle's merge and absorb_v; the last rows
    also against a call of their own (bitwise)."""
    mla = _mla()
    rows, heads, r, dn, dv = 260, 8, 512, 128, 128
    n_splits = [int(v) for v in gen.rng_for(SEED, gen.T_LENGTHS, layer=3).integers(1, 6, size=rows, endpoint=True)]
    s_max = max(n_splits)
    say(f"merge {rows} rows, s_max {s_max}")
    po = gen.normal_f32(SEED, gen.T_MISC, (rows, heads, s_max, r), layer=4)
    pl = 2.0 * gen.normal_f32(SEED, gen.T_MISC, (rows, heads, s_max), layer=5)
    for b in range(rows):
        pl[b, :, n_splits[b]:] = np.nan          # slots past a row's splits are never read
        po[b, :, n_splits[b]:] = np.nan
    w = cf.store(gen.normal_f32(SEED, gen.T_W_KVB, (heads * (dn + dv), r), std=r ** -0.5), cf.BF16)
    po_d, pl_d, w_d = dev(po), dev(pl), dev(w)
    o_lat, lse = mla.mla_decode_combine(po_d, pl_d, n_splits)
    ctx = mla.mla_decode_combine_v(po_d, pl_d, n_splits, w_d, dn, dv)
    torch.cuda.synchronize()
    po_ref = np.where(np.isnan(po), 0.0, po)
    pl_ref = np.where(np.isnan(pl), -np.inf, pl)
    o_ref, lse_ref = oracle.combine_partials(po_ref, pl_ref, n_splits)
    ctx_ref = oracle.absorb_v(o_ref, cf.values(w), dn, dv)
    assert_close(host_values(o_lat), o_ref, cf.F32, "o_lat", tol=1e-5)
    assert np.allclose(host_values(lse), lse_ref, rtol=0, atol=1e-5)
    assert_close(host_values(ctx), ctx_ref, cf.F32, "ctx", tol=1e-5)
    o2, l2 = mla.mla_decode_combine(po_d[256:], pl_d[256:], n_splits[256:])
    c2 = mla.mla_decode_combine_v(po_d[256:], pl_d[256:], n_splits[256:], w_d, dn, dv)
    torch.cuda.synchronize()
    assert bitwise_equal(o2, o_lat[256:]) and bitwise_equal(l2, lse[256:]) and bitwise_equal(c2, ctx[256:])
