"""GPU DSA top-k selection against the oracle (bit-exact: the output is
integer positions), and the selection feeding the latent attention."""

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf
from synth import generators as gen
from tests.gpu_util import assert_close, dev, host_values, say

pytestmark = pytest.mark.gpu


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


def _scores(n, layer, kind="normal"):
    s = gen.normal_f32(cf.DSA_BF16.config_id, gen.T_DSA_SCORES, (n,), layer=layer)
    if kind == "coarse":        # few distinct values: long runs of ties at the threshold
        s = np.round(s * 2.0).astype(np.float32) / np.float32(2.0)
    elif kind == "equal":
        s = np.full(n, 0.25, dtype=np.float32)
    elif kind == "zeros":       # +0, -0 and negatives: the threshold sits at zero
        s = np.where(s > 0.5, np.float32(0.0), np.where(s > -0.5, np.float32(-0.0), s)).astype(np.float32)
    elif kind == "negative":
        s = -np.abs(s) - np.float32(1.0)
    elif kind == "fine":        # a 1/1024 grid: short tie runs inside one score bucket
        s = np.round(s * 1024.0).astype(np.float32) / np.float32(1024.0)
    elif kind == "signed_zero_mix":   # normal scores with +0 / -0 pairs near the threshold of a 2048-of-131072 row
        s = s.copy()
        s[::97] = np.float32(2.0)
        s[1::97] = np.float32(0.0)
        s[2::97] = np.float32(-0.0)
    return np.ascontiguousarray(s, dtype=np.float32)


@pytest.mark.parametrize("two_stage", [True, False], ids=["two_stage", "one_workgroup"])
@pytest.mark.parametrize("n,k,kind", [
    (5000, 300, "normal"), (2049, 2048, "normal"), (1025, 1024, "coarse"), (10000, 1000, "coarse"),
    (3000, 64, "equal"), (4000, 700, "zeros"), (4000, 2000, "zeros"), (3333, 17, "negative"), (1, 1, "normal"),
    (131072, 2048, "normal"), (131072, 2048, "coarse"),
    # two-stage boundaries: a 1-score last segment, three segments of 5000
    # candidates, all ties, zeros and long tie runs across segment ends
    (16385, 64, "normal"), (40000, 5000, "coarse"), (131072, 2048, "equal"), (131072, 2048, "zeros"),
    (65543, 2048, "coarse"), (131072, 2048, "negative"),
    # the score-bucket select: ties inside the bucket, +-0 and a tie run at the threshold
    (131072, 2048, "fine"), (50000, 3000, "fine"), (131072, 2048, "signed_zero_mix"), (20000, 9000, "normal"),
])
def test_topk_matches_oracle_bitwise(n, k, kind, two_stage):
    say(f"dsa topk n={n} k={k} {kind} two_stage={two_stage}")
    s = _scores(n, layer=n % 97 + k, kind=kind)
    got, counts = _mla().mla_dsa_topk_select(dev(s).view(1, -1), [n], k, two_stage=two_stage)
    torch.cuda.synchronize()
    ref = oracle.dsa_select(s, k)
    if ref is None:
        assert counts == [-1] and got.numel() == 0
    else:
        assert counts == [k]
        assert got.cpu().numpy().tolist() == ref.tolist()


def test_topk_rows_mix_both_forms():
    """Rows taking the two-stage form and rows on one workgroup in one call."""
    lens = [131072, 5000, 20000, 100, 98304]
    k = 2048
    w = max(lens)
    s = np.zeros((len(lens), w), dtype=np.float32)
    for b, n in enumerate(lens):
        s[b, :n] = _scores(n, layer=400 + b, kind="coarse" if b % 2 else "normal")
    assert _mla().dsa_topk_workspace_bytes(lens, k) == 3 * 131328
    got, counts = _mla().mla_dsa_topk_select(dev(s), lens, k)
    torch.cuda.synchronize()
    ref_idx, ref_cnt = oracle.dsa_select_rows(s, lens, k)
    assert counts == ref_cnt.tolist()
    assert got.cpu().numpy().tolist() == ref_idx.tolist()


def test_topk_rows_concatenate_with_dense_rows():
    lens = [5000, 100, 3000, 64, 2048, 65]
    k = 64
    w = max(lens)
    s = np.zeros((len(lens), w), dtype=np.float32)
    for b, n in enumerate(lens):
        s[b, :n] = _scores(n, layer=200 + b, kind="coarse" if b % 2 else "normal")
    got, counts = _mla().mla_dsa_topk_select(dev(s), lens, k)
    torch.cuda.synchronize()
    ref_idx, ref_cnt = oracle.dsa_select_rows(s, lens, k)
    assert counts == ref_cnt.tolist()
    assert got.cpu().numpy().tolist() == ref_idx.tolist()


def test_selection_feeds_latent_attention():
    """Scores -> GPU selection -> latent attention over the selected tokens,
    against the oracle's reconstructed decode with the oracle's selection."""
    cfg = cf.with_shape(cf.DSA_BF16, tokens=8192, selected=None)
    inp = cf.decode_inputs(cfg, layer=3)
    n, k = int(inp.kv_len[0]), 512
    s = _scores(n, layer=300)
    mla = _mla()
    sel, counts = mla.mla_dsa_topk_select(dev(s).view(1, -1), [n], k)
    c = inp.cfg
    cache = dev(np.concatenate([inp.latent, inp.rope], axis=-1))
    q_rope = dev(inp.q_rope_raw)
    view = q_rope.view(1, 1, c.heads, c.qk_rope)
    mla.mla_rope_partial_interleaved(view, [int(o) for o in inp.offsets], c.qk_rope, c.theta, out=view)
    w = dev(inp.w_kvb)
    q_lat = mla.mla_absorb_q(dev(inp.q_nope), w, c.v_head)
    po, pl, ns = mla.mla_decode_latent_attn(q_lat, q_rope, cache[..., :512], cache[..., 512:], inp.kv_len,
                                            c.softmax_scale, 128, sel_idx=sel, sel_count=counts)
    o_lat, _ = mla.mla_decode_combine(po, pl, ns)
    ctx = mla.mla_absorb_v(o_lat, w, c.qk_nope, c.v_head)
    torch.cuda.synchronize()
    ref_sel = oracle.dsa_select(s, k)
    qr = oracle.rope_partial_interleaved(cf.values(inp.q_rope_raw)[:, None], [int(o) for o in inp.offsets],
                                         c.qk_rope, c.theta)[:, 0]
    ref = oracle.decode_reconstructed(cf.values(inp.q_nope), qr, cf.values(inp.latent), cf.values(inp.rope),
                                      cf.values(inp.w_kvb), inp.kv_len, [ref_sel], c.softmax_scale, c.qk_nope,
                                      c.v_head)
    assert_close(host_values(ctx), ref, c.dtype, "ctx over the GPU selection")
