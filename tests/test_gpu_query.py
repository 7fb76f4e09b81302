"""GPU parity of the fused decode query (mla_decode_query: absorb_q of the
no-PE part and RoPE of the rope part in one call) against the two separate
entries, bit for bit, and against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf
from synth import generators as gen
from tests.gpu_util import TOL, assert_close, bitwise_equal, dev, host_values, say

pytestmark = pytest.mark.gpu

ROPE_TOL = {cf.F32: 1e-6, cf.BF16: 8e-3}   # one rounding of each rotated value to the storage type


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


def _case(cfg, batch, layer, packed):
    """q_nope, q_rope (device views) of seeded queries, the kv_b weight, positions."""
    c = cfg
    inp = cf.decode_inputs(c, layer=layer, lengths=[3] * batch)
    rng = np.random.default_rng(layer)
    pos = [int(v) for v in rng.integers(0, 1 << 20, size=batch)]
    pos[0] = 0
    if packed:   # the page's query layout: [B, H, dn + dr], split into views
        q = dev(np.concatenate([inp.q_nope, inp.q_rope_raw], axis=-1))
        q_nope, q_rope = q[..., : c.qk_nope], q[..., c.qk_nope:]
    else:
        q_nope, q_rope = dev(inp.q_nope), dev(inp.q_rope_raw)
    return inp, q_nope, q_rope, dev(inp.w_kvb), pos


@pytest.mark.parametrize("cfg,batch,packed,in_place", [
    (cf.RAGGED_BF16, 8, False, False),     # one launch (MFMA absorb)
    (cf.RAGGED_BF16, 8, True, True),       # strided views of one query tensor, rotated in place
    (cf.DENSE_BF16, 130, False, False),    # more rows than one launch carries
    (cf.TINY_F32, 3, True, False),         # fp32: the two kernels in order
])
def test_decode_query_matches_entries_and_oracle(cfg, batch, packed, in_place):
    mla = _mla()
    c = cfg
    say(f"decode_query {c.name} B={batch} packed={packed} in_place={in_place}")
    inp, q_nope, q_rope, w, pos = _case(c, batch, 40 + batch, packed)
    rope_in = q_rope.clone()
    out = q_rope if in_place else None
    q_lat, q_rot = mla.mla_decode_query(q_nope, q_rope, w, c.v_head, pos, c.theta, q_rope_out=out)
    # the separate entries on the same inputs
    ref_lat = mla.mla_absorb_q(q_nope, w, c.v_head)
    ref_rot = mla.mla_rope_partial_interleaved(rope_in.view(batch, 1, c.heads, c.qk_rope), pos, c.qk_rope, c.theta)
    torch.cuda.synchronize()
    assert bitwise_equal(q_lat, ref_lat), "q_lat differs from mla_absorb_q"
    assert bitwise_equal(q_rot, ref_rot.view(batch, c.heads, c.qk_rope)), "q_rope differs from the RoPE entry"
    if in_place:
        assert q_rot.data_ptr() == q_rope.data_ptr()
    # the oracle
    lat = oracle.absorb_q(cf.values(inp.q_nope), cf.values(inp.w_kvb), c.qk_nope, c.v_head)
    assert_close(host_values(q_lat), lat, c.dtype, "q_lat")
    rot = oracle.rope_partial_interleaved(cf.values(inp.q_rope_raw)[:, None], pos, c.qk_rope, c.theta)[:, 0]
    assert_close(host_values(q_rot), rot, c.dtype, "rotated q_rope", tol=ROPE_TOL[c.dtype])


def test_decode_query_empty_batch_and_errors():
    mla = _mla()
    c = cf.RAGGED_BF16
    z = torch.empty((0, c.heads, c.qk_nope), dtype=torch.bfloat16, device="cuda")
    zr = torch.empty((0, c.heads, c.qk_rope), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((c.heads * (c.qk_nope + c.v_head), c.kv_lora_rank), dtype=torch.bfloat16, device="cuda")
    q_lat, q_rot = mla.mla_decode_query(z, zr, w, c.v_head, [], c.theta)
    assert q_lat.shape == (0, c.heads, c.kv_lora_rank) and q_rot.shape == zr.shape
    q = torch.zeros((1, c.heads, c.qk_nope), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((1, c.heads, c.qk_rope), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError):
        mla.mla_decode_query(q, qr, w, c.v_head, [-1], c.theta)
    with pytest.raises(ValueError):
        mla.mla_decode_query(q, qr, w, c.v_head, [1, 2], c.theta)
