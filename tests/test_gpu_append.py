"""GPU fused cache append against the oracle, and an appended token feeding
the latent decode attention."""

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf
from synth import generators as gen
from tests.gpu_util import assert_close, bitwise_equal, dev, host_values, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


def _inputs(dtype, batch, tokens, r, dr, layer):
    kv_a = cf.store(gen.normal_f32(20, gen.T_MISC, (batch, tokens, r + dr), layer=layer), dtype)
    w = cf.store(np.float32(1.0) + gen.normal_f32(20, gen.T_MISC, (r,), std=0.1, layer=layer + 1000), dtype)
    return kv_a, w


@pytest.mark.parametrize("dtype,batch,tokens,r,dr", [(cf.F32, 2, 3, 64, 16), (cf.BF16, 3, 1, 512, 64),
                                                     (cf.BF16, 2, 5, 512, 64), (cf.F32, 1, 1, 300, 8)])
def test_append_matches_oracle(dtype, batch, tokens, r, dr):
    say(f"append {dtype} B={batch} T={tokens} r={r} dr={dr}")
    kv_a, w = _inputs(dtype, batch, tokens, r, dr, layer=tokens)
    width, slot = 40, 33
    pos = [100 * (b + 1) + 7 for b in range(batch)]
    cache0 = cf.store(gen.normal_f32(21, gen.T_MISC, (batch, width, r + dr)), dtype)
    cache = dev(cache0)
    _mla().mla_append_compressed(dev(kv_a), dev(w), EPS, pos, 10000.0, cache[..., :r], cache[..., r:], slot)
    torch.cuda.synchronize()
    lat, rope = oracle.append_compressed(cf.values(kv_a), cf.values(w), EPS, pos, 10000.0, r, dr)
    got = host_values(cache)
    tol = 1e-5 if dtype == cf.F32 else None
    assert_close(got[:, slot:slot + tokens, :r], lat, dtype, "latent", tol=tol)
    assert_close(got[:, slot:slot + tokens, r:], rope, dtype, "rope", tol=tol)
    untouched = torch.ones(width, dtype=torch.bool)
    untouched[slot:slot + tokens] = False
    assert bitwise_equal(cache[:, untouched], dev(cache0)[:, untouched])


def test_appended_token_is_attended():
    """Append the step's token at slot = width of a right-aligned ragged cache,
    then attend over kv_len + 1 tokens; the oracle appends with its own values."""
    cfg = cf.RAGGED_BF16
    inp = cf.decode_inputs(cfg, layer=9, lengths=(300, 37, 1))
    c = inp.cfg
    b = len(inp.kv_len)
    r, dr = c.kv_lora_rank, c.qk_rope
    kv_a, w = _inputs(cf.BF16, b, 1, r, dr, layer=77)
    width = inp.latent.shape[1]
    cache_h = np.concatenate([inp.latent, inp.rope], axis=-1)
    cache_h = np.concatenate([cache_h, np.zeros((b, 1, r + dr), dtype=cache_h.dtype)], axis=1)
    cache = dev(cache_h)
    lens = [int(n) for n in inp.kv_len]
    mla = _mla()
    mla.mla_append_compressed(dev(kv_a), dev(w), EPS, lens, c.theta, cache[..., :r], cache[..., r:], width)
    new_len = [n + 1 for n in lens]
    q_rope = dev(inp.q_rope_raw)
    view = q_rope.view(b, 1, c.heads, dr)
    mla.mla_rope_partial_interleaved(view, lens, dr, c.theta, out=view)   # q and the new key share a position
    wk = dev(inp.w_kvb)
    q_lat = mla.mla_absorb_q(dev(inp.q_nope), wk, c.v_head)
    po, pl, ns = mla.mla_decode_latent_attn(q_lat, q_rope, cache[..., :r], cache[..., r:], new_len, c.softmax_scale, 64)
    o_lat, _ = mla.mla_decode_combine(po, pl, ns)
    ctx = mla.mla_absorb_v(o_lat, wk, c.qk_nope, c.v_head)
    torch.cuda.synchronize()
    lat_new, rope_new = oracle.append_compressed(cf.values(kv_a), cf.values(w), EPS, lens, c.theta, r, dr)
    lat_all = np.concatenate([cf.values(inp.latent), lat_new], axis=1)
    rope_all = np.concatenate([cf.values(inp.rope), rope_new], axis=1)
    qr = oracle.rope_partial_interleaved(cf.values(inp.q_rope_raw)[:, None], lens, dr, c.theta)[:, 0]
    ref = oracle.decode_reconstructed(cf.values(inp.q_nope), qr, lat_all, rope_all, cf.values(inp.w_kvb), new_len,
                                      None, c.softmax_scale, c.qk_nope, c.v_head)
    assert_close(host_values(ctx), ref, c.dtype, "ctx with the appended token")
