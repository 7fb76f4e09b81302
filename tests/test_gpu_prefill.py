"""GPU parity of mla_prefill_reconstructed against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf
from tests.gpu_util import assert_close, bitwise_equal, dev, host_values, say

pytestmark = pytest.mark.gpu

SMALL_F32 = cf.PrefillConfig("prefill_small_f32", 6, cf.F32, 2, 96, 120, 4, 64, 32, 16, 32, 64)
SMALL_BF16 = cf.PrefillConfig("prefill_small_bf16", 7, cf.BF16, 2, 200, 200, 3, 128, 128, 64, 128, 512)


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


def _gpu(inp: cf.PrefillInputs, left_pad=None, scale=None):
    """Rotate the raw rope keys at positions 0..K-1 on the GPU, then prefill."""
    c = inp.cfg
    mla = _mla()
    rope = dev(inp.k_rope_raw)
    mla.mla_rope_partial_interleaved(rope, 0, c.qk_rope, c.theta, out=rope)
    ctx = mla.mla_prefill_reconstructed(dev(inp.c_q), dev(inp.w_qb), dev(inp.latent), rope, dev(inp.w_kvb), c.heads,
                                        c.qk_nope, c.qk_rope, c.v_head, [int(o) for o in inp.q_offsets], c.theta,
                                        c.softmax_scale if scale is None else scale, left_pad=left_pad)
    torch.cuda.synchronize()
    return ctx


def _oracle(inp: cf.PrefillInputs, rows=None, left_pad=None, scale=None):
    c = inp.cfg
    rope = oracle.rope_partial_interleaved(cf.values(inp.k_rope_raw), 0, c.qk_rope, c.theta)
    return oracle.prefill_reconstructed(cf.values(inp.c_q), cf.values(inp.w_qb), cf.values(inp.latent), rope,
                                        cf.values(inp.w_kvb), inp.q_offsets, c.theta, left_pad,
                                        c.softmax_scale if scale is None else scale, c.heads, c.qk_nope, c.qk_rope,
                                        c.v_head, query_rows=rows)


@pytest.mark.parametrize("cfg,tokens,keys", [(SMALL_F32, 96, 120), (SMALL_F32, 1, 7), (SMALL_BF16, 200, 200),
                                             (SMALL_BF16, 130, 300)])
def test_prefill_small_matches_oracle(cfg, tokens, keys):
    say(f"prefill {cfg.name} T={tokens} K={keys}")
    inp = cf.prefill_inputs(cfg, tokens=tokens, keys=keys)
    got = _gpu(inp)
    assert_close(host_values(got), _oracle(inp), cfg.dtype, "ctx")


@pytest.mark.parametrize("scale", [-0.0721, 0.0])
def test_prefill_nonpositive_scale_matches_oracle(scale):
    """The kernel takes the softmax max from the raw scores (their min for a
    negative scale); a negative or zero scale is still a valid softmax."""
    say(f"prefill scale {scale}")
    inp = cf.prefill_inputs(SMALL_BF16, tokens=130, keys=300)
    pads = [0, 45]
    got = host_values(_gpu(inp, left_pad=pads, scale=scale))
    ref = _oracle(inp, left_pad=np.array(pads), scale=scale)
    assert_close(got[0], ref[0], cf.BF16, "row 0")
    assert_close(got[1, 45:], ref[1, 45:], cf.BF16, "row 1 past its pad")


def test_prefill_left_pad_matches_oracle():
    inp = cf.prefill_inputs(SMALL_BF16, tokens=150, keys=150)
    pads = [0, 37]
    got = host_values(_gpu(inp, left_pad=pads))
    ref = _oracle(inp, left_pad=np.array(pads))
    assert_close(got[0], ref[0], cf.BF16, "row 0")
    assert_close(got[1, 37:], ref[1, 37:], cf.BF16, "row 1 past its pad")
    assert not got[1, :37].any(), "queries inside the pad see no key and are defined as zero"


def test_prefill_future_tokens_do_not_leak_bitwise():
    inp = cf.prefill_inputs(SMALL_BF16, tokens=200, keys=200)
    base = _gpu(inp)
    lat = inp.latent.copy()
    lat[:, 150:] ^= np.uint16(0x0041)
    cq = inp.c_q.copy()
    cq[:, 150:] ^= np.uint16(0x0103)
    inp.latent, inp.c_q = lat, cq
    pert = _gpu(inp)
    assert bitwise_equal(base[:, :150], pert[:, :150])
    assert not torch.equal(base[:, 150:], pert[:, 150:])


def test_prefill_full_size_sampled_rows():
    """The 4096-token workload at full size; the oracle computes sampled query rows."""
    cfg = cf.PREFILL_BF16
    say("prefill full: generating")
    inp = cf.prefill_inputs(cfg)
    say("prefill full: gpu")
    got = host_values(_gpu(inp))
    rows = [0, 1, 2, 63, 64, 127, 128, 1000, 2047, 2048, 3071, 4094, 4095]
    say("prefill full: oracle")
    ref = _oracle(inp, rows=rows)
    assert_close(got[:, rows], ref, cfg.dtype, "ctx sampled rows")


def test_prefill_long_ragged_tiles_sampled_rows():
    """2200 tokens: the projections run on 256 x 256 GEMM tiles with a partial
    last row tile (2200 = 8 x 256 + 152); sampled rows against the oracle."""
    cfg = cf.PREFILL_BF16
    inp = cf.prefill_inputs(cfg, tokens=2200, keys=2200)
    got = host_values(_gpu(inp))
    rows = [0, 151, 152, 255, 256, 1500, 2047, 2048, 2199]
    assert_close(got[:, rows], _oracle(inp, rows=rows), cfg.dtype, "ctx sampled rows")
