"""Pins of the oracle's reconstructed causal prefill.

Page "mlx-bun 0.0.11 -> 0.0.13", glm52-mla.ts: project (q_b_proj, split, RoPE)
and attendReconstructed (kv_b_proj expansion, causal mask with last visible key
prefix + t); page "mlx-bun 0.2.0 -> 0.4.0", glm52-mla.ts: left-padding mask.
"""

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_q_split_hand_example.json")


def _val(v):
    """A number of the golden file: a float, or "lnX" for the natural log of X."""
    if isinstance(v, str):
        assert v.startswith("ln"), v
        return math.log(float(v[2:]))
    return float(v)


def _vals(x):
    return np.array([_vals(v) for v in x]) if isinstance(x, list) else _val(x)


def test_query_split_hand_example():
    """Head-major view of the q_b projection, no-PE part first, rope part last,
    RoPE at position 0 = the de-interleave; then the causal softmax over two keys."""
    g = json.load(open(GOLDEN))
    h, dn, dr, dv = g["heads"], g["qk_nope"], g["qk_rope"], g["v_head"]
    c_q = _vals(g["c_q"])[None, None]                    # [1, 1, ql]
    w_qb = _vals(g["w_qb"])                              # [H (dn+dr), ql]
    q_nope, q_rope = oracle.prefill_queries(c_q, w_qb, [g["q_offset"]], g["theta"], h, dn, dr)
    assert np.array_equal(q_nope[0, 0], _vals(g["expected_q_nope"]))
    assert np.array_equal(q_rope[0, 0], _vals(g["expected_q_rope"]))
    latent = _vals(g["latent"])[None]                    # [1, K=2, r]
    rope = _vals(g["rope"])[None]                        # [1, 2, dr]
    ctx = oracle.prefill_reconstructed(c_q, w_qb, latent, rope, _vals(g["kv_b"]), [g["q_offset"]], g["theta"], None,
                                       g["scale"], h, dn, dr, dv)
    np.testing.assert_allclose(ctx[0, 0], _vals(g["expected_ctx"]), rtol=1e-14, atol=1e-15)


def _problem(seed, batch=1, tokens=6, keys=6, heads=3, ql=7, dn=4, dr=4, dv=5, r=6, theta=10000.0):
    rng = np.random.default_rng(seed)
    return dict(
        c_q=rng.standard_normal((batch, tokens, ql)),
        w_qb=rng.standard_normal((heads * (dn + dr), ql)) / math.sqrt(ql),
        latent=rng.standard_normal((batch, keys, r)),
        rope=rng.standard_normal((batch, keys, dr)),
        w_kvb=rng.standard_normal((heads * (dn + dv), r)) / math.sqrt(r),
        q_offsets=np.full(batch, keys - tokens, dtype=np.int64),
        theta=theta, left_pad=None, scale=1 / math.sqrt(dn + dr), heads=heads, dn=dn, dr=dr, dv=dv,
    )


def _prefill(p, query_rows=None):
    return oracle.prefill_reconstructed(p["c_q"], p["w_qb"], p["latent"], p["rope"], p["w_kvb"], p["q_offsets"],
                                        p["theta"], p["left_pad"], p["scale"], p["heads"], p["dn"], p["dr"], p["dv"],
                                        query_rows=query_rows)


def _queries(p):
    """q_nope, rotated q_rope [B,T,H,*]: the query step the hand example pins."""
    return oracle.prefill_queries(p["c_q"], p["w_qb"], p["q_offsets"], p["theta"], p["heads"], p["dn"], p["dr"])


def test_query_step_rope_matches_rope_entry():
    """The queries' rope part equals the RoPE entry applied to the projected rope features."""
    p = _problem(6, batch=2, tokens=3, keys=5)
    _, q_rope = _queries(p)
    b, t, _ = p["c_q"].shape
    raw = (p["c_q"] @ p["w_qb"].T).reshape(b, t, p["heads"], p["dn"] + p["dr"])[..., p["dn"]:]
    ref = oracle.rope_partial_interleaved(raw, [int(o) for o in p["q_offsets"]], p["dr"], p["theta"])
    assert np.array_equal(q_rope, ref)


def test_matches_torch_sdpa_causal_with_prefix():
    p = _problem(0, batch=2, tokens=5, keys=8)
    ctx = _prefill(p)
    q_nope, q_rope = _queries(p)
    h, dn, dv = p["heads"], p["dn"], p["dv"]
    w = torch.tensor(p["w_kvb"]).reshape(h, dn + dv, -1)
    for b in range(2):
        lat = torch.tensor(p["latent"][b])
        k = torch.cat([torch.einsum("kr,hdr->hkd", lat, w[:, :dn]),
                       torch.tensor(p["rope"][b]).expand(h, 8, p["dr"])], dim=-1)
        v = torch.einsum("kr,hvr->hkv", lat, w[:, dn:])
        q = torch.cat([torch.tensor(q_nope[b]), torch.tensor(q_rope[b])], dim=-1).transpose(0, 1)   # [H,T,dqk]
        prefix = 8 - 5
        mask = torch.arange(8)[None, :] <= (prefix + torch.arange(5))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask,
                                                             scale=p["scale"])
        np.testing.assert_allclose(ctx[b], o[0].transpose(0, 1).reshape(5, -1).numpy(), rtol=1e-12, atol=1e-13)


def test_row_t_equals_decode_over_visible_prefix():
    p = _problem(1, tokens=4, keys=7)
    ctx = _prefill(p)
    q_nope, q_rope = _queries(p)
    for t in range(4):
        n = 7 - 4 + t + 1
        d = oracle.decode_reconstructed(q_nope[:, t], q_rope[:, t], p["latent"][:, :n], p["rope"][:, :n], p["w_kvb"],
                                        np.array([n]), None, p["scale"], p["dn"], p["dv"])
        np.testing.assert_allclose(ctx[0, t], d[0], rtol=1e-12, atol=1e-13)


def test_future_tokens_do_not_leak():
    p = _problem(2, tokens=6, keys=6)
    base = _prefill(p)
    q = dict(p)
    q["latent"] = p["latent"].copy()
    q["rope"] = p["rope"].copy()
    q["c_q"] = p["c_q"].copy()
    q["latent"][:, 4:] += 3.0
    q["rope"][:, 4:] -= 1.0
    q["c_q"][:, 4:] *= -2.0
    out = _prefill(q)
    assert np.array_equal(out[:, :4], base[:, :4])
    assert not np.allclose(out[:, 4:], base[:, 4:])


def test_left_padded_batch_equals_unpadded_rows():
    """Row b with pad[b] masked leading keys equals the unpadded run of its last T - pad[b] tokens.

    Query token pad+j of the padded row sits at position q_offset + pad + j, so the
    unpadded run uses offset q_offset + pad.  Queries inside the pad see no key and
    have no defined output; they are not compared.
    """
    p = _problem(3, batch=2, tokens=5, keys=5)
    pad = [0, 2]
    p["left_pad"] = np.array(pad)
    ctx = _prefill(p)
    for b in range(2):
        q = dict(p)
        q["c_q"] = p["c_q"][b:b + 1, pad[b]:]
        q["latent"] = p["latent"][b:b + 1, pad[b]:]
        q["rope"] = p["rope"][b:b + 1, pad[b]:]
        q["q_offsets"] = np.array([int(p["q_offsets"][b]) + pad[b]])
        q["left_pad"] = None
        np.testing.assert_allclose(ctx[b, pad[b]:], _prefill(q)[0], rtol=1e-12, atol=1e-13)


def test_single_token_prefill_equals_absorbed_decode():
    p = _problem(4, tokens=1, keys=9)
    ctx = _prefill(p)
    q_nope, q_rope = _queries(p)
    d = oracle.decode_absorbed(q_nope[:, 0], q_rope[:, 0], p["latent"], p["rope"], p["w_kvb"], np.array([9]), None,
                               p["scale"], p["dn"], p["dv"])
    np.testing.assert_allclose(ctx[:, 0], d["ctx"], rtol=1e-12, atol=1e-13)


def test_query_subset_equals_full_rows():
    p = _problem(5, batch=2, tokens=7, keys=9)
    full = _prefill(p)
    rows = [0, 3, 6]
    sub = _prefill(p, query_rows=rows)
    np.testing.assert_allclose(sub, full[:, rows], rtol=1e-13, atol=1e-14)
