"""Pins of the oracle's decode path (absorb, latent attention, split/combine).

Pages "mlx-bun 0.0.11 -> 0.0.13" (glm52-mla.ts: attendAbsorbed,
attendReconstructed, forward) and "mlx-bun 0.2.0 -> 0.4.0" (glm52-cache.ts:
right-aligned rows).  Each pin is a closed form, a hand-worked example, an
independent library routine (torch SDPA, scipy logsumexp) or the identity the
method rests on (absorbed == reconstructed).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import OracleError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse(v):
    if isinstance(v, str):
        if v.startswith("ln"):
            return math.log(float(v[2:]))
        if "/" in v:
            a, b = v.split("/")
            return float(a) / float(b)
    return float(v)


def _arr(x):
    return np.array([[_parse(v) for v in row] for row in x]) if isinstance(x[0], list) else np.array([_parse(v) for v in x])


def _random_problem(seed, batch=2, heads=3, dn=5, dv=4, r=6, dr=4, width=11, lengths=None):
    rng = np.random.default_rng(seed)
    lengths = np.array(lengths if lengths is not None else [width] * batch, dtype=np.int32)
    q_nope = rng.standard_normal((batch, heads, dn))
    q_rope = rng.standard_normal((batch, heads, dr))
    latent = rng.standard_normal((batch, width, r))
    rope = rng.standard_normal((batch, width, dr))
    for b in range(batch):            # pad slots are never read
        latent[b, : width - lengths[b]] = np.nan
        rope[b, : width - lengths[b]] = np.nan
    w_kvb = rng.standard_normal((heads * (dn + dv), r)) / math.sqrt(r)
    return dict(q_nope=q_nope, q_rope=q_rope, latent=latent, rope=rope, w_kvb=w_kvb, kv_len=lengths,
                scale=1 / math.sqrt(dn + dr), dn=dn, dv=dv)


def _decode(p, selections=None, form="absorbed"):
    args = (p["q_nope"], p["q_rope"], p["latent"], p["rope"], p["w_kvb"], p["kv_len"], selections, p["scale"],
            p["dn"], p["dv"])
    if form == "absorbed":
        return oracle.decode_absorbed(*args)
    return oracle.decode_reconstructed(*args)


# ---------------------------------------------------------------- absorb

def test_kv_b_layout_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "decode_hand_example.json")))
    latent = _arr(g["latent"])[None]          # [1, 2, 1]
    rope = _arr(g["rope"])[None]              # [1, 2, 2]
    w = _arr(g["kv_b"])                       # [4, 1]
    q_nope = _arr(g["q_nope"])[None]          # [1, 2, 1]
    q_rope = _arr(g["q_rope"])[None]          # [1, 2, 2]
    kv_len = np.array([2])
    out = oracle.decode_absorbed(q_nope, q_rope, latent, rope, w, kv_len, None, g["scale"], 1, 1)
    np.testing.assert_allclose(out["o_lat"][0, :, 0], [_parse(v) for v in g["expected_o_lat"]], rtol=1e-14)
    np.testing.assert_allclose(out["ctx"][0], [_parse(v) for v in g["expected_ctx"]], rtol=1e-14)
    np.testing.assert_allclose(out["lse"][0], [_parse(v) for v in g["expected_lse"]], rtol=1e-14)
    rec = oracle.decode_reconstructed(q_nope, q_rope, latent, rope, w, kv_len, None, g["scale"], 1, 1)
    np.testing.assert_allclose(rec[0], [_parse(v) for v in g["expected_ctx"]], rtol=1e-14)


def test_absorb_q_unit_query_selects_w_uk_row():
    heads, dn, dv, r = 3, 4, 2, 5
    rng = np.random.default_rng(10)
    w = rng.standard_normal((heads * (dn + dv), r))
    for h in range(heads):
        for i in range(dn):
            q = np.zeros((1, heads, dn))
            q[0, h, i] = 1.0
            out = oracle.absorb_q(q, w, dn, dv)
            assert np.array_equal(out[0, h], w[h * (dn + dv) + i])
            others = [x for x in range(heads) if x != h]
            assert not out[0, others].any()


def test_absorb_brute_force_loops():
    heads, dn, dv, r, batch = 2, 3, 2, 4, 2
    rng = np.random.default_rng(11)
    w = rng.standard_normal((heads * (dn + dv), r))
    q = rng.standard_normal((batch, heads, dn))
    o = rng.standard_normal((batch, heads, r))
    ql = oracle.absorb_q(q, w, dn, dv)
    ctx = oracle.absorb_v(o, w, dn, dv)
    for b in range(batch):
        for h in range(heads):
            base = h * (dn + dv)
            for c in range(r):
                acc = 0.0
                for d in range(dn):
                    acc += q[b, h, d] * w[base + d, c]
                assert abs(ql[b, h, c] - acc) < 1e-13
            for v in range(dv):
                acc = 0.0
                for c in range(r):
                    acc += o[b, h, c] * w[base + dn + v, c]
                assert abs(ctx[b, h * dv + v] - acc) < 1e-13


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("seed,lengths", [(0, None), (1, [11, 3]), (2, [1, 7])])
def test_absorbed_equals_reconstructed(seed, lengths):
    p = _random_problem(seed, lengths=lengths)
    a = _decode(p)["ctx"]
    r = _decode(p, form="reconstructed")
    np.testing.assert_allclose(a, r, rtol=1e-12, atol=1e-13)
    assert np.all(np.isfinite(a))


def test_reconstructed_matches_torch_sdpa():
    p = _random_problem(3, batch=2, heads=4, dn=8, dv=6, r=10, dr=4, width=9, lengths=[9, 5])
    ctx = _decode(p, form="reconstructed")
    heads, dn, dv = 4, 8, 6
    w = torch.tensor(p["w_kvb"]).reshape(heads, dn + dv, -1)
    for b in range(2):
        n = int(p["kv_len"][b])
        c = torch.tensor(p["latent"][b, -n:])
        rho = torch.tensor(p["rope"][b, -n:])
        k_nope = torch.einsum("nr,hdr->hnd", c, w[:, :dn])
        v = torch.einsum("nr,hvr->hnv", c, w[:, dn:])
        k = torch.cat([k_nope, rho.expand(heads, n, rho.shape[-1])], dim=-1)
        q = torch.cat([torch.tensor(p["q_nope"][b]), torch.tensor(p["q_rope"][b])], dim=-1)[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], scale=p["scale"])
        np.testing.assert_allclose(ctx[b], o[0, :, 0].reshape(-1).numpy(), rtol=1e-12, atol=1e-13)


def test_single_token_returns_it():
    p = _random_problem(4, lengths=[1, 1])
    out = _decode(p)
    for b in range(2):
        c0 = p["latent"][b, -1]
        assert np.array_equal(out["o_lat"][b], np.broadcast_to(c0, out["o_lat"][b].shape))
        _, w_uv = oracle.split_kv_b(p["w_kvb"], 3, p["dn"], p["dv"])
        np.testing.assert_allclose(out["ctx"][b], (w_uv @ c0).reshape(-1), rtol=1e-13)


def test_zero_query_is_uniform_mean():
    p = _random_problem(5, lengths=[11, 4])
    p["q_nope"][:] = 0
    p["q_rope"][:] = 0
    out = _decode(p)
    for b in range(2):
        n = int(p["kv_len"][b])
        mean = p["latent"][b, -n:].mean(axis=0)
        np.testing.assert_allclose(out["o_lat"][b], np.broadcast_to(mean, (3, mean.size)), rtol=1e-13)
        np.testing.assert_allclose(out["lse"][b], math.log(n), rtol=1e-13)


def test_identical_tokens_give_the_token():
    p = _random_problem(6)
    p["latent"][:] = p["latent"][:, :1]
    p["rope"][:] = p["rope"][:, :1]
    out = _decode(p)
    for b in range(2):
        np.testing.assert_allclose(out["o_lat"][b], np.broadcast_to(p["latent"][b, 0], (3, 6)), rtol=1e-13)


def test_rope_term_and_scale_enter_scores():
    """Scores are scale*(q_lat.c + q_rope.rope): checked through lse on one token pair."""
    p = _random_problem(7, batch=1, width=2)
    out = _decode(p)
    q_lat = oracle.absorb_q(p["q_nope"], p["w_kvb"], p["dn"], p["dv"])[0]
    s = p["scale"] * (q_lat @ p["latent"][0].T + p["q_rope"][0] @ p["rope"][0].T)
    np.testing.assert_allclose(out["lse"][0], logsumexp(s, axis=-1), rtol=1e-13)


def test_ragged_rows_equal_separate_rows():
    p = _random_problem(8, batch=3, lengths=[11, 2, 6])
    full = _decode(p)["ctx"]
    for b in range(3):
        n = int(p["kv_len"][b])
        q = {k: (v[b:b + 1] if isinstance(v, np.ndarray) and v.ndim == 3 and k in ("q_nope", "q_rope") else v)
             for k, v in p.items()}
        q["latent"] = p["latent"][b:b + 1, -n:]
        q["rope"] = p["rope"][b:b + 1, -n:]
        q["kv_len"] = np.array([n])
        np.testing.assert_allclose(full[b], _decode(q)["ctx"][0], rtol=1e-13)


# ---------------------------------------------------------------- selection (DSA gather)

def test_selection_of_all_equals_dense_and_compacted_equals_gathered():
    p = _random_problem(9, batch=2, lengths=[11, 8])
    dense = _decode(p)
    sel = [np.arange(11), np.arange(8)]
    assert np.array_equal(_decode(p, sel)["ctx"], dense["ctx"])
    pick = [np.array([0, 3, 4, 10]), np.array([7, 1])]
    gathered = _decode(p, pick)
    for b in range(2):
        n = int(p["kv_len"][b])
        q = dict(p)
        q["q_nope"], q["q_rope"] = p["q_nope"][b:b + 1], p["q_rope"][b:b + 1]
        q["latent"] = p["latent"][b:b + 1, -n:][:, pick[b]]
        q["rope"] = p["rope"][b:b + 1, -n:][:, pick[b]]
        q["kv_len"] = np.array([len(pick[b])])
        np.testing.assert_allclose(gathered["ctx"][b], _decode(q)["ctx"][0], rtol=1e-14, atol=1e-15)


def test_selection_order_invariant_and_duplicates_count_twice():
    p = _random_problem(10, batch=1)
    a = _decode(p, [np.array([1, 5, 9])])["ctx"]
    b = _decode(p, [np.array([9, 1, 5])])["ctx"]
    np.testing.assert_allclose(a, b, rtol=1e-13)
    dup = _decode(p, [np.array([1, 1, 5])])["o_lat"][0]
    q_lat = oracle.absorb_q(p["q_nope"], p["w_kvb"], p["dn"], p["dv"])[0]
    c = p["latent"][0][[1, 5]]
    s = p["scale"] * (q_lat @ c.T + p["q_rope"][0] @ p["rope"][0][[1, 5]].T)
    w = np.exp(s - s.max(axis=1, keepdims=True)) * np.array([2.0, 1.0])
    np.testing.assert_allclose(dup, (w @ c) / w.sum(axis=1, keepdims=True), rtol=1e-13)


@pytest.mark.parametrize("sel", [np.array([], dtype=np.int64), np.array([0, 11]), np.array([-1, 2])])
def test_selection_rejections(sel):
    p = _random_problem(11, batch=1)
    with pytest.raises(OracleError):
        _decode(p, [sel])


def test_row_needs_a_token():
    p = _random_problem(12, batch=1)
    p["kv_len"] = np.array([0])
    with pytest.raises(OracleError):
        _decode(p)


# ---------------------------------------------------------------- split / combine

@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 11, 64])
def test_split_then_combine_equals_single_pass(chunk):
    p = _random_problem(13, batch=2, lengths=[11, 4])
    q_lat = oracle.absorb_q(p["q_nope"], p["w_kvb"], p["dn"], p["dv"])
    o_ref, lse_ref = oracle.latent_attention(q_lat, p["q_rope"], p["latent"], p["rope"], p["kv_len"], None, p["scale"])
    po, pl, ns = oracle.latent_attention_partials(q_lat, p["q_rope"], p["latent"], p["rope"], p["kv_len"], None,
                                                  p["scale"], chunk)
    assert ns.tolist() == [-(-11 // chunk), -(-4 // chunk)]
    o, lse = oracle.combine_partials(po, pl, ns)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)


def test_combine_single_split_is_identity_and_lse_is_logsumexp():
    rng = np.random.default_rng(14)
    po = rng.standard_normal((2, 3, 1, 5))
    pl = rng.standard_normal((2, 3, 1))
    o, lse = oracle.combine_partials(po, pl, np.array([1, 1]))
    assert np.array_equal(o, po[:, :, 0])
    assert np.array_equal(lse, pl[:, :, 0])
    po = rng.standard_normal((1, 2, 4, 5))
    pl = rng.standard_normal((1, 2, 4)) * 10
    o, lse = oracle.combine_partials(po, pl, np.array([4]))
    np.testing.assert_allclose(lse[0], logsumexp(pl[0], axis=-1), rtol=1e-14)
    w = np.exp(pl[0] - logsumexp(pl[0], axis=-1, keepdims=True))
    np.testing.assert_allclose(o[0], np.einsum("hs,hsr->hr", w, po[0]), rtol=1e-13)


def test_combine_arbitrary_partition_and_empty_split():
    p = _random_problem(15, batch=1)
    q_lat = oracle.absorb_q(p["q_nope"], p["w_kvb"], p["dn"], p["dv"])
    o_ref, lse_ref = oracle.latent_attention(q_lat, p["q_rope"], p["latent"], p["rope"], p["kv_len"], None, p["scale"])
    parts = [np.array([4, 0, 9]), np.array([1]), np.array([10, 2, 3, 5, 6, 7, 8])]
    po = np.zeros((1, 3, 4, 6))
    pl = np.full((1, 3, 4), -np.inf)
    for s, idx in enumerate(parts):
        o_s, l_s = oracle.latent_attention(q_lat, p["q_rope"], p["latent"], p["rope"], p["kv_len"], [idx], p["scale"])
        po[0, :, s], pl[0, :, s] = o_s[0], l_s[0]
    o, lse = oracle.combine_partials(po, pl, np.array([4]))     # slot 3 is an empty split
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
