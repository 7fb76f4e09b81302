"""GPU parity of mla_rope_partial_interleaved against the oracle, plus its bitwise invariants."""

import numpy as np
import pytest
import torch

import oracle
from synth import configs as cf, generators as g
from tests.gpu_util import assert_close, bitwise_equal, dev, host_values, say

pytestmark = pytest.mark.gpu


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


@pytest.mark.parametrize("dtype", [cf.F32, cf.BF16])
@pytest.mark.parametrize("shape,rot,offs", [
    ((1, 1, 4, 16), 16, [128]),                 # tiny decode q rope, one row
    ((8, 1, 64, 64), 64, "ragged"),             # batched decode q rope, per-row offsets
    ((2, 37, 3, 80), 64, [5, 131072]),          # token axis with a tail, large positions
    ((1, 300, 2, 512), 512, [0]),               # widest rotary
])
def test_rope_matches_oracle(dtype, shape, rot, offs):
    say(f"rope {dtype} {shape} R={rot}")
    x32 = g.normal_f32(90, 1, shape)
    xs = cf.store(x32, dtype)
    if offs == "ragged":
        offs = [int(v) for v in g.ragged_lengths(3, shape[0], 1024, 32768)]
    ref = oracle.rope_partial_interleaved(cf.values(xs), offs if len(offs) > 1 else offs[0], rot, 10000.0)
    mla = _mla()
    x = dev(xs)
    y = mla.mla_rope_partial_interleaved(x, offs if len(offs) > 1 else offs[0], rot, 10000.0)
    torch.cuda.synchronize()
    # rounded once from double: f32 within ~1 ulp, bf16 within half a bf16 ulp
    assert_close(host_values(y), ref, dtype, "rope", tol=2e-7 if dtype == cf.F32 else 8e-3)
    yi = x.clone()
    mla.mla_rope_partial_interleaved(yi, offs if len(offs) > 1 else offs[0], rot, 10000.0, out=yi)
    assert bitwise_equal(yi, y), "in-place result differs from out-of-place"
    if rot < shape[-1]:
        assert bitwise_equal(y[..., rot:], x[..., rot:]), "tail not preserved"


@pytest.mark.parametrize("dtype", [cf.F32, cf.BF16])
def test_rope_position_zero_is_exact_permutation(dtype):
    xs = cf.store(g.normal_f32(91, 1, (3, 1, 5, 64)), dtype)
    x = dev(xs)
    y = _mla().mla_rope_partial_interleaved(x, 0, 64, 10000.0)
    perm = list(range(0, 64, 2)) + list(range(1, 64, 2))
    assert bitwise_equal(y, x[..., perm].contiguous())


def test_rope_per_row_offsets_equal_scalar_calls():
    mla = _mla()
    x = dev(cf.store(g.normal_f32(92, 1, (4, 3, 8, 64)), cf.BF16))
    offs = [0, 17, 4096, 99999]
    y = mla.mla_rope_partial_interleaved(x, offs, 64, 10000.0)
    for b in range(4):
        yb = mla.mla_rope_partial_interleaved(x[b:b + 1].contiguous(), offs[b], 64, 10000.0)
        assert bitwise_equal(y[b:b + 1], yb)


def test_rope_strided_slice_of_q():
    """RoPE applied to the rope slice of a [B,1,H,dn+dr] query in place, nope part untouched."""
    mla = _mla()
    qh = cf.store(g.normal_f32(93, 1, (2, 1, 64, 192)), cf.BF16)
    q = dev(qh)
    before = q.clone()
    view = q[..., 128:]
    mla.mla_rope_partial_interleaved(view, [4096, 7], 64, 10000.0, out=view)
    ref = oracle.rope_partial_interleaved(cf.values(qh[..., 128:]), [4096, 7], 64, 10000.0)
    assert_close(host_values(q[..., 128:]), ref, cf.BF16, "rope slice", tol=8e-3)
    assert bitwise_equal(q[..., :128], before[..., :128])


def test_rope_empty_and_errors():
    mla = _mla()
    x = torch.empty((0, 4, 2, 16), device="cuda", dtype=torch.float32)
    mla.mla_rope_partial_interleaved(x, 0, 16, 10000.0)
    with pytest.raises(mla.MlaError):
        mla.mla_rope_partial_interleaved(torch.zeros((1, 2, 1, 16), device="cuda"), 0, 15, 10000.0)
    with pytest.raises(mla.MlaError):
        mla.mla_rope_partial_interleaved(torch.zeros((1, 2, 1, 16), device="cuda"), -3, 16, 10000.0)
