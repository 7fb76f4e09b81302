"""GPU o_proj against the oracle: the weight-streaming path (decode rows), the
GEMM path (prefill rows, with partial tiles) and the generic kernels."""

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


@pytest.mark.parametrize("dtype,rows,width,hidden", [
    (cf.BF16, 8, 8192, 6144),      # decode rows: weight streaming on MFMA (256 blocks of 24 columns)
    (cf.BF16, 8, 1024, 4160),      # 24-column blocks, the last one partial (8 columns)
    (cf.BF16, 64, 1024, 512),
    (cf.BF16, 200, 8192, 6144),    # GEMM path, partial M tile
    (cf.BF16, 130, 512, 300),      # GEMM path, partial N tile
    (cf.BF16, 5, 200, 40),         # generic (shape outside the MFMA kernels)
    (cf.F32, 3, 100, 37),          # generic fp32
])
def test_o_proj_matches_oracle(dtype, rows, width, hidden):
    say(f"o_proj {dtype} rows={rows} in={width} hidden={hidden}")
    ctx = gen.normal_f32(30, gen.T_MISC, (rows, width), layer=rows)
    w = cf.store(gen.normal_f32(30, gen.T_MISC, (hidden, width), std=width ** -0.5, layer=rows + 1), dtype)
    got = _mla().mla_o_proj(dev(ctx), dev(w))
    torch.cuda.synchronize()
    assert_close(host_values(got), oracle.o_proj(ctx, cf.values(w)), dtype, "o_proj")


def test_o_proj_prefill_size_sampled_rows():
    rows, width, hidden = 4096, 8192, 6144
    ctx = gen.normal_f32(31, gen.T_MISC, (rows, width))
    w = cf.store(gen.normal_f32(31, gen.T_MISC, (hidden, width), std=width ** -0.5, layer=1), cf.BF16)
    got = host_values(_mla().mla_o_proj(dev(ctx), dev(w)))
    sample = [0, 1, 127, 128, 2047, 4095]
    assert_close(got[sample], oracle.o_proj(ctx[sample], cf.values(w)), cf.BF16, "o_proj sampled rows")


@pytest.mark.parametrize("hidden", [
    4100,   # 256 x 192 tiles: 16 x 22 = 352 tiles (2 rounds of 3 units) beat 16 x 17 (2 rounds of 4);
            # 4100 = 21 x 192 + 68 columns
    4000,   # 256 x 256 tiles: 16 x 16 = 256, one round; 4000 = 15 x 256 + 160 columns
])
def test_o_proj_long_gemm_partial_tiles_sampled_rows(hidden):
    """Enough rows and columns for the 256-row GEMM tiles, with a partial
    tile at both edges (4000 = 15 x 256 + 160 rows)."""
    rows, width = 4000, 512
    say(f"o_proj rows={rows} in={width} hidden={hidden}")
    ctx = gen.normal_f32(32, gen.T_MISC, (rows, width))
    w = cf.store(gen.normal_f32(32, gen.T_MISC, (hidden, width), std=width ** -0.5, layer=1), cf.BF16)
    got = host_values(_mla().mla_o_proj(dev(ctx), dev(w)))
    sample = [0, 1, 127, 128, 255, 256, 3839, 3840, 3967, 3999]
    assert_close(got[sample], oracle.o_proj(ctx[sample], cf.values(w)), cf.BF16, "o_proj sampled rows")
