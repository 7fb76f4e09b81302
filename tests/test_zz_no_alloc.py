"""mla_dsa_topk_select_noalloc (the fixed-scratch form of the DSA top-k, for
callers that cannot allocate) against mla_dsa_topk_select with a caller
workspace: the same positions and counts, bit for bit, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's
candidates, which the second call must not see)."""

import ctypes

import numpy as np
import pytest
import torch

from synth import generators as gen
from tests.gpu_util import say

TOP_K = 2048


def _mla():
    import mla_latent_kv_partial_amd as mla
    return mla


def _scores(rows, width, layer):
    x = gen.normal_f32(4, gen.T_DSA_SCORES, (rows, width), layer=layer)
    x[:, ::7] = np.round(x[:, ::7], 1)      # many equal scores: ties at the threshold
    return torch.from_numpy(x).cuda()


@pytest.mark.gpu
def test_noalloc_topk_equals_workspace_form_on_two_calls():
    mla = _mla()
    # call 1: six 131072-score rows (two-stage), one 5000-score row (one
    # workgroup), one row not longer than top_k (dense)
    # call 2: two 40000-score rows (three segments each)
    for call, (lens, width) in enumerate((([131072] * 6 + [5000, 1500], 131072), ([40000, 33000], 40000))):
        scores = _scores(len(lens), width, layer=call)
        total = sum(TOP_K for n in lens if n > TOP_K)
        say(f"noalloc top-k call {call}: rows {lens}")
        ref_idx, ref_cnt = mla.mla_dsa_topk_select(scores, lens, TOP_K, two_stage=True)
        buf = torch.full((total,), -7, dtype=torch.int32, device="cuda")
        got_idx, got_cnt = mla.mla_dsa_topk_select_noalloc(scores, lens, TOP_K, buf)
        torch.cuda.synchronize()
        assert got_cnt == ref_cnt
        assert torch.equal(got_idx, ref_idx)


@pytest.mark.gpu
def test_noalloc_topk_rejects_more_rows_than_the_scratch():
    from mla_latent_kv_partial_amd._lib import i32_array, lib
    lens = [131072] * 33
    counts = i32_array([0] * 33)
    code = lib.mla_dsa_topk_select_noalloc(ctypes.c_void_p(16), 131072, 33, i32_array(lens), TOP_K,
                                           ctypes.c_void_p(16), counts, None)
    assert code == -5 and b"scratch" in lib.mla_last_error()
