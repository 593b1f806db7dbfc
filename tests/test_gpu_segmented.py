"""GPU parity of the segment-parallel chunk forward (comba_chunk_fwd_segmented)
against the fp64 oracle, plus its structural properties. Same gates as the
plain chunk forward: the segment maps and the scan are carried in fp32.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
from _util import (BF16, BF16_IN_FP32_OUT, FP32, STATE_BF16, assert_close, cached, dev_inputs,
                   full_inputs, full_oracle, oracle_of, rel_l2, to_np)

pytestmark = pytest.mark.gpu

GATE_BF16 = 2e-3
GATE_FP32 = 1e-5
GATE_BF16_IN_FP32_OUT = 1e-4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(inp, out_dtype=None, **kw):
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                            out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def wl(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("T,S,s0", [(1000, 3, 0.02), (1000, 7, 0.0), (640, 2, 0.02), (130, 3, 0.02)])
def test_bf16_segmented_matches_oracle(K, V, T, S, s0):
    inp = make_inputs(wl("layer_340m", K=K, V=V, B=2, H=3), T=T, s0_std=s0, seed=31)
    ro, rs = oracle_of(inp)
    o, s = run(inp, segments=S)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")
    o32, s32 = run(inp, out_dtype=torch.float32, segments=S)
    assert_close(o32, ro, BF16_IN_FP32_OUT, "o (fp32 out)")
    assert_close(s32, rs, BF16_IN_FP32_OUT, "state (fp32 out)")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 64)])
@pytest.mark.parametrize("S", [2, 5])
def test_fp32_segmented_matches_oracle(K, V, S):
    inp = make_inputs(wl("tiny_fp32", K=K, V=V, B=2, H=2), T=500, s0_std=0.1, seed=32)
    ro, rs = oracle_of(inp)
    o, s = run(inp, segments=S)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


def test_long_context_automatic_segments_full():
    """One 64K-token sequence with slow decay, segments chosen automatically
    (8 of 8192 tokens); every head against the oracle over the whole sequence."""
    w = WORKLOADS["long_context"]
    assert comba.segmented_workspace_size(w.B, w.T, w.H, w.K, w.V, 0) > 0
    ro, rs = full_oracle("long_context")
    o, s = run(full_inputs("long_context"), segments=0)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_one_segment_is_the_plain_call():
    inp = make_inputs(wl("layer_340m", B=2, H=3), T=700, s0_std=0.02, seed=33)
    o_ref, s_ref = run(inp)
    o, s = run(inp, segments=1)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s, s_ref)


def test_segmented_close_to_plain():
    inp = make_inputs(wl("layer_340m", B=1, H=4), T=4096, s0_std=0.02, seed=34)
    o_ref, s_ref = run(inp, out_dtype=torch.float32)
    o, s = run(inp, out_dtype=torch.float32, segments=8)
    assert_close(o, o_ref, BF16_IN_FP32_OUT, "o")
    assert_close(s, s_ref, BF16_IN_FP32_OUT, "state")


def test_segmented_with_fused_inputs():
    inp = make_inputs(wl("layer_340m", B=2, H=2), T=900, s0_std=0.02, seed=35, raw=True)
    ro, rs = oracle_of(inp)
    o, s = run(inp, out_dtype=torch.float32, segments=4, gate_logits=True, qk_l2norm=True)
    assert_close(o, ro, BF16_IN_FP32_OUT, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")


def test_segmented_in_place_state_and_no_final_state():
    inp = make_inputs(wl("layer_340m", B=2, H=2), T=600, s0_std=0.02, seed=36)
    o_ref, s_ref = run(inp, segments=3)
    t = dev_inputs(inp)
    st = t["initial_state"]
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], st, final_state=st, segments=3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o), o_ref)
    np.testing.assert_array_equal(to_np(st), s_ref)
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                            output_final_state=False, segments=3)
    torch.cuda.synchronize()
    assert sf is None
    np.testing.assert_array_equal(to_np(o), o_ref)


def test_segmented_bitwise_deterministic():
    inp = make_inputs(wl("layer_340m", B=1, H=4), T=2000, s0_std=0.02, seed=37)
    o1, s1 = run(inp, segments=5)
    o2, s2 = run(inp, segments=5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
