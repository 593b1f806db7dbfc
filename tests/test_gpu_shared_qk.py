"""GPU parity with q / k heads shared by several value heads (comba_chunk_fwd_ex,
comba_recurrent_step_ex and the segmented forward) against the fp64 oracle,
which expands the shared heads first (oracle.expand_shared_qk). The kernels do
the same arithmetic per value head either way, so a shared-head call must also
match a plain call on expanded q / k bit for bit.
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


def run_chunk(inp, out_dtype=None, **kw):
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                            t["cu_seqlens"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def run_step(inp, out_dtype=None, **kw):
    t = dev_inputs(inp)
    o, sf = comba.recurrent_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                                 t["cu_seqlens"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def wl(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


def expanded(inp):
    """The same inputs with one q / k head per value head."""
    H = inp.v.shape[2]
    G = H // inp.q.shape[2]
    q, k = np.repeat(inp.q, G, axis=2), np.repeat(inp.k, G, axis=2)
    out = dataclasses.replace(inp, q=q, k=k)
    if inp.q_bits is not None:
        out.q_bits, out.k_bits = np.repeat(inp.q_bits, G, axis=2), np.repeat(inp.k_bits, G, axis=2)
    return out


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("Hk", [1, 2])
@pytest.mark.parametrize("T", [300, 64])
def test_bf16_shared_qk_chunk(K, V, Hk, T):
    inp = make_inputs(wl("layer_340m", K=K, V=V, B=2, H=4), T=T, s0_std=0.02, seed=41, qk_heads=Hk)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")
    o32, s32 = run_chunk(inp, out_dtype=torch.float32)
    assert_close(o32, ro, BF16_IN_FP32_OUT, "o (fp32 out)")
    assert_close(s32, rs, BF16_IN_FP32_OUT, "state (fp32 out)")
    # bit-equal to the plain call on expanded q / k
    oe, se = run_chunk(expanded(inp), out_dtype=torch.float32)
    np.testing.assert_array_equal(o32, oe)
    np.testing.assert_array_equal(s32, se)


@pytest.mark.parametrize("Hk", [1, 2])
def test_fp32_shared_qk_chunk_and_recurrent(Hk):
    inp = make_inputs(wl("tiny_fp32", B=2, H=4), T=200, s0_std=0.1, seed=42, qk_heads=Hk)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")
    o, s = run_step(inp, out_dtype=torch.float32)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")
    oe, se = run_chunk(expanded(inp))
    oc, sc = run_chunk(inp)
    np.testing.assert_array_equal(oc, oe)
    np.testing.assert_array_equal(sc, se)


def test_shared_qk_varlen_and_fused():
    lengths = np.array([70, 1, 0, 200, 64])
    inp = make_inputs(wl("varlen", H=4), lengths=lengths, s0_std=0.05, seed=43, qk_heads=1, raw=True)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp, out_dtype=torch.float32, gate_logits=True, qk_l2norm=True)
    assert_close(o, ro, BF16_IN_FP32_OUT, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")
    o, s = run_step(inp, out_dtype=torch.float32, gate_logits=True, qk_l2norm=True)
    assert_close(o, ro, BF16_IN_FP32_OUT, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")


def test_decode_multi_value_heads():
    """Decode with one q / k head shared by all 16 value heads, 256 sequences."""
    inp = make_inputs(WORKLOADS["decode"], qk_heads=1)
    ro, rs = oracle_of(inp)
    o, s = run_step(inp)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")
    oe, se = run_step(expanded(inp))
    np.testing.assert_array_equal(o, oe)
    np.testing.assert_array_equal(s, se)


def test_segmented_shared_qk():
    inp = make_inputs(wl("layer_340m", B=1, H=4), T=1500, s0_std=0.02, seed=44, qk_heads=2)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp, out_dtype=torch.float32, segments=4)
    assert_close(o, ro, BF16_IN_FP32_OUT, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")


def test_layer_1p3b_multi_value_heads_full_size():
    """The 1.3B layer shapes with one q / k head for all 16 value heads, every
    (batch row, head) pair over whole sequences."""
    inp = full_inputs("layer_1p3b", qk_heads=1)
    ro, rs = full_oracle("layer_1p3b", qk_heads=1)
    o, s = run_chunk(inp)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_shared_qk_shape_errors():
    inp = make_inputs(wl("layer_340m", B=1, H=4), T=64, seed=45, qk_heads=2)
    t = dev_inputs(inp)
    q3 = torch.zeros((1, 64, 3, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        comba.chunk_fwd(q3, q3, t["v"], t["alpha"], t["beta"], t["d"])
