"""GPU parity of the fused entry points (gate logits, in-kernel q/k L2
normalisation) against the fp64 oracle, which takes the same input steps in
fp64 (oracle.fused_inputs) before its recurrence. Same gates as the unfused
parity tests: the fused kernels never round a normalised q or k to bf16.
"""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
from bilinear_rnn_amd import api
from bilinear_rnn_amd.inputs import WORKLOADS, bf16_bits, bf16_bits_to_f32, make_inputs
from _util import (BF16, BF16_IN_FP32_OUT, FP32, STATE_BF16, assert_close, cached, dev_inputs,
                   full_inputs, full_oracle, oracle_of, rel_l2, to_np)

pytestmark = pytest.mark.gpu

GATE_BF16 = 2e-3
GATE_FP32 = 1e-5
GATE_BF16_IN_FP32_OUT = 1e-4

BOTH = dict(gate_logits=True, qk_l2norm=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_chunk(inp, out_dtype=None, **kw):
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"],
                            t["initial_state"], t["cu_seqlens"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def run_step(inp, out_dtype=None, **kw):
    t = dev_inputs(inp)
    o, sf = comba.recurrent_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"],
                                 t["initial_state"], t["cu_seqlens"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def wl(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


def mixed(w, gate_logits, qk_l2norm, **kw):
    """Inputs where only the chosen steps are left to the kernel: raw q/k if
    qk_l2norm, gate logits if gate_logits (both drawn from the same seed)."""
    raw = make_inputs(w, raw=True, **kw)
    ready = make_inputs(w, raw=False, **kw)
    src_qk = raw if qk_l2norm else ready
    src_ab = raw if gate_logits else ready
    return dataclasses.replace(src_qk, alpha=src_ab.alpha, beta=src_ab.beta, raw=False)


# --- chunk forward -------------------------------------------------------------------------

@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [300, 64, 1, 129])
def test_bf16_fused_chunk_shapes_ragged(K, V, T):
    inp = make_inputs(wl("layer_340m", K=K, V=V, B=2, H=3), T=T, s0_std=0.02, seed=21, raw=True)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp, **BOTH)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")
    o32, s32 = run_chunk(inp, out_dtype=torch.float32, **BOTH)
    assert_close(o32, ro, BF16_IN_FP32_OUT, "o (fp32 out)")
    assert_close(s32, rs, BF16_IN_FP32_OUT, "state (fp32 out)")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 200])
def test_fp32_fused_chunk_shapes_ragged(K, V, T):
    inp = make_inputs(wl("tiny_fp32", K=K, V=V, B=2, H=2), T=T, s0_std=0.1, seed=22, raw=True)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp, **BOTH)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("gate_logits,qk_l2norm", [(True, False), (False, True)])
def test_single_fusion_flags(dtype, gate_logits, qk_l2norm):
    inp = mixed(wl("layer_340m", B=2, H=3, dtype=dtype), gate_logits, qk_l2norm, T=200, s0_std=0.02, seed=23)
    ro, rs = oracle_of(inp, gate_logits=gate_logits, qk_l2norm=qk_l2norm)
    flags = dict(gate_logits=gate_logits, qk_l2norm=qk_l2norm)
    o, s = run_chunk(inp, out_dtype=torch.float32, **flags)
    gate = FP32 if dtype == "fp32" else BF16_IN_FP32_OUT
    assert_close(o, ro, gate, "o")
    assert_close(s, rs, gate, "state")
    o, s = run_step(inp, out_dtype=torch.float32, **flags)
    assert_close(o, ro, (FP32 if dtype == "fp32" else BF16_IN_FP32_OUT), "o")
    assert_close(s, rs, (FP32 if dtype == "fp32" else BF16_IN_FP32_OUT), "state")


def test_fused_layer_1p3b_full_size():
    """The 1.3B layer at full size with raw q/k and gate logits, every
    (batch row, head) pair over whole sequences."""
    inp = full_inputs("layer_1p3b", raw=True)
    ro, rs = full_oracle("layer_1p3b", raw=True)
    o, s = run_chunk(inp, **BOTH)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_fused_varlen_workload_full():
    inp = full_inputs("varlen", raw=True)
    ro, rs = full_oracle("varlen", raw=True)
    o, s = run_chunk(inp, **BOTH)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_fused_wide_logits_and_zero_rows():
    """Gate logits over +-25 (alpha from ~1e-11 to 1 - 1e-11, beta likewise)
    and some all-zero q and k rows, which normalise to zero."""
    w = wl("layer_340m", B=2, H=2)
    inp = make_inputs(w, T=190, s0_std=0.02, seed=24, raw=True)
    rng = np.random.default_rng(24)
    a = rng.uniform(-25, 25, inp.alpha.shape).astype(np.float32)
    b = rng.uniform(-25, 25, inp.beta.shape).astype(np.float32)
    q, k = inp.q.copy(), inp.k.copy()
    q[0, 5:9, 1] = 0
    k[1, 60:70, 0] = 0
    k[0, 100, :] = 0
    inp = dataclasses.replace(inp, alpha=a, beta=b, q=q, k=k, q_bits=bf16_bits(q), k_bits=bf16_bits(k))
    assert np.array_equal(bf16_bits_to_f32(inp.q_bits), q)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp, out_dtype=torch.float32, **BOTH)
    assert_close(o, ro, BF16_IN_FP32_OUT, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")
    o, s = run_step(inp, out_dtype=torch.float32, **BOTH)
    assert_close(o, ro, BF16_IN_FP32_OUT, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fused_gate_logits_below_float_range(dtype):
    """alpha logits of -90 and -120 give sigmoids below the smallest normal
    float (about 8e-40, and 8e-53, which fp32 cannot hold), mixed with
    ordinary logits inside every chunk; the kernels clamp alpha to the
    smallest normal float, so the state is forgotten and nothing turns
    non-finite. Chunk and recurrent paths against the oracle, which takes the
    sigmoid in fp64."""
    w = wl("layer_340m", K=64, V=64, B=2, H=2, dtype=dtype)
    inp = make_inputs(w, T=200, s0_std=0.05, seed=31, raw=True)
    rng = np.random.default_rng(31)
    shape = inp.alpha.shape
    a = np.choose(rng.integers(0, 3, shape), [np.full(shape, -90.0), np.full(shape, -120.0),
                                             rng.normal(3.0, 0.5, shape)]).astype(np.float32)
    inp = dataclasses.replace(inp, alpha=a)
    ro, rs = oracle_of(inp)
    og, sg = (BF16, STATE_BF16) if dtype == "bf16" else (FP32, FP32)
    for path, (o, s) in (("chunk", run_chunk(inp, **BOTH)), ("recurrent", run_step(inp, **BOTH))):
        assert_close(o, ro, og, f"{path} o")
        assert_close(s, rs, sg, f"{path} state")


# --- recurrent step ------------------------------------------------------------------------

def test_fused_decode_workload_full_size():
    inp = full_inputs("decode", raw=True)
    ro, rs = full_oracle("decode", raw=True)
    o, s = run_step(inp, **BOTH)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_recurrent_multi_token(K, V, dtype):
    inp = make_inputs(wl("tiny_fp32", K=K, V=V, B=2, H=2, dtype=dtype), T=70, s0_std=0.1, seed=25, raw=True)
    ro, rs = oracle_of(inp)
    o, s = run_step(inp, out_dtype=torch.float32, **BOTH)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


def test_fused_recurrent_varlen():
    lengths = np.array([3, 0, 40, 1])
    inp = make_inputs(wl("varlen", H=2), lengths=lengths, s0_std=0.05, seed=26, raw=True)
    ro, rs = oracle_of(inp)
    o, s = run_step(inp, out_dtype=torch.float32, **BOTH)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


# --- structure -----------------------------------------------------------------------------

def test_fused_chunk_equals_fused_recurrent():
    inp = make_inputs(wl("layer_340m", B=2, H=4), T=257, s0_std=0.02, seed=27, raw=True)
    oc, sc = run_chunk(inp, out_dtype=torch.float32, **BOTH)
    orr, sr = run_step(inp, out_dtype=torch.float32, **BOTH)
    assert_close(oc, orr, BF16_IN_FP32_OUT, "o chunk vs recurrent")
    assert_close(sc, sr, BF16_IN_FP32_OUT, "state chunk vs recurrent")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fusion_zero_is_the_plain_entry_point(dtype):
    """comba_*_fused with fusion == 0 gives the plain entry points' bits."""
    inp = make_inputs(wl("layer_340m", B=2, H=3, dtype=dtype), T=150, s0_std=0.02, seed=28)
    o_ref, s_ref = run_chunk(inp)
    r_ref, rs_ref = run_step(inp)
    t = dev_inputs(inp)
    B, T, H, K = t["q"].shape
    V = t["v"].shape[-1]
    dt = api.COMBA_BF16 if dtype == "bf16" else api.COMBA_FP32
    o = torch.empty((B, T, H, V), dtype=t["q"].dtype, device="cuda")
    sf = torch.empty((B, H, V, K), dtype=torch.float32, device="cuda")
    p = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    common = (p(t["q"]), p(t["k"]), p(t["v"]), p(t["alpha"]), p(t["beta"]), p(t["d"]),
              p(t["initial_state"]), None, 0, B, T, H, K, V, dt, dt, p(o), p(sf))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = comba.lib()
    assert L.comba_chunk_fwd_fused(*common, None, 0, 0, stream) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o), o_ref)
    np.testing.assert_array_equal(to_np(sf), s_ref)
    assert L.comba_recurrent_step_fused(*common, 0, stream) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o), r_ref)
    np.testing.assert_array_equal(to_np(sf), rs_ref)


def test_fused_bitwise_deterministic():
    inp = make_inputs(wl("layer_340m", B=2, H=4), T=500, s0_std=0.02, seed=29, raw=True)
    o1, s1 = run_chunk(inp, **BOTH)
    o2, s2 = run_chunk(inp, **BOTH)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
