"""GPU parity of the HIP path against the fp64 CPU oracle, through the C ABI.

Gates (rel-L2 over a whole tensor, fp64): 2e-3 for bf16 q/k/v (o in bf16),
1e-5 for fp32 q/k/v. For bf16 inputs with an fp32 output, the only error
left is the rounding of the kernels' non-input operands, each carried as a
hi+lo bf16 pair (about 2^-17 relative) and accumulated in fp32; a 1e-4 gate
there checks that no operand silently dropped to a single bf16 (which costs
about 2e-4 to 2e-3 in an fp64 experiment that rounds one intermediate of the
chunk form at a time). Beside every whole-tensor figure, the largest error of
a single token-head row (or state row) is bounded too (``_util.assert_close``).
Every workload the benchmark times is compared whole, at full size, in the
launch configuration the benchmark uses.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
from _util import (BF16, BF16_IN_FP32_OUT, FP32, STATE_BF16, Gates, assert_close, dev_inputs, full_inputs,
                   full_oracle, oracle_of, rel_l2, to_np)

pytestmark = pytest.mark.gpu

GATE_BF16 = 2e-3
GATE_FP32 = 1e-5
GATE_BF16_IN_FP32_OUT = 1e-4
FLT_MIN = float(np.finfo(np.float32).tiny)


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


# ---------------------------------------------------------------------------------------

def test_tiny_fp32_workload_exact():
    inp = make_inputs(WORKLOADS["tiny_fp32"])
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 64, 200])
def test_fp32_shapes_ragged(K, V, T):
    inp = make_inputs(wl("tiny_fp32", K=K, V=V, B=2, H=2), T=T, s0_std=0.1, seed=7)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T,s0", [(300, 0.02), (64, 0.0), (1, 0.02), (129, 0.02)])
def test_bf16_shapes_ragged(K, V, T, s0):
    inp = make_inputs(wl("layer_340m", K=K, V=V, B=2, H=3), T=T, s0_std=s0, seed=11)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")
    o32, s32 = run_chunk(inp, out_dtype=torch.float32)
    assert_close(o32, ro, BF16_IN_FP32_OUT, "o (fp32 out)")
    assert_close(s32, rs, BF16_IN_FP32_OUT, "state (fp32 out)")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_gates(dtype):
    """Decays and write strengths at their limits: alpha from half the
    smallest normal float (a subnormal, which the kernels clamp to the
    smallest normal) and 1e-6 (the state forgotten within a token, in-chunk
    decay products far below fp32's range) to exactly 1 (no decay), beta
    exactly 0 and 1, mixed within every chunk; chunk and recurrent paths
    against the oracle."""
    base = wl("layer_340m", K=64, V=64, B=2, H=2) if dtype == "bf16" else wl("tiny_fp32", B=2, H=2)
    inp = make_inputs(base, T=200, s0_std=0.05, seed=41)
    rng = np.random.default_rng(42)
    shape = inp.alpha.shape
    alpha = np.choose(rng.integers(0, 5, shape), [np.full(shape, 1e-6), np.ones(shape),
                                                  rng.uniform(0.0, 1.0, shape), np.full(shape, 0.5),
                                                  np.full(shape, FLT_MIN / 2)])
    beta = np.choose(rng.integers(0, 3, shape), [np.zeros(shape), np.ones(shape), rng.uniform(0.0, 1.0, shape)])
    inp = dataclasses.replace(inp, alpha=alpha.astype(np.float32), beta=beta.astype(np.float32))
    assert (inp.alpha == np.float32(FLT_MIN / 2)).any()
    ro, rs = oracle_of(inp)
    og, sg = (BF16, STATE_BF16) if dtype == "bf16" else (FP32, FP32)
    for path, (o, s) in (("chunk", run_chunk(inp)), ("recurrent", run_step(inp))):
        assert_close(o, ro, og, f"{path} o")
        assert_close(s, rs, sg, f"{path} state")


def test_layer_340m_full_size():
    """The 340M layer at full size (B=4, H=16, T=2048, K = V = 128), whole tensors."""
    ro, rs = full_oracle("layer_340m")
    o, s = run_chunk(full_inputs("layer_340m"))
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_layer_1p3b_full_size():
    """The 1.3B layer at full size (B=8, H=16, T=4096, non-zero initial state),
    launched exactly as the benchmark launches it; the oracle checks every
    (batch row, head) pair over whole sequences."""
    ro, rs = full_oracle("layer_1p3b")
    o, s = run_chunk(full_inputs("layer_1p3b"))
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_long_context_full():
    """One 64K-token sequence with slow decay: long inter-chunk scan and fp32
    accumulation drift, every head over the whole sequence."""
    ro, rs = full_oracle("long_context")
    o, s = run_chunk(full_inputs("long_context"))
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_varlen_workload_full():
    """64 packed sequences, lognormal lengths, H = 32, K = V = 64."""
    ro, rs = full_oracle("varlen")
    o, s = run_chunk(full_inputs("varlen"))
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")


def test_varlen_edge_lengths_and_initial_state():
    lengths = np.array([16, 70, 1, 0, 130, 64, 200, 0, 63, 65])
    inp = make_inputs(wl("varlen", H=4), lengths=lengths, s0_std=0.05, seed=5)
    ro, rs = oracle_of(inp)
    o, s = run_chunk(inp)
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, STATE_BF16, "state")
    # empty sequences return their initial state unchanged
    for n in np.flatnonzero(lengths == 0):
        np.testing.assert_array_equal(s[n], inp.s0[n].astype(np.float64))


def test_varlen_equals_separate_calls():
    lengths = np.array([33, 200, 64, 1])
    inp = make_inputs(wl("varlen", H=2, K=128, V=128), lengths=lengths, s0_std=0.02, seed=6)
    o, s = run_chunk(inp)
    cu = inp.cu_seqlens
    for n in range(len(lengths)):
        sl = slice(cu[n], cu[n + 1])
        sub = dataclasses.replace(inp, q=inp.q[:, sl], k=inp.k[:, sl], v=inp.v[:, sl],
                                  alpha=inp.alpha[:, sl], beta=inp.beta[:, sl], s0=inp.s0[n:n + 1],
                                  cu_seqlens=None, q_bits=inp.q_bits[:, sl], k_bits=inp.k_bits[:, sl],
                                  v_bits=inp.v_bits[:, sl])
        on, sn = run_chunk(sub)
        np.testing.assert_array_equal(o[:, sl], on)
        np.testing.assert_array_equal(s[n:n + 1], sn)


def test_varlen_order_is_longest_first():
    lengths = np.array([5, 300, 300, 0, 17, 4096, 5])
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    order = comba.varlen_order(cu).cpu().numpy()
    expect = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    np.testing.assert_array_equal(order, expect)


# --- recurrent step ------------------------------------------------------------------------

def test_decode_workload_full_size():
    """Decode step: 256 sequences x 16 heads, K = V = 128, fp32 state in HBM."""
    ro, rs = full_oracle("decode")
    o, s = run_step(full_inputs("decode"))
    assert_close(o, ro, BF16, "o")
    assert_close(s, rs, BF16_IN_FP32_OUT, "state")


def test_decode_in_place_state():
    inp = make_inputs(WORKLOADS["decode"], B=8)
    ro, rs = oracle_of(inp)
    t = dev_inputs(inp)
    st = t["initial_state"]
    o, sf = comba.recurrent_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], st, in_place=True)
    torch.cuda.synchronize()
    assert sf.data_ptr() == st.data_ptr()
    assert_close(to_np(st), rs, BF16_IN_FP32_OUT, "state")
    assert_close(to_np(o), ro, BF16, "o")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_recurrent_multi_token(K, V, dtype):
    inp = make_inputs(wl("tiny_fp32", K=K, V=V, B=2, H=2, dtype=dtype), T=70, s0_std=0.1, seed=3)
    ro, rs = oracle_of(inp)
    o, s = run_step(inp, out_dtype=torch.float32)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


def test_recurrent_varlen():
    lengths = np.array([3, 0, 40, 1])
    inp = make_inputs(wl("varlen", H=2), lengths=lengths, s0_std=0.05, seed=8)
    ro, rs = oracle_of(inp)
    o, s = run_step(inp, out_dtype=torch.float32)
    assert_close(o, ro, FP32, "o")
    assert_close(s, rs, FP32, "state")


# --- cross-entry-point and structural checks ----------------------------------------------

def test_chunk_equals_recurrent_path():
    inp = make_inputs(wl("layer_340m", B=2, H=4), T=257, s0_std=0.02, seed=9)
    oc, sc = run_chunk(inp, out_dtype=torch.float32)
    orr, sr = run_step(inp, out_dtype=torch.float32)
    assert_close(oc, orr, BF16_IN_FP32_OUT, "o chunk vs recurrent")
    assert_close(sc, sr, BF16_IN_FP32_OUT, "state chunk vs recurrent")


def test_split_and_resume():
    inp = make_inputs(wl("layer_340m", B=2, H=4), T=320, s0_std=0.02, seed=10)
    o, s = run_chunk(inp, out_dtype=torch.float32)
    cut = 192

    def part(sl, s0):
        return dataclasses.replace(inp, q=inp.q[:, sl], k=inp.k[:, sl], v=inp.v[:, sl],
                                   alpha=inp.alpha[:, sl], beta=inp.beta[:, sl], s0=s0,
                                   q_bits=inp.q_bits[:, sl], k_bits=inp.k_bits[:, sl], v_bits=inp.v_bits[:, sl])

    oa, sa = run_chunk(part(slice(0, cut), inp.s0), out_dtype=torch.float32)
    ob, sb = run_chunk(part(slice(cut, 320), sa.astype(np.float32)), out_dtype=torch.float32)
    assert rel_l2(np.concatenate([oa, ob], axis=1), o) <= 1e-5
    assert rel_l2(sb, s) <= 1e-5


def test_in_place_chunk_state():
    inp = make_inputs(wl("layer_340m", B=2, H=2), T=130, s0_std=0.02, seed=12)
    o, s = run_chunk(inp)
    t = dev_inputs(inp)
    st = t["initial_state"]
    o2, s2 = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], st, final_state=st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o2), o)
    np.testing.assert_array_equal(to_np(st), s)


def test_bitwise_deterministic():
    inp = make_inputs(wl("layer_340m", B=2, H=4), T=500, s0_std=0.02, seed=13)
    o1, s1 = run_chunk(inp)
    o2, s2 = run_chunk(inp)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_no_final_state_requested():
    inp = make_inputs(wl("layer_340m", B=1, H=2), T=100, seed=14)
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], output_final_state=False)
    torch.cuda.synchronize()
    assert sf is None
    ro, _ = oracle_of(inp)
    assert_close(to_np(o), ro, BF16, "o")
