"""comba_chunk_fwd_noalloc, the entry point for callers that cannot allocate,
against comba_chunk_fwd: the same kernels, so the same bits, call after call
(the library's device scratch keeps the previous call's contents; a smaller
second call must not read past its own sequences). Also against the oracle,
and the host-side rejection of more packed sequences than the scratch holds."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
from bilinear_rnn_amd import api
from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
from _util import BF16, FP32, STATE_BF16, assert_close, dev_inputs, oracle_of, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _p(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def noalloc(inp):
    """One call of comba_chunk_fwd_noalloc through the C ABI; outputs allocated
    here, by the caller."""
    t = dev_inputs(inp)
    B, T, H, K = t["q"].shape
    V = t["v"].shape[-1]
    N = inp.num_seqs
    dt = api.COMBA_BF16 if inp.dtype == "bf16" else api.COMBA_FP32
    o = torch.empty((B, T, H, V), dtype=t["q"].dtype, device="cuda")
    sf = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    packed = t["cu_seqlens"] is not None
    rc = comba.lib().comba_chunk_fwd_noalloc(
        _p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["alpha"]), _p(t["beta"]), _p(t["d"]), _p(t["initial_state"]),
        _p(t["cu_seqlens"]), N if packed else 0, B, T, H, K, V, dt, dt, _p(o), _p(sf), stream)
    assert rc == 0, api.last_error()
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def with_workspace(inp):
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                            t["cu_seqlens"])
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def wl(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_equals_workspace_entry_point_twice_shrinking(dtype):
    """A packed batch of 40 sequences, then one of 7 shorter ones: each call
    bit-equal to comba_chunk_fwd, and within the parity gates of the oracle."""
    gates = (BF16, STATE_BF16) if dtype == "bf16" else (FP32, FP32)
    rng = np.random.default_rng(501)
    first = make_inputs(wl("varlen", H=4, dtype=dtype), lengths=rng.integers(0, 300, 40), s0_std=0.05, seed=502)
    second = make_inputs(wl("varlen", H=4, dtype=dtype), lengths=np.array([65, 1, 0, 130, 7, 64, 20]),
                         s0_std=0.05, seed=503)
    for inp in (first, second):
        print(f"noalloc: {inp.num_seqs} sequences, {inp.q.shape[1]} tokens, {dtype}", flush=True)
        o, s = noalloc(inp)
        ow, sw = with_workspace(inp)
        np.testing.assert_array_equal(o, ow)
        np.testing.assert_array_equal(s, sw)
        ro, rs = oracle_of(inp)
        assert_close(o, ro, gates[0], "o")
        assert_close(s, rs, gates[1], "state")


def test_noalloc_fixed_length_batch():
    inp = make_inputs(wl("layer_340m", B=3, H=2), T=200, s0_std=0.02, seed=504)
    o, s = noalloc(inp)
    ow, sw = with_workspace(inp)
    np.testing.assert_array_equal(o, ow)
    np.testing.assert_array_equal(s, sw)


def test_noalloc_binding_matches():
    rng = np.random.default_rng(505)
    inp = make_inputs(wl("varlen", H=2, K=128, V=128), lengths=rng.integers(1, 200, 9), s0_std=0.02, seed=506)
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                                    t["cu_seqlens"])
    torch.cuda.synchronize()
    ow, sw = with_workspace(inp)
    np.testing.assert_array_equal(to_np(o), ow)
    np.testing.assert_array_equal(to_np(sf), sw)


def test_noalloc_rejects_more_sequences_than_its_scratch():
    """16385 packed sequences exceed the 16384 the scratch holds: rejected on
    the host, before anything is enqueued."""
    N, H, K, V = 16385, 1, 64, 64
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    q = torch.zeros((1, 1, H, K), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, 1, H, V), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((1, 1, H), dtype=torch.float32, device="cuda")
    d = torch.zeros((H,), dtype=torch.float32, device="cuda")
    o = torch.empty_like(v)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = comba.lib().comba_chunk_fwd_noalloc(_p(q), _p(q), _p(v), _p(a), _p(a), _p(d), None, _p(cu), N, 1, 1, H,
                                             K, V, api.COMBA_BF16, api.COMBA_BF16, _p(o), None, stream)
    assert rc == api.COMBA_ERR_UNSUPPORTED
    assert "16384" in api.last_error()
