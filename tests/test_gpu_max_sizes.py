"""The largest shapes the C ABI admits, on the GPU, against the oracle on
sampled heads:

- the most heads per token (H * max(K, V) = 2^22: 32768 heads of 128), where
  the byte offsets inside one chunk are largest, through the chunk forward,
  the recurrent path and the backward, in bf16 and fp32;
- q, k, v and o above 4 GiB each (one sequence of about 2.1 M tokens, 16
  heads), where token offsets need 64 bits, through the plain and the
  segment-parallel forward;
- a decode state above 4 GiB (4100 sequences x 16 heads x 128 x 128 fp32).

Outputs are sliced on the device before they are copied back. The long
sequence is the seeded draw of an 8229-token sequence repeated 255 times on
the device; 8229 is odd, so a token offset that wrapped at 2^32 bytes would
read a different token of the period and fail the comparison."""
import dataclasses

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
import oracle
from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
from _util import BF16, FP32, STATE_BF16, assert_close, dev_inputs, rel_l2
from test_gpu_backward import check, cotangents

pytestmark = pytest.mark.gpu

GATE_BF16 = 2e-3
GATE_FP32 = 1e-5


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def head_slice(inp, heads):
    """The same inputs restricted to some heads (all tokens, all sequences)."""
    sl = {name: getattr(inp, name)[:, :, heads] for name in ("q", "k", "v", "alpha", "beta")}
    for name in ("q_bits", "k_bits", "v_bits"):
        if getattr(inp, name) is not None:
            sl[name] = getattr(inp, name)[:, :, heads]
    return dataclasses.replace(inp, d=inp.d[heads], s0=None if inp.s0 is None else inp.s0[:, heads], **sl)


MAX_H = (1 << 22) // 128
HEADS = [0, 12345, MAX_H - 1]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_most_heads_forward_recurrent_backward(dtype):
    print(f"max heads: H={MAX_H} K=V=128 T=100 {dtype}", flush=True)
    w = dataclasses.replace(WORKLOADS["layer_1p3b"], dtype=dtype)
    inp = make_inputs(w, B=1, T=100, H=MAX_H, s0_std=0.02, seed=2201)
    t = dev_inputs(inp)
    o, sf = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"])
    ro_, rs_ = comba.recurrent_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"])
    torch.cuda.synchronize()
    sub = head_slice(inp, HEADS)
    ro, rs = oracle.comba_forward_c(sub.q, sub.k, sub.v, sub.alpha, sub.beta, sub.d, sub.s0)
    for got_o, got_s in ((o, sf), (ro_, rs_)):
        assert_close(f64(got_o[:, :, HEADS]), ro, BF16 if dtype == "bf16" else FP32, "o")
        assert_close(f64(got_s[:, HEADS]), rs, STATE_BF16 if dtype == "bf16" else FP32, "state")
    del o, sf, ro_, rs_

    do, do_bits, dsf = cotangents(inp, 2202)
    dod = (torch.from_numpy(np.ascontiguousarray(do_bits).view(np.int16)).view(torch.bfloat16).cuda()
           if do_bits is not None else torch.from_numpy(do).cuda())
    g = comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], dod, t["initial_state"],
                        None, torch.from_numpy(dsf).cuda())
    torch.cuda.synchronize()
    got = {key: f64(x[:, :, HEADS]) for key, x in g.items() if key in ("dq", "dk", "dv", "dalpha", "dbeta")}
    got["dd"] = f64(g["dd"][HEADS])
    got["ds0"] = f64(g["dinitial_state"][:, HEADS])
    ref = oracle.comba_backward(sub.q, sub.k, sub.v, sub.alpha, sub.beta, sub.d, do[:, :, HEADS], sub.s0,
                                dsf[:, HEADS], None)
    check(got, ref, sub)


PERIOD, REPEATS = 8229, 255


def test_tensors_above_4gib_plain_and_segmented():
    w = WORKLOADS["layer_1p3b"]
    T = PERIOD * REPEATS
    assert T * w.H * w.K * 2 > (1 << 32)
    print(f"long sequence: T={T} H={w.H} K=V=128 bf16 ({T * w.H * w.K * 2 / 2**30:.1f} GiB per tensor)", flush=True)
    base = make_inputs(w, B=1, T=PERIOD, s0_std=0.02, seed=2203)
    t = dev_inputs(base)
    big = {key: t[key].repeat(1, REPEATS, 1, 1) for key in ("q", "k", "v")}
    big.update({key: t[key].repeat(1, REPEATS, 1) for key in ("alpha", "beta")})
    h, rows = 7, slice(0, 16)
    # the oracle on value rows 0..15 of head h (rows of the state evolve independently)
    rep = lambda x: np.tile(x[:, :, h:h + 1], (1, REPEATS) + (1,) * (x.ndim - 2))  # noqa: E731
    ro, rs = oracle.comba_forward_c(rep(base.q), rep(base.k), rep(base.v)[..., rows], rep(base.alpha),
                                    rep(base.beta), base.d[h:h + 1], base.s0[:, h:h + 1, rows])
    for segments in (None, 0):
        print(f"segments={segments}", flush=True)
        o, sf = comba.chunk_fwd(big["q"], big["k"], big["v"], big["alpha"], big["beta"], t["d"],
                                t["initial_state"], segments=segments)
        torch.cuda.synchronize()
        assert_close(f64(o[:, :, h:h + 1, rows]), ro, BF16, "o")
        assert_close(f64(sf[:, h:h + 1, rows]), rs, STATE_BF16, "state")
        # the last period, all heads, is finite (offsets past 4 GiB were written)
        assert torch.isfinite(o[:, -PERIOD:].float()).all()
        del o, sf


def test_decode_state_above_4gib():
    w = WORKLOADS["decode"]
    N = 4100
    assert N * w.H * w.V * w.K * 4 > (1 << 32)
    print(f"decode: N={N} H={w.H} state {N * w.H * w.V * w.K * 4 / 2**30:.1f} GiB", flush=True)
    inp = make_inputs(w, B=N, seed=2204)
    t = dev_inputs(inp)
    o, sf = comba.recurrent_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                                 in_place=True)
    torch.cuda.synchronize()
    for n, h in [(0, 0), (2222, 5), (N - 1, w.H - 1)]:
        ro, rs = oracle.comba_forward_c(inp.q[n:n + 1, :, h:h + 1], inp.k[n:n + 1, :, h:h + 1],
                                        inp.v[n:n + 1, :, h:h + 1], inp.alpha[n:n + 1, :, h:h + 1],
                                        inp.beta[n:n + 1, :, h:h + 1], inp.d[h:h + 1], inp.s0[n:n + 1, h:h + 1])
        assert_close(f64(o[n:n + 1, :, h:h + 1]), ro, BF16, "o")
        assert_close(f64(sf[n:n + 1, h:h + 1]), rs, STATE_BF16, "state")
