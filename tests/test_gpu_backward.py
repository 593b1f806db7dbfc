"""GPU parity of the chunk backward (comba_chunk_bwd) against the fp64
reverse-mode oracle of the token recurrence (oracle.comba_backward), on the
same seeded inputs and cotangents. The gradients are accumulated in fp32.

fp32 inputs: every product is an exact-fp32 matrix-core product, so the gate
is rel-L2 <= 1e-5 per gradient tensor (fp32 rounding, 6e-8, accumulated over
sums of a few hundred terms, the chunk inverse and the scan over the chunks).
Measured: 4e-8 to 8e-7.

bf16 inputs: q, k, v and dO enter the bf16 matrix cores exactly; every fp32
operand (states, state gradients, the chunk inverse, scores and the
intermediate products) enters as hi + lo bf16, about 16 significant bits (a
relative error up to u = 2^-17 = 7.6e-6 per operand); a product of two split
operands carries about 3u relative to the product of their magnitudes, and a
gradient that is a short sum of such products with cancellation (dq of a
one-token sequence: the state term against the score term) more. The gate is
rel-L2 <= 5e-5 (about 6.6u) per per-token gradient tensor; measured: up to
5e-6, and 1.1e-5 for one-token sequences. dd is a signed sum over every token
and key of a head, so cancellation scales its relative error by
sum |dq k| / |dd|; it is gated by |dd - dd_ref| <= 5e-5 sum |dq k| per head
(measured up to 1.1e-5). All of these lie far inside the bf16 tolerance of
the forward (rel-L2 2e-3).

Beside each whole-tensor figure, the largest error of one row (one
token-head row of dq, dk or dv; one value channel of dS_0) is bounded at ten
times the whole-tensor gate (oracle.row_rel_err), so that a single wrong row
cannot hide in a tensor of a million rows. dalpha and dbeta hold one scalar
per token and head and are checked whole.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
import oracle
from bilinear_rnn_amd.inputs import WORKLOADS, bf16_bits, bf16_bits_to_f32, make_inputs
from _util import dev_inputs, rel_l2, to_np

pytestmark = pytest.mark.gpu

GATE = 1e-5        # fp32 inputs
GATE_BF16 = 5e-5   # bf16 inputs: hi / lo bf16 matrix-core products
DD_COND = 5e-5     # bf16 inputs, dd: error relative to sum |dq (.) k| of the head
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dd", "ds0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def wl(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


def cotangents(inp, seed, with_dsf=True):
    """dL/do (rounded to the input dtype) and dL/dS_final, seeded."""
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(inp.v.shape, dtype=np.float32)
    do_bits = None
    if inp.dtype == "bf16":
        do_bits = bf16_bits(do)
        do = bf16_bits_to_f32(do_bits)
    N, H, V, K = inp.num_seqs, inp.v.shape[2], inp.v.shape[3], inp.q.shape[3]
    dsf = rng.standard_normal((N, H, V, K), dtype=np.float32) if with_dsf else None
    return do, do_bits, dsf


def run_bwd(inp, do, do_bits, dsf):
    t = dev_inputs(inp)
    if do_bits is not None:
        dod = torch.from_numpy(np.ascontiguousarray(do_bits).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dod = torch.from_numpy(np.ascontiguousarray(do)).cuda()
    dsfd = None if dsf is None else torch.from_numpy(dsf).cuda()
    g = comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], dod, t["initial_state"],
                        t["cu_seqlens"], dsfd)
    torch.cuda.synchronize()
    g["ds0"] = g.pop("dinitial_state")
    return {key: to_np(x) for key, x in g.items()}


def oracle_bwd(inp, do, dsf):
    """The reverse-mode oracle; the C one (equal to the numpy one to 1e-12 on
    the CPU pins) for anything beyond a few thousand head-tokens."""
    if inp.q.shape[0] * inp.q.shape[1] * inp.q.shape[2] > 4096:
        return oracle.comba_backward_c(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.d, do, inp.s0, dsf,
                                       inp.cu_seqlens)
    return oracle.comba_backward(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.d, do, inp.s0, dsf, inp.cu_seqlens)


def check(got, ref, inp, names=NAMES):
    bf16 = inp.dtype == "bf16"
    gate = GATE_BF16 if bf16 else GATE
    errs = {key: rel_l2(got[key], ref[key]) for key in names if not (bf16 and key == "dd")}
    limits = dict.fromkeys(errs, gate)
    if bf16 and "dd" in names:
        # per head: sum over batch rows, tokens and keys of |dq (.) k|
        scale = np.abs(np.asarray(ref["dq"], np.float64) * np.asarray(inp.k, np.float64)).sum(axis=(0, 1, 3))
        errs["dd/cond"] = float(np.max(np.abs(np.asarray(got["dd"], np.float64) - ref["dd"]) / scale))
        limits["dd/cond"] = DD_COND
    for key in ("dq", "dk", "dv", "ds0"):
        if key in names:
            errs[key + "/row"] = oracle.row_rel_err(got[key], ref[key])
            limits[key + "/row"] = 10 * gate
    print(" ".join(f"{key}={e:.2e}" for key, e in errs.items()), flush=True)
    bad = {key: e for key, e in errs.items() if not e <= limits[key]}
    assert not bad, bad


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 64, 150])
def test_fp32_backward_shapes(K, V, T):
    inp = make_inputs(wl("tiny_fp32", K=K, V=V, B=2, H=2), T=T, s0_std=0.1, seed=71)
    do, do_bits, dsf = cotangents(inp, 72)
    check(run_bwd(inp, do, do_bits, dsf), oracle_bwd(inp, do, dsf), inp)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T,s0", [(130, 0.02), (64, 0.0), (1, 0.02), (300, 0.02)])
def test_bf16_backward_shapes(K, V, T, s0):
    inp = make_inputs(wl("layer_340m", K=K, V=V, B=2, H=2), T=T, s0_std=s0, seed=73)
    do, do_bits, dsf = cotangents(inp, 74, with_dsf=s0 > 0)
    check(run_bwd(inp, do, do_bits, dsf), oracle_bwd(inp, do, dsf), inp)


def test_bf16_backward_many_chunks():
    """Eight chunks of the 340M-layer head shape: the reverse scan's carry."""
    inp = make_inputs(wl("layer_340m", B=1, H=2), T=512, s0_std=0.02, seed=75)
    do, do_bits, dsf = cotangents(inp, 76)
    check(run_bwd(inp, do, do_bits, dsf), oracle_bwd(inp, do, dsf), inp)


def test_backward_varlen_edge_lengths():
    lengths = np.array([16, 70, 1, 0, 130, 64, 0, 63, 65])
    inp = make_inputs(wl("varlen", H=3), lengths=lengths, s0_std=0.05, seed=77)
    do, do_bits, dsf = cotangents(inp, 78)
    got = run_bwd(inp, do, do_bits, dsf)
    check(got, oracle_bwd(inp, do, dsf), inp)
    # an empty sequence passes its final-state gradient straight to its initial state
    for n in np.flatnonzero(lengths == 0):
        np.testing.assert_array_equal(got["ds0"][n], dsf[n].astype(np.float64))


def test_backward_without_final_state_gradient():
    inp = make_inputs(wl("layer_340m", B=2, H=2), T=200, s0_std=0.02, seed=79)
    do, do_bits, _ = cotangents(inp, 80, with_dsf=False)
    check(run_bwd(inp, do, do_bits, None), oracle_bwd(inp, do, None), inp)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_extreme_gates(dtype):
    """alpha from 1e-6 to exactly 1 and beta exactly 0 and 1, mixed within every
    chunk (in-chunk decay products far below fp32's range)."""
    base = wl("layer_340m", K=64, V=64, B=2, H=2) if dtype == "bf16" else wl("tiny_fp32", B=2, H=2)
    inp = make_inputs(base, T=150, s0_std=0.05, seed=85)
    rng = np.random.default_rng(86)
    shape = inp.alpha.shape
    alpha = np.choose(rng.integers(0, 4, shape), [np.full(shape, 1e-6), np.ones(shape),
                                                  rng.uniform(0.0, 1.0, shape), np.full(shape, 0.5)])
    beta = np.choose(rng.integers(0, 3, shape), [np.zeros(shape), np.ones(shape), rng.uniform(0.0, 1.0, shape)])
    inp = dataclasses.replace(inp, alpha=alpha.astype(np.float32), beta=beta.astype(np.float32))
    do, do_bits, dsf = cotangents(inp, 87)
    got = run_bwd(inp, do, do_bits, dsf)
    assert all(np.isfinite(x).all() for x in got.values())
    check(got, oracle_bwd(inp, do, dsf), inp)


CACHED_CASES = [
    ("layer_340m", dict(K=128, V=128, B=2, H=2), dict(T=300, s0_std=0.02), None),
    ("layer_340m", dict(K=64, V=128, B=3, H=2), dict(T=65, s0_std=0.0), None),
    ("tiny_fp32", dict(K=128, V=64, B=2, H=2), dict(T=150, s0_std=0.1), None),
    ("varlen", dict(H=3), dict(s0_std=0.05), np.array([16, 70, 1, 0, 130, 64, 0, 63, 65])),
]


@pytest.mark.parametrize("case", range(len(CACHED_CASES)))
def test_cached_chunk_states_backward(case):
    """The forward that keeps the chunk states writes the plain forward's
    output and final state, and the backward that reads them gives the
    recomputing backward's gradients, bit for bit (the same state chain
    either way), and so passes the oracle gates."""
    name, wkw, ikw, lengths = CACHED_CASES[case]
    inp = make_inputs(wl(name, **wkw), lengths=lengths, seed=90 + case, **ikw)
    print(f"cached states: {name} {wkw} {ikw} lengths={lengths}", flush=True)
    do, do_bits, dsf = cotangents(inp, 95 + case)
    t = dev_inputs(inp)
    B, T, H, K = inp.q.shape
    V = inp.v.shape[-1]
    nseq = inp.num_seqs if inp.cu_seqlens is not None else 0
    cs = torch.empty((comba.chunk_states_size(B, T, H, K, V, nseq) // 4,), dtype=torch.float32, device="cuda")
    o1, s1 = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                             t["cu_seqlens"])
    o2, s2 = comba.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"],
                             t["cu_seqlens"], chunk_states=cs)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    dod = (torch.from_numpy(np.ascontiguousarray(do_bits).view(np.int16)).view(torch.bfloat16).cuda()
           if do_bits is not None else torch.from_numpy(np.ascontiguousarray(do)).cuda())
    dsfd = torch.from_numpy(dsf).cuda()
    g1 = comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], dod, t["initial_state"],
                         t["cu_seqlens"], dsfd)
    g2 = comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], dod, t["initial_state"],
                         t["cu_seqlens"], dsfd, chunk_states=cs)
    torch.cuda.synchronize()
    for key in g1:
        assert torch.equal(g1[key], g2[key]), key
    got = {key: to_np(x) for key, x in g2.items()}
    got["ds0"] = got.pop("dinitial_state")
    check(got, oracle_bwd(inp, do, dsf), inp)


def test_backward_deterministic():
    inp = make_inputs(wl("layer_340m", B=2, H=2), T=333, s0_std=0.02, seed=81)
    do, do_bits, dsf = cotangents(inp, 82)
    g1 = run_bwd(inp, do, do_bits, dsf)
    g2 = run_bwd(inp, do, do_bits, dsf)
    for key in NAMES:
        np.testing.assert_array_equal(g1[key], g2[key])


def test_backward_layer_1p3b_full_size():
    """The 1.3B layer at full size (B=8, T=4096, H=16); the C reverse-mode
    oracle checks every gradient of every (batch row, head) pair."""
    w = WORKLOADS["layer_1p3b"]
    inp = make_inputs(w)
    do, do_bits, dsf = cotangents(inp, 83)
    got = run_bwd(inp, do, do_bits, dsf)
    assert all(np.isfinite(x).all() for x in got.values())
    check(got, oracle_bwd(inp, do, dsf), inp)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_workspace_contents_do_not_matter(dtype):
    """The prep kernel stores only the 16x16 blocks of Tinv and P on or below
    the diagonal, and every buffer of the workspace is written before it is
    read: a workspace filled with NaN bytes gives the same gradients, bit for
    bit, as a zeroed one (ragged tail, packed batch with an empty sequence)."""
    for case in ("ragged", "packed"):
        if case == "ragged":
            inp = make_inputs(wl("layer_340m", B=2, H=2, dtype=dtype), T=150, s0_std=0.02, seed=91)
        else:
            inp = make_inputs(wl("varlen", H=2, dtype=dtype), lengths=np.array([70, 0, 129, 1]), s0_std=0.02,
                              seed=92)
        do, do_bits, dsf = cotangents(inp, 93)
        t = dev_inputs(inp)
        if do_bits is not None:
            dod = torch.from_numpy(np.ascontiguousarray(do_bits).view(np.int16)).view(torch.bfloat16).cuda()
        else:
            dod = torch.from_numpy(np.ascontiguousarray(do)).cuda()
        dsfd = torch.from_numpy(dsf).cuda()
        B, T, H, K = inp.q.shape
        V = inp.v.shape[3]
        nseq = inp.num_seqs if inp.cu_seqlens is not None else 0
        nws = int(comba.lib().comba_chunk_bwd_workspace_size(B, T, H, K, V, nseq))
        out = []
        for fill in (0x00, 0xFF):
            ws = torch.full((nws,), fill, dtype=torch.uint8, device="cuda")
            g = comba.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], dod, t["initial_state"],
                                t["cu_seqlens"], dsfd, workspace=ws)
            torch.cuda.synchronize()
            out.append({key: x.clone() for key, x in g.items()})
        for key in out[0]:
            assert torch.equal(out[0][key], out[1][key]), (case, key)
        got = {key: to_np(x) for key, x in out[1].items()}
        got["ds0"] = got.pop("dinitial_state")
        check(got, oracle_bwd(inp, do, dsf), inp)
