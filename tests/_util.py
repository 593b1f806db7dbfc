"""Helpers shared by the tests: device copies of seeded inputs and oracle calls."""
import numpy as np
import torch

import oracle
from oracle import rel_l2  # noqa: F401


def dev_inputs(inp, device="cuda"):
    """Device tensors holding exactly the values in ``inp`` (bf16 via its bit patterns)."""
    def floats(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    if inp.dtype == "bf16":
        def qkv(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
        q, k, v = qkv(inp.q_bits), qkv(inp.k_bits), qkv(inp.v_bits)
    else:
        q, k, v = floats(inp.q), floats(inp.k), floats(inp.v)
    out = dict(q=q, k=k, v=v, alpha=floats(inp.alpha), beta=floats(inp.beta), d=floats(inp.d))
    out["initial_state"] = None if inp.s0 is None else floats(inp.s0)
    out["cu_seqlens"] = None if inp.cu_seqlens is None else torch.from_numpy(
        np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)).to(device)
    return out


def oracle_of(inp, heads=None, seqs=None, nthreads=0, gate_logits=None, qk_l2norm=None):
    """fp64 oracle on the exact inputs, optionally restricted to some heads and
    batch rows (full sequences). Returns (o, final_state) in the same order.

    For raw inputs (``inp.raw``) the oracle's own input steps run first: gate
    logits and q/k normalisation both default to on, each can be switched off."""
    q, k, v, a, b, d, s0 = inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.d, inp.s0
    gate_logits = inp.raw if gate_logits is None else gate_logits
    qk_l2norm = inp.raw if qk_l2norm is None else qk_l2norm
    if q.shape[2] != v.shape[2]:  # q / k heads shared by several value heads
        q, k = oracle.expand_shared_qk(q, k, v.shape[2])
    cu = inp.cu_seqlens
    if seqs is not None:
        assert cu is None
        q, k, v, a, b = (x[seqs] for x in (q, k, v, a, b))
        s0 = None if s0 is None else s0[seqs]
    if heads is not None:
        q, k, v, a, b = (x[:, :, heads] for x in (q, k, v, a, b))
        d = d[heads]
        s0 = None if s0 is None else s0[:, heads]
    if gate_logits or qk_l2norm:
        q, k, a, b = oracle.fused_inputs(q, k, a, b, gate_logits=gate_logits, qk_l2norm=qk_l2norm)
    return oracle.comba_forward_c(q, k, v, a, b, d, s0, cu, nthreads=nthreads)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# --- parity gates ------------------------------------------------------------------------
# Each gate is a pair: rel-L2 over the whole tensor, and the largest relative
# error of one row (the last axis: one token-head row of o or of a gradient,
# one value channel of a state; oracle.row_rel_err). Row gates:
#   - bf16 output: rounding to nearest bf16 moves each element by at most
#     2^-8 of its magnitude, so a row by at most 2^-8 of its norm; 1e-3 more
#     covers the arithmetic before rounding (ten times its whole-tensor gate);
#   - fp32 outputs: ten times the whole-tensor gate of the same arithmetic,
#     room for the tail rows of a tensor of a million rows whose typical row
#     sits at the whole-tensor figure.
# A row that is wrong altogether scores about 1 and fails every one of them.
import collections
import functools

Gates = collections.namedtuple("Gates", "whole row")
BF16 = Gates(2e-3, 2.0 ** -8 + 1e-3)          # bf16 q/k/v, bf16 o
FP32 = Gates(1e-5, 1e-4)                      # fp32 q/k/v, fp32 o and state
BF16_IN_FP32_OUT = Gates(1e-4, 1e-3)          # bf16 q/k/v, fp32 o
STATE_BF16 = Gates(2e-3, 1e-3)                # fp32 state from bf16 q/k/v


def assert_close(got, ref, gates, what=""):
    """Whole-tensor rel-L2 and per-row bound of ``got`` against the oracle's
    ``ref``; non-finite values fail both."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    e = rel_l2(got, ref)
    r = oracle.row_rel_err(got, ref)
    print(f"{what}: rel-L2 {e:.3e} (gate {gates.whole:.1e}), worst row {r:.3e} (gate {gates.row:.1e})", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert e <= gates.whole, f"{what}: rel-L2 {e:.3e} > {gates.whole:.1e}"
    assert r <= gates.row, f"{what}: worst row {r:.3e} > {gates.row:.1e}"


_CACHE = {}


def cached(key, make):
    """A value computed once per test session (seeded full-size inputs and
    their oracle results, shared by several tests)."""
    if key not in _CACHE:
        _CACHE[key] = make()
    return _CACHE[key]


def full_inputs(name, **kw):
    from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
    return cached(("inputs", name, tuple(sorted(kw.items()))), lambda: make_inputs(WORKLOADS[name], **kw))


def full_oracle(name, **kw):
    """Oracle (o, final_state) over the whole of a named workload."""
    return cached(("oracle", name, tuple(sorted(kw.items()))), lambda: oracle_of(full_inputs(name, **kw)))
