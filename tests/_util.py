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
