"""Seeded synthetic inputs for the Comba mixer workloads.

This module only draws random numbers and arranges them into the tensors the
mixer consumes. It holds none of the recurrence's arithmetic, so both the
CPU oracle (through the tests) and the HIP path are fed from it.

Workloads are layer shapes of the 340M and 1.3B Comba language models
(Comba arXiv abstract; PaperWeekly write-up, section on experiments). The
language-model corpora those models were trained on are not used: every
tensor is synthetic, with the distributions stated per workload below.

Draw order for one workload, from ``numpy.random.Generator(PCG64(seed))``:
lengths (variable-length workloads only) -> q -> k -> v -> alpha logits ->
beta logits -> initial state. All draws are float32. q and k are
L2-normalised per (token, head) in float32 and then rounded to the workload's
dtype; alpha = sigmoid(logit) and beta = sigmoid(logit) stay float32.

With ``raw=True`` the same draws are returned before those two steps: q and
k un-normalised (rounded to the workload's dtype), alpha and beta holding the
logits. That is the input of the fused entry points, which normalise and
apply the sigmoid themselves.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CHUNK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    T: int
    K: int
    V: int
    dtype: str                      # "fp32" or "bf16" for q, k, v and o
    alpha_mu: float = 3.0           # alpha = sigmoid(N(alpha_mu, 0.5))
    d_value: float = 0.5            # output-correction factor, same for all heads
    s0_std: float = 0.0             # 0 means no initial state (zeros)
    num_seqs: int = 0               # > 0: packed variable-length batch (B == 1)
    len_mu: float = 6.0             # lognormal parameters of sequence lengths
    len_sigma: float = 1.0
    len_min: int = 16
    len_max: int = 4096
    decode: bool = False            # one token per sequence (recurrent step)


WORKLOADS = {
    # tiny fp32 forward, used for exactness checks against the oracle
    "tiny_fp32": Workload("tiny_fp32", 1000, B=1, H=2, T=256, K=64, V=64, dtype="fp32"),
    # one mixer layer of the 340M model
    "layer_340m": Workload("layer_340m", 1001, B=4, H=16, T=2048, K=128, V=128, dtype="bf16"),
    # one mixer layer of the 1.3B model, non-zero initial state (throughput workload)
    "layer_1p3b": Workload("layer_1p3b", 1002, B=8, H=16, T=4096, K=128, V=128, dtype="bf16",
                           s0_std=0.02),
    # a single 64K-token sequence with slow decay
    "long_context": Workload("long_context", 1003, B=1, H=16, T=65536, K=128, V=128,
                             dtype="bf16", alpha_mu=5.0),
    # 64 packed sequences of lognormal length
    "varlen": Workload("varlen", 1004, B=1, H=32, T=0, K=64, V=64, dtype="bf16", num_seqs=64),
    # single-token decode for 256 sequences with the state resident in device memory
    "decode": Workload("decode", 1005, B=256, H=16, T=1, K=128, V=128, dtype="bf16",
                       s0_std=0.02, decode=True),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs here are finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x.astype(np.float32)))).astype(np.float32)


def varlen_lengths(rng: np.random.Generator, w: Workload) -> np.ndarray:
    raw = rng.lognormal(mean=w.len_mu, sigma=w.len_sigma, size=w.num_seqs)
    return np.clip(np.rint(raw), w.len_min, w.len_max).astype(np.int64)


@dataclasses.dataclass
class Inputs:
    """One batch. Floating tensors are float32 numpy arrays holding exactly the
    values the device receives (bf16 workloads are already rounded);
    ``*_bits`` carry the bf16 bit patterns for the device copy."""
    q: np.ndarray                   # [B, T, Hqk, K] (Hqk = H unless q / k heads are shared)
    k: np.ndarray                   # [B, T, Hqk, K]
    v: np.ndarray                   # [B, T, H, V]
    alpha: np.ndarray               # [B, T, H]
    beta: np.ndarray                # [B, T, H]
    d: np.ndarray                   # [H]
    s0: Optional[np.ndarray]        # [N, H, V, K] or None
    cu_seqlens: Optional[np.ndarray]  # int32 [N + 1] or None
    dtype: str
    raw: bool = False               # q, k un-normalised; alpha, beta are logits
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else len(self.cu_seqlens) - 1


def make_inputs(w: Workload, *, B: Optional[int] = None, T: Optional[int] = None,
                H: Optional[int] = None, num_seqs: Optional[int] = None,
                seed: Optional[int] = None, s0_std: Optional[float] = None,
                lengths: Optional[np.ndarray] = None, raw: bool = False,
                qk_heads: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``w``; keyword overrides shrink it for tests.

    ``qk_heads`` (a divisor of H) draws q and k with that many heads, shared by
    consecutive value heads; v, alpha, beta, d and the state keep H heads."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    seed = w.seed if seed is None else seed
    s0_std = w.s0_std if s0_std is None else s0_std
    rng = np.random.Generator(np.random.PCG64(seed))

    cu = None
    nseq = B
    if w.num_seqs or lengths is not None or num_seqs is not None:
        if lengths is None:
            wl = dataclasses.replace(w, num_seqs=num_seqs or w.num_seqs)
            lengths = varlen_lengths(rng, wl)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T, nseq = 1, int(cu[-1]), len(lengths)

    K, V = w.K, w.V
    Hk = H if qk_heads is None else qk_heads
    assert H % Hk == 0
    q = rng.standard_normal((B, T, Hk, K), dtype=np.float32)
    k = rng.standard_normal((B, T, Hk, K), dtype=np.float32)
    v = rng.standard_normal((B, T, H, V), dtype=np.float32)
    a_logit = rng.standard_normal((B, T, H), dtype=np.float32) * np.float32(0.5) + np.float32(w.alpha_mu)
    b_logit = rng.standard_normal((B, T, H), dtype=np.float32)
    s0 = None
    if s0_std > 0:
        s0 = rng.standard_normal((nseq, H, V, K), dtype=np.float32) * np.float32(s0_std)

    if raw:
        alpha, beta = a_logit, b_logit
    else:
        q, k = _l2_normalise(q), _l2_normalise(k)
        alpha, beta = _sigmoid(a_logit), _sigmoid(b_logit)
    out = Inputs(q=q, k=k, v=v, alpha=alpha, beta=beta,
                 d=np.full((H,), w.d_value, dtype=np.float32), s0=s0,
                 cu_seqlens=cu, dtype=w.dtype, raw=raw)
    if w.dtype == "bf16":
        out.q_bits, out.k_bits, out.v_bits = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        out.q = bf16_bits_to_f32(out.q_bits)
        out.k = bf16_bits_to_f32(out.k_bits)
        out.v = bf16_bits_to_f32(out.v_bits)
    return out


def head_tokens(inp: Inputs) -> int:
    B, T, H, _ = inp.q.shape
    return B * T * H
