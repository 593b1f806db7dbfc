"""Plain fp64 CPU oracle for the Comba mixer. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The library's device path never calls it.

What is computed (Comba: Improving Bilinear RNNs with Closed-loop Control;
PaperWeekly write-up, section "Comba架构：基于闭环控制理论"; arXiv abstract):
the state transition is scalar-plus-low-rank, the feedback vector is the key,
and the same key feedback corrects first the value and then the output. The
write-up's printed recurrence was lost from the page text, so the oracle
takes the plainest form consistent with those three facts:

    S_t = S_{t-1} (alpha_t I - beta_t k_t k_t^T) + beta_t v_t k_t^T
        = alpha_t S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T
    o_t = S_t (q_t - d k_t)

S_t has one row per value channel (V x K). alpha_t, beta_t are scalars per
(token, head) and d is one scalar per head. No query scale is applied.

Tensor layouts (row-major): q, k [B, T, H, K]; v [B, T, H, V];
alpha, beta [B, T, H]; d [H]; state [N, H, V, K]. With ``cu_seqlens``
(int [N + 1], B == 1) sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
and starts from its own initial state; otherwise N == B.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _segments(B: int, T: int, cu_seqlens):
    """Yield (n, b, t0, t1) for every sequence."""
    if cu_seqlens is None:
        for b in range(B):
            yield b, b, 0, T
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        for n in range(len(cu) - 1):
            yield n, 0, int(cu[n]), int(cu[n + 1])


def comba_forward(q, k, v, alpha, beta, d, s0=None, cu_seqlens=None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token recurrence in fp64 (the definition above, rank-1 form).

    Returns (o [B, T, H, V], final_state [N, H, V, K]), both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, V), dtype=np.float64)
    s_final = np.zeros((N, H, V, K), dtype=np.float64)
    for n, b, t0, t1 in _segments(B, T, cu_seqlens):
        S = np.zeros((H, V, K)) if s0 is None else np.array(s0[n], dtype=np.float64)
        for t in range(t0, t1):
            kk = k[b, t]                                   # [H, K]
            u = v[b, t] - np.einsum("hvk,hk->hv", S, kk)   # value corrected by key feedback
            S = alpha[b, t][:, None, None] * S + beta[b, t][:, None, None] * u[:, :, None] * kk[:, None, :]
            qt = q[b, t] - d[:, None] * kk                 # output corrected by the same feedback
            o[b, t] = np.einsum("hvk,hk->hv", S, qt)
        s_final[n] = S
    return o, s_final


def comba_forward_chunked(q, k, v, alpha, beta, d, s0=None, cu_seqlens=None,
                          chunk: int = 64, return_intermediates: bool = False):
    """Chunk-wise form in fp64: recurrent across chunks, parallel inside one.

    The write-up (section "硬件高效的分块并行计算") evaluates Comba chunk by
    chunk through intermediates W and U, with a single matrix inverse per
    chunk. Written out for one chunk of n tokens with incoming state
    h = S^T (K x V), g = log alpha, G the inclusive and Gx the exclusive
    within-chunk cumulative sums of g:

        A[s, r] = beta_s exp(Gx_s - G_r) (k_s . k_r)   for r < s, else 0
        Tinv    = (I + A)^-1                           (unit lower triangular)
        W       = Tinv diag(beta * exp(Gx)) K          U = Tinv diag(beta) V
        Ubar    = U - W h                  (row s equals beta_s (v_s - S_{s-1} k_s))
        O       = diag(exp(G)) (Q - dK) h + [((Q - dK) K^T) * M] Ubar,
                  M[t, s] = exp(G_t - G_s) for s <= t, else 0
        h'      = exp(G_n) h + K^T diag(exp(G_n - G)) Ubar

    Equal to :func:`comba_forward` up to rounding. With
    ``return_intermediates`` it also returns, per (sequence, head), a list of
    dicts holding the per-chunk Tinv, W, U, Ubar and incoming h.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, V), dtype=np.float64)
    s_final = np.zeros((N, H, V, K), dtype=np.float64)
    inter = {}
    for n, b, t0, t1 in _segments(B, T, cu_seqlens):
        for hh in range(H):
            h = np.zeros((K, V)) if s0 is None else np.array(s0[n, hh], dtype=np.float64).T
            recs = []
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                Q, Kc, Vc = q[b, c0:c1, hh], k[b, c0:c1, hh], v[b, c0:c1, hh]
                bet = beta[b, c0:c1, hh]
                g = np.log(alpha[b, c0:c1, hh])
                G = np.cumsum(g)
                Gx = G - g
                nrow = c1 - c0
                low = np.tril(np.ones((nrow, nrow), dtype=bool), -1)
                A = np.where(low, bet[:, None] * np.exp(Gx[:, None] - G[None, :]) * (Kc @ Kc.T), 0.0)
                Tinv = np.linalg.solve(np.eye(nrow) + A, np.eye(nrow))
                W = Tinv @ ((bet * np.exp(Gx))[:, None] * Kc)
                U = Tinv @ (bet[:, None] * Vc)
                Ubar = U - W @ h
                Qt = Q - d[hh] * Kc
                M = np.where(np.tril(np.ones((nrow, nrow), dtype=bool)),
                             np.exp(np.minimum(G[:, None] - G[None, :], 0.0)), 0.0)
                o[b, c0:c1, hh] = np.exp(G)[:, None] * (Qt @ h) + ((Qt @ Kc.T) * M) @ Ubar
                if return_intermediates:
                    recs.append(dict(Tinv=Tinv, W=W, U=U, Ubar=Ubar, h=h.copy()))
                h = np.exp(G[-1]) * h + Kc.T @ (np.exp(G[-1] - G)[:, None] * Ubar)
            s_final[n, hh] = h.T
            if return_intermediates:
                inter[(n, hh)] = recs
    if return_intermediates:
        return o, s_final, inter
    return o, s_final


def comba_backward(q, k, v, alpha, beta, d, do, s0=None, dsf=None, cu_seqlens=None):
    """Gradients of the token recurrence of :func:`comba_forward`, in fp64.

    Reverse-mode differentiation of the definition, one token at a time and
    backwards, for a loss L with dL/do = ``do`` [B, T, H, V] and dL/dS_final =
    ``dsf`` [N, H, V, K] (None: 0). Per head, with S_t the V x K state, a_t =
    S_{t-1} k_t, u_t = v_t - a_t, S_t = alpha_t S_{t-1} + beta_t u_t k_t^T,
    qt_t = q_t - d k_t and o_t = S_t qt_t, and X the running dL/dS_t:

        X     += do_t qt_t^T                 (o_t reads S_t)
        dqt    = S_t^T do_t   ->  dq_t = dqt, dk_t -= d dqt, dd -= dqt . k_t
        dalpha_t = <X, S_{t-1}>,   dbeta_t = u_t . (X k_t)
        du     = beta_t X k_t     ->  dv_t = du, da = -du
        dk_t  += beta_t X^T u_t + S_{t-1}^T da
        X      = alpha_t X + da k_t^T        (dL/dS_{t-1})

    and dS_0 is X after the first token. The states S_{t-1} are kept from a
    forward pass over the sequence.

    Returns a dict of float64 arrays: dq, dk, dv, dalpha, dbeta ([B, T, H, ...]),
    dd [H] (summed over the batch) and ds0 [N, H, V, K].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    g = {name: np.zeros_like(x) for name, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha),
                                                  ("dbeta", beta))}
    g["dd"] = np.zeros((H,))
    g["ds0"] = np.zeros((N, H, V, K))
    for n, b, t0, t1 in _segments(B, T, cu_seqlens):
        S = np.zeros((H, V, K)) if s0 is None else np.asarray(s0[n], dtype=np.float64).copy()
        states = [S]
        for t in range(t0, t1):  # forward, keeping every state
            kt = k[b, t]
            ut = v[b, t] - np.einsum("hvk,hk->hv", S, kt)
            S = S * alpha[b, t][:, None, None] + (beta[b, t][:, None] * ut)[:, :, None] * kt[:, None, :]
            states.append(S)
        X = np.zeros((H, V, K)) if dsf is None else np.array(dsf[n], dtype=np.float64)
        for t in range(t1 - 1, t0 - 1, -1):
            S_prev, S_t = states[t - t0], states[t - t0 + 1]
            kk, qv, al, be = k[b, t], q[b, t], alpha[b, t], beta[b, t]
            qt = qv - d[:, None] * kk
            dot = do[b, t]                                           # [H, V]
            X = X + dot[:, :, None] * qt[:, None, :]
            dqt = np.einsum("hvk,hv->hk", S_t, dot)
            g["dq"][b, t] += dqt
            g["dk"][b, t] -= d[:, None] * dqt
            g["dd"] -= np.einsum("hk,hk->h", dqt, kk)
            ur = v[b, t] - np.einsum("hvk,hk->hv", S_prev, kk)
            Xk = np.einsum("hvk,hk->hv", X, kk)
            g["dalpha"][b, t] += np.einsum("hvk,hvk->h", X, S_prev)
            g["dbeta"][b, t] += np.einsum("hv,hv->h", ur, Xk)
            du = be[:, None] * Xk
            g["dv"][b, t] += du
            da = -du
            g["dk"][b, t] += be[:, None] * np.einsum("hvk,hv->hk", X, ur) + np.einsum("hvk,hv->hk", S_prev, da)
            X = al[:, None, None] * X + da[:, :, None] * kk[:, None, :]
        g["ds0"][n] = X
    return g


def expand_shared_qk(q, k, H: int):
    """q, k with Hqk heads shared by H value heads -> one q, k head per value head.

    The Comba write-up (section "硬件高效的分块并行计算", last paragraph) has its
    Mamba-form models share one query and key across value heads, like
    multi-value attention. Value head h reads q / k head h // (H // Hqk):
    consecutive value heads share a head. With Hqk == H this is the identity.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    Hk = q.shape[2]
    if H % Hk != 0:
        raise ValueError("the q/k head count must divide H")
    return np.repeat(q, H // Hk, axis=2), np.repeat(k, H // Hk, axis=2)


L2NORM_EPS = 1e-6


def fused_inputs(q, k, alpha, beta, gate_logits: bool = False, qk_l2norm: bool = False):
    """Input-side steps that the fused entry points take inside their kernels, in fp64.

    - ``qk_l2norm``: q and k are L2-normalised per (token, head), x / sqrt(sum x^2 + eps)
      with eps = 1e-6. The pages do not spell this step out; it is the plainest
      reading of the unit-norm keys that keep the transition alpha I - beta k k^T
      of the Comba write-up (section "Comba架构") a contraction for beta <= 1.
    - ``gate_logits``: alpha and beta arrive as logits and become sigmoid(logit),
      the gate of the GLA/KDA comparison (sections 2.1 and 3.1) that CARVE
      evaluates inside its kernel (GDN-2/CARVE summary, section 2.3).

    Returns (q, k, alpha, beta) as float64 arrays ready for :func:`comba_forward`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if qk_l2norm:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + L2NORM_EPS)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + L2NORM_EPS)
    if gate_logits:
        with np.errstate(over="ignore"):
            alpha = 1.0 / (1.0 + np.exp(-alpha))
            beta = 1.0 / (1.0 + np.exp(-beta))
    return q, k, alpha, beta


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if not np.isfinite(num):
        return float("inf")
    return float(num / den) if den > 0 else float(num)


def row_rel_err(x, ref, floor: float = 1e-2) -> float:
    """Largest relative error of one row, rows being the last axis, in fp64.

    Row i scores ||x_i - ref_i||_2 / max(||ref_i||_2, floor * r), where r is
    the root mean square of the reference row norms: a row is judged against
    its own norm unless that norm is below ``floor`` times the typical one.
    A whole-tensor rel-L2 spreads one wrong row over all of them; this does not.
    Any non-finite value in x gives inf.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if x.size == 0:
        return 0.0
    if not np.isfinite(x).all():
        return float("inf")
    n = x.shape[-1]
    xr, rr = x.reshape(-1, n), ref.reshape(-1, n)
    rn = np.sqrt(np.sum(rr * rr, axis=1))
    en = np.sqrt(np.sum((xr - rr) ** 2, axis=1))
    typical = float(np.sqrt(np.mean(rn * rn)))
    den = np.maximum(rn, floor * typical)
    if typical == 0.0:
        return float(np.max(en))
    return float(np.max(en / den))
