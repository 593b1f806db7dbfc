"""The oracle pins catch plausible mistakes.

Each case plants one mistake in a scratch copy of the numpy oracle (a sign,
a dropped term, a wrong index or decay, a transposed operand) and runs the
pin suite against that copy in a subprocess: at least one pin must fail.
CPU only; the repository's own oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    # token loop (definition of the recurrence)
    "erase_sign": ("u = v[b, t] - np.einsum", "u = v[b, t] + np.einsum"),
    "no_decay": ("S = alpha[b, t][:, None, None] * S + ", "S = S + "),
    "correction_sign": ("qt = q[b, t] - d[:, None] * kk", "qt = q[b, t] + d[:, None] * kk"),
    "no_correction": ("qt = q[b, t] - d[:, None] * kk", "qt = q[b, t] + 0 * kk"),
    "transposed_write": ("u[:, :, None] * kk[:, None, :]", "kk[:, :, None] * u[:, None, :]"),
    "wrong_head_d": ("d[:, None] * kk  ", "d[::-1][:, None] * kk  "),
    "no_initial_state": ("S = np.zeros((H, V, K)) if s0 is None else np.array(s0[n], dtype=np.float64)",
                         "S = np.zeros((H, V, K))"),
    "output_before_update": ('o[b, t] = np.einsum("hvk,hk->hv", S, qt)',
                             'o[b, t] = np.einsum("hvk,hk->hv", S - beta[b, t][:, None, None] * u[:, :, None]'
                             ' * kk[:, None, :], qt)'),
    # chunk form
    "chunk_A_inclusive_decay": ("np.exp(Gx[:, None] - G[None, :]) * (Kc @ Kc.T)",
                                "np.exp(G[:, None] - G[None, :]) * (Kc @ Kc.T)"),
    "chunk_mask_strict": ("M = np.where(np.tril(np.ones((nrow, nrow), dtype=bool)),",
                          "M = np.where(np.tril(np.ones((nrow, nrow), dtype=bool), -1),"),
    "chunk_state_weights": ("Kc.T @ (np.exp(G[-1] - G)[:, None] * Ubar)",
                            "Kc.T @ (np.exp(G[-1] - Gx)[:, None] * Ubar)"),
    "chunk_W_without_decay": ("W = Tinv @ ((bet * np.exp(Gx))[:, None] * Kc)", "W = Tinv @ (bet[:, None] * Kc)"),
    # input-side steps of the fused entry points
    "l2norm_eps_outside_sqrt": ("q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + L2NORM_EPS)",
                                "q = q / (np.sqrt(np.sum(q * q, axis=-1, keepdims=True)) + L2NORM_EPS)"),
    "l2norm_k_by_q_norm": ("k = k / np.sqrt(np.sum(k * k, axis=-1",
                           "k = k / np.sqrt(np.sum(q * q, axis=-1"),
    "sigmoid_sign": ("alpha = 1.0 / (1.0 + np.exp(-alpha))", "alpha = 1.0 / (1.0 + np.exp(alpha))"),
    # backward
    "bwd_no_feedback_term": ("X = al[:, None, None] * X + da[:, :, None] * kk[:, None, :]",
                             "X = al[:, None, None] * X"),
    "bwd_dalpha_from_new_state": ('g["dalpha"][b, t] += np.einsum("hvk,hvk->h", X, S_prev)',
                                  'g["dalpha"][b, t] += np.einsum("hvk,hvk->h", X, S_t)'),
    "bwd_dk_write_sign": ('g["dk"][b, t] += be[:, None] * np.einsum("hvk,hv->hk", X, ur) +',
                          'g["dk"][b, t] -= be[:, None] * np.einsum("hvk,hv->hk", X, ur) -'),
    "bwd_no_correction_in_dk": ('g["dk"][b, t] -= d[:, None] * dqt', 'g["dk"][b, t] -= 0 * dqt'),
    # shared q / k heads
    "shared_qk_interleaved": ("return np.repeat(q, H // Hk, axis=2), np.repeat(k, H // Hk, axis=2)",
                              "return np.tile(q, (1, 1, H // Hk, 1)), np.tile(k, (1, 1, H // Hk, 1))"),
}


def _run_pins_on_copy(tmp_path, before=None, after=None):
    for d in ("oracle", "tests", "bilinear_rnn_amd"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "*.so", "csrc", "test_oracle_mutations.py"))
    if before is not None:
        ref = tmp_path / "oracle" / "reference.py"
        src = ref.read_text()
        assert src.count(before) == 1, f"mutation anchor not found: {before!r}"
        ref.write_text(src.replace(before, after))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-k", "numpy or chunk or fused or shared or backward", "tests/test_oracle_pins.py"],
                          cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes(tmp_path):
    r = _run_pins_on_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    r = _run_pins_on_copy(tmp_path, *MUTATIONS[name])
    # exit status 1: tests ran and at least one failed (2 would be a collection error)
    assert r.returncode == 1, f"pins did not catch '{name}':\n{r.stdout[-2000:]}"
